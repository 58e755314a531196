// fa_layout.h - index arithmetic shared by the gfx950 attention kernel and its
// host-side layout self-test. Everything here is plain integer math usable on
// the host and on the device; nothing touches memory.
//
// Conventions (all verified lane by lane on gfx950):
//  * v_mfma_f32_32x32x16_{f16,bf16}: lane l holds A[m = l%32][k = 8*(l/32) + e]
//    and B[k = 8*(l/32) + e][n = l%32] for e = 0..7; accumulator register r of
//    lane l is C[m = 8*(r/4) + 4*(l/32) + r%4][n = l%32], r = 0..15.
//  * ds_read_b64_tr_b16: within each group of 16 lanes, lane j receives as its
//    element e (e = 0..3) element j%4 of the 8-byte chunk addressed by lane
//    16*(j/16) + 4*e + (j%16)/4.
//  * global_load_lds (16 bytes): lane l's 16 bytes land at LDS base + 16*l.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define FA_HD __host__ __device__ __forceinline__
#else
#define FA_HD inline
#endif

namespace fa {

// ---------------------------------------------------------------------------
// LDS tile layout. A [ROWS x D] tile of 16-bit elements is stored as columns of
// row segments: segment column `seg` holds bytes [seg*SEG, (seg+1)*SEG) of every
// row, rows SEG bytes apart, columns ROWS*SEG bytes apart (SEG = 64 bytes, or
// 32 for D = 16). LDS serves 64 banks x 4 bytes, so a 256-byte line holds
// 256/SEG rows of a column and what matters for conflicts is the 16-byte slot.
//
// Row tiles (Q and K) are read 16 bytes per lane, one chunk column of 16
// consecutive rows per access phase; the 16-byte chunks inside a segment are
// XOR-swizzled with the row's line index so those rows hit 16 distinct slots.
// Transposed tiles (V) are read with ds_read_b64_tr_b16, 4 consecutive rows x
// 32 contiguous bytes per 16-lane group; 4 rows of one line already cover 16
// distinct slots, so they are stored unswizzled.
//
// Every address the kernel needs splits into a per-lane part, fixed for the
// whole kernel, plus a part known at compile time (or uniform across the
// wave), so LDS accesses use immediate offsets and copies use scalar offsets.

template <int D>
FA_HD constexpr int seg_bytes() { return D * 2 < 64 ? D * 2 : 64; }
template <int D>
FA_HD constexpr int chunks_per_seg() { return seg_bytes<D>() / 16; }
template <int D>
FA_HD constexpr int rows_per_line() { return 256 / seg_bytes<D>(); }

// Swizzle of the chunk inside a segment for row tiles.
template <int D>
FA_HD int row_swizzle(int row) { return (row / rows_per_line<D>()) % chunks_per_seg<D>(); }

// Byte offset of logical 16-byte chunk c (elements 8c .. 8c+7) of row `row`.
template <int D, int ROWS, bool TR>
FA_HD int tile_chunk_offset(int row, int c) {
  constexpr int cps = chunks_per_seg<D>();
  const int seg = c / cps, cin = c % cps;
  const int slot = TR ? cin : (cin ^ row_swizzle<D>(row));
  return seg * (ROWS * seg_bytes<D>()) + row * seg_bytes<D>() + slot * 16;
}

// Byte offset of the 8 bytes holding elements [col, col+4) of row `row` of a
// transposed tile (col a multiple of 4).
template <int D, int ROWS>
FA_HD int tile_quad_offset(int row, int col) {
  return tile_chunk_offset<D, ROWS, true>(row, col / 8) + (col % 8) * 2;
}

// ---------------------------------------------------------------------------
// Direct-to-LDS copy of a tile: 64 lanes x 16 bytes per instruction, lane l of
// instruction i landing at byte 1024*i + 16*l of the tile. Instruction i covers
// row group rg = i % IPS (64/cps consecutive rows) of segment column i / IPS.
template <int D, int ROWS>
FA_HD constexpr int dma_insts() { return ROWS * (D / 8) / 64; }

struct RowChunk {
  int row;
  int chunk;
};
template <int D, int ROWS, bool TR>
FA_HD RowChunk dma_source(int inst, int lane) {
  constexpr int cps = chunks_per_seg<D>();
  constexpr int ips = ROWS * cps / 64;
  const int seg = inst / ips, rg = inst % ips;
  const int row = rg * (64 / cps) + lane / cps;
  const int slot = lane % cps;
  const int cin = TR ? slot : (slot ^ row_swizzle<D>(row));
  return RowChunk{row, seg * cps + cin};
}
// The byte offset in global memory of dma_source(inst, lane) relative to the
// tile's first row, split as lane part + instruction part.
template <int D, bool TR>
FA_HD int64_t dma_lane_offset(int lane, int64_t row_stride_bytes) {
  constexpr int cps = chunks_per_seg<D>();
  const int slot = lane % cps;
  // row_swizzle of the lane's row depends only on lane / 16 (see dma_source)
  const int cin = TR ? slot : (slot ^ ((lane / 16) % cps));
  return (int64_t)(lane / cps) * row_stride_bytes + cin * 16;
}
template <int D, int ROWS>
FA_HD int64_t dma_inst_offset(int inst, int64_t row_stride_bytes) {
  constexpr int cps = chunks_per_seg<D>();
  constexpr int ips = ROWS * cps / 64;
  return (int64_t)((inst % ips) * (64 / cps)) * row_stride_bytes + (inst / ips) * seg_bytes<D>();
}

// ---------------------------------------------------------------------------
// MFMA operand fragments (32x32x16 shape).
// K as the A operand of S^T = K Q^T: lane reads key row (32*kb + lane%32),
// head-dim chunk 2*s + lane/32 (elements 16*s + 8*(lane/32) .. +7).
FA_HD int kfrag_row(int kb, int lane) { return 32 * kb + (lane & 31); }
FA_HD int kfrag_chunk(int s, int lane) { return 2 * s + (lane >> 5); }
// Split of that read's LDS offset: a per-lane part that depends on the slice
// only through its parity (s % kfrag_parities), plus a compile-time part.
template <int D>
FA_HD constexpr int kfrag_parities() { return chunks_per_seg<D>() / 2; }
template <int D, int ROWS>
FA_HD int kfrag_lane_offset(int parity, int lane) {
  return tile_chunk_offset<D, ROWS, false>(lane & 31, 2 * parity + (lane >> 5));
}
template <int D, int ROWS>
FA_HD int kfrag_const_offset(int kb, int s) {
  return (2 * s / chunks_per_seg<D>()) * (ROWS * seg_bytes<D>()) + 32 * kb * seg_bytes<D>();
}

// Q as the B operand: query row (32*qb + lane%32) of the wave's rows, same chunk rule.
FA_HD int qfrag_row(int qb, int lane) { return 32 * qb + (lane & 31); }

// Accumulator register r of lane `lane` sits at row 8*(r/4) + 4*(lane/32) + r%4
// of a 32x32 block (the key index for S^T, the head-dim index for O^T) and at
// column lane%32 (the query).
FA_HD int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Reduction order of the P.V product. The 16-wide key slice ks of the P^T
// operand is taken straight from the S^T accumulators, so operand position
// k = 8*(lane/32) + e holds key 16*ks + 4*(lane/32) + e%4 + 8*(e/4), which is
// accumulator register 8*(ks%2) + e of the 32-key block ks/2.
FA_HD int pv_key(int ks, int lane, int e) { return 16 * ks + 4 * (lane >> 5) + (e & 3) + 8 * (e >> 2); }
FA_HD int pv_src_reg(int ks, int e) { return 8 * (ks & 1) + e; }

// V^T as the A operand of O^T = V^T P^T, read with two ds_read_b64_tr_b16.
// Read `half` (0 or 1) of head-dim block db and key slice ks: lane `lane`
// supplies the address of V[row][col .. col+3]. For D = 16 the column is taken
// mod 16 (the lanes that would address columns 16..31 carry padding).
FA_HD int vtr_row(int ks, int half, int lane) {
  const int g = lane >> 4, i = lane & 15;
  return 16 * ks + 8 * half + 4 * (g >> 1) + (i >> 2);
}
FA_HD int vtr_col(int db, int lane) {
  const int g = lane >> 4, i = lane & 15;
  return 32 * db + 16 * (g & 1) + 4 * (i & 3);
}
template <int D>
FA_HD int vtr_col_clamped(int db, int lane) { return D < 32 ? (vtr_col(db, lane) & 15) : vtr_col(db, lane); }
// per-lane part and compile-time part of the transposed read's LDS offset
template <int D, int ROWS>
FA_HD int vtr_lane_offset(int lane) { return tile_quad_offset<D, ROWS>(vtr_row(0, 0, lane), vtr_col_clamped<D>(0, lane)); }
template <int D, int ROWS>
FA_HD int vtr_const_offset(int ks, int half, int db) {
  return (16 * ks + 8 * half) * seg_bytes<D>() + db * (ROWS * seg_bytes<D>());
}

// Transposing reads of a swizzled row tile, i.e. a tile that is read both as MFMA row fragments
// (16 bytes per lane, conflict-free only with the swizzle) and transposed (the backward's Q, dO
// and K tiles). The rows of one transposing read lie in one 256-byte line, which shares a single
// swizzle value, so the read stays conflict-free; the swizzle depends on the read's half but not on
// its key slice or head-dim block. Offset = per-lane part for the half + compile-time part.
template <int D, int ROWS>
FA_HD int vtr_swz_lane_offset(int half, int lane) {
  const int row = vtr_row(0, half, lane), col = vtr_col_clamped<D>(0, lane);
  return tile_chunk_offset<D, ROWS, false>(row, col / 8) + (col % 8) * 2;
}
template <int D, int ROWS>
FA_HD int vtr_swz_const_offset(int ks, int db) {
  return 16 * ks * seg_bytes<D>() + db * (ROWS * seg_bytes<D>());
}

// Key tiles a query tile [q0, q0 + bq) visits: all of [0, Nkv) without the mask;
// with the top-left causal mask only keys <= the tile's last row.
FA_HD int64_t kv_tiles_for_qtile(int64_t q0, int64_t bq, int64_t nkv, int64_t bkv, bool causal) {
  int64_t end = nkv;
  if (causal) {
    const int64_t last_row = q0 + bq - 1;
    if (last_row + 1 < end) end = last_row + 1;
  }
  return (end + bkv - 1) / bkv;
}

// ---------------------------------------------------------------------------
// Work schedule. An item is one (batch, query head, query tile). A "unit" is
// one (batch, key/value head) pair with its `group` query heads; all items of
// a unit read the same K/V. Workgroup ids are dealt round-robin to the 8 XCDs,
// each with its own L2, so the XCD that runs an item decides which L2 its K/V
// stream goes through.
//
// Placement. The first 8*W units (W = n_units / 8) are whole units: unit
// x + 8m belongs to XCD x, which keeps its K/V in one L2. The R = n_units % 8
// leftover units are dealt so that every XCD holds the same work to within one
// item:
//  * R = 1, 2 or 4: leftover unit r takes its own share of s = 8 / R XCDs,
//    its items (longest query tile first under the causal mask) dealt over
//    them in a snake (still one unit per L2);
//  * R = 3, 5, 6 or 7: over all eight XCDs. Under the causal mask the leftover
//    items are listed longest query tile first (then unit, then head) and
//    dealt over the XCDs in a snake; without it they are listed unit by unit
//    and XCD x takes a contiguous run of (L - x + 7) / 8 of the L items.
//
// Order of an XCD's list:
//  * causal, all of the XCD's items running at once (no more items than
//    workgroups): longest query tile first over all of them;
//  * causal, several rounds: the leftover items first (longest first), then
//    the whole units one at a time (the XCD's workgroups stream one unit's K/V
//    together, which its L2 holds), longest first within a unit and all query
//    heads of the group at each query tile;
//  * without the mask: the whole units unit by unit (head, then query tile),
//    then the leftover items.
//
// The grid holds at most a few workgroups per CU. The dispatcher deals an
// XCD's workgroups k = 0, 1, ... over its 32 CUs first (k and k + 32 share a
// CU when two are resident). Workgroup k takes position pos(k) in the XCD's
// item list in even rounds and the mirrored position in odd rounds (a snake),
// where pos() snakes over the CU-major order, so the workgroups that share a
// CU take mirrored positions: with the causal mask, where items are listed
// longest first, every CU gets a long query tile paired with a short one.
// The placement only affects balance and cache reuse, never which items are
// computed.
constexpr int kCUsPerXCD = 32;

struct Item {
  int b, h, qt;
};

struct Schedule {
  // All counts are 32-bit: the host keeps the number of items below 2^31, so every item index,
  // and an index one round of workgroups past the last item, fits (32-bit division is several
  // times cheaper than 64-bit on the GPU, and the decode runs before each item's first load).
  int n_units;  // B * Hkv
  int hkv;      // Hkv
  int group;    // Hq / Hkv
  int n_qt;     // query tiles per head
  bool causal;
  int grid;     // workgroups launched

  typedef uint32_t u32;
  FA_HD u32 whole() const { return (u32)n_units / 8; }  // whole units per XCD
  FA_HD u32 rest() const { return (u32)n_units % 8; }   // leftover units
  FA_HD u32 per_unit() const { return (u32)group * (u32)n_qt; }
  FA_HD u32 n_items() const { return (u32)n_units * per_unit(); }
  FA_HD u32 n_whole_of() const { return whole() * per_unit(); }  // whole-unit items per XCD
  // leftover units with their own XCD share (R divides 8), and the share
  FA_HD bool shared_rest() const { return rest() == 1 || rest() == 2 || rest() == 4; }
  FA_HD u32 share() const { return rest() > 0 ? 8 / rest() : 8; }

  // The leftover entries of XCD x are taken from a leftover list (one unit's items when the
  // leftover units have their own shares, else all leftover items) in a snake over its m XCDs:
  // sweep k of m consecutive entries goes to XCDs 0 .. m-1 for even k and m-1 .. 0 for odd k, so no
  // XCD always receives the longer item of a sweep. The entries of XCD-in-share a are therefore
  // 2m*k + a and 2m*k + 2m-1-a (k = 0, 1, ...). m is 8 / R (shared) or 8, a power of two.
  FA_HD u32 lo_shift() const { return !shared_rest() ? 3 : rest() == 1 ? 3 : rest() == 2 ? 2 : 1; }
  FA_HD u32 lo_a(int x) const { return shared_rest() ? (u32)x % share() : (u32)x; }
  FA_HD u32 lo_len() const { return shared_rest() ? per_unit() : rest() * per_unit(); }
  // entries e < n of XCD x's sequence
  FA_HD u32 lo_count_below(int x, u32 n) const {
    const u32 a = lo_a(x), period = 2u << lo_shift();
    const u32 q = n >> (lo_shift() + 1), r = n & (period - 1);
    return 2 * q + (r > a ? 1 : 0) + (r > period - 1 - a ? 1 : 0);
  }
  // entry number k of XCD x's sequence
  FA_HD u32 lo_entry(int x, u32 k) const {
    const u32 a = lo_a(x), period = 2u << lo_shift();
    return (k >> 1) * period + ((k & 1) ? period - 1 - a : a);
  }
  // leftover items of XCD x
  FA_HD u32 left_of(int x) const {
    if (rest() == 0) return 0;
    if (!causal && !shared_rest()) {  // a contiguous run
      const u32 L = lo_len();
      return L > (u32)x ? (L - (u32)x + 7) / 8 : 0;
    }
    return lo_count_below(x, lo_len());
  }
  // number of items of XCD x
  FA_HD u32 items_of(int x) const { return n_whole_of() + left_of(x); }
  // one more than the highest XCD that receives items (the grid must reach it)
  FA_HD int xcds_used() const {
    for (int x = 7; x > 0; --x)
      if (items_of(x) > 0) return x + 1;
    return 1;
  }
  // workgroups of XCD x
  FA_HD int wgs_of(int x) const { return x < grid ? (grid - x + 7) / 8 : 0; }
  // grid for at most `max_grid` workgroups: no more than there are items, but at least one
  // workgroup on every XCD that has items
  FA_HD int choose_grid(int64_t max_grid) const {
    int64_t g = max_grid < (int64_t)n_items() ? max_grid : (int64_t)n_items();
    if (g < xcds_used()) g = xcds_used();
    return (int)g;
  }
  // does XCD x hold no more items than workgroups, so that all of them run at once?
  FA_HD bool one_round(int x) const { return items_of(x) <= (u32)wgs_of(x); }

  FA_HD Item make(u32 unit, u32 g, u32 t) const {
    Item it;
    it.b = (int)(unit / (u32)hkv);
    it.h = (int)((unit % (u32)hkv) * (u32)group + g);
    it.qt = causal ? n_qt - 1 - (int)t : (int)t;  // t is the rank (longest first) under the causal mask
    return it;
  }
  // entry e of the leftover list of XCD x's sequence
  FA_HD Item left_item(int x, u32 e) const {
    const u32 base = 8 * whole();
    if (shared_rest()) {
      const u32 unit = base + (u32)x / share();
      return causal ? make(unit, e % (u32)group, e / (u32)group) : make(unit, e / (u32)n_qt, e % (u32)n_qt);
    }
    if (causal) {
      const u32 per_rank = rest() * (u32)group;
      const u32 r = e % per_rank;
      return make(base + r / (u32)group, r % (u32)group, e / per_rank);
    }
    const u32 r = e % per_unit();
    return make(base + e / per_unit(), r / (u32)n_qt, r % (u32)n_qt);
  }
  // whole-unit item i of XCD x (0 <= i < n_whole_of()), unit by unit
  FA_HD Item whole_item(int x, u32 i) const {
    const u32 m = i / per_unit(), r = i % per_unit();
    const u32 unit = (u32)x + 8 * m;
    return causal ? make(unit, r % (u32)group, r / (u32)group) : make(unit, r / (u32)n_qt, r % (u32)n_qt);
  }
  // causal: items of XCD x whose rank is below t (the whole units' and the leftover ones)
  FA_HD u32 rank_prefix(int x, u32 t) const {
    const u32 per_rank = shared_rest() ? (u32)group : rest() * (u32)group;
    return t * whole() * (u32)group + (rest() ? lo_count_below(x, t * per_rank) : 0);
  }
  // item number i of XCD x (0 <= i < items_of(x))
  FA_HD Item item(int x, u32 i) const {
    const u32 nw = n_whole_of();
    if (!causal) {
      if (i < nw) return whole_item(x, i);
      const u32 k = i - nw;
      if (shared_rest()) return left_item(x, lo_entry(x, k));
      const u32 L = lo_len();
      return left_item(x, (u32)x * (L / 8) + ((u32)x < L % 8 ? (u32)x : L % 8) + k);  // x's contiguous run
    }
    if (one_round(x)) {
      // longest first over all of the XCD's items: the rank is the largest t with rank_prefix <= i
      u32 lo = 0, hi = (u32)n_qt - 1;
      while (lo < hi) {
        const u32 mid = lo + (hi - lo + 1) / 2;
        if (rank_prefix(x, mid) <= i)
          lo = mid;
        else
          hi = mid - 1;
      }
      const u32 off = i - rank_prefix(x, lo);
      const u32 wg = whole() * (u32)group;
      if (off < wg) return make((u32)x + 8 * (off / (u32)group), off % (u32)group, lo);
      const u32 per_rank = shared_rest() ? (u32)group : rest() * (u32)group;
      const u32 k = lo_count_below(x, lo * per_rank) + (off - wg);
      return left_item(x, lo_entry(x, k));
    }
    const u32 nl = left_of(x);
    if (i < nl) return left_item(x, lo_entry(x, i));
    return whole_item(x, i - nl);
  }
  // position of the XCD's k-th workgroup among its gx workgroups (a bijection of [0, gx))
  FA_HD static int cu_snake(int k, int gx) {
    const int full = gx / kCUsPerXCD * kCUsPerXCD;  // workgroups in complete CU rounds
    if (k >= full) return k;
    const int s = k / kCUsPerXCD, c = k % kCUsPerXCD;
    return s * kCUsPerXCD + ((s & 1) ? kCUsPerXCD - 1 - c : c);
  }
  // index into the XCD's item list of workgroup `wg` in round r (may be >= items_of, by less than
  // one round of workgroups)
  FA_HD u32 item_index(int wg, u32 r) const {
    const int x = wg % 8, k = wg / 8, gx = wgs_of(x);
    const int pos = cu_snake(k, gx);
    return r * (u32)gx + (u32)((r & 1) ? (gx - 1 - pos) : pos);
  }
};

}  // namespace fa
