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
// a unit read the same K/V, so they are kept on one XCD (workgroup ids are
// dealt round-robin to the 8 XCDs, each with its own L2). With fewer than 8
// units, each unit's items are spread over 8 / n_units XCDs.
//
// The grid holds at most a few workgroups per CU. The dispatcher deals an
// XCD's workgroups k = 0, 1, ... over its 32 CUs first (k and k + 32 share a
// CU when two are resident). Workgroup k takes position pos(k) in the XCD's
// item list in even rounds and the mirrored position in odd rounds (a snake),
// where pos() snakes over the CU-major order, so the workgroups that share a
// CU take mirrored positions, so with the causal mask, where items are listed
// longest first, every CU gets a long query tile paired with a short one.
// Items are listed unit by unit, longest first within a unit, so that the XCD
// streams one unit's K/V at a time; when all of an XCD's items run at once
// (no more items than workgroups) the causal items are instead listed longest
// first across the XCD's units.
// The placement only affects balance, never which items are computed.
constexpr int kCUsPerXCD = 32;

struct Item {
  int b, h, qt;
};

struct Schedule {
  int n_units;  // B * Hkv
  int hkv;      // Hkv
  int group;    // Hq / Hkv
  int n_qt;     // query tiles per head
  bool causal;
  int grid;     // workgroups launched

  FA_HD int xcd_share() const { return n_units >= 8 ? 1 : 8 / n_units; }
  // XCDs that receive items
  FA_HD int xcds_used() const { return n_units >= 8 ? 8 : n_units * xcd_share(); }
  // number of items of XCD x
  FA_HD int64_t items_of(int x) const {
    if (x >= xcds_used()) return 0;
    const int64_t per_unit = (int64_t)group * n_qt;
    if (n_units >= 8) {
      const int64_t units_x = (n_units - x + 7) / 8;
      return units_x * per_unit;
    }
    const int s = xcd_share(), sub = x % s;
    return (per_unit - sub + s - 1) / s;
  }
  // workgroups of XCD x
  FA_HD int wgs_of(int x) const { return x < grid ? (grid - x + 7) / 8 : 0; }
  // grid for at most `max_grid` workgroups: no more than there are items, but at least one
  // workgroup on every XCD that has items
  FA_HD int choose_grid(int64_t max_grid) const {
    const int64_t n_items = (int64_t)n_units * group * n_qt;
    int64_t g = max_grid < n_items ? max_grid : n_items;
    if (g < xcds_used()) g = xcds_used();
    return (int)g;
  }
  // does XCD x hold no more items than workgroups, so that all of them run at once?
  FA_HD bool one_round(int x) const { return items_of(x) <= wgs_of(x); }
  // item number i of XCD x (0 <= i < items_of(x))
  FA_HD Item item(int x, int64_t i) const {
    int unit, g, rank;  // rank: position of the query tile in the order items are listed
    if (n_units >= 8) {
      const int units_x = (n_units - x + 7) / 8;
      int64_t m;
      if (causal && one_round(x)) {
        // every item of the XCD runs at once: the longest query tiles first across its units
        rank = (int)(i / ((int64_t)units_x * group));
        const int64_t rest = i % ((int64_t)units_x * group);
        m = rest / group;
        g = (int)(rest % group);
      } else if (causal) {
        // unit by unit (the XCD's workgroups stream one unit's K/V together, which its L2 holds),
        // and within a unit the longest query tiles first, all query heads of the group at each
        m = i / ((int64_t)group * n_qt);
        const int64_t rest = i % ((int64_t)group * n_qt);
        rank = (int)(rest / group);
        g = (int)(rest % group);
      } else {
        m = i / ((int64_t)group * n_qt);
        const int64_t rest = i % ((int64_t)group * n_qt);
        g = (int)(rest / n_qt);
        rank = (int)(rest % n_qt);
      }
      unit = x + 8 * (int)m;
    } else {
      const int s = xcd_share();
      unit = x / s;
      const int64_t f = x % s + i * s;
      if (causal) {
        rank = (int)(f / group);
        g = (int)(f % group);
      } else {
        g = (int)(f / n_qt);
        rank = (int)(f % n_qt);
      }
    }
    Item it;
    it.b = unit / hkv;
    it.h = (unit % hkv) * group + g;
    it.qt = causal ? n_qt - 1 - rank : rank;
    return it;
  }
  // position of the XCD's k-th workgroup among its gx workgroups (a bijection of [0, gx))
  FA_HD static int cu_snake(int k, int gx) {
    const int full = gx / kCUsPerXCD * kCUsPerXCD;  // workgroups in complete CU rounds
    if (k >= full) return k;
    const int s = k / kCUsPerXCD, c = k % kCUsPerXCD;
    return s * kCUsPerXCD + ((s & 1) ? kCUsPerXCD - 1 - c : c);
  }
  // index into the XCD's item list of workgroup `wg` in round r (may be >= items_of)
  FA_HD int64_t item_index(int wg, int64_t r) const {
    const int x = wg % 8, k = wg / 8, gx = wgs_of(x);
    const int pos = cu_snake(k, gx);
    return r * gx + ((r & 1) ? (gx - 1 - pos) : pos);
  }
};

}  // namespace fa
