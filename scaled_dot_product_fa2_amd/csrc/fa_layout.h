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

// Workgroup id -> logical work id. Consecutive workgroup ids go round-robin
// to the 8 XCDs; this bijection hands each XCD a contiguous range of logical
// ids, so the query tiles that share a K/V head run on one XCD's L2.
FA_HD int64_t xcd_remap(int64_t wg, int64_t n) {
  const int64_t nx = 8;
  const int64_t per = n / nx, rem = n % nx;
  const int64_t x = wg % nx, k = wg / nx;
  return x * per + (x < rem ? x : rem) + k;
}

}  // namespace fa
