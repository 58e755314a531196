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

// 16-byte chunks per tile row of D 16-bit elements.
template <int D>
FA_HD constexpr int chunks_per_row() { return D / 8; }

// XOR swizzle of the chunk index within a row: 16 consecutive rows spread over
// the 16 chunk slots of a 256-byte LDS line, so the 16 lanes that one LDS
// access phase serves never collide on a bank.
template <int D>
FA_HD int chunk_swizzle(int row) {
  constexpr int cpr = chunks_per_row<D>();
  constexpr int rows_per_line = cpr >= 16 ? 1 : 16 / cpr;
  constexpr int slots = cpr >= 16 ? 16 : cpr;
  return (row / rows_per_line) % slots;
}

// Byte offset of 16-byte chunk c of row `row` inside a tile stored in LDS.
template <int D>
FA_HD int tile_chunk_offset(int row, int c) {
  return (row * chunks_per_row<D>() + (c ^ chunk_swizzle<D>(row))) * 16;
}

// Byte offset of the 8-byte group holding elements [col, col+4) of row `row`
// (col a multiple of 4).
template <int D>
FA_HD int tile_quad_offset(int row, int col) {
  return tile_chunk_offset<D>(row, col / 8) + (col % 8) * 2;
}

// Direct-to-LDS copy of a tile: instruction `inst` of the copy, lane `lane`.
// Slot p = 64*inst + lane of the LDS tile holds (row, logical chunk).
struct RowChunk {
  int row;
  int chunk;
};
template <int D>
FA_HD RowChunk dma_source(int inst, int lane) {
  constexpr int cpr = chunks_per_row<D>();
  const int p = inst * 64 + lane;
  const int row = p / cpr;
  const int slot = p % cpr;
  return RowChunk{row, slot ^ chunk_swizzle<D>(row)};
}

// MFMA operand fragments (32x32x16 shape).
// K as the A operand of S^T = K Q^T: lane reads key row (32*kb + lane%32),
// head-dim chunk 2*s + lane/32 (elements 16*s + 8*(lane/32) .. +7).
FA_HD int kfrag_row(int kb, int lane) { return 32 * kb + (lane & 31); }
FA_HD int kfrag_chunk(int s, int lane) { return 2 * s + (lane >> 5); }

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
// supplies the address of V[row][col .. col+3].
FA_HD int vtr_row(int ks, int half, int lane) {
  const int g = lane >> 4, i = lane & 15;
  return 16 * ks + 8 * half + 4 * (g >> 1) + (i >> 2);
}
FA_HD int vtr_col(int db, int lane) {
  const int g = lane >> 4, i = lane & 15;
  return 32 * db + 16 * (g & 1) + 4 * (i & 3);
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
