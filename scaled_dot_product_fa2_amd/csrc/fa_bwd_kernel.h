// fa_bwd_kernel.h - gfx950 (CDNA4) attention backward: dQ, dK, dV.
//
// The gradients follow the backward of the Ascend notes ("FlashAttention on
// Ascend: Triton-Ascend CV pipeline", section 2): Delta = rowsum(O * dO), the
// probabilities recomputed from the saved logsumexp, dP = dO V^T,
// dS = scale * P * (dP - Delta), dQ = dS K, dK = dS^T Q, dV = P^T dO.
// Following the principle the notes settle on (section 2: every gradient tile
// written once, no atomics and no cross-program reduction), the work is split
// by owner:
//  * fa_bwd_delta_kernel: Delta per query row, fp32, from the 16-bit O and dO;
//  * fa_bwd_dkdv_kernel: one workgroup per (batch, kv head, 32*NW keys). Each
//    wave keeps its 32 keys' K and V rows in VGPRs as MFMA operands and streams
//    the Q and dO tiles of every query head of the group past them, so dK and dV
//    accumulate in registers and are written once (grouped heads summed there);
//  * fa_bwd_dq_kernel: one workgroup per (batch, query head, 32*NW rows), the
//    forward's structure with dO next to Q in VGPRs, streaming K and V tiles;
//    dQ accumulates in registers and is written once.
// S and dP are recomputed in both gradient kernels (two extra products against
// a scheme with atomic dQ updates) in exchange for deterministic results.
// WINDOW and VARLEN instances of both gradient kernels mirror the forward's:
// only the band's tiles are visited, or each packed sequence is addressed
// through its cu_seqlens offsets with its own lengths.
//
// MI355X mapping (32x32x16 MFMAs, fp32 accumulate; P and dS rounded to the
// input dtype before they enter an MFMA, like P in the forward):
//  * dK/dV kernel: S = Q K^T and dP = dO V^T with Q/dO fragments read from LDS
//    and K/V fragments in VGPRs, so each lane owns one key and holds 16 query
//    rows; then dV^T += dO^T P and dK^T += Q^T dS take P and dS straight from
//    those accumulators (the query order of the reduction permuted as the key
//    order is in the forward's P.V product) against transposing LDS reads of
//    the dO and Q tiles.
//  * dQ kernel: S^T = K Q^T and dP^T = V dO^T (each lane owns one query row, as
//    in the forward), then dQ^T += K^T dS^T with transposing reads of the K tile.
#pragma once

#include <type_traits>

#include "fa_fwd_kernel.h"

namespace fa {

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;  // natural-log logsumexp of the forward, row i of (b, h) at b*lse_sb + h*lse_sh + i
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // workspace, laid out like lse
  int64_t q_sb, q_sh, q_sn;  // element strides; the head-dim stride is 1
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t o_sb, o_sh, o_sn;
  int64_t do_sb, do_sh, do_sn;
  int64_t dq_sb, dq_sh, dq_sn;
  int64_t dk_sb, dk_sh, dk_sn;
  int64_t dv_sb, dv_sh, dv_sn;
  int32_t B, Hq, Hkv, Nq, Nkv;
  int32_t group;  // Hq / Hkv
  float c;        // scale * log2(e)
  float scale;
  // order of the 1-D gradient grids: nonzero = row block slowest (longest first under the causal
  // mask; L2 sharing between the blocks of a head when the grid is about one wave of workgroups)
  int32_t dkdv_block_slowest, dq_block_slowest;
  // sliding window (the WINDOW instances only): row i sees keys i - win_left .. i + win_right
  int32_t win_left, win_right;
  // packed variable-length sequences (the VARLEN instances only): sequence b owns tokens
  // cu_q[b] .. cu_q[b+1]-1 of Q/O/dO/dQ and cu_k[b] .. cu_k[b+1]-1 of K/V/dK/dV; Nq and Nkv hold the
  // longest lengths, the batch strides are 0
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t total_q, total_k;
  int64_t lse_sb, lse_sh;  // element offsets of (b, h) in lse and delta; the row index is added
};

// Lengths and first tokens of sequence b: the dense lengths, or those of the packed sequence read
// from the offsets, clamped to the token counts so that no offset array can address out of bounds.
struct SeqSpan {
  int nq, nkv, q_tok0, k_tok0;
};
template <bool VARLEN>
__device__ __forceinline__ SeqSpan seq_span(const BwdParams& p, int b) {
  if (!VARLEN) return SeqSpan{p.Nq, p.Nkv, 0, 0};
  const int cq0 = min(max(p.cu_q[b], 0), p.total_q), cq1 = min(max(p.cu_q[b + 1], cq0), p.total_q);
  const int ck0 = min(max(p.cu_k[b], 0), p.total_k), ck1 = min(max(p.cu_k[b + 1], ck0), p.total_k);
  return SeqSpan{min(cq1 - cq0, p.Nq), min(ck1 - ck0, p.Nkv), cq0, ck0};
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) f32x4 lds_f32x4_t;

constexpr float kLog2e = 1.44269504088896340736f;

// Fragment read-ahead of the gradient kernels, in fragments (as in the forward's loops).
constexpr int kBwdLead = 3;
// The transposed reads of the dK/dV form with K and V in LDS, which holds its partial dK and dV at
// two waves per SIMD and has registers for less read-ahead.
constexpr int kBwdLeadKvl = 2;
// The dQ kernel's score loop at D >= 128 under a mask holds the mask's row bounds as well; one
// fragment less read-ahead there keeps it inside the register file.
constexpr int kBwdDqMaskedLead = 2;

// Delta_i = sum_d O_id * dO_id for every (batch, head, row), fp32. D/8 lanes per row, one
// 16-byte vector of O and of dO per lane, then a butterfly sum over those lanes.
template <typename T, int D>
__global__ void __launch_bounds__(256) fa_bwd_delta_kernel(const BwdParams p) {
  constexpr int LPR = D / 8;          // lanes per row
  constexpr int RPB = 256 / LPR;      // rows per workgroup
  typedef typename Elem<T>::vec8 vec8;
  const int tid = threadIdx.x;
  const int64_t g = (int64_t)blockIdx.x * RPB + tid / LPR;  // row over (B, Hq, Nq)
  const int64_t total = (int64_t)p.B * p.Hq * p.Nq;
  float acc = 0.f;
  if (g < total) {
    const int i = (int)(g % p.Nq);
    const int64_t bh = g / p.Nq;
    const int h = (int)(bh % p.Hq), b = (int)(bh / p.Hq);
    const int col = 8 * (tid % LPR);
    const vec8 o = *(const vec8*)((const T*)p.o + b * p.o_sb + h * p.o_sh + i * p.o_sn + col);
    const vec8 d = *(const vec8*)((const T*)p.dout + b * p.do_sb + h * p.do_sh + i * p.do_sn + col);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)o[e], (float)d[e], acc);
  }
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) acc += __shfl_xor(acc, m, LPR);
  if (g < total && tid % LPR == 0) p.delta[g] = acc;
}

// Workgroup shape of the gradient kernels: NW waves of 32 rows each (keys for dK/dV, query rows
// for dQ), tiles of BT rows streamed past them (query rows for dK/dV, keys for dQ). In the KVL form
// of dK/dV, NW/2 groups of 32 keys with two waves each, one per 32-row half of every tile.
template <int D_, int NW_, int BT_, int WAVES_PER_SIMD_, bool KVL_ = false>
struct BwdCfg {
  static constexpr int D = D_;
  static constexpr int NW = NW_;
  static constexpr int BT = BT_;
  static constexpr int WAVES_PER_SIMD = WAVES_PER_SIMD_;
  // dK/dV only: K and V of the workgroup's keys staged in LDS instead of each wave's registers,
  // and two waves per 32-key group, each taking one 32-row half of every query tile
  static constexpr bool KVL = KVL_;
  static constexpr int NKG = KVL ? NW / 2 : NW;  // 32-row groups the workgroup owns
  static constexpr int THREADS = NW * 64;
  static constexpr int BW = NKG * 32;  // rows owned by the workgroup
  static constexpr int TILE_BYTES = BT * D * 2;
  static_assert(BT % 32 == 0 && dma_insts<D, BT>() * 64 == BT * (D / 8), "tile rows must fill whole copies");
};

// ------------------------------------------------------------------------------------------------
// dK, dV. Grid: ceil(Nkv / BW) * Hkv * B workgroups (1-D). PART selects the outputs: kBwdBoth, or one of
// kBwdOnlyV / kBwdOnlyK (two launches, S recomputed in each, to fit wide heads in registers).
constexpr int kBwdBoth = 0, kBwdOnlyV = 1, kBwdOnlyK = 2;

template <typename T, bool CAUSAL, class Cfg, int PART, bool WINDOW = false, bool VARLEN = false>
__global__ void __launch_bounds__(Cfg::THREADS)
    __attribute__((amdgpu_waves_per_eu(Cfg::WAVES_PER_SIMD, Cfg::WAVES_PER_SIMD)))
    fa_bwd_dkdv_kernel(const BwdParams p) {
  constexpr int D = Cfg::D, NW = Cfg::NW, BQ = Cfg::BT, BK = Cfg::BW;
  constexpr bool DO_V = PART != kBwdOnlyK, DO_K = PART != kBwdOnlyV;
  constexpr int NS = D / 16;
  constexpr bool DPAD = D < 32;
  constexpr int NDB = DPAD ? 1 : D / 32;
  constexpr int NQB = BQ / 32;  // 32-row query blocks per tile
  constexpr int TB = Cfg::TILE_BYTES;
  constexpr bool KVL = Cfg::KVL;
  constexpr int NKG = Cfg::NKG;
  static_assert(!KVL || (PART == kBwdBoth && NW == 2 * NKG && NQB == 2), "K/V in LDS: both outputs, two row halves");
  typedef typename Elem<T>::vec8 vec8;

  // Q and dO tiles in the transposing layout (read both as row fragments and transposed), two
  // stages each, plus the tile's logsumexp and Delta.
  __shared__ __attribute__((aligned(1024))) char q_st0_raw[TB];
  __shared__ __attribute__((aligned(1024))) char q_st1_raw[TB];
  __shared__ __attribute__((aligned(1024))) char o_st0_raw[TB];
  __shared__ __attribute__((aligned(1024))) char o_st1_raw[TB];
  __shared__ __attribute__((aligned(256))) float ls_st0[BQ];
  __shared__ __attribute__((aligned(256))) float ls_st1[BQ];
  __shared__ __attribute__((aligned(256))) float dl_st0[BQ];
  __shared__ __attribute__((aligned(256))) float dl_st1[BQ];
  // K and V rows of the workgroup's keys (the KVL form; a stub otherwise)
  constexpr int KVB = KVL ? BK * D * 2 : 16;
  __shared__ __attribute__((aligned(1024))) char k_lds_raw[KVB];
  __shared__ __attribute__((aligned(1024))) char v_lds_raw[KVB];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int kg = KVL ? wave % NKG : wave;  // 32-key group of this wave
  const int rh = KVL ? wave / NKG : 0;     // (KVL) the 32-row half of each query tile it takes
  // 1-D grid over (key block, kv head, batch). Key block slowest: under the causal mask the early
  // key blocks, which see the most query tiles, are dispatched first (longest first). Key block
  // fastest: the key blocks of one head are dispatched together and share its Q/dO stream in cache.
  const int64_t lin = blockIdx.x;
  const int n_kb = (p.Nkv + BK - 1) / BK;
  int kvh, b, k0;
  if (p.dkdv_block_slowest) {
    const int64_t per_kb = (int64_t)p.Hkv * p.B;
    kvh = (int)(lin % p.Hkv);
    b = (int)((lin % per_kb) / p.Hkv);
    k0 = (int)(lin / per_kb) * BK;
  } else {
    const int64_t rest = lin / n_kb;
    k0 = (int)(lin % n_kb) * BK;
    kvh = (int)(rest % p.Hkv);
    b = (int)(rest / p.Hkv);
  }
  const SeqSpan sq = seq_span<VARLEN>(p, b);
  const int nq = sq.nq, nkv = sq.nkv;
  if (VARLEN && k0 >= nkv) return;  // a key block past this sequence's end (workgroup-uniform)
  const int kw0 = k0 + 32 * kg;  // first key of this wave
  const int my_key = kw0 + (lane & 31);

  // K and V rows of the wave's keys as B operands: lane holds row (lane % 32), elements
  // 16*s + 8*(lane/32) .. +7. Keys past the sequence read as zero.
  vec8 kf[NS], vf[NS];
  if constexpr (!KVL) {
    const T* krow = (const T*)p.k + b * p.k_sb + kvh * p.k_sh + (int64_t)(sq.k_tok0 + my_key) * p.k_sn;
    const T* vrow = (const T*)p.v + b * p.v_sb + kvh * p.v_sh + (int64_t)(sq.k_tok0 + my_key) * p.v_sn;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int col = 16 * s + 8 * (lane >> 5);
      kf[s] = my_key < nkv ? *(const vec8*)(krow + col) : vec8{};
      if (DO_K) vf[s] = my_key < nkv ? *(const vec8*)(vrow + col) : vec8{};
    }
  }
  f32x16 dkT[NDB], dvT[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dkT[db] = f32x16{};
    dvT[db] = f32x16{};
  }

  // Work list: (query head of the group, query tile), tiles that can see one of the keys only.
  const int n_qt = (nq + BQ - 1) / BQ;
  int qt0 = CAUSAL ? (k0 / BQ < n_qt ? k0 / BQ : n_qt) : 0, qt_end = n_qt;
  if (WINDOW) {
    // rows that see one of the workgroup's keys: key - win_right <= row <= key + win_left
    const int first = max(0, k0 - p.win_right);
    const int last = min(nq - 1, k0 + BK - 1 + p.win_left);
    qt0 = min(first / BQ, n_qt);
    qt_end = first > last ? qt0 : last / BQ + 1;
  }
  const int per_head = qt_end - qt0;
  const int n_work = p.group * per_head;
  const int q_stride = (int)(p.q_sn * 2), o_stride = (int)(p.do_sn * 2);
  const int q_dma_off = (int)dma_lane_offset<D, false>(lane, q_stride);
  const int o_dma_off = (int)dma_lane_offset<D, false>(lane, o_stride);

  auto issue = [&](int w, lds_char_t* qt, lds_char_t* ot, float* ls, float* dl) {
    const int h = kvh * p.group + w / per_head;
    const int q0 = (qt0 + w % per_head) * BQ;
    const char* qbase = (const char*)p.q + (b * p.q_sb + h * p.q_sh + (int64_t)sq.q_tok0 * p.q_sn) * 2;
    const char* obase = (const char*)p.dout + (b * p.do_sb + h * p.do_sh + (int64_t)sq.q_tok0 * p.do_sn) * 2;
    dma_tile<D, BQ, NW>(qt, qbase, q_stride, q0, nq, wave_u, q_dma_off);
    dma_tile<D, BQ, NW>(ot, obase, o_stride, q0, nq, wave_u, o_dma_off);
    // logsumexp and Delta of the tile's rows: 4 bytes per lane, rows past the sequence read as zero
    const int64_t row0 = b * p.lse_sb + h * p.lse_sh + sq.q_tok0 + q0;
    const int valid = nq - q0 < BQ ? nq - q0 : BQ;
#pragma unroll
    for (int part = 0; part < BQ / 64; ++part) {
      if (wave_u == (2 * part) % NW) {
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(p.lse + row0 + 64 * part), (short)0, (int)(4 * (valid - 64 * part > 0 ? valid - 64 * part : 0)),
            0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(ls + 64 * part), 4, 4 * lane, 0, 0, 0);
      }
      if (wave_u == (2 * part + 1) % NW) {
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(p.delta + row0 + 64 * part), (short)0,
            (int)(4 * (valid - 64 * part > 0 ? valid - 64 * part : 0)), 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(dl + 64 * part), 4, 4 * lane, 0, 0, 0);
      }
    }
  };

  // per-lane parts of the tile reads. The Q and dO tiles are read as row fragments and transposed;
  // both kinds of read are free of bank conflicts on the swizzled layout (fa_layout.h).
  constexpr int KP = kfrag_parities<D>();
  int q_lane[KP];
#pragma unroll
  for (int par = 0; par < KP; ++par) q_lane[par] = kfrag_lane_offset<D, BQ>(par, lane);
  const int t_lane[2] = {vtr_swz_lane_offset<D, BQ>(0, lane), vtr_swz_lane_offset<D, BQ>(1, lane)};
  const float c = p.c;

  // KVL: the workgroup's K and V rows, copied once with the first query tile and read as the same
  // B-operand fragments the register form holds
  const lds_char_t* const k_lds = (const lds_char_t*)k_lds_raw;
  const lds_char_t* const v_lds = (const lds_char_t*)v_lds_raw;
  int kv_lane[KP];
#pragma unroll
  for (int par = 0; par < KP; ++par) kv_lane[par] = KVL ? kfrag_lane_offset<D, BK>(par, lane) : 0;
  if (KVL && n_work > 0) {
    const int k_stride = (int)(p.k_sn * 2), v_stride = (int)(p.v_sn * 2);
    const char* kbase = (const char*)p.k + (b * p.k_sb + kvh * p.k_sh + (int64_t)sq.k_tok0 * p.k_sn) * 2;
    const char* vbase = (const char*)p.v + (b * p.v_sb + kvh * p.v_sh + (int64_t)sq.k_tok0 * p.v_sn) * 2;
    dma_tile<D, BK, NW>((lds_char_t*)k_lds_raw, kbase, k_stride, k0, nkv, wave_u,
                        (int)dma_lane_offset<D, false>(lane, k_stride));
    dma_tile<D, BK, NW>((lds_char_t*)v_lds_raw, vbase, v_stride, k0, nkv, wave_u,
                        (int)dma_lane_offset<D, false>(lane, v_stride));
  }

  auto step = [&](auto stage_c, int w) {
    constexpr int S = decltype(stage_c)::value;
    lds_char_t* const qt = (lds_char_t*)(S == 0 ? q_st0_raw : q_st1_raw);
    lds_char_t* const ot = (lds_char_t*)(S == 0 ? o_st0_raw : o_st1_raw);
    const float* const ls = S == 0 ? ls_st0 : ls_st1;
    const float* const dl = S == 0 ? dl_st0 : dl_st1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (w + 1 < n_work) {
      if (S == 0)
        issue(w + 1, (lds_char_t*)q_st1_raw, (lds_char_t*)o_st1_raw, ls_st1, dl_st1);
      else
        issue(w + 1, (lds_char_t*)q_st0_raw, (lds_char_t*)o_st0_raw, ls_st0, dl_st0);
    }
    const int q0 = (qt0 + w % per_head) * BQ;
#pragma unroll
    for (int qi = 0; qi < (KVL ? 1 : NQB); ++qi) {
      const int qb = KVL ? rh : qi;
      const int qrow0 = q0 + 32 * qb;
      // every query row of the block is before the wave's first key: nothing visible
      if (CAUSAL && qrow0 + 31 < kw0) continue;
      // with a window: the block's rows are all outside every key's window
      if (WINDOW && (qrow0 + 31 < kw0 - p.win_right || qrow0 > kw0 + 31 + p.win_left)) continue;
      if (qrow0 >= nq) continue;
      f32x16 s_acc = f32x16{}, dp_acc = f32x16{};
      {
        vec8 qa[NS], oa[NS], ka[NS], va[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const int off = q_lane[s % KP] + kfrag_const_offset<D, BQ>(qb, s);
          qa[s] = __builtin_bit_cast(vec8, lds_read16(qt + off));
          if (DO_K) oa[s] = __builtin_bit_cast(vec8, lds_read16(ot + off));
          if (KVL) {
            const int koff = kv_lane[s % KP] + kfrag_const_offset<D, BK>(kg, s);
            ka[s] = __builtin_bit_cast(vec8, lds_read16(k_lds + koff));
            va[s] = __builtin_bit_cast(vec8, lds_read16(v_lds + koff));
          }
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          s_acc = Elem<T>::mfma(qa[s], KVL ? ka[s] : kf[s], s_acc);
          if (DO_K) dp_acc = Elem<T>::mfma(oa[s], KVL ? va[s] : vf[s], dp_acc);
        }
        // Pinned read-ahead. The KVL form, which reads K and V fragments here as well, is left to
        // the compiler's pressure-aware placement: pinned, its reads are all hoisted ahead of the
        // first MFMA and spill.
        if constexpr (!KVL) {
          constexpr int PER = DO_K ? 2 : 1;
          constexpr int LEAD = kBwdLead < NS ? kBwdLead : NS;
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, PER * LEAD, 0);
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, PER, 0);
            if (s + LEAD < NS) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, PER, 0);
          }
        }
      }
      // register r holds query row qrow0 + acc_row(r, lane) against the lane's key; registers
      // 4g .. 4g+3 are four consecutive rows, so their logsumexp and Delta are one 16-byte read
      vec8 pf[2], sf[2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int m0 = 8 * g + 4 * (lane >> 5);
        const float4 l4 = *(const float4*)(ls + 32 * qb + m0);
        const float4 d4 = DO_K ? *(const float4*)(dl + 32 * qb + m0) : float4{};
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s_acc[r], c, -lv[e] * kLog2e));
          if (CAUSAL && my_key > qrow0 + m0 + e) pv = 0.f;
          if (WINDOW && (my_key > qrow0 + m0 + e + p.win_right || my_key < qrow0 + m0 + e - p.win_left)) pv = 0.f;
          const float ds = pv * (dp_acc[r] - dv4[e]);
          pf[r >> 3][r & 7] = (T)pv;
          sf[r >> 3][r & 7] = (T)ds;
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS over the block's 32 query rows (two 16-row slices)
      {
        vec8 oT[2][NDB], qT[2][NDB];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            i16x4 olo{}, ohi{}, qlo{}, qhi{};
            if (DO_V) {
              olo = lds_read_tr(ot + t_lane[0] + vtr_swz_const_offset<D, BQ>(2 * qb + ks, db));
              ohi = lds_read_tr(ot + t_lane[1] + vtr_swz_const_offset<D, BQ>(2 * qb + ks, db));
            }
            if (DO_K) {
              qlo = lds_read_tr(qt + t_lane[0] + vtr_swz_const_offset<D, BQ>(2 * qb + ks, db));
              qhi = lds_read_tr(qt + t_lane[1] + vtr_swz_const_offset<D, BQ>(2 * qb + ks, db));
            }
            if (DPAD && ((lane >> 4) & 1)) {
              olo = i16x4{};
              ohi = i16x4{};
              qlo = i16x4{};
              qhi = i16x4{};
            }
            oT[ks][db] = __builtin_bit_cast(vec8, __builtin_shufflevector(olo, ohi, 0, 1, 2, 3, 4, 5, 6, 7));
            qT[ks][db] = __builtin_bit_cast(vec8, __builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7));
          }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            if (DO_V) dvT[db] = Elem<T>::mfma(oT[ks][db], pf[ks], dvT[db]);
            if (DO_K) dkT[db] = Elem<T>::mfma(qT[ks][db], sf[ks], dkT[db]);
          }
        constexpr int PER = (DO_V ? 1 : 0) + (DO_K ? 1 : 0);
        constexpr int NF = 2 * NDB;
        constexpr int LEAD = (KVL ? kBwdLeadKvl : kBwdLead) < NF ? (KVL ? kBwdLeadKvl : kBwdLead) : NF;
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * PER * LEAD, 0);
#pragma unroll
        for (int i = 0; i < NF; ++i) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, PER, 0);
          if (i + LEAD < NF) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * PER, 0);
        }
      }
    }
  };

  if (n_work > 0) issue(0, (lds_char_t*)q_st0_raw, (lds_char_t*)o_st0_raw, ls_st0, dl_st0);
  int w = 0;
  for (; w + 1 < n_work; w += 2) {
    step(IC<0>(), w);
    step(IC<1>(), w + 1);
  }
  if (w < n_work) step(IC<0>(), w);

  if constexpr (KVL) {
    // The two row halves of a key group hold partial sums of its dK and dV: the first half keeps dV
    // and hands its dK over, the second keeps dK and hands its dV over, through 16 KiB exchange
    // slots carved from the (now idle) tile buffers; each then adds the other's part to its own
    // (a fixed order, so results repeat) and writes one of the two outputs.
    static_assert(NDB * 4 * 64 * 16 == 16384 && TB >= 16384 && KVB >= 2 * 16384 && NKG <= 4, "exchange slots");
    __syncthreads();  // every wave is done with the tiles
    auto xslot = [&](int i) {
      lds_char_t* const base = (lds_char_t*)(i < 2 ? k_lds_raw : i < 4 ? v_lds_raw : i == 4 ? q_st0_raw : i == 5 ? q_st1_raw : i == 6 ? o_st0_raw : o_st1_raw);
      return (lds_f32x4_t*)(base + (i < 4 ? (i & 1) * 16384 : 0));
    };
    lds_f32x4_t* const out = xslot(2 * kg + rh);
    lds_f32x4_t* const in = xslot(2 * kg + 1 - rh);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 give;
#pragma unroll
        for (int e = 0; e < 4; ++e) give[e] = rh == 0 ? dkT[db][4 * r4 + e] : dvT[db][4 * r4 + e];
        out[(db * 4 + r4) * 64 + lane] = give;
      }
    __syncthreads();
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 o = in[(db * 4 + r4) * 64 + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dvT[db][4 * r4 + e] += rh == 0 ? o[e] : 0.f;
          dkT[db][4 * r4 + e] += rh == 0 ? 0.f : o[e];
        }
      }
  }

  // ---- epilogue: lane owns key my_key; register r of block db is head-dim 32*db + acc_row(r)
  if (my_key < nkv) {
    char* dkrow = (char*)p.dk + (b * p.dk_sb + kvh * p.dk_sh + (int64_t)(sq.k_tok0 + my_key) * p.dk_sn) * 2;
    char* dvrow = (char*)p.dv + (b * p.dv_sb + kvh * p.dv_sh + (int64_t)(sq.k_tok0 + my_key) * p.dv_sn) * 2;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < (DPAD ? D / 8 : 4); ++g4) {
        typename Elem<T>::vec4 kv, vv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kv[e] = (T)(dkT[db][4 * g4 + e] * p.scale);
          vv[e] = (T)dvT[db][4 * g4 + e];
        }
        const int col = 32 * db + acc_row(4 * g4, lane);
        if (DO_K && (!KVL || rh == 1)) *(i32x2*)(dkrow + col * 2) = __builtin_bit_cast(i32x2, kv);
        if (DO_V && (!KVL || rh == 0)) *(i32x2*)(dvrow + col * 2) = __builtin_bit_cast(i32x2, vv);
      }
  }
}

// ------------------------------------------------------------------------------------------------
// dQ. Grid: ceil(Nq / BW) * Hq * B workgroups (1-D).
template <typename T, bool CAUSAL, class Cfg, bool WINDOW = false, bool VARLEN = false>
__global__ void __launch_bounds__(Cfg::THREADS)
    __attribute__((amdgpu_waves_per_eu(Cfg::WAVES_PER_SIMD, Cfg::WAVES_PER_SIMD)))
    fa_bwd_dq_kernel(const BwdParams p) {
  constexpr int D = Cfg::D, NW = Cfg::NW, BKV = Cfg::BT, BQ = Cfg::BW;
  constexpr int NS = D / 16;
  constexpr bool DPAD = D < 32;
  constexpr int NDB = DPAD ? 1 : D / 32;
  constexpr int NKB = BKV / 32;
  constexpr int NKS = BKV / 16;
  constexpr int TB = Cfg::TILE_BYTES;
  typedef typename Elem<T>::vec8 vec8;

  // K in the transposing layout (row fragments for S^T, transposed for dQ^T), V in the row layout.
  __shared__ __attribute__((aligned(1024))) char k_st0_raw[TB];
  __shared__ __attribute__((aligned(1024))) char k_st1_raw[TB];
  __shared__ __attribute__((aligned(1024))) char v_st0_raw[TB];
  __shared__ __attribute__((aligned(1024))) char v_st1_raw[TB];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // 1-D grid over (query tile, head, batch). Query tile slowest, last tile first: under the causal
  // mask the last tiles, which see the most key tiles, go first (longest first). Query tile fastest:
  // the tiles of one head are dispatched together and share its K/V stream in cache.
  const int64_t lin = blockIdx.x;
  const int n_qt_all = (p.Nq + BQ - 1) / BQ;
  int h, b, q0;
  if (p.dq_block_slowest) {
    const int64_t per_qt = (int64_t)p.Hq * p.B;
    h = (int)(lin % p.Hq);
    b = (int)((lin % per_qt) / p.Hq);
    q0 = (n_qt_all - 1 - (int)(lin / per_qt)) * BQ;
  } else {
    const int64_t rest = lin / n_qt_all;
    q0 = (int)(lin % n_qt_all) * BQ;
    h = (int)(rest % p.Hq);
    b = (int)(rest / p.Hq);
  }
  const SeqSpan sq = seq_span<VARLEN>(p, b);
  const int nq = sq.nq, nkv = sq.nkv;
  if (VARLEN && q0 >= nq) return;  // a query block past this sequence's end (workgroup-uniform)
  const int kvh = h / p.group;
  const int wq0 = q0 + 32 * wave;
  const int my_row = wq0 + (lane & 31);
  const bool row_ok = my_row < nq;

  // Q and dO rows of the wave as B operands (lane holds row lane % 32); rows past the sequence are zero.
  vec8 qf[NS], of[NS];
  {
    const T* qrow = (const T*)p.q + b * p.q_sb + h * p.q_sh + (int64_t)(sq.q_tok0 + my_row) * p.q_sn;
    const T* orow = (const T*)p.dout + b * p.do_sb + h * p.do_sh + (int64_t)(sq.q_tok0 + my_row) * p.do_sn;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int col = 16 * s + 8 * half;
      qf[s] = row_ok ? *(const vec8*)(qrow + col) : vec8{};
      of[s] = row_ok ? *(const vec8*)(orow + col) : vec8{};
    }
  }
  const int64_t stat = b * p.lse_sb + h * p.lse_sh + sq.q_tok0 + my_row;
  const float lse2 = row_ok ? p.lse[stat] * kLog2e : 0.f;
  const float dlt = row_ok ? p.delta[stat] : 0.f;
  f32x16 dqT[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqT[db] = f32x16{};

  const char* kbase = (const char*)p.k + (b * p.k_sb + kvh * p.k_sh + (int64_t)sq.k_tok0 * p.k_sn) * 2;
  const char* vbase = (const char*)p.v + (b * p.v_sb + kvh * p.v_sh + (int64_t)sq.k_tok0 * p.v_sn) * 2;
  const int k_stride = (int)(p.k_sn * 2), v_stride = (int)(p.v_sn * 2);
  const int k_dma_off = (int)dma_lane_offset<D, false>(lane, k_stride);
  const int v_dma_off = (int)dma_lane_offset<D, false>(lane, v_stride);
  // key tiles this workgroup visits: [t0, t0 + n_tiles)
  int t0 = 0, n_tiles;
  if (WINDOW) {
    const int first = max(0, q0 - p.win_left);
    const int last = min(nkv - 1, min(q0 + BQ, nq) - 1 + p.win_right);
    t0 = first / BKV;
    n_tiles = first > last ? 0 : last / BKV + 1 - t0;
  } else {
    n_tiles = (int)kv_tiles_for_qtile(q0, BQ, nkv, BKV, CAUSAL);
  }
  const int wq_last = wq0 + 31;
  const float c = p.c;

  // per-lane parts of the tile reads: K and V row fragments (both tiles swizzled), and the
  // transposing reads of the K tile, conflict-free on the swizzled layout as well (fa_layout.h)
  constexpr int KP = kfrag_parities<D>();
  int frag_lane[KP];
#pragma unroll
  for (int par = 0; par < KP; ++par) frag_lane[par] = kfrag_lane_offset<D, BKV>(par, lane);
  const int kt_lane[2] = {vtr_swz_lane_offset<D, BKV>(0, lane), vtr_swz_lane_offset<D, BKV>(1, lane)};

  auto step = [&](auto stage_c, int j) {
    constexpr int S = decltype(stage_c)::value;
    lds_char_t* const kt = (lds_char_t*)(S == 0 ? k_st0_raw : k_st1_raw);
    lds_char_t* const vt = (lds_char_t*)(S == 0 ? v_st0_raw : v_st1_raw);
    const int kpos = (t0 + j) * BKV;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 1 < n_tiles) {
      lds_char_t* const kn = (lds_char_t*)(S == 0 ? k_st1_raw : k_st0_raw);
      lds_char_t* const vn = (lds_char_t*)(S == 0 ? v_st1_raw : v_st0_raw);
      dma_tile<D, BKV, NW>(kn, kbase, k_stride, kpos + BKV, nkv, wave_u, k_dma_off);
      dma_tile<D, BKV, NW>(vn, vbase, v_stride, kpos + BKV, nkv, wave_u, v_dma_off);
    }
    if (CAUSAL && kpos > wq_last) return;
    if (WINDOW && (kpos > wq_last + p.win_right || kpos + BKV - 1 < wq0 - p.win_left)) return;
    f32x16 st[NKB], dpt[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      st[kb] = f32x16{};
      dpt[kb] = f32x16{};
    }
    {
      vec8 ka[NS][NKB], va[NS][NKB];
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          ka[s][kb] = __builtin_bit_cast(vec8, lds_read16(kt + frag_lane[s % KP] + kfrag_const_offset<D, BKV>(kb, s)));
          va[s][kb] = __builtin_bit_cast(vec8, lds_read16(vt + frag_lane[s % KP] + kfrag_const_offset<D, BKV>(kb, s)));
        }
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          st[kb] = Elem<T>::mfma(ka[s][kb], qf[s], st[kb]);
          dpt[kb] = Elem<T>::mfma(va[s][kb], of[s], dpt[kb]);
        }
      constexpr int LEAD_S = D >= 128 && (CAUSAL || WINDOW) ? kBwdDqMaskedLead : kBwdLead;
      constexpr int LEAD = LEAD_S < NS ? LEAD_S : NS;
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * NKB * LEAD, 0);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2 * NKB, 0);
        if (s + LEAD < NS) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * NKB, 0);
      }
    }
    // register r of block kb: key kpos + 32*kb + acc_row(r, lane) against the lane's row
    const int base = kpos + 4 * half;
    int limit = nkv - 1 - base;
    if (CAUSAL) limit = min(limit, my_row - base);
    if (WINDOW) limit = min(limit, my_row + p.win_right - base);
    const int lower = WINDOW ? my_row - p.win_left - base : -1;  // keys below the window
    // The per-key test runs only for a tile that crosses the sequence end, the diagonal of the
    // wave's rows or a window edge (wave-uniform choice between two versions of the loop).
    auto probs = [&](auto masked_c) {
      constexpr bool MASKED = decltype(masked_c)::value != 0;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int koff = 32 * kb + 8 * (r >> 2) + (r & 3);
          float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][r], c, -lse2));
          if (MASKED) pv = (koff > limit || koff < lower) ? 0.f : pv;
          st[kb][r] = pv * (dpt[kb][r] - dlt);  // dS^T / scale
        }
      // (fp16) dS as opaque fp32 registers, from which both of its dtype terms below are converted
      if constexpr (std::is_same<T, _Float16>::value) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) __asm__("" : "+v"(st[kb]));
      }
    };
    if (WINDOW || kpos + BKV > nkv || (CAUSAL && kpos + BKV - 1 > wq0))
      probs(IC<1>());
    else
      probs(IC<0>());
    // dS enters the dQ product as two terms of the input dtype, hi = round(dS) and lo = round(dS - hi),
    // so the product sees dS to about twice the dtype's precision: where dQ is a sum of terms that
    // cancel (keys sharing a large component), one rounding of dS would dominate the result.
    // Both terms must come from one fp32 value. The backend can fold a conversion to fp16 into the
    // multiply that formed dS (a mixed-precision multiply-add: one rounding of the exact product)
    // for one use of hi and not for another, so that the operand hi and the hi the remainder is
    // taken from differ by one unit in the last place where the product lies next to a rounding
    // midpoint; the empty asm at the end of probs() makes dS opaque fp32 registers, from which every
    // use converts. (bf16 has no such fused conversion: its conversions take fp32 operands.)
    auto ds_terms = [&](int ks, vec8& hi_v, vec8& lo_v) {
#pragma clang fp contract(off)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = st[ks >> 1][pv_src_reg(ks, e)];
        const T hi = (T)x;
        hi_v[e] = hi;
        lo_v[e] = (T)(x - (float)hi);
      }
    };
    {
      vec8 kT[NKS][NDB];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          i16x4 lo = lds_read_tr(kt + kt_lane[0] + vtr_swz_const_offset<D, BKV>(ks, db));
          i16x4 hi = lds_read_tr(kt + kt_lane[1] + vtr_swz_const_offset<D, BKV>(ks, db));
          if (DPAD && ((lane >> 4) & 1)) {
            lo = i16x4{};
            hi = i16x4{};
          }
          kT[ks][db] = __builtin_bit_cast(vec8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        vec8 sfr, sfl;
        ds_terms(ks, sfr, sfl);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          dqT[db] = Elem<T>::mfma(kT[ks][db], sfr, dqT[db]);
          dqT[db] = Elem<T>::mfma(kT[ks][db], sfl, dqT[db]);
        }
      }
      constexpr int NF = NKS * NDB;
      // the window instance at D >= 128 holds the band's bounds as well: less read-ahead there
      constexpr int LEAD_F = D >= 128 && WINDOW ? kBwdLead : kBwdLead + 1;
      constexpr int LEAD = LEAD_F < NF ? LEAD_F : NF;
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * LEAD, 0);
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
        if (i + LEAD < NF) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
      }
    }
  };

  if (n_tiles > 0) {
    dma_tile<D, BKV, NW>((lds_char_t*)k_st0_raw, kbase, k_stride, t0 * BKV, nkv, wave_u, k_dma_off);
    dma_tile<D, BKV, NW>((lds_char_t*)v_st0_raw, vbase, v_stride, t0 * BKV, nkv, wave_u, v_dma_off);
  }
  int j = 0;
  for (; j + 1 < n_tiles; j += 2) {
    step(IC<0>(), j);
    step(IC<1>(), j + 1);
  }
  if (j < n_tiles) step(IC<0>(), j);

  // ---- epilogue: dQ = scale * (dS K), lane owns row my_row; register r of block db is
  // head-dim 32*db + acc_row(r)
  if (row_ok) {
    char* drow = (char*)p.dq + (b * p.dq_sb + h * p.dq_sh + (int64_t)(sq.q_tok0 + my_row) * p.dq_sn) * 2;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < (DPAD ? D / 8 : 4); ++g4) {
        typename Elem<T>::vec4 qv;
#pragma unroll
        for (int e = 0; e < 4; ++e) qv[e] = (T)(dqT[db][4 * g4 + e] * p.scale);
        const int col = 32 * db + acc_row(4 * g4, lane);
        *(i32x2*)(drow + col * 2) = __builtin_bit_cast(i32x2, qv);
      }
  }
}

}  // namespace fa
