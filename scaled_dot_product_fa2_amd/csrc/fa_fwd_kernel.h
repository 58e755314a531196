// fa_fwd_kernel.h - gfx950 (CDNA4) fused attention forward.
//
// One workgroup owns one (batch, query head, query tile) and streams the key /
// value tiles of its key/value head past the query tile, as in the tiled
// forward of "Write Triton Attention Kernel" (Required reasoning process,
// steps 1-9) and the Ascend notes, section 1: the Q tile stays on chip, scores
// and probabilities never leave registers, and O and LSE are written once.
//
// MI355X mapping:
//  * Scores are computed transposed, S^T = K Q^T, with 32x32x16 MFMAs (fp32
//    accumulate). Every lane then owns one query row: the running maximum,
//    denominator and rescale factor are per-lane scalars, and a row reduction
//    is an in-register reduction plus one swap between the two wave halves.
//  * The output is accumulated transposed as well, O^T += V^T P^T. The
//    probability operand is taken from the score accumulators without any
//    data movement (the reduction order of keys is permuted identically on
//    both operands), and V^T fragments come from ds_read_b64_tr_b16
//    transposing reads of a row-major V tile.
//  * Q, K and V tiles move HBM -> LDS with 16-byte direct-to-LDS loads
//    (global_load_lds), K/V double-buffered so the next tile streams in while
//    the current one is consumed. Q is staged through LDS once and then kept in
//    VGPRs for the whole key loop.
//  * Softmax runs in base 2 with scale*log2(e) folded into one FMA per score
//    (Ascend notes, section 1). m, l and the accumulator are fp32; P is rounded
//    to the input dtype before the P.V product (all three pages).
//  * Causal tiles above the diagonal are never visited; only key tiles that
//    cross a wave's rows are masked ("Build Triton-Ascend Fused Attention",
//    Workflow step 5; "Write Triton Attention Kernel", step 9 and Performance
//    requirements).
//  * D = 256 keeps eight 32-row accumulator blocks per query block, i.e. the two
//    D128 halves of the Ascend notes (sections 1 and 7) each as four blocks.
//  * Persistent grid: each workgroup loops over (batch, query head, query tile)
//    items dealt by an XCD-aware schedule (fa_layout.h), longest first under the
//    causal mask.
//  * Two more instances of the same kernel: WINDOW (a sliding-window mask, row i
//    sees keys i - left .. i + right; only the band's key tiles are visited) and
//    VARLEN (packed sequences addressed through cu_seqlens offsets, each with its
//    own length), the masking variants "Write Triton Attention Kernel" lists
//    among its inputs (items 3 and 6).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_layout.h"

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) i32x4 lds_i32x4_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

// Element traits: MFMA and round-to-nearest-even conversions per input type.
template <typename T>
struct Elem;

template <>
struct Elem<__bf16> {
  typedef bf16x8 vec8;
  typedef bf16x4 vec4;
  static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Elem<_Float16> {
  typedef f16x8 vec8;
  typedef f16x4 vec4;
  static __device__ __forceinline__ f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t q_sb, q_sh, q_sn;  // element strides; the head-dim stride is 1
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t o_sb, o_sh, o_sn;
  int32_t B, Hq, Hkv, Nq, Nkv;
  int32_t group;     // Hq / Hkv
  int32_t n_qtiles;  // ceil(Nq / BQ)
  float c;           // scale * log2(e)
  // sliding window (the WINDOW instances only): row i sees keys i - win_left .. i + win_right; an
  // unbounded side is passed as Nq (left) or Nkv (right), which no row can reach past
  int32_t win_left, win_right;
  // packed variable-length sequences (the VARLEN instances only): sequence b owns tokens
  // cu_q[b] .. cu_q[b+1]-1 of Q/O and cu_k[b] .. cu_k[b+1]-1 of K/V; Nq and Nkv hold the longest
  // lengths, the batch strides are 0
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t total_q, total_k;
  int64_t lse_sb, lse_sh;  // LSE element offset of (b, h); the row index is added to it
  // balanced instances only: claim counters, zero on entry and left zero on exit (kBalanceCounters)
  uint32_t* balance;
};

// Balanced instances (dense launches with long key ranges and many rounds of items). The
// XCDs of one chip hold different shader clocks under load, so a schedule that gives every
// workgroup the same work ends when the slowest XCD does. In these instances each XCD runs the
// static schedule below for all but the last kBalanceTailRounds rounds of its list (the shortest
// items, the list being longest first); those are claimed from a per-XCD counter, the next claim
// issued while the current item runs, and a workgroup whose own XCD has none left takes them from
// the XCD with the most left. Counter words: 0..7 the claims of each XCD's tail, 8 the workgroups
// that have finished; the last one to finish zeroes them all.
constexpr uint32_t kBalanceTailRounds = 3;
constexpr int kBalanceCounters = 16;

// Tile configuration: NW waves per workgroup, QB 32-row query blocks per wave,
// BKV keys per inner-loop tile.
template <int D_, int NW_, int QB_, int BKV_, int WAVES_PER_SIMD_>
struct TileCfg {
  static constexpr int D = D_;
  static constexpr int NW = NW_;
  static constexpr int QB = QB_;
  static constexpr int BKV = BKV_;
  static constexpr int WAVES_PER_SIMD = WAVES_PER_SIMD_;
  static constexpr int THREADS = NW * 64;
  static constexpr int BQ = NW * QB * 32;
  static constexpr int KV_TILE_BYTES = BKV * D * 2;
  // two stages of K and of V; the Q tile is staged in the same buffers before the key loop
  static constexpr int LDS_BYTES = 4 * KV_TILE_BYTES;
  // a tile copy is whole 64-lane instructions, each within one segment column
  static_assert((BKV * chunks_per_seg<D>()) % 64 == 0, "K/V tile rows must fill whole copy instructions");
  static_assert(BKV % 32 == 0 && BQ % BKV == 0 && (D % 32 == 0 || D == 16), "tile shape");
};

__device__ __forceinline__ float wave_half_max(float x) {
  // max of the value in lane l and lane l^32
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Copy rows [row0, row0 + ROWS) of a [rows x D] 16-bit tensor slice (row stride
// `stride` bytes) into an LDS tile with direct-to-LDS 16-byte buffer loads; the
// copy's instructions are spread over the NW waves. The buffer descriptor
// covers only the valid rows, so rows at or past `n_rows` read as zeros
// (they are masked out of every result). `lane_off` is dma_lane_offset for this
// lane and stride; `wave` must be wave-uniform.
template <int D, int ROWS, int NW>
__device__ __forceinline__ void dma_tile(lds_char_t* tile, const char* gbase, int stride, int row0, int n_rows,
                                         int wave, int lane_off) {
  constexpr int n_inst = dma_insts<D, ROWS>();
  constexpr int per_wave = (n_inst + NW - 1) / NW;
  const int valid = n_rows - row0 < ROWS ? n_rows - row0 : ROWS;
  const uint32_t nbytes = (uint32_t)(valid - 1) * (uint32_t)stride + (uint32_t)(D * 2);
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(gbase + (int64_t)row0 * stride), (short)0, (int)nbytes, 0x00020000);
#pragma unroll
  for (int t = 0; t < per_wave; ++t) {
    const int i = wave + t * NW;
    if (n_inst % NW != 0 && i >= n_inst) break;
    const int soff = (int)dma_inst_offset<D, ROWS>(i, stride);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(tile + i * 1024), 16, lane_off, soff, 0, 0);
  }
}

__device__ __forceinline__ i32x4 lds_read16(const lds_char_t* p) { return *(const lds_i32x4_t*)p; }
__device__ __forceinline__ i16x4 lds_read_tr(const lds_char_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p);
}

template <int V>
struct IC {
  static constexpr int value = V;
};

// Headroom of the lazily updated running maximum, in log2 units: a row's
// reference maximum is raised (and its accumulator rescaled) only when a tile
// exceeds it by more than this, so probabilities stay below 2^8.
constexpr float kRescaleHeadroom = 8.0f;
// Bound on a lane's sum of tile probabilities under which the fast softmax path keeps them without
// a tile maximum: every probability is then at most 2^14, inside fp16's range (and bf16's).
constexpr float kFastSumLimit = 16384.0f;

// Fragment read-ahead in the two MFMA loops, in head-dim slices of K (S^T) and in V fragments
// (P V). Left to itself the compiler issues each LDS read right before the MFMA that consumes it,
// into the same few registers, so every MFMA waits out a full LDS round trip; scheduling-group
// barriers pin an order with the reads this far ahead instead.
constexpr int kQkLead = 3;
constexpr int kPvLead = 4;
constexpr int kPvLeadD256 = 3;  // one fragment less at D = 256, which is at the register limit
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

#ifdef FA_TIMELINE
// Timeline build only (a separate library compiled with -DFA_TIMELINE; the kernels of libfa.so have
// none of this). Per workgroup, words of g_timeline: 0 and 3 the fixed 100 MHz clock
// (s_memrealtime) at its start and end, 6 and 7 the shader clock (s_memtime) at the same points,
// 1 and 2 the fixed clock when its first item's Q tile is in registers and when that item's key
// loop ends, 4 the shader clocks that item spent waiting for tile copies and at the per-tile
// barrier, 5 that item's key tiles. Written with ordinary vector stores by thread 0.
constexpr int kTimelineWgs = 65536;
constexpr int kTimelineWords = 8;
static __device__ unsigned long long g_timeline[kTimelineWgs * kTimelineWords];
#define FA_TL_STAMP(word, value)                                                \
  do {                                                                          \
    if (threadIdx.x == 0 && blockIdx.x < kTimelineWgs)                          \
      g_timeline[(size_t)blockIdx.x * kTimelineWords + (word)] = (value);       \
  } while (0)
#endif

template <typename T, bool CAUSAL, class Cfg, bool WINDOW = false, bool VARLEN = false, bool BALANCED = false>
__global__ void __launch_bounds__(Cfg::THREADS)
    __attribute__((amdgpu_waves_per_eu(Cfg::WAVES_PER_SIMD, Cfg::WAVES_PER_SIMD)))
    fa_fwd_kernel(const FwdParams p) {
  constexpr int D = Cfg::D, NW = Cfg::NW, QB = Cfg::QB, BKV = Cfg::BKV, BQ = Cfg::BQ;
  constexpr int NS = D / 16;     // 16-wide head-dim slices (QK^T reduction steps)
  constexpr bool DPAD = D < 32;  // D = 16: one 32-row O^T block, half of it padding
  constexpr int NDB = DPAD ? 1 : D / 32;  // 32-row head-dim blocks of O^T
  constexpr int NKB = BKV / 32;  // 32-row key blocks of S^T
  constexpr int NKS = BKV / 16;  // 16-wide key slices (P.V reduction steps)
  constexpr int KVB = Cfg::KV_TILE_BYTES;
  typedef typename Elem<T>::vec8 vec8;

  // Four separately declared LDS buffers (K and V, two stages each), so the
  // compiler can tell a read of one stage from the copy into the other.
  __shared__ __attribute__((aligned(1024))) char k_st0_raw[KVB];
  __shared__ __attribute__((aligned(1024))) char k_st1_raw[KVB];
  __shared__ __attribute__((aligned(1024))) char v_st0_raw[KVB];
  __shared__ __attribute__((aligned(1024))) char v_st1_raw[KVB];
  lds_char_t* const k_st0 = (lds_char_t*)k_st0_raw;
  lds_char_t* const k_st1 = (lds_char_t*)k_st1_raw;
  lds_char_t* const v_st0 = (lds_char_t*)v_st0_raw;
  lds_char_t* const v_st1 = (lds_char_t*)v_st1_raw;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int half = lane >> 5;

  // ---- persistent loop over this workgroup's items (batch, query head, query tile); see Schedule
  const Schedule sched{p.B * p.Hkv, p.Hkv, p.group, p.n_qtiles, CAUSAL, (int)gridDim.x};
  const int xcd = blockIdx.x % 8;
  const uint32_t n_mine = sched.items_of(xcd);
#ifdef FA_TIMELINE
  FA_TL_STAMP(0, __builtin_amdgcn_s_memrealtime());
  FA_TL_STAMP(6, __builtin_amdgcn_s_memtime());
#endif
  static_assert(!BALANCED || (!WINDOW && !VARLEN), "balanced instances: dense launches only");
  // (BALANCED) static rounds of XCD y's list: all but the last min(kBalanceTailRounds, rounds - 1)
  auto head_items_of = [&](int y) -> uint32_t {
    const uint32_t gy = (uint32_t)sched.wgs_of(y);
    if (gy == 0) return 0;
    const uint32_t r = (sched.items_of(y) + gy - 1) / gy;
    if (r == 0) return 0;
    const uint32_t t = r - 1 < kBalanceTailRounds ? r - 1 : kBalanceTailRounds;
    return (r - t) * gy;
  };
  __shared__ int s_claim[2];
  uint32_t my_head_rounds = 0, my_head_items = 0;
  if constexpr (BALANCED) {
    my_head_items = head_items_of(xcd);
    my_head_rounds = my_head_items / (uint32_t)sched.wgs_of(xcd);
  }
  int steal_from = 0;  // (thread 0) 0 while the own XCD's tail has items, then 1
  uint32_t pre = 0;    // (thread 0) an own-tail claim issued one item ahead
  bool pre_valid = false;
  for (uint32_t round = 0;; ++round) {
    uint32_t idx;
    int ix = xcd;  // the XCD whose list the item comes from
    if (!BALANCED || round < my_head_rounds) {
      idx = sched.item_index(blockIdx.x, round);
      if (idx >= n_mine) break;
    } else {
      if (tid == 0) {
        int got_x = -1;
        uint32_t got = 0;
        if (steal_from == 0) {
          if (my_head_items < n_mine) {
            const uint32_t cl = pre_valid ? pre : __hip_atomic_fetch_add(&p.balance[xcd], 1u, __ATOMIC_RELAXED,
                                                                         __HIP_MEMORY_SCOPE_AGENT);
            pre_valid = false;
            if (my_head_items + cl < n_mine) {
              got_x = xcd;
              got = my_head_items + cl;
            }
          }
          if (got_x < 0) steal_from = 1;
        }
        // the XCD with the most unclaimed items (all eight counters read at once). A claim fails
        // only on a tail this thread then sees exhausted, so the loop ends within eight failures.
        for (int attempt = 0; got_x < 0 && attempt < 64; ++attempt) {
          uint32_t cnt[8];
#pragma unroll
          for (int y = 0; y < 8; ++y) cnt[y] = __hip_atomic_load(&p.balance[y], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          int best = -1;
          uint32_t best_rem = 0;
#pragma unroll
          for (int y = 0; y < 8; ++y) {
            const uint32_t ny = sched.items_of(y), hy = head_items_of(y);
            const uint32_t rem = hy + cnt[y] < ny ? ny - hy - cnt[y] : 0;
            if (rem > best_rem) {
              best_rem = rem;
              best = y;
            }
          }
          if (best < 0) break;
          const uint32_t cl = __hip_atomic_fetch_add(&p.balance[best], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (head_items_of(best) + cl < sched.items_of(best)) {
            got_x = best;
            got = head_items_of(best) + cl;
          }
        }
        s_claim[0] = got_x;
        s_claim[1] = (int)got;
      }
      __syncthreads();
      ix = s_claim[0];
      idx = (uint32_t)s_claim[1];
      __syncthreads();  // s_claim is read by every wave before thread 0 writes it again
      if (ix < 0) break;
    }
    const Item item = sched.item(ix, idx);
    if constexpr (BALANCED) {
      // claim the next own-tail item while this one runs, from the last static round on
      if (tid == 0 && steal_from == 0 && !pre_valid && round + 1 >= my_head_rounds && my_head_items < n_mine) {
        pre = __hip_atomic_fetch_add(&p.balance[xcd], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        pre_valid = true;
      }
    }
    const int b = item.b, h = item.h, qt = item.qt;
    const int kvh = h / p.group;
    const int q0 = qt * BQ;
    // the item's sequence lengths and first tokens; packed sequences read them from the offsets,
    // clamped to the token counts so that no offset array can send a copy out of bounds
    int nq = p.Nq, nkv = p.Nkv, q_tok0 = 0, k_tok0 = 0;
    if (VARLEN) {
      const int cq0 = min(max(p.cu_q[b], 0), p.total_q), cq1 = min(max(p.cu_q[b + 1], cq0), p.total_q);
      const int ck0 = min(max(p.cu_k[b], 0), p.total_k), ck1 = min(max(p.cu_k[b + 1], ck0), p.total_k);
      q_tok0 = cq0;
      k_tok0 = ck0;
      nq = min(cq1 - cq0, p.Nq);
      nkv = min(ck1 - ck0, p.Nkv);
      if (q0 >= nq) continue;  // a query tile past this sequence's end
    }
    __syncthreads();  // every wave is done with the previous item's LDS tiles

    const char* qbase =
        (const char*)p.q + ((int64_t)b * p.q_sb + (int64_t)h * p.q_sh + (int64_t)q_tok0 * p.q_sn) * 2;
    const char* kbase =
        (const char*)p.k + ((int64_t)b * p.k_sb + (int64_t)kvh * p.k_sh + (int64_t)k_tok0 * p.k_sn) * 2;
    const char* vbase =
        (const char*)p.v + ((int64_t)b * p.v_sb + (int64_t)kvh * p.v_sh + (int64_t)k_tok0 * p.v_sn) * 2;

    // Row strides in bytes (validated on the host to keep every tile offset in 31 bits).
    const int q_stride = (int)(p.q_sn * 2), k_stride = (int)(p.k_sn * 2), v_stride = (int)(p.v_sn * 2);
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int k_dma_off = (int)dma_lane_offset<D, false>(lane, k_stride);
    const int v_dma_off = (int)dma_lane_offset<D, true>(lane, v_stride);

    // ---- Q tile: HBM -> LDS with coalesced 16-byte loads, staged in parts of BKV rows across
    // the K/V buffers; then LDS -> VGPRs in the MFMA B-operand layout, kept for the whole key loop.
    // When Q fits the two stage-1 buffers, key/value tile 0 streams into stage 0 at the same time,
    // so the workgroup pays one memory round trip before its first tile instead of two.
    constexpr int Q_PARTS = BQ / BKV;
    static_assert(Q_PARTS >= 1 && Q_PARTS <= 4 && Q_PARTS * BKV == BQ, "Q tile must fit the four K/V buffers");
    constexpr bool KV0_WITH_Q = Q_PARTS <= 2;
    // key tiles this item visits: [t0, t0 + n_tiles)
    int t0 = 0, n_tiles;
    if (WINDOW) {
      const int q_last = min(q0 + BQ, nq) - 1;
      const int first = max(0, q0 - p.win_left);
      const int last = min(nkv - 1, q_last + p.win_right);
      t0 = first / BKV;
      n_tiles = first > last ? 0 : last / BKV + 1 - t0;
    } else {
      n_tiles = (int)kv_tiles_for_qtile(q0, BQ, nkv, BKV, CAUSAL);
    }
    auto qpart = [&](int part) {
      if (KV0_WITH_Q) return part == 0 ? k_st1 : v_st1;
      return part == 0 ? k_st0 : part == 1 ? k_st1 : part == 2 ? v_st0 : v_st1;
    };
    {
      const int q_dma_off = (int)dma_lane_offset<D, false>(lane, q_stride);
#pragma unroll
      for (int part = 0; part < Q_PARTS; ++part)
        if (q0 + part * BKV < nq)
          dma_tile<D, BKV, NW>(qpart(part), qbase, q_stride, q0 + part * BKV, nq, wave_u, q_dma_off);
      if (KV0_WITH_Q && n_tiles > 0) {
        dma_tile<D, BKV, NW>(k_st0, kbase, k_stride, t0 * BKV, nkv, wave_u, k_dma_off);
        dma_tile<D, BKV, NW>(v_st0, vbase, v_stride, t0 * BKV, nkv, wave_u, v_dma_off);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    vec8 qf[QB][NS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = wave * QB * 32 + qfrag_row(qb, lane);
      const lds_char_t* qsrc = qpart(row / BKV);
#pragma unroll
      for (int s = 0; s < NS; ++s)
        qf[qb][s] = __builtin_bit_cast(
            vec8, lds_read16(qsrc + tile_chunk_offset<D, BKV, false>(row % BKV, kfrag_chunk(s, lane))));
    }
    __syncthreads();  // the Q staging area takes K/V tiles below
#ifdef FA_TIMELINE
    if (round == 0) FA_TL_STAMP(1, __builtin_amdgcn_s_memrealtime());
    unsigned long long tl_wait = 0;
#endif

    // leading tiles in which every (row, key) pair of the workgroup is visible and in range
    int n_full = nkv / BKV;
    if (CAUSAL && (q0 + 1) / BKV < n_full) n_full = (q0 + 1) / BKV;
    if (n_full > n_tiles) n_full = n_tiles;

    // per-lane softmax state of each query block: reference maximum (log2 units), partial denominator
    float m_run[QB], l_run[QB];
    f32x16 acc[QB][NDB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      m_run[qb] = -INFINITY;
      l_run[qb] = 0.f;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[qb][db] = f32x16{};
    }
    const int wq_first = q0 + wave * QB * 32;  // first and last query row owned by this wave
    const int wq_last = wq_first + QB * 32 - 1;
    const float c = p.c;

    if (!KV0_WITH_Q && n_tiles > 0) {
      dma_tile<D, BKV, NW>(k_st0, kbase, k_stride, t0 * BKV, nkv, wave_u, k_dma_off);
      dma_tile<D, BKV, NW>(v_st0, vbase, v_stride, t0 * BKV, nkv, wave_u, v_dma_off);
    }
    // per-lane parts of the fragment read offsets
    constexpr int KP = kfrag_parities<D>();
    int k_lane[KP];
#pragma unroll
    for (int par = 0; par < KP; ++par) k_lane[par] = kfrag_lane_offset<D, BKV>(par, lane);
    const int v_lane = vtr_lane_offset<D, BKV>(lane);

    // One key tile: wait for its copy, start the next tile's copy into the other stage, then
    // S^T = K Q^T, online softmax, O^T += V^T P^T.
    auto step = [&](auto stage_c, int j) {
      constexpr int S = decltype(stage_c)::value;
      lds_char_t* const kcur = S == 0 ? k_st0 : k_st1;
      lds_char_t* const vcur = S == 0 ? v_st0 : v_st1;
      lds_char_t* const knext = S == 0 ? k_st1 : k_st0;
      lds_char_t* const vnext = S == 0 ? v_st1 : v_st0;
      const int kpos = (t0 + j) * BKV;
      // wave-uniform: does any (row, key) pair of this wave and tile fall outside the visible set?
      const bool mask = WINDOW ? !(kpos >= wq_last - p.win_left && kpos + BKV - 1 <= wq_first + p.win_right &&
                                   kpos + BKV <= nkv)
                               : j >= n_full;
#ifdef FA_TIMELINE
      const unsigned long long tl_w0 = __builtin_amdgcn_s_memtime();
#endif
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
#ifdef FA_TIMELINE
      tl_wait += __builtin_amdgcn_s_memtime() - tl_w0;
#endif
      if (j + 1 < n_tiles) {
        dma_tile<D, BKV, NW>(knext, kbase, k_stride, kpos + BKV, nkv, wave_u, k_dma_off);
        dma_tile<D, BKV, NW>(vnext, vbase, v_stride, kpos + BKV, nkv, wave_u, v_dma_off);
      }
      // a causal tile wholly to the right of this wave's last row contributes nothing; with a
      // window, neither does a tile wholly outside every row's band
      if (CAUSAL && kpos > wq_last) return;
      if (WINDOW && (kpos > wq_last + p.win_right || kpos + BKV - 1 < wq_first - p.win_left)) return;

      // ---- S^T = K Q^T (a lambda: the rare slow softmax path below computes it a second time)
      f32x16 sc[QB][NKB];
      auto scores = [&]() {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) sc[qb][kb] = f32x16{};
        vec8 kf[NS][NKB];
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
            kf[s][kb] = __builtin_bit_cast(vec8, lds_read16(kcur + k_lane[s % KP] + kfrag_const_offset<D, BKV>(kb, s)));
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) sc[qb][kb] = Elem<T>::mfma(kf[s][kb], qf[qb][s], sc[qb][kb]);
        // Issue order: the reads of the first kQkLead slices, then per slice its MFMAs followed by
        // the reads of slice s + kQkLead, so every MFMA finds its operand already in flight.
        constexpr int LEAD = kQkLead < NS ? kQkLead : NS;
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, LEAD * NKB, 0);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, NKB * QB, 0);
          if (s + LEAD < NS) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, NKB, 0);
        }
      };
      scores();

      // ---- online softmax in base 2, one query row per lane
      // Scores hidden by the mask become -inf before any maximum or exponential is taken.
      auto apply_mask = [&](int qb) {
        // key = kpos + 4*(lane/32) + koff(kb, r) with koff a compile-time constant; the key is
        // hidden iff koff > limit, where limit folds the causal bound (key <= row) and the
        // sequence end (key < Nkv) into one per-lane value.
        const int qrow = wq_first + qfrag_row(qb, lane);
        const int base = kpos + 4 * half;
        int limit = nkv - 1 - base;
        if (CAUSAL) limit = min(limit, qrow - base);
        if (WINDOW) limit = min(limit, qrow + p.win_right - base);
        // with a window, keys below the band are hidden too: koff < lower
        const int lower = WINDOW ? qrow - p.win_left - base : -1;
        const int r0 = wq_first + 32 * qb, r1 = r0 + 31;  // rows of this block (wave-uniform)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          // Without a window, a 32-key block whose every (row, key) pair is visible needs no
          // mask and one whose every pair is hidden is cleared whole; only the others are masked
          // key by key. (The window instances mask every key: their registers are tighter.)
          if (!WINDOW) {
            const int k0 = kpos + 32 * kb, k1 = k0 + 31;
            if (k1 < nkv && (!CAUSAL || k1 <= r0)) continue;
            if (k0 >= nkv || (CAUSAL && k0 > r1)) {
              sc[qb][kb] = f32x16{} - INFINITY;
              continue;
            }
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int koff = 32 * kb + 8 * (r >> 2) + (r & 3);
            const bool hidden = WINDOW ? (koff > limit || koff < lower) : koff > limit;
            sc[qb][kb][r] = hidden ? -INFINITY : sc[qb][kb][r];
          }
        }
      };
      // Probabilities against the current reference maximum m, P = 2^(c*s - m), and their sum over
      // the lane's keys.
      auto probabilities = [&](int qb) {
        // a row that has seen no visible key yet keeps -inf; its scores are all -inf here too
        const float m_use = m_run[qb] == -INFINITY ? 0.f : m_run[qb];
        // four partial sums: four independent add chains instead of one
        float part[4];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[qb][kb][r], c, -m_use));
            sc[qb][kb][r] = pv;
            if (kb == 0 && r < 4)
              part[r] = pv;
            else
              part[r & 3] += pv;
          }
        return (part[0] + part[1]) + (part[2] + part[3]);
      };
      vec8 pf[QB][NKS];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (mask) apply_mask(qb);
        // Fast path: once a row has a finite reference maximum, the tile's probabilities are taken
        // against it without computing the tile's maximum first. They are kept when the lane's sum
        // stays at most kFastSumLimit, which bounds every one of them by it; otherwise (or while a
        // row has no reference yet, or on a non-finite sum) the tile is scored again and goes
        // through the maximum below. Either way every probability of the tile is finite and at
        // most kFastSumLimit, and numerator and denominator share the reference.
        bool slow = __any(m_run[qb] == -INFINITY);
        float rs = 0.f;
        if (!slow) {
          rs = probabilities(qb);
          slow = __any(!(rs <= kFastSumLimit));
          if (slow) {
            scores();
            if (mask) apply_mask(qb);
          }
        }
        if (slow) {
          float mx = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[qb][kb][r]);
          const float mt = wave_half_max(mx) * c;  // tile maximum of the scaled scores, log2 units
          const bool grow = mt > m_run[qb] + kRescaleHeadroom;
          if (__any(grow)) {
            const float alpha = grow ? __builtin_amdgcn_exp2f(m_run[qb] - mt) : 1.f;
            m_run[qb] = grow ? mt : m_run[qb];
            l_run[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[qb][db] *= alpha;
          }
          rs = probabilities(qb);
        }
        l_run[qb] += rs;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          vec8 t;
#pragma unroll
          for (int e = 0; e < 8; ++e) t[e] = (T)sc[qb][ks >> 1][pv_src_reg(ks, e)];
          pf[qb][ks] = t;
        }
      }

      // ---- O^T += V^T P^T
      // The wave runs this block at raised issue priority: while it streams P V MFMAs, the other
      // wave on the SIMD fills the gaps with its softmax or score work instead of competing for
      // the MFMA pipe.
      __builtin_amdgcn_s_setprio(1);
      {
        vec8 vf[NKS][NDB];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            // D = 16 fills only the first 16 rows of the 32-row block; the other lanes read a
            // valid address and contribute zeros.
            i16x4 lo = lds_read_tr(vcur + v_lane + vtr_const_offset<D, BKV>(ks, 0, db));
            i16x4 hi = lds_read_tr(vcur + v_lane + vtr_const_offset<D, BKV>(ks, 1, db));
            if (DPAD && ((lane >> 4) & 1)) {
              lo = i16x4{};
              hi = i16x4{};
            }
            vf[ks][db] = __builtin_bit_cast(vec8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) acc[qb][db] = Elem<T>::mfma(vf[ks][db], pf[qb][ks], acc[qb][db]);
        // the same read-ahead for V: two transposing reads per fragment, PV_LEAD fragments ahead
        constexpr int NV = NKS * NDB;
        constexpr int PV_LEAD = D >= 256 ? kPvLeadD256 : kPvLead;
        constexpr int LEAD = PV_LEAD < NV ? PV_LEAD : NV;
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * LEAD, 0);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, QB, 0);
          if (i + LEAD < NV) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
    };

    // key tiles two at a time (stage 0 then stage 1); an odd last tile uses stage 0
    int j = 0;
    for (; j + 1 < n_tiles; j += 2) {
      step(IC<0>(), j);
      step(IC<1>(), j + 1);
    }
    if (j < n_tiles) step(IC<0>(), j);
#ifdef FA_TIMELINE
    if (round == 0) {
      FA_TL_STAMP(2, __builtin_amdgcn_s_memrealtime());
      FA_TL_STAMP(4, tl_wait);
      FA_TL_STAMP(5, (unsigned long long)n_tiles);
    }
#endif

    // ---- epilogue: O = acc / l (rounded once to T), LSE = (m + log2 l) * ln 2
    const float LN2 = 0.69314718055994530942f;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qrow = wq_first + qfrag_row(qb, lane);
      const float l_tot = wave_half_sum(l_run[qb]);
      // a window, or a packed sequence without keys, can leave a row without visible keys:
      // O = 0 and LSE = -inf there
      const bool empty = (WINDOW || VARLEN) && !(l_tot > 0.f);
      const float inv = empty ? 0.f : 1.f / l_tot;
      if (qrow < nq) {
        char* orow =
            (char*)p.o + ((int64_t)b * p.o_sb + (int64_t)h * p.o_sh + (int64_t)(q_tok0 + qrow) * p.o_sn) * 2;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int g4 = 0; g4 < (DPAD ? D / 8 : 4); ++g4) {
            typename Elem<T>::vec4 ov;
#pragma unroll
            for (int e = 0; e < 4; ++e) ov[e] = (T)(acc[qb][db][4 * g4 + e] * inv);
            const int col = 32 * db + acc_row(4 * g4, lane);
            *(i32x2*)(orow + col * 2) = __builtin_bit_cast(i32x2, ov);
          }
        if (half == 0)
          p.lse[(int64_t)b * p.lse_sb + (int64_t)h * p.lse_sh + q_tok0 + qrow] =
              empty ? -INFINITY : (m_run[qb] + __log2f(l_tot)) * LN2;
      }
    }
  }  // item loop
  if constexpr (BALANCED) {
    if (tid == 0) {
      // every workgroup's claims are done before it counts itself finished, so the last one to
      // finish can zero the counters for the next launch
      const uint32_t done = __hip_atomic_fetch_add(&p.balance[8], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (done == gridDim.x - 1) {
        for (int y = 0; y < 9; ++y) __hip_atomic_store(&p.balance[y], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
#ifdef FA_TIMELINE
  FA_TL_STAMP(3, __builtin_amdgcn_s_memrealtime());
  FA_TL_STAMP(7, __builtin_amdgcn_s_memtime());
#endif
}

}  // namespace fa
