// fa_api.hip - C ABI of the gfx950 attention forward and backward: validation,
// launch plan, dispatch over (dtype, head_dim, mask) instances (defined in
// fa_fwd_inst.hip and fa_bwd_inst.hip). The declarations and the contract of
// every entry point are in include/fa.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <limits>
#include <mutex>

#include "fa.h"
#include "fa_launch.h"
#include "fa_layout.h"

namespace {

using fa::CfgFor;
using fa::FwdParams;
using fa::kNumCUs;

struct PlanInfo {
  int threads, bq, bkv, lds, wgs_per_cu;
};

template <int D>
PlanInfo plan_info() {
  typedef typename CfgFor<D>::type C;
  return PlanInfo{C::THREADS, C::BQ, C::BKV, C::LDS_BYTES, C::WAVES_PER_SIMD * 4 / C::NW};
}

bool plan_for_d(int64_t D, PlanInfo* out) {
  switch (D) {
    case 16: *out = plan_info<16>(); return true;
    case 32: *out = plan_info<32>(); return true;
    case 64: *out = plan_info<64>(); return true;
    case 128: *out = plan_info<128>(); return true;
    case 256: *out = plan_info<256>(); return true;
    default: return false;
  }
}

constexpr int64_t kMaxDim = (int64_t)std::numeric_limits<int32_t>::max();

bool mul_ok(int64_t a, int64_t b, int64_t* r) { return !__builtin_mul_overflow(a, b, r); }
bool add_ok(int64_t a, int64_t b, int64_t* r) { return !__builtin_add_overflow(a, b, r); }

// Largest element offset addressed through a (b, h, n, d) stride set; false on overflow.
bool extent_ok(int64_t B, int64_t H, int64_t N, int64_t D, const int64_t* st) {
  int64_t acc = D - 1, t;
  if (!mul_ok(B - 1, st[0], &t) || !add_ok(acc, t, &acc)) return false;
  if (!mul_ok(H - 1, st[1], &t) || !add_ok(acc, t, &acc)) return false;
  if (!mul_ok(N - 1, st[2], &t) || !add_ok(acc, t, &acc)) return false;
  return mul_ok(acc + 1, 2, &t);
}

int check_shape(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, int dtype, bool causal,
                PlanInfo* pi, int64_t* n_qtiles, int64_t* grid) {
  if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (!plan_for_d(D, pi)) return FA_ERR_HEAD_DIM;
  if (B < 1 || Hq < 1 || Nq < 1 || Nkv < 1 || Hkv < 0) return FA_ERR_SHAPE;
  if (B > kMaxDim || Hq > kMaxDim || Hkv > kMaxDim || Nq > kMaxDim || Nkv > kMaxDim) return FA_ERR_SHAPE;
  if (Hkv < 1 || Hq % Hkv != 0) return FA_ERR_GQA;
  *n_qtiles = (Nq + pi->bq - 1) / pi->bq;
  int64_t g;
  if (!mul_ok(B, Hq, &g) || !mul_ok(g, *n_qtiles, &g) || g > kMaxDim) return FA_ERR_SHAPE;
  int64_t lse_n;
  if (!mul_ok(B, Hq, &lse_n) || !mul_ok(lse_n, Nq, &lse_n) || !mul_ok(lse_n, 4, &lse_n)) return FA_ERR_SHAPE;
  if (B * Hkv > kMaxDim) return FA_ERR_SHAPE;
  // persistent grid: as many workgroups as are resident at once (or fewer, for small problems)
  const fa::Schedule sched{(int)(B * Hkv), (int)Hkv, (int)(Hq / Hkv), (int)*n_qtiles, causal, 0};
  *grid = sched.choose_grid((int64_t)kNumCUs * pi->wgs_per_cu);
  return FA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Largest sequence stride (elements): a tile of up to 256 rows is addressed with 32-bit offsets.
constexpr int64_t kMaxRowStride = (int64_t)1 << 22;

// Sequence lengths of a windowed forward: row + window stays within 32 bits.
constexpr int64_t kMaxWindowSeq = (int64_t)1 << 30;

int check_strides(const int64_t* st, bool is_output, int64_t B, int64_t H, int64_t N) {
  if (st[3] != 1) return FA_ERR_LAYOUT;
  for (int i = 0; i < 3; ++i) {
    if (st[i] < 0) return FA_ERR_LAYOUT;
    if (st[i] % 8 != 0) return FA_ERR_LAYOUT;  // 16-byte multiples of 2-byte elements
  }
  if (st[2] > kMaxRowStride) return FA_ERR_LAYOUT;
  if (is_output) {
    if ((B > 1 && st[0] == 0) || (H > 1 && st[1] == 0) || (N > 1 && st[2] == 0)) return FA_ERR_LAYOUT;
  }
  return FA_OK;
}

template <typename T, bool CAUSAL, bool WINDOW = false, bool VARLEN = false, bool BALANCED = false>
int launch_d(int64_t D, const FwdParams& p, int64_t grid, hipStream_t stream) {
  switch (D) {
    case 16: return fa::launch_fwd<T, CAUSAL, 16, WINDOW, VARLEN, BALANCED>(p, grid, stream);
    case 32: return fa::launch_fwd<T, CAUSAL, 32, WINDOW, VARLEN, BALANCED>(p, grid, stream);
    case 64: return fa::launch_fwd<T, CAUSAL, 64, WINDOW, VARLEN, BALANCED>(p, grid, stream);
    case 128: return fa::launch_fwd<T, CAUSAL, 128, WINDOW, VARLEN, BALANCED>(p, grid, stream);
    case 256: return fa::launch_fwd<T, CAUSAL, 256, WINDOW, VARLEN, BALANCED>(p, grid, stream);
    default: return FA_ERR_HEAD_DIM;
  }
}

// Whether a dense launch takes the balanced instance: at D <= 128, with a key range of at least
// kBalanceMinKvTiles tiles and at least kBalanceMinRounds rounds of items on some XCD, with or
// without the causal mask. Shorter launches lose more to the claims, and under the mask to the
// long/short pairing the claimed tail gives up, than the uneven XCD clocks cost them; at D = 256
// (32-key tiles, 16 MiB of K and V per unit at N = 16384) a stolen item's cold K/V stream costs
// more than it saves.
static_assert(fa::kBalanceCounters == FA_BALANCE_COUNTERS, "counter buffer size");
constexpr int64_t kBalanceMinKvTiles = 128;
constexpr uint32_t kBalanceMinRounds = 8;

bool use_balance(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nkv, int64_t D, int64_t n_qt, int64_t grid, int bkv,
                 bool causal) {
  if (D > 128 || (Nkv + bkv - 1) / bkv < kBalanceMinKvTiles) return false;
  const fa::Schedule sched{(int)(B * Hkv), (int)Hkv, (int)(Hq / Hkv), (int)n_qt, causal, (int)grid};
  uint32_t rounds = 0;
  for (int x = 0; x < 8; ++x) {
    const int gx = sched.wgs_of(x);
    if (gx > 0) rounds = std::max(rounds, (sched.items_of(x) + (uint32_t)gx - 1) / (uint32_t)gx);
  }
  return rounds >= kBalanceMinRounds;
}

// Shared validation and parameter setup of the forward entry points.
int prepare_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq, int64_t Hkv,
                int64_t Nq, int64_t Nkv, int64_t D, const int64_t* q_stride, const int64_t* k_stride,
                const int64_t* v_stride, const int64_t* o_stride, float scale, bool causal, int dtype, FwdParams* p,
                int64_t* grid) {
  if (!q || !k || !v || !o || !lse || !q_stride || !k_stride || !v_stride || !o_stride) return FA_ERR_NULL;
  PlanInfo pi;
  int64_t n_qt = 0;
  int rc = check_shape(B, Hq, Hkv, Nq, Nkv, D, dtype, causal, &pi, &n_qt, grid);
  if (rc != FA_OK) return rc;
  if (!(std::isfinite(scale) && scale > 0.f)) return FA_ERR_SCALE;
  if ((rc = check_strides(q_stride, false, B, Hq, Nq)) != FA_OK) return rc;
  if ((rc = check_strides(k_stride, false, B, Hkv, Nkv)) != FA_OK) return rc;
  if ((rc = check_strides(v_stride, false, B, Hkv, Nkv)) != FA_OK) return rc;
  if ((rc = check_strides(o_stride, true, B, Hq, Nq)) != FA_OK) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FA_ERR_LAYOUT;
  if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return FA_ERR_LAYOUT;
  if (!extent_ok(B, Hq, Nq, D, q_stride) || !extent_ok(B, Hkv, Nkv, D, k_stride) ||
      !extent_ok(B, Hkv, Nkv, D, v_stride) || !extent_ok(B, Hq, Nq, D, o_stride))
    return FA_ERR_SHAPE;
  p->q = q;
  p->k = k;
  p->v = v;
  p->o = o;
  p->lse = lse;
  p->q_sb = q_stride[0]; p->q_sh = q_stride[1]; p->q_sn = q_stride[2];
  p->k_sb = k_stride[0]; p->k_sh = k_stride[1]; p->k_sn = k_stride[2];
  p->v_sb = v_stride[0]; p->v_sh = v_stride[1]; p->v_sn = v_stride[2];
  p->o_sb = o_stride[0]; p->o_sh = o_stride[1]; p->o_sn = o_stride[2];
  p->B = (int32_t)B;
  p->Hq = (int32_t)Hq;
  p->Hkv = (int32_t)Hkv;
  p->Nq = (int32_t)Nq;
  p->Nkv = (int32_t)Nkv;
  p->group = (int32_t)(Hq / Hkv);
  p->n_qtiles = (int32_t)n_qt;
  // scores enter the base-2 softmax as s * scale * log2(e), one fp32 FMA per score
  p->c = (float)((double)scale * 1.4426950408889634074);
  p->win_left = (int32_t)Nq;
  p->win_right = (int32_t)Nkv;
  p->cu_q = nullptr;
  p->cu_k = nullptr;
  p->total_q = 0;
  p->total_k = 0;
  p->lse_sb = Hq * Nq;
  p->lse_sh = Nq;
  p->balance = nullptr;
  return FA_OK;
}

template <typename T, bool CAUSAL, bool WINDOW = false, bool VARLEN = false>
int launch_bwd_d(int64_t D, const fa::BwdParams& p, hipStream_t stream) {
  switch (D) {
    case 16: return fa::launch_bwd<T, CAUSAL, 16, WINDOW, VARLEN>(p, stream);
    case 32: return fa::launch_bwd<T, CAUSAL, 32, WINDOW, VARLEN>(p, stream);
    case 64: return fa::launch_bwd<T, CAUSAL, 64, WINDOW, VARLEN>(p, stream);
    case 128: return fa::launch_bwd<T, CAUSAL, 128, WINDOW, VARLEN>(p, stream);
    case 256: return fa::launch_bwd<T, CAUSAL, 256, WINDOW, VARLEN>(p, stream);
    default: return FA_ERR_HEAD_DIM;
  }
}

// ---- fa_bwd_noalloc: Delta in a fixed device array instead of a caller workspace. Each GPU holds
// its own copy at its own address; host code must use that address (looked up once per device with
// hipGetSymbolAddress), never the array's name, which on the host is only a stand-in.
static __device__ __align__(256) float scratch[FA_NOALLOC_MAX_ROWS];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the device that `stream` belongs to (the current device for the
// null stream); nullptr on a HIP error.
float* scratch_for(hipStream_t stream) {
  int dev = -1;
  const hipError_t qe = stream == nullptr ? hipGetDevice(&dev) : hipStreamGetDevice(stream, &dev);
  if (qe != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) return nullptr;
    if (prev != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (prev != dev && hipSetDevice(prev) != hipSuccess) return nullptr;
    if (e != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch_ptr[dev] = static_cast<float*>(ptr);
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int fa_version(void) { return FA_ABI_VERSION; }

const char* fa_strerror(int code) {
  switch (code) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_DTYPE: return "unsupported dtype (expected FA_DTYPE_F16 or FA_DTYPE_BF16)";
    case FA_ERR_HEAD_DIM: return "unsupported head dim (expected 16, 32, 64, 128 or 256)";
    case FA_ERR_GQA: return "query heads must be a positive multiple of key/value heads";
    case FA_ERR_SHAPE: return "sizes must be >= 1 and < 2^31, and addressed extents must not overflow";
    case FA_ERR_LAYOUT:
      return "unsupported layout (head-dim stride must be 1; strides >= 0 and pointers 16-byte aligned; "
             "no zero output strides)";
    case FA_ERR_SCALE: return "scale must be a finite number > 0";
    case FA_ERR_HIP: return "HIP kernel launch failed";
    case FA_ERR_SCRATCH:
      return "fa_bwd_noalloc: B * Hq * Nq exceeds the fixed Delta array of FA_NOALLOC_MAX_ROWS (4194304) rows";
    default: return "unknown error code";
  }
}

int64_t fa_tile_pairs(int64_t Nq, int64_t Nkv, int64_t bq, int64_t bkv, int causal) {
  if (Nq < 1 || Nkv < 1 || bq < 1 || bkv < 1) return -1;
  const int64_t n_qt = (Nq + bq - 1) / bq;
  int64_t total = 0;
  for (int64_t t = 0; t < n_qt; ++t) total += fa::kv_tiles_for_qtile(t * bq, bq, Nkv, bkv, causal != 0);
  return total;
}

int fa_fwd_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, int causal, int dtype,
                fa_plan* out) {
  if (!out) return FA_ERR_NULL;
  PlanInfo pi;
  int64_t n_qt = 0, grid = 0;
  const int rc = check_shape(B, Hq, Hkv, Nq, Nkv, D, dtype, causal != 0, &pi, &n_qt, &grid);
  if (rc != FA_OK) return rc;
  out->grid = grid;
  out->block_threads = pi.threads;
  out->block_q = pi.bq;
  out->block_kv = pi.bkv;
  out->lds_bytes = pi.lds;
  out->tile_pairs = fa_tile_pairs(Nq, Nkv, pi.bq, pi.bkv, causal) * B * Hq;
  return FA_OK;
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq, int64_t Hkv,
           int64_t Nq, int64_t Nkv, int64_t D, const int64_t q_stride[4], const int64_t k_stride[4],
           const int64_t v_stride[4], const int64_t o_stride[4], float scale, int causal, int dtype,
           void* stream) {
  FwdParams p;
  int64_t grid = 0;
  const int rc = prepare_fwd(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, q_stride, k_stride, v_stride, o_stride, scale,
                             causal != 0, dtype, &p, &grid);
  if (rc != FA_OK) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool cz = causal != 0;
  if (dtype == FA_DTYPE_BF16)
    return cz ? launch_d<__bf16, true>(D, p, grid, s) : launch_d<__bf16, false>(D, p, grid, s);
  return cz ? launch_d<_Float16, true>(D, p, grid, s) : launch_d<_Float16, false>(D, p, grid, s);
}

int fa_fwd_balance_applies(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, int causal,
                           int dtype) {
  PlanInfo pi;
  int64_t n_qt = 0, grid = 0;
  const int rc = check_shape(B, Hq, Hkv, Nq, Nkv, D, dtype, causal != 0, &pi, &n_qt, &grid);
  if (rc != FA_OK) return rc;
  return use_balance(B, Hq, Hkv, Nkv, D, n_qt, grid, pi.bkv, causal != 0) ? 1 : 0;
}

int fa_fwd_balanced(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                    int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, const int64_t q_stride[4],
                    const int64_t k_stride[4], const int64_t v_stride[4], const int64_t o_stride[4], float scale,
                    int causal, int dtype, uint32_t* counters, void* stream) {
  if (!counters) return FA_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(counters) & 63u) != 0) return FA_ERR_LAYOUT;
  FwdParams p;
  int64_t grid = 0;
  const int rc = prepare_fwd(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, q_stride, k_stride, v_stride, o_stride, scale,
                             causal != 0, dtype, &p, &grid);
  if (rc != FA_OK) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  PlanInfo pi;
  plan_for_d(D, &pi);
  if (!use_balance(B, Hq, Hkv, Nkv, D, p.n_qtiles, grid, pi.bkv, causal != 0)) {
    const bool cz = causal != 0;
    if (dtype == FA_DTYPE_BF16)
      return cz ? launch_d<__bf16, true>(D, p, grid, s) : launch_d<__bf16, false>(D, p, grid, s);
    return cz ? launch_d<_Float16, true>(D, p, grid, s) : launch_d<_Float16, false>(D, p, grid, s);
  }
  p.balance = counters;
  if (causal) {
    if (dtype == FA_DTYPE_BF16) return launch_d<__bf16, true, false, false, true>(D, p, grid, s);
    return launch_d<_Float16, true, false, false, true>(D, p, grid, s);
  }
  if (dtype == FA_DTYPE_BF16) return launch_d<__bf16, false, false, false, true>(D, p, grid, s);
  return launch_d<_Float16, false, false, false, true>(D, p, grid, s);
}

int fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                  int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, const int64_t q_stride[4],
                  const int64_t k_stride[4], const int64_t v_stride[4], const int64_t o_stride[4], float scale,
                  int64_t window_left, int64_t window_right, int dtype, void* stream) {
  FwdParams p;
  int64_t grid = 0;
  const int rc = prepare_fwd(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, q_stride, k_stride, v_stride, o_stride, scale,
                             false, dtype, &p, &grid);
  if (rc != FA_OK) return rc;
  if (window_left < -1 || window_right < -1) return FA_ERR_SHAPE;
  if (Nq > kMaxWindowSeq || Nkv > kMaxWindowSeq) return FA_ERR_SHAPE;
  // a side wider than the sequences reaches every key, the same as an unbounded side
  p.win_left = (int32_t)(window_left < 0 || window_left > Nq ? Nq : window_left);
  p.win_right = (int32_t)(window_right < 0 || window_right > Nkv ? Nkv : window_right);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == FA_DTYPE_BF16) return launch_d<__bf16, false, true>(D, p, grid, s);
  return launch_d<_Float16, false, true>(D, p, grid, s);
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* cu_seqlens_q,
                  const int32_t* cu_seqlens_k, int64_t B, int64_t Hq, int64_t Hkv, int64_t total_q,
                  int64_t total_k, int64_t max_seqlen_q, int64_t max_seqlen_k, int64_t D,
                  const int64_t q_stride[3], const int64_t k_stride[3], const int64_t v_stride[3],
                  const int64_t o_stride[3], float scale, int causal, int dtype, void* stream) {
  if (!cu_seqlens_q || !cu_seqlens_k || !q_stride || !k_stride || !v_stride || !o_stride) return FA_ERR_NULL;
  if (total_q < 1 || total_k < 1 || total_q > kMaxDim || total_k > kMaxDim) return FA_ERR_SHAPE;
  if (max_seqlen_q < 1 || max_seqlen_k < 1 || max_seqlen_q > total_q || max_seqlen_k > total_k) return FA_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) != 0 || (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u) != 0)
    return FA_ERR_LAYOUT;
  // token-major tensors: strides (token, head, dim), viewed as one batch of total tokens for the
  // layout and extent checks, and as B sequences with batch stride 0 by the kernel
  const int64_t qs[4] = {0, q_stride[1], q_stride[0], q_stride[2]};
  const int64_t ks[4] = {0, k_stride[1], k_stride[0], k_stride[2]};
  const int64_t vs[4] = {0, v_stride[1], v_stride[0], v_stride[2]};
  const int64_t os[4] = {0, o_stride[1], o_stride[0], o_stride[2]};
  // every token writes its own output row: the token stride of O is checked against all tokens here
  // (the per-sequence check below sees only the longest sequence, which may be one token long)
  if (total_q > 1 && o_stride[0] == 0) return FA_ERR_LAYOUT;
  if (!extent_ok(1, Hq, total_q, D, qs) || !extent_ok(1, Hkv, total_k, D, ks) || !extent_ok(1, Hkv, total_k, D, vs) ||
      !extent_ok(1, Hq, total_q, D, os))
    return FA_ERR_SHAPE;
  int64_t lse_n;
  if (!mul_ok(Hq, total_q, &lse_n) || lse_n > ((int64_t)1 << 62)) return FA_ERR_SHAPE;
  // strides, alignment and scale as one sequence of the longest lengths, then the grid for B sequences
  FwdParams p;
  int64_t grid = 0;
  int rc = prepare_fwd(q, k, v, o, lse, 1, Hq, Hkv, max_seqlen_q, max_seqlen_k, D, qs, ks, vs, os, scale, causal != 0,
                       dtype, &p, &grid);
  if (rc != FA_OK) return rc;
  PlanInfo pi;
  int64_t n_qt = 0;
  if ((rc = check_shape(B, Hq, Hkv, max_seqlen_q, max_seqlen_k, D, dtype, causal != 0, &pi, &n_qt, &grid)) != FA_OK)
    return rc;
  p.B = (int32_t)B;
  p.n_qtiles = (int32_t)n_qt;
  if (B + 1 > kMaxDim) return FA_ERR_SHAPE;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.total_q = (int32_t)total_q;
  p.total_k = (int32_t)total_k;
  p.lse_sb = 0;
  p.lse_sh = total_q;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool cz = causal != 0;
  if (dtype == FA_DTYPE_BF16)
    return cz ? launch_d<__bf16, true, false, true>(D, p, grid, s) : launch_d<__bf16, false, false, true>(D, p, grid, s);
  return cz ? launch_d<_Float16, true, false, true>(D, p, grid, s) : launch_d<_Float16, false, false, true>(D, p, grid, s);
}

// Validation and parameters of a backward call over B batches of Nq query / Nkv key rows (dense
// lengths; the window and the packed-sequence fields are filled in by the callers).
static int prepare_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                       const void* dout, void* dq, void* dk, void* dv, float* delta, int64_t B, int64_t Hq,
                       int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, const int64_t* q_stride,
                       const int64_t* k_stride, const int64_t* v_stride, const int64_t* o_stride,
                       const int64_t* do_stride, const int64_t* dq_stride, const int64_t* dk_stride,
                       const int64_t* dv_stride, float scale, bool causal, int dtype, fa::BwdParams* out) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !delta || !q_stride || !k_stride ||
      !v_stride || !o_stride || !do_stride || !dq_stride || !dk_stride || !dv_stride)
    return FA_ERR_NULL;
  PlanInfo pi;
  int64_t n_qt = 0, grid = 0;
  int rc = check_shape(B, Hq, Hkv, Nq, Nkv, D, dtype, causal, &pi, &n_qt, &grid);
  if (rc != FA_OK) return rc;
  // the gradient kernels use 1-D grids of (row block, head, batch) workgroups
  if (((Nkv + 127) / 128) * Hkv * B > kMaxDim || ((Nq + 127) / 128) * Hq * B > kMaxDim) return FA_ERR_SHAPE;
  if (!(std::isfinite(scale) && scale > 0.f)) return FA_ERR_SCALE;
  if ((rc = check_strides(q_stride, false, B, Hq, Nq)) != FA_OK) return rc;
  if ((rc = check_strides(k_stride, false, B, Hkv, Nkv)) != FA_OK) return rc;
  if ((rc = check_strides(v_stride, false, B, Hkv, Nkv)) != FA_OK) return rc;
  if ((rc = check_strides(o_stride, false, B, Hq, Nq)) != FA_OK) return rc;
  if ((rc = check_strides(do_stride, false, B, Hq, Nq)) != FA_OK) return rc;
  if ((rc = check_strides(dq_stride, true, B, Hq, Nq)) != FA_OK) return rc;
  if ((rc = check_strides(dk_stride, true, B, Hkv, Nkv)) != FA_OK) return rc;
  if ((rc = check_strides(dv_stride, true, B, Hkv, Nkv)) != FA_OK) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv))
    return FA_ERR_LAYOUT;
  if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0 || (reinterpret_cast<uintptr_t>(delta) & 3u) != 0)
    return FA_ERR_LAYOUT;
  if (!extent_ok(B, Hq, Nq, D, q_stride) || !extent_ok(B, Hkv, Nkv, D, k_stride) ||
      !extent_ok(B, Hkv, Nkv, D, v_stride) || !extent_ok(B, Hq, Nq, D, o_stride) ||
      !extent_ok(B, Hq, Nq, D, do_stride) || !extent_ok(B, Hq, Nq, D, dq_stride) ||
      !extent_ok(B, Hkv, Nkv, D, dk_stride) || !extent_ok(B, Hkv, Nkv, D, dv_stride))
    return FA_ERR_SHAPE;

  fa::BwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.dout = dout; p.lse = lse;
  p.dq = dq; p.dk = dk; p.dv = dv; p.delta = delta;
  p.q_sb = q_stride[0]; p.q_sh = q_stride[1]; p.q_sn = q_stride[2];
  p.k_sb = k_stride[0]; p.k_sh = k_stride[1]; p.k_sn = k_stride[2];
  p.v_sb = v_stride[0]; p.v_sh = v_stride[1]; p.v_sn = v_stride[2];
  p.o_sb = o_stride[0]; p.o_sh = o_stride[1]; p.o_sn = o_stride[2];
  p.do_sb = do_stride[0]; p.do_sh = do_stride[1]; p.do_sn = do_stride[2];
  p.dq_sb = dq_stride[0]; p.dq_sh = dq_stride[1]; p.dq_sn = dq_stride[2];
  p.dk_sb = dk_stride[0]; p.dk_sh = dk_stride[1]; p.dk_sn = dk_stride[2];
  p.dv_sb = dv_stride[0]; p.dv_sh = dv_stride[1]; p.dv_sn = dv_stride[2];
  p.B = (int32_t)B;
  p.Hq = (int32_t)Hq;
  p.Hkv = (int32_t)Hkv;
  p.Nq = (int32_t)Nq;
  p.Nkv = (int32_t)Nkv;
  p.group = (int32_t)(Hq / Hkv);
  p.c = (float)((double)scale * 1.4426950408889634074);
  p.scale = scale;
  p.win_left = (int32_t)Nq;
  p.win_right = (int32_t)Nkv;
  p.cu_q = nullptr;
  p.cu_k = nullptr;
  p.lse_sb = Hq * Nq;  // contiguous (B, Hq, Nq)
  p.lse_sh = Nq;
  *out = p;
  return FA_OK;
}

static int bwd_entry(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, float* delta, int64_t B, int64_t Hq,
                     int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, const int64_t* q_stride,
                     const int64_t* k_stride, const int64_t* v_stride, const int64_t* o_stride,
                     const int64_t* do_stride, const int64_t* dq_stride, const int64_t* dk_stride,
                     const int64_t* dv_stride, float scale, int causal, bool window, int64_t window_left,
                     int64_t window_right, int dtype, void* stream) {
  fa::BwdParams p;
  const int rc = prepare_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, Hq, Hkv, Nq, Nkv, D, q_stride, k_stride,
                             v_stride, o_stride, do_stride, dq_stride, dk_stride, dv_stride, scale, causal != 0,
                             dtype, &p);
  if (rc != FA_OK) return rc;
  if (window) {
    if (window_left < -1 || window_right < -1) return FA_ERR_SHAPE;
    if (Nq > kMaxWindowSeq || Nkv > kMaxWindowSeq) return FA_ERR_SHAPE;
    p.win_left = (int32_t)(window_left < 0 || window_left > Nq ? Nq : window_left);
    p.win_right = (int32_t)(window_right < 0 || window_right > Nkv ? Nkv : window_right);
  }

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool cz = causal != 0;
  if (window) return dtype == FA_DTYPE_BF16 ? launch_bwd_d<__bf16, false, true>(D, p, s)
                                            : launch_bwd_d<_Float16, false, true>(D, p, s);
  if (dtype == FA_DTYPE_BF16)
    return cz ? launch_bwd_d<__bf16, true>(D, p, s) : launch_bwd_d<__bf16, false>(D, p, s);
  return cz ? launch_bwd_d<_Float16, true>(D, p, s) : launch_bwd_d<_Float16, false>(D, p, s);
}


int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
           void* dq, void* dk, void* dv, float* delta, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
           int64_t Nkv, int64_t D, const int64_t q_stride[4], const int64_t k_stride[4],
           const int64_t v_stride[4], const int64_t o_stride[4], const int64_t do_stride[4],
           const int64_t dq_stride[4], const int64_t dk_stride[4], const int64_t dv_stride[4], float scale,
           int causal, int dtype, void* stream) {
  return bwd_entry(q, k, v, o, lse, dout, dq, dk, dv, delta, B, Hq, Hkv, Nq, Nkv, D, q_stride, k_stride, v_stride,
                   o_stride, do_stride, dq_stride, dk_stride, dv_stride, scale, causal, false, -1, -1, dtype, stream);
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                   void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv,
                   int64_t D, const int64_t q_stride[4], const int64_t k_stride[4], const int64_t v_stride[4],
                   const int64_t o_stride[4], const int64_t do_stride[4], const int64_t dq_stride[4],
                   const int64_t dk_stride[4], const int64_t dv_stride[4], float scale, int causal, int dtype,
                   void* stream) {
  // validate as fa_bwd does, with a placeholder (non-null, aligned) workspace pointer
  fa::BwdParams p;
  float* const placeholder = reinterpret_cast<float*>(uintptr_t(256));
  int rc = prepare_bwd(q, k, v, o, lse, dout, dq, dk, dv, placeholder, B, Hq, Hkv, Nq, Nkv, D, q_stride, k_stride,
                       v_stride, o_stride, do_stride, dq_stride, dk_stride, dv_stride, scale, causal != 0, dtype, &p);
  if (rc != FA_OK) return rc;
  if (B * Hq * Nq > (int64_t)FA_NOALLOC_MAX_ROWS) return FA_ERR_SCRATCH;  // no overflow: check_shape bounds it
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  float* const delta = scratch_for(s);
  if (delta == nullptr) return FA_ERR_HIP;
  p.delta = delta;
  const bool cz = causal != 0;
  if (dtype == FA_DTYPE_BF16)
    return cz ? launch_bwd_d<__bf16, true>(D, p, s) : launch_bwd_d<__bf16, false>(D, p, s);
  return cz ? launch_bwd_d<_Float16, true>(D, p, s) : launch_bwd_d<_Float16, false>(D, p, s);
}

int fa_bwd_window(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, float* delta, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
                  int64_t Nkv, int64_t D, const int64_t q_stride[4], const int64_t k_stride[4],
                  const int64_t v_stride[4], const int64_t o_stride[4], const int64_t do_stride[4],
                  const int64_t dq_stride[4], const int64_t dk_stride[4], const int64_t dv_stride[4], float scale,
                  int64_t window_left, int64_t window_right, int dtype, void* stream) {
  return bwd_entry(q, k, v, o, lse, dout, dq, dk, dv, delta, B, Hq, Hkv, Nq, Nkv, D, q_stride, k_stride, v_stride,
                   o_stride, do_stride, dq_stride, dk_stride, dv_stride, scale, 0, true, window_left, window_right,
                   dtype, stream);
}

int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, float* delta, const int32_t* cu_seqlens_q,
                  const int32_t* cu_seqlens_k, int64_t B, int64_t Hq, int64_t Hkv, int64_t total_q, int64_t total_k,
                  int64_t max_seqlen_q, int64_t max_seqlen_k, int64_t D, const int64_t q_stride[3],
                  const int64_t k_stride[3], const int64_t v_stride[3], const int64_t o_stride[3],
                  const int64_t do_stride[3], const int64_t dq_stride[3], const int64_t dk_stride[3],
                  const int64_t dv_stride[3], float scale, int causal, int dtype, void* stream) {
  if (!cu_seqlens_q || !cu_seqlens_k || !q_stride || !k_stride || !v_stride || !o_stride || !do_stride ||
      !dq_stride || !dk_stride || !dv_stride)
    return FA_ERR_NULL;
  if (total_q < 1 || total_k < 1 || total_q > kMaxDim || total_k > kMaxDim) return FA_ERR_SHAPE;
  if (max_seqlen_q < 1 || max_seqlen_k < 1 || max_seqlen_q > total_q || max_seqlen_k > total_k) return FA_ERR_SHAPE;
  if (B < 1 || B + 1 > kMaxDim) return FA_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) != 0 || (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u) != 0)
    return FA_ERR_LAYOUT;
  // token-major tensors, strides (token, head, dim): validated as one batch of all the tokens, then
  // run as B sequences with batch stride 0 and the longest lengths
  auto st4 = [](const int64_t* s3, int64_t* s4) {
    s4[0] = 0;
    s4[1] = s3[1];
    s4[2] = s3[0];
    s4[3] = s3[2];
  };
  int64_t qs[4], ks[4], vs[4], os[4], dos[4], dqs[4], dks[4], dvs[4];
  st4(q_stride, qs);
  st4(k_stride, ks);
  st4(v_stride, vs);
  st4(o_stride, os);
  st4(do_stride, dos);
  st4(dq_stride, dqs);
  st4(dk_stride, dks);
  st4(dv_stride, dvs);
  fa::BwdParams p;
  int rc = prepare_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, 1, Hq, Hkv, total_q, total_k, D, qs, ks, vs, os, dos,
                       dqs, dks, dvs, scale, causal != 0, dtype, &p);
  if (rc != FA_OK) return rc;
  // the grids cover B sequences of the longest lengths
  if (((max_seqlen_k + 127) / 128) * Hkv * B > kMaxDim || ((max_seqlen_q + 127) / 128) * Hq * B > kMaxDim)
    return FA_ERR_SHAPE;
  p.B = (int32_t)B;
  p.Nq = (int32_t)max_seqlen_q;
  p.Nkv = (int32_t)max_seqlen_k;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.total_q = (int32_t)total_q;
  p.total_k = (int32_t)total_k;
  p.lse_sb = 0;  // (Hq, total_q), as fa_fwd_varlen writes it
  p.lse_sh = total_q;
  p.win_left = (int32_t)max_seqlen_q;
  p.win_right = (int32_t)max_seqlen_k;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool cz = causal != 0;
  if (dtype == FA_DTYPE_BF16)
    return cz ? launch_bwd_d<__bf16, true, false, true>(D, p, s) : launch_bwd_d<__bf16, false, false, true>(D, p, s);
  return cz ? launch_bwd_d<_Float16, true, false, true>(D, p, s) : launch_bwd_d<_Float16, false, false, true>(D, p, s);
}

}  // extern "C"
