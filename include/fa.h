/*
 * fa.h - C ABI of the gfx950 (MI355X) attention library (libfa.so): the fused
 * forward (fa_fwd) and its backward (fa_bwd).
 *
 * The library computes, for every batch b, query head h and query row i,
 *
 *     s_ij   = scale * <q[b,h,i,:], k[b,kvh,j,:]>       for the visible keys j
 *     o[b,h,i,:] = sum_j softmax_j(s_ij) * v[b,kvh,j,:]
 *     lse[b,h,i] = ln sum_j exp(s_ij)
 *
 * with kvh = h / (Hq / Hkv) (grouped-query / multi-query heads). This is the
 * fused attention forward described in "Build Triton-Ascend Fused Attention"
 * (Goal, Workflow, Implementation Pattern) and "Write Triton Attention Kernel"
 * (Required reasoning process, steps 1-9; Correctness requirements); the
 * score/softmax/output definition is the three-line forward of the
 * "FlashAttention on Ascend: Triton-Ascend CV pipeline" notes, section 1.
 * Without the causal flag every key is visible; with it, key j is visible to
 * query row i iff j <= i (zero-based positions, mask anchored at the top-left
 * corner, as in step 5c of "Write Triton Attention Kernel").
 *
 * Numerics: scores, the running row maximum, the softmax denominator and the
 * output accumulator are fp32; probabilities are rounded to the input dtype
 * (round to nearest even) before the P.V product; O is rounded to the input
 * dtype only at the final store; LSE is fp32 in natural-log units.
 */
#ifndef FA_H_
#define FA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 8

/* Element types of Q, K, V and O (all four share one type). */
#define FA_DTYPE_F16 0
#define FA_DTYPE_BF16 1

/* Return codes. 0 is success; every error is negative. A validation error is
 * reported before any HIP call: nothing is enqueued and O/LSE are untouched. */
#define FA_OK 0
#define FA_ERR_NULL -1      /* a required pointer (a tensor, lse, delta, a stride array, out) is NULL */
#define FA_ERR_DTYPE -2     /* dtype is not FA_DTYPE_F16 or FA_DTYPE_BF16 */
#define FA_ERR_HEAD_DIM -3  /* D is not one of 16, 32, 64, 128, 256 */
#define FA_ERR_GQA -4       /* Hkv < 1 or Hq is not a multiple of Hkv */
#define FA_ERR_SHAPE -5     /* a size is < 1, or a size or an addressed extent overflows */
#define FA_ERR_LAYOUT -6    /* a d-stride is not 1, a base address or b/h/n stride is not 16-byte aligned,
                               a stride is negative, the n-stride exceeds 2^22, or O has a zero stride */
#define FA_ERR_SCALE -7     /* scale is not a finite number > 0 */
#define FA_ERR_HIP -8       /* the kernel launch failed (hipGetLastError after the launch), or a HIP
                               query of fa_bwd_noalloc's set-up failed */
#define FA_ERR_SCRATCH -9   /* fa_bwd_noalloc: B * Hq * Nq exceeds FA_NOALLOC_MAX_ROWS */

/*
 * fa_fwd - enqueue one attention forward on `stream` and return.
 *
 * q   : device pointer, Q viewed as (B, Hq, Nq, D) with element strides q_stride
 * k   : device pointer, K viewed as (B, Hkv, Nkv, D) with element strides k_stride
 * v   : device pointer, V viewed as (B, Hkv, Nkv, D) with element strides v_stride
 * o   : device pointer, output O viewed as (B, Hq, Nq, D) with element strides o_stride
 * lse : device pointer, fp32 logsumexp, contiguous (B, Hq, Nq): lse[(b*Hq + h)*Nq + i]
 * *_stride : host arrays of 4 int64 element strides ordered (batch, head, sequence, dim).
 *       The dim stride must be 1; the other strides must be >= 0 and, like every
 *       base pointer, multiples of 16 bytes (the kernel moves 16-byte vectors).
 *       Otherwise strides are free (BSND storage viewed as BNSD is fine). Zero
 *       strides (broadcast views) are allowed for Q, K and V, not for O over a
 *       dimension of size > 1. The sequence stride must be at most 2^22 elements.
 * scale : score scale, a finite float > 0 (typically 1/sqrt(D)).
 * causal: 0 = every key visible; nonzero = top-left causal mask (key j visible to row i iff j <= i).
 * dtype : FA_DTYPE_F16 or FA_DTYPE_BF16, the element type of q, k, v and o.
 * stream: a hipStream_t of the device that holds the buffers (NULL = the default stream of the
 *         current device, which must then hold them).
 *
 * Sizes: 1 <= B, Hq, Hkv, Nq, Nkv < 2^31; D in {16, 32, 64, 128, 256}; Hq % Hkv == 0.
 * Nq and Nkv need not be multiples of any tile size, and Nq may differ from Nkv.
 *
 * Ownership: the caller owns every buffer; the library keeps no state, allocates
 * nothing and never synchronises. O and LSE must not overlap Q, K or V or each other.
 * Calls are thread-safe. The launch is asynchronous: errors in the running kernel
 * surface at the caller's next synchronisation, launch errors as FA_ERR_HIP.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D,
           const int64_t q_stride[4], const int64_t k_stride[4],
           const int64_t v_stride[4], const int64_t o_stride[4],
           float scale, int causal, int dtype, void* stream);

/*
 * fa_fwd_balanced - fa_fwd for callers that can lend it a small counter buffer, with which long
 * launches even out the uneven clocks of the chip's XCDs. The schedule of fa_fwd gives
 * every workgroup the same work, so a launch ends when its slowest XCD does; here, in a dense
 * launch (either mask) at D <= 128 with a key range of at least 128 tiles and at least 8 rounds of items, the last
 * rounds of each XCD's list (its shortest items) are claimed through the counters instead, and
 * an XCD that runs out takes items from the one with the most left. The outputs are bitwise those
 * of fa_fwd: every item is computed the same way whichever workgroup runs it. Other launches use
 * fa_fwd's schedule and leave the counters alone.
 *
 * counters: device pointer to FA_BALANCE_COUNTERS uint32 words, 64-byte aligned, zero before the
 *           buffer's first use; every call leaves them zero when its kernel ends. Calls that may
 *           run at the same time (other streams) need buffers of their own; calls in order on one
 *           stream can share one. FA_ERR_NULL / FA_ERR_LAYOUT for a NULL or misaligned pointer.
 *
 * Everything else (arguments, layout, ownership, errors) as in fa_fwd; the library allocates
 * nothing and keeps no state of its own.
 */
#define FA_BALANCE_COUNTERS 16

/* 1 if fa_fwd_balanced would claim items through its counters for this launch (a dense launch
 * at D <= 128 with a key range of at least 128 tiles and at least 8 rounds of items), 0 if it would use
 * fa_fwd's schedule; a negative FA_ERR_* code for arguments fa_fwd would reject. */
int fa_fwd_balance_applies(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D,
                           int causal, int dtype);
int fa_fwd_balanced(const void* q, const void* k, const void* v, void* o, float* lse,
                    int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D,
                    const int64_t q_stride[4], const int64_t k_stride[4],
                    const int64_t v_stride[4], const int64_t o_stride[4],
                    float scale, int causal, int dtype, uint32_t* counters, void* stream);

/*
 * fa_fwd_window - fa_fwd with a sliding-window mask in place of the causal flag: query row i
 * sees the keys j with i - window_left <= j <= i + window_right (zero-based positions, the same
 * top-left anchoring as the causal mask). window_left / window_right = -1 leaves that side
 * unbounded, so (-1, 0) is the causal mask and (-1, -1) no mask. The sliding-window mask is
 * one of the masking variants "Write Triton Attention Kernel" lists among its inputs (item 3).
 * A row whose window holds no key (e.g. row i >= Nkv with window_left = 0) has no softmax:
 * its O row is written as zeros and its LSE as -inf.
 *
 * Arguments, layout, ownership and errors as in fa_fwd; additionally window_left and
 * window_right must be >= -1 and Nq, Nkv <= 2^30 (FA_ERR_SHAPE otherwise).
 */
int fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                  int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D,
                  const int64_t q_stride[4], const int64_t k_stride[4],
                  const int64_t v_stride[4], const int64_t o_stride[4],
                  float scale, int64_t window_left, int64_t window_right, int dtype, void* stream);

/*
 * fa_fwd_varlen - the forward over packed variable-length sequences (the CSR layout "Write
 * Triton Attention Kernel" lists among its inputs, item 6; per its correctness requirements each
 * sequence's key loop ends at that sequence's own length and padding never contributes).
 *
 * q   : (total_q, Hq, D) token-major, strides q_stride = {token, head, dim} in elements
 * k, v: (total_k, Hkv, D), strides k_stride / v_stride likewise
 * o   : (total_q, Hq, D), strides o_stride
 * lse : fp32, contiguous (Hq, total_q): lse[h * total_q + token]
 * cu_seqlens_q, cu_seqlens_k : device int32 arrays of B + 1 offsets; sequence b owns query tokens
 *       [cu_seqlens_q[b], cu_seqlens_q[b+1]) and key/value tokens [cu_seqlens_k[b], cu_seqlens_k[b+1]).
 *       The caller guarantees 0 = cu[0] <= cu[1] <= ... <= cu[B] = total and every length <= the
 *       matching max_seqlen; the kernel clamps offsets to [0, total] and lengths to max_seqlen, so
 *       arrays breaking this give unspecified values but never an access outside the tensors.
 * max_seqlen_q, max_seqlen_k : the longest sequence lengths (>= 1, <= the totals); they size the grid.
 * causal: top-left causal mask per sequence (positions counted from each sequence's start).
 * A sequence with queries but no keys gets O = 0 and LSE = -inf on its rows. Other rules
 * (dtype, head dims, GQA, 16-byte strides and pointers, scale, stream, ownership, errors) as in
 * fa_fwd; 1 <= total_q, total_k < 2^31.
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                  int64_t B, int64_t Hq, int64_t Hkv, int64_t total_q, int64_t total_k,
                  int64_t max_seqlen_q, int64_t max_seqlen_k, int64_t D,
                  const int64_t q_stride[3], const int64_t k_stride[3],
                  const int64_t v_stride[3], const int64_t o_stride[3],
                  float scale, int causal, int dtype, void* stream);

/*
 * fa_bwd - enqueue the attention backward on `stream` and return: given the
 * forward's inputs, its output O and logsumexp LSE, and the gradient dO of a
 * loss with respect to O, write
 *
 *     dq = dS K,   dk = dS^T Q,   dv = P^T dO   (per query head; for grouped
 *                                              heads dk and dv sum the group)
 *
 * where P is the forward's softmax (recomputed from Q, K and LSE), dP = dO V^T,
 * Delta_i = sum_d O_id dO_id and dS = scale * P * (dP - Delta): the backward of
 * the Ascend notes ("FlashAttention on Ascend: Triton-Ascend CV pipeline",
 * section 2). LSE receives no gradient. Every gradient element is written once
 * by one workgroup (no atomics), so results are bitwise reproducible.
 *
 * q, k, v, o : the forward's tensors, as in fa_fwd (o with strides o_stride)
 * lse        : fp32 (B, Hq, Nq) contiguous, natural log, as written by fa_fwd
 * dout       : dO viewed as (B, Hq, Nq, D) with strides do_stride
 * dq, dk, dv : outputs, shaped like q, k, v, with strides dq_stride, dk_stride, dv_stride;
 *              every element is overwritten (no accumulation into existing values)
 * delta      : caller-provided fp32 workspace of B * Hq * Nq floats (4-byte aligned),
 *              overwritten with Delta, contiguous (B, Hq, Nq)
 * scale, causal, dtype, stream, and the stride and alignment rules: as in fa_fwd,
 *              with o and dout read-only inputs and dq, dk, dv outputs (no zero strides).
 *
 * Sizes as in fa_fwd, and ceil(N/128) * heads * B < 2^31 for both sequences. Ownership: the caller owns every
 * buffer; outputs and the workspace must not overlap any input or each other.
 * The library allocates nothing and never synchronises. Three kernels are
 * enqueued in order (Delta, then dK/dV, then dQ). Validation errors return
 * before any HIP call with nothing written.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
           void* dq, void* dk, void* dv, float* delta,
           int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D,
           const int64_t q_stride[4], const int64_t k_stride[4], const int64_t v_stride[4],
           const int64_t o_stride[4], const int64_t do_stride[4], const int64_t dq_stride[4],
           const int64_t dk_stride[4], const int64_t dv_stride[4],
           float scale, int causal, int dtype, void* stream);

/*
 * fa_bwd_window - fa_bwd for a forward run by fa_fwd_window: the same arguments, with the
 * window (window_left, window_right; -1 = unbounded side) in place of the causal flag. P is the
 * softmax over each row's window; a row whose window holds no key (LSE = -inf) gets dQ = 0 and
 * adds nothing to dK or dV. Validation as fa_bwd plus the window rules of fa_fwd_window.
 */
int fa_bwd_window(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, float* delta,
                  int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D,
                  const int64_t q_stride[4], const int64_t k_stride[4], const int64_t v_stride[4],
                  const int64_t o_stride[4], const int64_t do_stride[4], const int64_t dq_stride[4],
                  const int64_t dk_stride[4], const int64_t dv_stride[4],
                  float scale, int64_t window_left, int64_t window_right, int dtype, void* stream);

/*
 * fa_bwd_varlen - the backward of fa_fwd_varlen (packed variable-length sequences, "Write Triton
 * Attention Kernel", Inputs item 6): the tensors and offsets of that call plus
 *
 * dout       : dO, token-major (total_q, Hq, D) with strides do_stride (token, head, dim)
 * dq         : (total_q, Hq, D), strides dq_stride; dk, dv: (total_k, Hkv, D), strides dk_stride, dv_stride
 * lse        : fp32 (Hq, total_q) contiguous, as written by fa_fwd_varlen
 * delta      : caller-provided fp32 workspace of Hq * total_q floats, overwritten, laid out like lse
 *
 * Each sequence's gradients depend on its own tokens only: dk and dv of a sequence with keys but no
 * queries are zero, and dq of a sequence with queries but no keys is zero. Tokens outside every
 * sequence (before cu_seqlens[0] or after cu_seqlens[B]) are not written. Validation as
 * fa_fwd_varlen plus the output rules of fa_bwd; ceil(max_seqlen/128) * heads * B < 2^31.
 */
int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, float* delta,
                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                  int64_t B, int64_t Hq, int64_t Hkv, int64_t total_q, int64_t total_k,
                  int64_t max_seqlen_q, int64_t max_seqlen_k, int64_t D,
                  const int64_t q_stride[3], const int64_t k_stride[3], const int64_t v_stride[3],
                  const int64_t o_stride[3], const int64_t do_stride[3], const int64_t dq_stride[3],
                  const int64_t dk_stride[3], const int64_t dv_stride[3],
                  float scale, int causal, int dtype, void* stream);

/*
 * fa_bwd_noalloc - fa_bwd without the caller's Delta workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. The arguments, validation, results and kernels are those of fa_bwd without `delta`;
 * Delta is kept instead in a fixed device array of FA_NOALLOC_MAX_ROWS floats (16 MiB) inside the
 * library, which every GPU the library runs this on holds until the process ends. The entry point
 * itself allocates nothing: on its first call on a device it looks up that device's copy of the
 * array (hipStreamGetDevice, hipGetSymbolAddress) and remembers it.
 *
 * Limit: B * Hq * Nq <= FA_NOALLOC_MAX_ROWS, else FA_ERR_SCRATCH (checked after the other
 * validation, before any HIP call, nothing enqueued).
 * Sharing: all calls on one GPU use that GPU's single array, which keeps the last call's Delta.
 * Calls that overlap in time on one GPU (on different streams, or from several threads without
 * ordering) race on it and must not be issued; calls ordered on one stream are safe. Every Delta
 * row a call reads is written by the same call first, so nothing needs clearing between calls.
 */
#define FA_NOALLOC_MAX_ROWS 4194304
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                   void* dq, void* dk, void* dv,
                   int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D,
                   const int64_t q_stride[4], const int64_t k_stride[4], const int64_t v_stride[4],
                   const int64_t o_stride[4], const int64_t do_stride[4], const int64_t dq_stride[4],
                   const int64_t dk_stride[4], const int64_t dv_stride[4],
                   float scale, int causal, int dtype, void* stream);

/* Launch plan of fa_fwd for a shape, computed on the host without any HIP call. */
typedef struct fa_plan {
  int64_t grid;          /* workgroups launched */
  int32_t block_threads; /* threads per workgroup */
  int32_t block_q;       /* query rows per workgroup tile */
  int32_t block_kv;      /* key/value rows per inner-loop tile */
  int32_t lds_bytes;     /* LDS per workgroup */
  int64_t tile_pairs;    /* (query tile, key tile) pairs the kernel visits, summed over all workgroups */
} fa_plan;

/* Fill *out with the plan fa_fwd would use. Same validation codes as fa_fwd
 * (pointer and layout checks aside). */
int fa_fwd_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D,
                int causal, int dtype, fa_plan* out);

/*
 * Number of (query tile, key tile) pairs of an Nq x Nkv score matrix cut into
 * bq x bkv tiles that a forward visits: all of them without the mask; with the
 * top-left causal mask, for each query tile only the key tiles up to the one
 * holding its last visible key (the loop bound of "Write Triton Attention
 * Kernel", step 9, and the lower-triangle count of the Ascend notes, section 8).
 * Returns -1 on sizes < 1.
 */
int64_t fa_tile_pairs(int64_t Nq, int64_t Nkv, int64_t bq, int64_t bkv, int causal);

/* Static description of a return code (never NULL). */
const char* fa_strerror(int code);

/* FA_ABI_VERSION of the loaded library. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
