// fa_bwd_inst.hip - the backward kernel instances of one (element type, head
// dim): Delta, dK/dV and dQ for the dense non-causal and causal masks, the
// sliding window, and packed sequences with and without the causal mask.
// Compiled once per -DFA_INST_T (0 = fp16, 1 = bf16) and -DFA_INST_D.
#include "fa.h"
#include "fa_launch.h"

#if !defined(FA_INST_T) || !defined(FA_INST_D)
#error "compile with -DFA_INST_T=<0|1> -DFA_INST_D=<head dim>"
#endif

namespace fa {

template <typename T, bool CAUSAL, int D, bool WINDOW, bool VARLEN>
int launch_bwd(BwdParams p, hipStream_t stream) {
  typedef typename BwdCfgFor<D>::dkdv CK;
  typedef typename BwdCfgFor<D>::dq CQ;
  // row block slowest under the causal mask (longest first), and when a grid is at most about two
  // rounds of resident workgroups (the blocks of a head then run together on one XCD and share its
  // streamed tiles in L2); otherwise the blocks of a head are dispatched consecutively
  const int64_t kv_wgs = (int64_t)((p.Nkv + CK::BW - 1) / CK::BW) * p.Hkv * p.B;
  const int64_t q_wgs = (int64_t)((p.Nq + CQ::BW - 1) / CQ::BW) * p.Hq * p.B;
  p.dkdv_block_slowest = CAUSAL || kv_wgs <= 2 * kNumCUs * (CK::WAVES_PER_SIMD * 4 / CK::NW);
  p.dq_block_slowest = CAUSAL || q_wgs <= 2 * kNumCUs * (CQ::WAVES_PER_SIMD * 4 / CQ::NW);
  constexpr int RPB = 256 / (D / 8);
  // Delta is per token: packed sequences run it as one batch of total_q rows, which is the
  // (Hq, total_q) layout of their logsumexp
  BwdParams pd = p;
  if (VARLEN) {
    pd.B = 1;
    pd.Nq = p.total_q;
    pd.o_sb = 0;
    pd.do_sb = 0;
  }
  const int64_t rows = (int64_t)pd.B * pd.Hq * pd.Nq;
  hipLaunchKernelGGL((fa_bwd_delta_kernel<T, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, stream, pd);
  if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
  const dim3 kv_grid((unsigned)kv_wgs);
  if constexpr (BwdCfgFor<D>::SPLIT_KV) {
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<T, CAUSAL, CK, kBwdOnlyV, WINDOW, VARLEN>), kv_grid, dim3(CK::THREADS), 0,
                       stream, p);
    if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<T, CAUSAL, CK, kBwdOnlyK, WINDOW, VARLEN>), kv_grid, dim3(CK::THREADS), 0,
                       stream, p);
  } else {
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<T, CAUSAL, CK, kBwdBoth, WINDOW, VARLEN>), kv_grid, dim3(CK::THREADS), 0,
                       stream, p);
  }
  if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
  hipLaunchKernelGGL((fa_bwd_dq_kernel<T, CAUSAL, CQ, WINDOW, VARLEN>), dim3((unsigned)q_wgs), dim3(CQ::THREADS), 0,
                     stream, p);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

#if FA_INST_T == 1
typedef __bf16 InstT;
#else
typedef _Float16 InstT;
#endif

template int launch_bwd<InstT, false, FA_INST_D, false, false>(BwdParams, hipStream_t);
template int launch_bwd<InstT, true, FA_INST_D, false, false>(BwdParams, hipStream_t);
template int launch_bwd<InstT, false, FA_INST_D, true, false>(BwdParams, hipStream_t);
template int launch_bwd<InstT, false, FA_INST_D, false, true>(BwdParams, hipStream_t);
template int launch_bwd<InstT, true, FA_INST_D, false, true>(BwdParams, hipStream_t);

}  // namespace fa
