// fa_fwd_inst.hip - the forward kernel instances of one (element type, head dim):
// dense non-causal and causal, sliding window, packed sequences with and
// without the causal mask. Compiled once per -DFA_INST_T (0 = fp16, 1 = bf16)
// and -DFA_INST_D (16, 32, 64, 128, 256).
#include "fa.h"
#include "fa_launch.h"

#if !defined(FA_INST_T) || !defined(FA_INST_D)
#error "compile with -DFA_INST_T=<0|1> -DFA_INST_D=<head dim>"
#endif

namespace fa {

template <typename T, bool CAUSAL, int D, bool WINDOW, bool VARLEN, bool BALANCED>
int launch_fwd(const FwdParams& p, int64_t grid, hipStream_t stream) {
  typedef typename CfgFor<D>::type C;
  hipLaunchKernelGGL((fa_fwd_kernel<T, CAUSAL, C, WINDOW, VARLEN, BALANCED>), dim3((unsigned)grid), dim3(C::THREADS),
                     0, stream, p);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

#if FA_INST_T == 1
typedef __bf16 InstT;
#else
typedef _Float16 InstT;
#endif

template int launch_fwd<InstT, false, FA_INST_D, false, false>(const FwdParams&, int64_t, hipStream_t);
template int launch_fwd<InstT, true, FA_INST_D, false, false>(const FwdParams&, int64_t, hipStream_t);
template int launch_fwd<InstT, false, FA_INST_D, true, false>(const FwdParams&, int64_t, hipStream_t);
template int launch_fwd<InstT, false, FA_INST_D, false, true>(const FwdParams&, int64_t, hipStream_t);
template int launch_fwd<InstT, true, FA_INST_D, false, true>(const FwdParams&, int64_t, hipStream_t);
template int launch_fwd<InstT, true, FA_INST_D, false, false, true>(const FwdParams&, int64_t, hipStream_t);
template int launch_fwd<InstT, false, FA_INST_D, false, false, true>(const FwdParams&, int64_t, hipStream_t);

}  // namespace fa

#ifdef FA_TIMELINE
// Timeline build only: copy this instance's timeline words (see g_timeline) to host memory.
#define FA_TL_JOIN(a, b, c, d) a##b##c##d
#define FA_TL_NAME(t, d) FA_TL_JOIN(fa_timeline_read_t, t, _d, d)
extern "C" int FA_TL_NAME(FA_INST_T, FA_INST_D)(void* dst, int64_t n_words) {
  if (dst == nullptr || n_words < 0 || n_words > (int64_t)fa::kTimelineWgs * fa::kTimelineWords) return FA_ERR_SHAPE;
  return hipMemcpyFromSymbol(dst, HIP_SYMBOL(fa::g_timeline), (size_t)n_words * 8, 0, hipMemcpyDeviceToHost) ==
                 hipSuccess
             ? FA_OK
             : FA_ERR_HIP;
}
#endif
