// fa_launch.h - tile configuration per head dim and the typed launchers of
// every kernel instance.
//
// The launchers are defined in fa_fwd_inst.hip and fa_bwd_inst.hip. The build
// compiles each of those once per (element type, head dim), selected with
// -DFA_INST_T and -DFA_INST_D, so the instances compile in parallel; the C ABI
// in fa_api.hip (validation, planning, dispatch) only declares them here.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_bwd_kernel.h"
#include "fa_fwd_kernel.h"

namespace fa {

constexpr int kNumCUs = 256;  // MI355X

// Forward tile configuration per head dim: four waves per workgroup, one 32-row query block per
// wave, and as many waves per SIMD as the registers allow (occupancy is what hides the softmax
// behind the other waves' MFMAs). D <= 32: four waves per SIMD; D = 64: three; D = 128: two
// (64 KiB of LDS per workgroup, two per CU); D = 256: two, with 32-key tiles.
template <int D>
struct CfgFor;
template <> struct CfgFor<16> { typedef TileCfg<16, 4, 1, 64, 4> type; };
template <> struct CfgFor<32> { typedef TileCfg<32, 4, 1, 64, 4> type; };
template <> struct CfgFor<64> { typedef TileCfg<64, 4, 1, 64, 3> type; };
template <> struct CfgFor<128> { typedef TileCfg<128, 4, 1, 64, 2> type; };
template <> struct CfgFor<256> { typedef TileCfg<256, 4, 1, 32, 2> type; };

// Backward, per head dim: the dK/dV kernel (32 keys per wave group, 64-row query tiles) and the dQ
// kernel (32 query rows per wave, 64-key tiles; 32 at D = 256). At D = 128 the dK/dV workgroup
// stages its 128 keys' K and V in LDS and runs eight waves, two per 32-key group (one per 32-row
// half of each query tile), so that it fits two waves per SIMD; below that a wave keeps its keys'
// K and V in registers at two waves per SIMD. At D = 256 dV and dK run as two launches (S
// recomputed in each) at one wave per SIMD. dQ: two waves per SIMD up to D = 128, otherwise one.
template <int D>
struct BwdCfgFor {
  static constexpr bool SPLIT_KV = D >= 256;
  static constexpr bool KV_LDS = D == 128;
  static constexpr int W_KV = D <= 128 ? 2 : 1;
  static constexpr int W_Q = D <= 128 ? 2 : 1;
  typedef BwdCfg<D, KV_LDS ? 8 : 4, 64, W_KV, KV_LDS> dkdv;
  typedef BwdCfg<D, 4, D >= 256 ? 32 : 64, W_Q> dq;
};

// Enqueue one forward instance on `stream` with a 1-D grid of `grid` workgroups (BALANCED: the
// instance with the claimed tail, dense launches only; p.balance must then hold the counters).
template <typename T, bool CAUSAL, int D, bool WINDOW, bool VARLEN, bool BALANCED = false>
int launch_fwd(const FwdParams& p, int64_t grid, hipStream_t stream);

// Enqueue the backward's kernels (Delta, dK/dV, dQ) of one instance on `stream`.
template <typename T, bool CAUSAL, int D, bool WINDOW, bool VARLEN>
int launch_bwd(BwdParams p, hipStream_t stream);

}  // namespace fa
