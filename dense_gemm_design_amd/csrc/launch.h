// Tile configurations of the kernels and the wide-wave kernels' launch helpers, shared by the
// library's translation units: gemm.hip (planner, ABI, every kernel but the source-reading ones)
// and gemm_src_bf16.hip / gemm_src_fp8.hip (the wide-wave kernels' instantiations that read a
// source matrix, compiled on their own so that the build runs them in parallel).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_kernel.h"

namespace dg {

// Tile configurations: TileCfg<dtype, BM, BN, BK, wave rows, wave columns, stages, swizzle>.
// SWZ spreads the 16 rows one 16-lane LDS read phase touches over 16 distinct 16-byte bank groups
// (1 for 128-byte rows, 2 for 64-byte rows).  Defaults (first match per tile shape): 8 waves of
// 128 x 64 sub-tiles with 2 stages of 64 KiB -- two waves per SIMD hide each other's LDS waits.
// The ping-pong kernel (GEMM_FLAG_PINGPONG) runs the same 256 x 256 tiles with two wave groups.
using CfgBf16_256pp = TileCfg<DT_BF16, 256, 256, 64, 2, 4, 2, 1>;
using CfgBf16_256 = TileCfg<DT_BF16, 256, 256, 64, 2, 4, 2, 1>;
using CfgBf16_128 = TileCfg<DT_BF16, 128, 128, 64, 2, 2, 2, 1>;
using CfgFp8_256pp = TileCfg<DT_FP8, 256, 256, 128, 2, 4, 2, 1>;
using CfgFp8_256 = TileCfg<DT_FP8, 256, 256, 128, 2, 4, 2, 1>;
using CfgFp8_128 = TileCfg<DT_FP8, 128, 128, 128, 2, 2, 2, 1>;
// The wide-wave kernel (GEMM_FLAG_WIDE): four waves of 128 x 128, two stages of 64 KiB.
using CfgBf16_256w = TileCfg<DT_BF16, 256, 256, 64, 2, 2, 2, 1, 16>;  // 16 x 16 x 32 MFMAs
using CfgFp8_256w = TileCfg<DT_FP8, 256, 256, 128, 2, 2, 2, 1, 16>;  // 16 x 16 x 128 MFMAs
// ... and on 128 x 128 tiles: four waves of 64 x 64, four stages of 32 KiB (a k-step of this
// tile is a quarter as long, so its loads need three k-steps of lead to land: measured 17 % faster
// at 4096^3 and 34 % on 1024 x 1024 x 16384 e4m3 than two stages)
using CfgBf16_128w = TileCfg<DT_BF16, 128, 128, 64, 2, 2, 4, 1, 16>;
using CfgFp8_128w = TileCfg<DT_FP8, 128, 128, 128, 2, 2, 4, 1, 16>;
// ... and on 256 x 224 tiles (waves of 128 x 112): a block width from the heuristic's aligned set
// below 256 that fills whole waves where 256 does not -- N = 14336 is 64 such columns, so
// 4096 x 14336 makes 1024 tiles, four full waves of 256 CUs, where 256 x 256 tiles leave the
// fourth wave half empty
using CfgBf16_224w = TileCfg<DT_BF16, 256, 224, 64, 2, 2, 2, 1, 16>;
using CfgFp8_224w = TileCfg<DT_FP8, 256, 224, 128, 2, 2, 2, 1, 16>;
// ... and on 256 x 192 tiles (waves of 128 x 96), the next width of that set: N a multiple of
// 6,144 makes whole waves of them (4096 x 6144: 512 tiles, two waves, where 256 x 256 tiles make
// one and a half)
using CfgBf16_192w = TileCfg<DT_BF16, 256, 192, 64, 2, 2, 2, 1, 16>;
using CfgFp8_192w = TileCfg<DT_FP8, 256, 192, 128, 2, 2, 2, 1, 16>;

// k-tiles one MFMA deep (e4m3 16 x 16 x 128) take the single-A-buffer form of the schedule
template <class CFG, bool RAGGED_K, int FUSE = FUSE_OFF>
constexpr auto wide_kernel() {
  if constexpr (CFG::KSUB == 1)
    return &gemm_kernel_wide1<CFG, RAGGED_K, FUSE>;
  else
    return &gemm_kernel_wide<CFG, RAGGED_K, FUSE>;
}
// activation of a fused plan, the wide-wave kernels' FUSE argument
inline int act_of(uint32_t epi) {
  return (epi & EPI_RELU) ? ACT_RELU : (epi & EPI_GELU) ? ACT_GELU : (epi & EPI_SILU) ? ACT_SILU
                                                                                   : ACT_NONE;
}
template <class CFG, int FUSE>
void launch_wide_as(const KernelArgs &a, int grid, bool ragged_k, hipStream_t s) {
  if (ragged_k)
    hipLaunchKernelGGL((wide_kernel<CFG, true, FUSE>()), dim3(grid), dim3(CFG::THREADS), 0, s, a);
  else
    hipLaunchKernelGGL((wide_kernel<CFG, false, FUSE>()), dim3(grid), dim3(CFG::THREADS), 0, s, a);
}
template <class CFG, int SRC>
void launch_wide_act(const KernelArgs &a, int grid, bool ragged_k, hipStream_t s) {
  switch (act_of(a.epi)) {
    case ACT_RELU: launch_wide_as<CFG, ACT_RELU | SRC>(a, grid, ragged_k, s); break;
    case ACT_GELU: launch_wide_as<CFG, ACT_GELU | SRC>(a, grid, ragged_k, s); break;
    case ACT_SILU: launch_wide_as<CFG, ACT_SILU | SRC>(a, grid, ragged_k, s); break;
    default: launch_wide_as<CFG, ACT_NONE | SRC>(a, grid, ragged_k, s); break;
  }
}

// Launch of a wide-wave plan whose epilogue reads a source matrix (EPI_SRC_* bits), defined in
// gemm_src_bf16.hip and gemm_src_fp8.hip for the wide-wave tile configurations.
template <class CFG>
hipError_t launch_wide_src(const KernelArgs &a, int grid, bool ragged_k, hipStream_t s);

}  // namespace dg
