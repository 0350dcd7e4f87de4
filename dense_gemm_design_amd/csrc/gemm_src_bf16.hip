// The wide-wave kernels' source-reading instantiations for BF16 operands (fused epilogue
// with Z = alpha * Acc + beta * S, "H100 Kernel Design" lesson, section 12.2 step 2): one kernel
// per activation and K raggedness for each tile configuration, in a translation unit of their
// own so that they compile in parallel with the rest of the library.
#include "launch.h"

namespace dg {

template <class CFG>
hipError_t launch_wide_src(const KernelArgs &a, int grid, bool ragged_k, hipStream_t s) {
  launch_wide_act<CFG, FUSE_SRC>(a, grid, ragged_k, s);
  return hipGetLastError();
}

template hipError_t launch_wide_src<CfgBf16_256w>(const KernelArgs &, int, bool, hipStream_t);
template hipError_t launch_wide_src<CfgBf16_128w>(const KernelArgs &, int, bool, hipStream_t);
template hipError_t launch_wide_src<CfgBf16_224w>(const KernelArgs &, int, bool, hipStream_t);
template hipError_t launch_wide_src<CfgBf16_192w>(const KernelArgs &, int, bool, hipStream_t);

}  // namespace dg
