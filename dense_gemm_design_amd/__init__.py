"""MI355X-native tiled dense GEMM (BF16, FP8 e4m3 with per-tensor FP32 scales, FP32 accumulate).

The compute path is the HIP library libdgemm.so (csrc/, C ABI in include/gemm.h); this package
is its Python binding.  See gemm() for a one-call helper on torch tensors.
"""
from . import _lib
from ._lib import (GemmDesc, GemmError, Plan, make_desc, load,  # noqa: F401
                   GEMM_BF16, GEMM_FP8_E4M3, GEMM_F32, GEMM_MAP_LINEAR_N, GEMM_MAP_LINEAR_M,
                   GEMM_MAP_GROUPED_M, GEMM_MAP_GROUPED_N, GEMM_SCHED_STATIC,
                   GEMM_SCHED_PERSISTENT, GEMM_SCHED_STREAMK, GEMM_SCHED_AUTO, GEMM_FLAG_TRACE,
                   GEMM_FLAG_NO_XCD_REMAP, GEMM_FLAG_STREAMK_CHAIN, GEMM_FLAG_PINGPONG,
                   GEMM_FLAG_COOPERATIVE, GEMM_FLAG_REGSTAGED, GEMM_FLAG_WIDE)

MAPPINGS = {"linear_n": GEMM_MAP_LINEAR_N, "linear_m": GEMM_MAP_LINEAR_M,
            "grouped_m": GEMM_MAP_GROUPED_M, "grouped_n": GEMM_MAP_GROUPED_N}
SCHEDS = {"static": GEMM_SCHED_STATIC, "persistent": GEMM_SCHED_PERSISTENT,
          "streamk": GEMM_SCHED_STREAMK, "auto": GEMM_SCHED_AUTO}


def gemm(A, B, out_dtype="f32", scale_a=None, scale_b=None, mapping="grouped_m", group=8,
         sched="auto", tile=0, flags=0):
    """C = alpha * A x B for torch device tensors: A (M, K) row-major; B given as (N, K), i.e. the
    K x N operand in column-major storage; bf16 or uint8-coded e4m3 (then scale_a / scale_b are
    one-element float32 device tensors).  Returns C (M, N) in float32 or bfloat16."""
    import torch
    M, K = A.shape
    N = B.shape[0]
    fp8 = A.dtype in (torch.uint8, torch.float8_e4m3fn)
    desc = make_desc(M, N, K, GEMM_FP8_E4M3 if fp8 else GEMM_BF16,
                     GEMM_BF16 if out_dtype == "bf16" else GEMM_F32, MAPPINGS[mapping], group,
                     SCHEDS[sched], 0, tile, tile, 0, flags)
    plan = Plan(desc)
    C = torch.empty((M, N), device=A.device,
                    dtype=torch.bfloat16 if out_dtype == "bf16" else torch.float32)
    ws = None
    if plan.workspace_bytes:
        ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=A.device)
    plan.run(A, B, C, scale_a, scale_b, ws)
    return C
