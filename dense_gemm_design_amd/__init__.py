"""MI355X-native tiled dense GEMM (BF16, FP8 e4m3 with per-tensor FP32 scales, FP32 accumulate).

The compute path is the HIP library libdgemm.so (csrc/, C ABI in include/gemm.h); this package
is its Python binding.  See gemm() for a one-call helper on torch tensors.
"""
from . import _lib
from ._lib import (GemmDesc, GemmError, Plan, make_desc, load,  # noqa: F401
                   GEMM_BF16, GEMM_FP8_E4M3, GEMM_F32, GEMM_MAP_LINEAR_N, GEMM_MAP_LINEAR_M,
                   GEMM_MAP_GROUPED_M, GEMM_MAP_GROUPED_N, GEMM_MAP_BLOCKED, GEMM_MAP_MORTON,
                   GEMM_SCHED_STATIC,
                   GEMM_SCHED_PERSISTENT, GEMM_SCHED_STREAMK, GEMM_SCHED_AUTO, GEMM_FLAG_TRACE,
                   GEMM_FLAG_NO_XCD_REMAP, GEMM_FLAG_STREAMK_CHAIN, GEMM_FLAG_PINGPONG,
                   GEMM_FLAG_COOPERATIVE, GEMM_FLAG_WIDE,
                   GEMM_EPI_BIAS_ROW, GEMM_EPI_BIAS_COL, GEMM_EPI_RELU, GEMM_EPI_GELU,
                   GEMM_EPI_SILU, GEMM_EPI_AMAX, GEMM_EPI_SOURCE_F32, GEMM_EPI_SOURCE_BF16,
                   GemmEpilogueArgs)

KERNEL_NAMES = {0: "cooperative", 1: "ping-pong", 3: "wide-wave"}  # gemm_plan_info.kernel
MAPPINGS = {"linear_n": GEMM_MAP_LINEAR_N, "linear_m": GEMM_MAP_LINEAR_M,
            "grouped_m": GEMM_MAP_GROUPED_M, "grouped_n": GEMM_MAP_GROUPED_N,
            "blocked": GEMM_MAP_BLOCKED, "morton": GEMM_MAP_MORTON}
SCHEDS = {"static": GEMM_SCHED_STATIC, "persistent": GEMM_SCHED_PERSISTENT,
          "streamk": GEMM_SCHED_STREAMK, "auto": GEMM_SCHED_AUTO}
ACTIVATIONS = {None: 0, "relu": GEMM_EPI_RELU, "gelu": GEMM_EPI_GELU, "silu": GEMM_EPI_SILU}
OUT_DTYPES = {"f32": GEMM_F32, "bf16": GEMM_BF16, "e4m3": GEMM_FP8_E4M3}


def gemm(A, B, out_dtype="f32", scale_a=None, scale_b=None, mapping="grouped_m", group=8,
         sched="auto", tile=0, flags=0, bias_row=None, bias_col=None, activation=None,
         scale_d=None, amax=None, group_n=0, sk_groups=0, source=None, beta=1.0):
    """D = epilogue(alpha * A x B + beta * source) for torch device tensors: A (M, K) row-major; B given as (N, K),
    i.e. the K x N operand in column-major storage; bf16 or uint8-coded e4m3 (then scale_a /
    scale_b are one-element float32 device tensors).  Optional fused epilogue: a float32 bias per
    row (M) or per column (N), an activation ("relu", "gelu", "silu"), amax (a one-element float32
    device tensor the kernel max-combines max |Y| into), and out_dtype "e4m3" (uint8 codes of
    Y / scale_d, scale_d a one-element float32 device tensor).  tile: 0 (the planner's), an int
    for square tiles, or (bm, bn), e.g. (256, 224).  sk_groups: Stream-K groups (0 = the
    planner's count, 1-8) of a plan with a Stream-K band.  source: an (M, N) float32 or
    bfloat16 device tensor added as beta * source before the bias (it may be C's own storage
    only through Plan.run; here C is a new tensor).  Returns C (M, N): float32,
    bfloat16, or uint8 e4m3 codes.  Shapes, element types, contiguity and devices are checked
    before anything is launched (ValueError)."""
    import torch
    if not isinstance(A, torch.Tensor) or not isinstance(B, torch.Tensor):
        raise ValueError("A and B must be torch tensors")
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError(f"A and B must be 2-D; got {tuple(A.shape)} and {tuple(B.shape)}")
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError(f"B must be (N, K) = (N, {K}), the K x N operand stored column-major; "
                         f"got {tuple(B.shape)}")
    fp8 = A.dtype in (torch.uint8, torch.float8_e4m3fn)
    if fp8 != (B.dtype in (torch.uint8, torch.float8_e4m3fn)):
        raise ValueError(f"A and B must both be bf16 or both e4m3; got {A.dtype} and {B.dtype}")
    if out_dtype not in OUT_DTYPES:
        raise ValueError(f"out_dtype must be one of {sorted(OUT_DTYPES)}")
    if bias_row is not None and bias_col is not None:
        raise ValueError("one bias at most (bias_row or bias_col)")
    epi = ACTIVATIONS[activation]
    epi |= GEMM_EPI_BIAS_ROW if bias_row is not None else 0
    epi |= GEMM_EPI_BIAS_COL if bias_col is not None else 0
    epi |= GEMM_EPI_AMAX if amax is not None else 0
    if source is not None:
        epi |= GEMM_EPI_SOURCE_F32 if source.dtype == torch.float32 else GEMM_EPI_SOURCE_BF16
    bm, bn = tile if isinstance(tile, tuple) else (tile, tile)
    desc = make_desc(M, N, K, GEMM_FP8_E4M3 if fp8 else GEMM_BF16, OUT_DTYPES[out_dtype],
                     MAPPINGS[mapping], group, SCHEDS[sched], 0, bm, bn, 0, flags,
                     epilogue=epi, group_n=group_n, sk_groups=sk_groups)
    plan = Plan(desc)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "e4m3": torch.uint8}[out_dtype]
    C = torch.empty((M, N), device=A.device, dtype=dt)
    ws = None
    if plan.workspace_bytes:
        ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=A.device)
    plan.run(A, B, C, scale_a, scale_b, ws, bias=bias_row if bias_row is not None else bias_col,
             scale_d=scale_d, amax=amax, source=source, beta=beta if source is not None else 0.0)
    return C
