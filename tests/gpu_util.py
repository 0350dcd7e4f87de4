"""Helpers for the GPU tests: moving generator operands to the device, running the library
through its C ABI, and comparing against the oracle."""
import numpy as np

import oracle
from dense_gemm_design_amd import _lib as L


def to_device(op, torch, device):
    if op.dtype == "bf16":
        A = torch.from_numpy(op.A.view(np.int16).reshape(op.M, op.K)).to(device)
        B = torch.from_numpy(op.B.view(np.int16).reshape(op.N, op.K)).to(device)
    else:
        A = torch.from_numpy(op.A.reshape(op.M, op.K)).to(device)
        B = torch.from_numpy(op.B.reshape(op.N, op.K)).to(device)
    sa = torch.tensor([op.scale_a], dtype=torch.float32, device=device)
    sb = torch.tensor([op.scale_b], dtype=torch.float32, device=device)
    return A, B, sa, sb


def decode_output(C, torch):
    if C.dtype == torch.bfloat16:
        return C.float().cpu().numpy().astype(np.float64)
    return C.cpu().numpy().astype(np.float64)


def run_gpu(op, torch, device, out="f32", mapping=L.GEMM_MAP_LINEAR_N, group=1,
            sched=L.GEMM_SCHED_PERSISTENT, workers=0, tile=0, flags=0, plan=None, keep=False,
            bk=0, group_n=0, sk_groups=0, bn=0):
    """Runs C = alpha * A x B on the GPU; returns (C decoded to float64, plan, workspace)."""
    A, B, sa, sb = to_device(op, torch, device)
    if plan is None:
        desc = L.make_desc(op.M, op.N, op.K,
                           L.GEMM_BF16 if op.dtype == "bf16" else L.GEMM_FP8_E4M3,
                           L.GEMM_BF16 if out == "bf16" else L.GEMM_F32, mapping, group, sched,
                           workers, tile, bn or tile, bk, flags, group_n=group_n,
                           sk_groups=sk_groups)
        plan = L.Plan(desc)
    C = torch.empty((op.M, op.N), device=device,
                    dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    C.fill_(float("nan"))
    ws = None
    if plan.workspace_bytes:
        ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=device)
    plan.run(A, B, C, sa, sb, ws)
    torch.cuda.synchronize()
    res = decode_output(C, torch)
    if keep:
        return res, plan, ws, C
    return res, plan, ws


def oracle_dtype(op):
    return oracle.BF16 if op.dtype == "bf16" else oracle.E4M3


def reference(op):
    return oracle.gemm_ref(op.M, op.N, op.K, oracle_dtype(op), op.A, op.B,
                           scale_a=op.scale_a, scale_b=op.scale_b)


def assert_within_tolerance(C, C_ref, op, what=""):
    amax_a = oracle.max_abs_decoded(op.A, oracle_dtype(op), op.scale_a)
    amax_b = oracle.max_abs_decoded(op.B, oracle_dtype(op), op.scale_b)
    tol = oracle.tolerance(C_ref, op.K, amax_a, amax_b)
    err = np.abs(C - C_ref)
    assert np.isfinite(C).all(), f"{what}: non-finite outputs"
    bad = err > tol
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} elements outside tolerance; first {idx.tolist()}"
                             f" got {C[tuple(idx[0])]} want {C_ref[tuple(idx[0])]}")
    return float((err / tol).max()) if err.size else 0.0
