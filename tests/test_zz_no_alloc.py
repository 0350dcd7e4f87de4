"""gemm_run_noalloc: the entry point for callers that cannot allocate (its workspace is the
library's own per-GPU scratch array) against gemm_run_ex with a caller-allocated workspace --
the same plan, kernels and summation order, so the outputs (and amax) must agree bit for bit.
Two calls in a row, the second on a smaller problem, so the second finds the first's scratch
contents (its Stream-K counters must be cleared again) -- then a plan with no workspace."""
import numpy as np
import pytest

import gemm_inputs as gi
from dense_gemm_design_amd import _lib as L
from gpu_util import to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CALLS = [
    # M, N, K, dtype, out, sched, workers, tile, epilogue bits
    (512, 512, 16384, "bf16", "f32", L.GEMM_SCHED_STREAMK, 256, 128, 0),
    (256, 384, 4096, "e4m3", "e4m3", L.GEMM_SCHED_STREAMK, 64, 128,
     L.GEMM_EPI_BIAS_COL | L.GEMM_EPI_GELU | L.GEMM_EPI_AMAX),
    (520, 776, 1000, "bf16", "bf16", L.GEMM_SCHED_PERSISTENT, 3, 256, 0),
]
OUT = {"f32": (L.GEMM_F32, "float32"), "bf16": (L.GEMM_BF16, "bfloat16"),
       "e4m3": (L.GEMM_FP8_E4M3, "uint8")}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()
    return torch.device("cuda:0")


def test_noalloc_matches_run_ex_on_consecutive_calls(dev):
    for i, (M, N, K, dt, out, sched, workers, tile, epi) in enumerate(CALLS):
        print(f"no-alloc call {i}: {M}x{N}x{K} {dt}->{out} sched {sched} P {workers}", flush=True)
        dist = ("normal", 1.0) if dt == "e4m3" else ("uniform",)
        op = gi.make_operands(M, N, K, dt, dist, dist, seed=700 + i)
        A, B, sa, sb = to_device(op, torch, dev)
        plan = L.Plan(L.make_desc(M, N, K, L.GEMM_BF16 if dt == "bf16" else L.GEMM_FP8_E4M3,
                                  OUT[out][0], L.GEMM_MAP_GROUPED_M, 2, sched, workers, tile,
                                  tile, 0, 0, epilogue=epi))
        need = plan.workspace_bytes
        assert need <= L.GEMM_NOALLOC_SCRATCH_BYTES
        if sched == L.GEMM_SCHED_STREAMK:
            assert need > 0 and plan.info.sk_tiles > 0
        dtype = getattr(torch, OUT[out][1])
        bias = torch.from_numpy(gi.make_vector(N, seed=800 + i)).to(dev)
        scale_d = torch.tensor([4.0 * K ** 0.5 / 448.0], dtype=torch.float32, device=dev)
        am_ref = torch.zeros(1, dtype=torch.float32, device=dev)
        am_na = torch.zeros(1, dtype=torch.float32, device=dev)
        C_ref = torch.full((M, N), 0x7F if out == "e4m3" else float("nan"), dtype=dtype,
                           device=dev)
        C_na = torch.full_like(C_ref, 0x7F if out == "e4m3" else float("nan"))
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        plan.run(A, B, C_ref, sa, sb, ws if need else None, bias=bias if epi else None,
                 scale_d=scale_d if out == "e4m3" else None, amax=am_ref if epi else None)
        plan.run_noalloc(A, B, C_na, sa, sb, bias=bias if epi else None,
                         scale_d=scale_d if out == "e4m3" else None,
                         amax=am_na if epi else None)
        torch.cuda.synchronize()
        view = {torch.float32: torch.int32, torch.bfloat16: torch.int16, torch.uint8: torch.uint8}
        diff = int((C_na.view(view[dtype]) != C_ref.view(view[dtype])).sum())
        assert diff == 0, f"call {i}: {diff} outputs differ from gemm_run_ex"
        if epi & L.GEMM_EPI_AMAX:
            assert float(am_na.cpu()[0]) == float(am_ref.cpu()[0]) > 0.0
        if out != "e4m3":
            assert bool(torch.isfinite(C_na.float()).all())
