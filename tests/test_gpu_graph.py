"""Launches recorded into a HIP graph (torch.cuda.CUDAGraph) and replayed: the library's run path
enqueues only kernels on the caller's stream (the Stream-K counters are cleared by a fill kernel,
not by a memset), so every replay must give the bits of an eager launch of the same plan.  Each
replay follows eager work of the program's own (C refilled with a canary, amax reset, an unrelated
product) and is checked on its own."""
import numpy as np
import pytest

import gemm_inputs as gi
from dense_gemm_design_amd import _lib as L
from gpu_util import assert_within_tolerance, decode_output, reference, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REPLAYS = 3
EPI = L.GEMM_EPI_BIAS_COL | L.GEMM_EPI_GELU | L.GEMM_EPI_AMAX
CASES = [
    # id, M, N, K, dtype, out, sched, workers, tile, flags, epilogue, entry point
    ("dp_bf16", 1000, 1032, 520, "bf16", "bf16", L.GEMM_SCHED_PERSISTENT, 0, 256, 0, 0, "run"),
    ("streamk_separate", 512, 512, 16384, "bf16", "f32", L.GEMM_SCHED_STREAMK, 256, 128, 0, 0,
     "run"),
    ("streamk_chain", 384, 256, 4096, "bf16", "f32", L.GEMM_SCHED_STREAMK, 40, 128,
     L.GEMM_FLAG_STREAMK_CHAIN, 0, "run"),
    ("fp8_fused_e4m3", 520, 776, 1040, "e4m3", "e4m3", L.GEMM_SCHED_PERSISTENT, 0, 256, 0, EPI,
     "run"),
    ("noalloc_streamk", 512, 512, 16384, "bf16", "f32", L.GEMM_SCHED_STREAMK, 256, 128, 0, 0,
     "noalloc"),
]
OUT = {"f32": (L.GEMM_F32, "float32", float("nan")), "bf16": (L.GEMM_BF16, "bfloat16",
                                                                float("nan")),
       "e4m3": (L.GEMM_FP8_E4M3, "uint8", 0x7F)}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()
    return torch.device("cuda:0")


def bits(C):
    return C.view(torch.uint8).cpu().numpy().copy()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(dev, case):
    name, M, N, K, dt, out, sched, workers, tile, flags, epi, entry = case
    print(f"graph case {name}: {M}x{N}x{K} {dt}->{out}", flush=True)
    dist = ("normal", 1.0) if dt == "e4m3" else ("uniform",)
    op = gi.make_operands(M, N, K, dt, dist, dist, seed=900 + CASES.index(case))
    A, B, sa, sb = to_device(op, torch, dev)
    plan = L.Plan(L.make_desc(M, N, K, L.GEMM_BF16 if dt == "bf16" else L.GEMM_FP8_E4M3,
                              OUT[out][0], L.GEMM_MAP_GROUPED_M, 2, sched, workers, tile, tile,
                              0, flags, epilogue=epi))
    if sched == L.GEMM_SCHED_STREAMK:
        assert plan.info.sk_tiles > 0 and plan.workspace_bytes > 0
    dtype = getattr(torch, OUT[out][1])
    canary = OUT[out][2]
    bias = torch.from_numpy(gi.make_vector(N, seed=950)).to(dev) if epi else None
    scale_d = (torch.tensor([4.0 * K ** 0.5 / 448.0], dtype=torch.float32, device=dev)
               if out == "e4m3" else None)
    amax = torch.zeros(1, dtype=torch.float32, device=dev) if epi else None
    ws = (torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
          if plan.workspace_bytes and entry == "run" else None)
    C = torch.full((M, N), canary, dtype=dtype, device=dev)

    def launch():
        if entry == "run":
            plan.run(A, B, C, sa, sb, ws, bias=bias, scale_d=scale_d, amax=amax)
        else:
            plan.run_noalloc(A, B, C, sa, sb, bias=bias, scale_d=scale_d, amax=amax)

    # eager launch: the bits every replay must reproduce
    launch()
    torch.cuda.synchronize()
    want = bits(C)
    want_amax = float(amax.item()) if epi else None
    if not epi:
        assert_within_tolerance(decode_output(C, torch), reference(op), op, f"{name} eager")

    g = torch.cuda.CUDAGraph()
    C.fill_(canary)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        launch()
    torch.cuda.synchronize()
    X = torch.randn(256, 256, device=dev)
    for r in range(REPLAYS):
        C.fill_(canary)
        if epi:
            amax.zero_()
        Y = X @ X  # eager work of the program's own between replays
        g.replay()
        torch.cuda.synchronize()
        assert np.isfinite(float(Y.sum().item()))
        got = bits(C)
        assert np.array_equal(got, want), f"{name}: replay {r} differs from the eager launch"
        if epi:
            assert float(amax.item()) == want_amax, f"{name}: replay {r} amax"
    # and an eager launch after the replays still agrees
    C.fill_(canary)
    if epi:
        amax.zero_()
    launch()
    torch.cuda.synchronize()
    assert np.array_equal(bits(C), want), f"{name}: eager launch after the replays"
