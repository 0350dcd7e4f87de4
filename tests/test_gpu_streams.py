"""Plans are read-only after gemm_create: one plan, or several, may run on several HIP streams at
once.  Data-parallel launches on two streams (both kernel families, plain and fused), issued so
that they overlap, must store the bits that the same launches store one at a time.  (Stream-K
plans are left out here: their units wait on each other and rely on sharing the GPU with no
other launch, as gemm.h states for num_workers.)"""
import numpy as np
import pytest

import gemm_inputs as gi
from dense_gemm_design_amd import _lib as L
from gpu_util import to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()
    return torch.device("cuda:0")


def make_job(dev, M, N, K, dt, out, flags, tile, epi, seed):
    dist = ("normal", 1.0) if dt == "e4m3" else ("uniform",)
    op = gi.make_operands(M, N, K, dt, dist, dist, seed=seed)
    A, B, sa, sb = to_device(op, torch, dev)
    plan = L.Plan(L.make_desc(M, N, K, L.GEMM_BF16 if dt == "bf16" else L.GEMM_FP8_E4M3,
                              {"f32": L.GEMM_F32, "bf16": L.GEMM_BF16}[out],
                              L.GEMM_MAP_GROUPED_M, 2, L.GEMM_SCHED_PERSISTENT, 0, tile, tile, 0,
                              flags, epilogue=epi))
    assert plan.workspace_bytes == 0
    bias = torch.from_numpy(gi.make_vector(N, seed=seed + 1)).to(dev) if epi else None
    dtype = torch.float32 if out == "f32" else torch.bfloat16

    def run(C, stream):
        plan.run(A, B, C, sa, sb, None, stream=stream, bias=bias)
    return run, (M, N), dtype


def bits(C):
    return C.view(torch.uint8).cpu().numpy().copy()


def test_overlapping_streams_match_one_at_a_time(dev):
    jobs = [
        make_job(dev, 1000, 1032, 2056, "bf16", "bf16", L.GEMM_FLAG_WIDE, 256, 0, 41),
        make_job(dev, 776, 520, 1040, "e4m3", "f32", L.GEMM_FLAG_COOPERATIVE, 128,
                 L.GEMM_EPI_BIAS_COL | L.GEMM_EPI_GELU, 43),
        make_job(dev, 520, 904, 1000, "bf16", "f32", 0, 128, L.GEMM_EPI_SILU, 47),
    ]
    # one at a time, on the default stream
    want = []
    for run, shape, dtype in jobs:
        C = torch.full(shape, float("nan"), dtype=dtype, device=dev)
        run(C, torch.cuda.current_stream())
        torch.cuda.synchronize()
        want.append(bits(C))
    # all at once: each job twice, on its own stream (default priority), into separate outputs;
    # the same plan also runs on two streams
    streams = [torch.cuda.Stream() for _ in range(2 * len(jobs))]
    for rep in range(3):
        outs = []
        for j, (run, shape, dtype) in enumerate(jobs):
            for copy in range(2):
                C = torch.full(shape, float("nan"), dtype=dtype, device=dev)
                outs.append((j, C))
        torch.cuda.synchronize()
        for s, (j, C) in zip(streams, outs):
            jobs[j][0](C, s)
        torch.cuda.synchronize()
        for j, C in outs:
            assert np.array_equal(bits(C), want[j]), f"job {j}, repetition {rep}"
