"""Full-size parity: every workload in the launch configuration bench.py times, checked on
sampled outputs (tile corners and edges plus seeded random positions) that the oracle computes
one element at a time, and for finiteness everywhere."""
import numpy as np
import pytest

import gemm_inputs as gi
import oracle
from dense_gemm_design_amd import _lib as L
import dense_gemm_design_amd as dg
from gpu_util import oracle_dtype, run_gpu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import bench  # noqa: E402  (the launch table the benchmark uses)

SAMPLES = 1536


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()
    return torch.device("cuda:0")


_ops = {}


def operands(name):
    if name not in _ops:
        _ops.clear()
        _ops[name] = gi.make_workload(name)
    return _ops[name]


@pytest.mark.parametrize("run", list(bench.RUNS))
def test_fullsize_sampled(dev, run):
    wl, mapping, group, sched, tile, out, workers = bench.RUNS[run][:7]
    bk = bench.RUNS[run][7] if len(bench.RUNS[run]) > 7 else 0
    chain = len(bench.RUNS[run]) > 8 and bench.RUNS[run][8] == "chain"
    op = operands(wl)
    C, plan, _ = run_gpu(op, torch, dev, out, dg.MAPPINGS[mapping], group, dg.SCHEDS[sched],
                         workers, tile, bk=bk, flags=L.GEMM_FLAG_STREAMK_CHAIN if chain else 0)
    if bk:
        assert plan.info.bk == bk
    assert np.isfinite(C).all()
    rows, cols = gi.sample_positions(op.M, op.N, SAMPLES, seed=len(run), BM=plan.info.bm,
                                     BN=plan.info.bn)
    ref = oracle.gemm_ref_sampled(op.M, op.N, op.K, oracle_dtype(op), op.A, op.B, rows, cols,
                                  scale_a=op.scale_a, scale_b=op.scale_b)
    amax_a = oracle.max_abs_decoded(op.A, oracle_dtype(op), op.scale_a)
    amax_b = oracle.max_abs_decoded(op.B, oracle_dtype(op), op.scale_b)
    tol = oracle.tolerance(ref, op.K, amax_a, amax_b)
    err = np.abs(C[rows, cols] - ref)
    assert (err <= tol).all(), f"{run}: {(err > tol).sum()} sampled elements outside tolerance"
    print(f"{run}: max err/tol {(err / tol).max():.3f}")


def test_streamk_workload_bit_exact_small_integers(dev):
    """The 512 x 512 x 65536 Stream-K launch on integer operands in [-2, 2]: exact in FP32, so
    the full output must equal the oracle bit for bit."""
    op = gi.make_operands(512, 512, 65536, "bf16", ("smallint", -2, 2), ("smallint", -2, 2),
                          seed=55)
    wl, mapping, group, sched, tile, out, workers = bench.RUNS["bf16_streamk"][:7]
    C, plan, _ = run_gpu(op, torch, dev, out, dg.MAPPINGS[mapping], group, dg.SCHEDS[sched],
                         workers, tile)
    assert plan.info.sk_tiles == 16 and plan.info.dp_tiles == 0
    rows, cols = gi.sample_positions(512, 512, 4096, seed=3, BM=128, BN=128)
    ref = oracle.gemm_ref_sampled(512, 512, 65536, oracle.BF16, op.A, op.B, rows, cols)
    assert np.array_equal(C[rows, cols], ref)
