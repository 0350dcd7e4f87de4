"""Full-size parity: every workload in the launch configuration bench.py times, checked on
sampled outputs (tile corners and edges plus seeded random positions) that the oracle computes
one element at a time, and for finiteness everywhere."""
import numpy as np
import pytest

import gemm_inputs as gi
import oracle
from dense_gemm_design_amd import _lib as L
import dense_gemm_design_amd as dg
from gpu_util import oracle_dtype, run_gpu, to_device

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
    op = operands(wl)
    C, plan, _ = run_gpu(op, torch, dev, out, dg.MAPPINGS[mapping], group, dg.SCHEDS[sched],
                         workers, tile, bk=bk, flags=bench.run_flags(run, dg))
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


REPEAT_RUNS = [r for r in bench.RUNS if bench.RUNS[r][0] in ("bf16_4096", "fp8_8192",
                                                            "bf16_mlp_up", "bf16_streamk")]


@pytest.mark.parametrize("run", REPEAT_RUNS)
def test_repeated_launches_bit_identical(dev, run):
    """Every launch configuration is deterministic by construction (fixed summation order, no
    atomics on data), so three launches must give identical bits; a race between waves (a stage
    refilled or reused while another wave still reads it) shows up as a difference."""
    wl, mapping, group, sched, tile, out, workers = bench.RUNS[run][:7]
    bk = bench.RUNS[run][7] if len(bench.RUNS[run]) > 7 else 0
    op = operands(wl)
    A, B, sa, sb = to_device(op, torch, dev)
    desc = L.make_desc(op.M, op.N, op.K, L.GEMM_BF16 if op.dtype == "bf16" else L.GEMM_FP8_E4M3,
                       L.GEMM_BF16 if out == "bf16" else L.GEMM_F32, dg.MAPPINGS[mapping], group,
                       dg.SCHEDS[sched], workers, tile, tile, bk, bench.run_flags(run, dg))
    plan = L.Plan(desc)
    ws = None
    if plan.workspace_bytes:
        ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
    outs = []
    for i in range(3):
        C = torch.full((op.M, op.N), float("nan"), device=dev,
                       dtype=torch.bfloat16 if out == "bf16" else torch.float32)
        plan.run(A, B, C, sa, sb, ws)
        outs.append(C)
    torch.cuda.synchronize()
    for i in (1, 2):
        diff = int((outs[i].view(torch.int16 if out == "bf16" else torch.int32)
                    != outs[0].view(torch.int16 if out == "bf16" else torch.int32)).sum())
        assert diff == 0, f"{run}: launch {i} differs from launch 0 in {diff} elements"


@pytest.mark.parametrize("run", [r for r in bench.RUNS if bench.RUNS[r][0] == "bf16_4096"])
def test_bf16_4096_every_output(dev, run):
    """bf16 4096^3: every one of the 16.8M outputs against the oracle (a few seconds of fp64 on
    the host's cores), so a wrong row band or tile anywhere fails."""
    wl, mapping, group, sched, tile, out, workers = bench.RUNS[run][:7]
    op = operands(wl)
    if not hasattr(test_bf16_4096_every_output, "ref"):
        test_bf16_4096_every_output.ref = oracle.gemm_ref(op.M, op.N, op.K, oracle.BF16, op.A,
                                                          op.B)
    ref = test_bf16_4096_every_output.ref
    C, plan, _ = run_gpu(op, torch, dev, out, dg.MAPPINGS[mapping], group, dg.SCHEDS[sched],
                         workers, tile, flags=bench.run_flags(run, dg))
    amax_a = oracle.max_abs_decoded(op.A, oracle.BF16)
    amax_b = oracle.max_abs_decoded(op.B, oracle.BF16)
    tol = oracle.tolerance(ref, op.K, amax_a, amax_b)
    bad = ~(np.abs(C - ref) <= tol)
    assert not bad.any(), f"{run}: {int(bad.sum())} outputs outside tolerance, first at " \
                          f"{np.argwhere(bad)[0].tolist()}"
