"""Full-size parity: every launch configuration bench.py times, at its full size, with every
output element compared against the fp64 oracle (cached per workload and seed, tests/cref_cache).

Plain runs: |C - C_ref| <= 4e-3 |C_ref| + 1e-3 sqrt(K) max|a| max|b| per element.  Fused runs go
through the epilogue oracle (oracle.epilogue) in the order of the "H100 Kernel Design" lesson,
section 12.2 -- Z = alpha * Acc, Z += bias, Y = act(Z), amax, then the output scale and cast:
  * float outputs: |Y - Y_ref| within oracle.epilogue.tolerance (bf16 rounding included);
  * e4m3 outputs: every stored code between the oracle's codes of (Y_ref -+ tol) / scale_d, and
    the amax between max(|Y_ref| - tol) and max(|Y_ref| + tol).
Also: the Stream-K launch on small-integer operands equals the oracle bit for bit everywhere, and
three launches of every configuration give identical bits (and identical amax).
"""
import numpy as np
import pytest

import gemm_inputs as gi
import oracle
from oracle import epilogue as E
from dense_gemm_design_amd import _lib as L
import dense_gemm_design_amd as dg
from cref_cache import cref
from gpu_util import run_gpu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import bench  # noqa: E402  (the launch table and set-up the benchmark uses)

# runs grouped by workload, so one workload's operands and reference are live at a time
_WL_ORDER = ["bf16_256", "bf16_4096", "bf16_streamk", "bf16_mlp_up", "fp8_8192"]
RUN_ORDER = sorted(bench.RUNS, key=lambda r: _WL_ORDER.index(bench.RUNS[r][0]))


def e4m3_table():
    """The oracle's value of every e4m3 code (NaN for the NaN codes)."""
    return np.array([oracle.decode_e4m3(c) for c in range(256)], dtype=np.float64)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()
    return torch.device("cuda:0")


_dev_cache = {}


def setup(name):
    """bench.setup_run for `name`, keeping only its workload's operands on the device."""
    wl = bench.RUNS[name][0]
    for k in [k for k in _dev_cache if k != wl]:
        del _dev_cache[k]
    return bench.setup_run(name, torch, dg, gi, _dev_cache)


def fill_poison(C):
    """NaN everywhere (bf16 / f32), or the e4m3 NaN code 0xFF, so an unwritten element fails."""
    if C.dtype == torch.uint8:
        C.fill_(0xFF)
    else:
        C.fill_(float("nan"))


def operand_maxima(op):
    code = oracle.BF16 if op.dtype == "bf16" else oracle.E4M3
    return (oracle.max_abs_decoded(op.A, code, op.scale_a),
            oracle.max_abs_decoded(op.B, code, op.scale_b))


def first_bad(bad, got, want):
    idx = tuple(np.argwhere(bad)[0])
    return f"first at {list(idx)}: got {got[idx]!r}, want {want[idx]!r}"


def check_every_output(run):
    """Compares every element of run["C"] with the oracle; returns max err / tol."""
    op, C, out = run["op"], run["C"], run["out"]
    ref = cref(run["workload"], op)
    amax_a, amax_b = operand_maxima(op)
    epi = run["epi"]
    if not epi and out != "e4m3":
        got = C.float().cpu().numpy().astype(np.float64)
        tol = oracle.tolerance(ref, op.K, amax_a, amax_b)
        err = np.abs(got - ref)
        bad = ~(err <= tol)
        assert not bad.any(), f"{run['name']}: {int(bad.sum())} of {bad.size} outputs outside " \
                              f"tolerance; {first_bad(bad, got, ref)}"
        return float((err / tol).max())
    bias_host = run["bias_host"]
    bias = {} if bias_host is None else {
        ("bias_row" if epi["bias"] == "row" else "bias_col"): bias_host.astype(np.float64)}
    src = {} if run.get("source_host") is None else {
        "source": run["source_host"].astype(np.float64), "beta": run["beta"]}
    z, y = E.apply(ref, act=epi.get("act"), **bias, **src)
    s_ref = src["beta"] * src["source"] if src else None
    if out == "e4m3":
        scale_d = float(run["scale_d"].cpu()[0])
        tol = E.tolerance(y, z, op.K, amax_a, amax_b, out="f32", s_ref=s_ref)
        lo, hi = E.quantized_bounds(y, tol, scale_d)
        got = e4m3_table()[C.cpu().numpy()]
        bad = ~((lo <= got) & (got <= hi))
        assert not bad.any(), f"{run['name']}: {int(bad.sum())} of {bad.size} e4m3 codes " \
                              f"outside the oracle's code bounds; {first_bad(bad, got, y / scale_d)}"
        worst = 0.0
    else:
        got = C.float().cpu().numpy().astype(np.float64)
        tol = E.tolerance(y, z, op.K, amax_a, amax_b, out=out, s_ref=s_ref)
        err = np.abs(got - y)
        bad = ~(err <= tol)
        assert not bad.any(), f"{run['name']}: {int(bad.sum())} of {bad.size} outputs outside " \
                              f"the epilogue tolerance; {first_bad(bad, got, y)}"
        worst = float((err / tol).max())
    if epi.get("amax"):
        got_amax = float(run["amax"].cpu()[0])
        ay = np.abs(y)
        lo_a, hi_a = float((ay - tol).max()), float((ay + tol).max())
        assert lo_a <= got_amax <= hi_a, \
            f"{run['name']}: amax {got_amax} outside [{lo_a}, {hi_a}] (oracle {E.amax(y)})"
    return worst


@pytest.mark.parametrize("name", RUN_ORDER)
def test_fullsize_every_output(dev, name):
    run = setup(name)
    fill_poison(run["C"])
    if run["amax"] is not None:
        run["amax"].zero_()
    run["launch"]()
    torch.cuda.synchronize()
    plan = run["plan"]
    if len(bench.RUNS[name]) > 7 and bench.RUNS[name][7]:
        assert plan.info.bk == bench.RUNS[name][7]
    worst = check_every_output(run)
    print(f"{name}: every output of {run['op'].M}x{run['op'].N} checked, max err/tol {worst:.3f}")


REPEAT_RUNS = [r for r in RUN_ORDER if bench.RUNS[r][0] in ("bf16_4096", "fp8_8192",
                                                           "bf16_mlp_up", "bf16_streamk")]


@pytest.mark.parametrize("name", REPEAT_RUNS)
def test_repeated_launches_bit_identical(dev, name):
    """Every launch configuration is deterministic by construction (fixed summation order, no
    atomics on data), so three launches must give identical bits -- outputs and amax alike; a
    race between waves (a stage refilled or reused while another wave still reads it) shows up
    as a difference."""
    run = setup(name)
    outs, amaxes = [], []
    for _ in range(3):
        C = torch.empty_like(run["C"])
        fill_poison(C)
        if run["amax"] is not None:
            run["amax"].zero_()
        run["launch"](None, C)
        outs.append(C)
        if run["amax"] is not None:
            amaxes.append(run["amax"].clone())
    torch.cuda.synchronize()
    view = {torch.bfloat16: torch.int16, torch.float32: torch.int32, torch.uint8: torch.uint8}[
        run["C"].dtype]
    for i in (1, 2):
        diff = int((outs[i].view(view) != outs[0].view(view)).sum())
        assert diff == 0, f"{name}: launch {i} differs from launch 0 in {diff} elements"
        if amaxes:
            assert float(amaxes[i][0]) == float(amaxes[0][0]), f"{name}: amax differs"


def test_streamk_workload_bit_exact_small_integers(dev):
    """The 512 x 512 x 65536 Stream-K launch on integer operands in [-2, 2]: every partial sum is
    an integer below 2^24, exact in FP32 whatever the split and order, so every output must equal
    the oracle bit for bit."""
    op = gi.make_operands(512, 512, 65536, "bf16", ("smallint", -2, 2), ("smallint", -2, 2),
                          seed=55)
    wl, mapping, group, sched, tile, out, workers = bench.RUNS["bf16_streamk"][:7]
    C, plan, _ = run_gpu(op, torch, dev, out, dg.MAPPINGS[mapping], group, dg.SCHEDS[sched],
                         workers, tile)
    assert plan.info.sk_tiles == 16 and plan.info.dp_tiles == 0
    ref = oracle.gemm_ref(512, 512, 65536, oracle.BF16, op.A, op.B)
    bad = C != ref
    assert not bad.any(), f"{int(bad.sum())} outputs differ; {first_bad(bad, C, ref)}"
