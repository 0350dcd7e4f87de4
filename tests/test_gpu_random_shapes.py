"""Seeded random sweep of the launch space against the oracle: operand type, M, N, K (ragged),
tile, kernel flag, scheduler, worker count, mapping, group, and for half the cases a fused
epilogue (source term in fp32 or bf16, in place or not, bias row/column, activation, amax,
fp32 / bf16 / e4m3 output).  Every combination the
planner accepts must match the oracle within the same bounds as the fixed-shape tests
(plain: |C - C_ref| <= 4e-3 |C_ref| + 1e-3 sqrt(K) max|a| max|b|; fused: oracle.epilogue's
bounds, e4m3 code bounds and the amax interval); combinations it refuses (GEMM_ERR_UNSUPPORTED)
are counted, not run.  The parameters come from a fixed seed, so a failing case names itself
and reruns the same way."""
import random

import numpy as np
import pytest

import gemm_inputs as gi
from dense_gemm_design_amd import _lib as L
from gpu_util import assert_within_tolerance, reference, run_gpu
import test_gpu_epilogue as TE

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CASES_PER_SEED = 40


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()
    return torch.device("cuda:0")


def draw(rng):
    dt = rng.choice(["bf16", "e4m3"])
    return dict(
        dt=dt,
        M=rng.choice([rng.randint(1, 64), rng.randint(1, 1100), rng.randint(200, 1100)]),
        N=8 * rng.randint(1, 137),
        K=(8 if dt == "bf16" else 16) * rng.randint(1, 190),
        tile=rng.choice([0, 128, 256, (256, 224), (256, 192)]),
        flags=rng.choice([0, 0, L.GEMM_FLAG_WIDE, L.GEMM_FLAG_COOPERATIVE]),
        sched=rng.choice([L.GEMM_SCHED_PERSISTENT, L.GEMM_SCHED_STREAMK, L.GEMM_SCHED_STATIC,
                          L.GEMM_SCHED_AUTO]),
        workers=rng.choice([0, rng.randint(1, 300)]),
        mapping=rng.choice([L.GEMM_MAP_LINEAR_N, L.GEMM_MAP_GROUPED_M, L.GEMM_MAP_GROUPED_N,
                            L.GEMM_MAP_BLOCKED, L.GEMM_MAP_MORTON]),
        group=rng.choice([0, 1, 2, 4, 8]),
        fused=rng.random() < 0.5,
        out_plain=rng.choice(["f32", "bf16"]),
        out_fused=rng.choice(["f32", "bf16", "e4m3"]),
        bias_kind=rng.choice([None, "row", "col"]),
        act=rng.choice([None, "relu", "gelu", "silu"]),
        scale_d=rng.choice([1.0, 0.25, 3.0]),
        source=rng.choice([None, None, "f32", "bf16"]),
        beta=rng.choice([1.0, -0.5, 0.0]),
        in_place=rng.random() < 0.5)


@pytest.mark.parametrize("seed", [11, 12, 13])
def test_random_launches_match_the_oracle(dev, seed):
    rng = random.Random(seed)
    ran = refused = 0
    for i in range(CASES_PER_SEED):
        c = draw(rng)
        dist = ("normal", 1.0) if c["dt"] == "e4m3" else ("uniform",)
        what = f"seed {seed} case {i}: {c}"
        print(what, flush=True)
        op = gi.make_operands(c["M"], c["N"], c["K"], c["dt"], dist, dist, seed=1000 * seed + i)
        bm, bn = c["tile"] if isinstance(c["tile"], tuple) else (c["tile"], c["tile"])
        try:
            if not c["fused"]:
                C, _, _ = run_gpu(op, torch, dev, c["out_plain"], c["mapping"], c["group"],
                                  c["sched"], c["workers"], bm, flags=c["flags"], bn=bn)
                assert_within_tolerance(C, reference(op), op, what)
            else:
                n_b = c["M"] if c["bias_kind"] == "row" else c["N"]
                bias = None
                if c["bias_kind"]:
                    bias = (np.random.default_rng(1000 * seed + i).standard_normal(n_b) * 0.5
                            ).astype(np.float32)
                S = s_vals = None
                if c["source"]:
                    S, s_vals = TE.make_source(c["M"], c["N"], c["source"], seed=2000 * seed + i)
                in_place = S is not None and c["in_place"] and c["source"] == c["out_fused"]
                got, am, _ = TE.run_epi(op, dev, c["out_fused"], c["bias_kind"], bias, c["act"],
                                        True, c["scale_d"], c["flags"], c["sched"], c["workers"],
                                        c["tile"], mapping=c["mapping"], group=c["group"],
                                        source=S, beta=c["beta"], in_place=in_place)
                TE.check(op, got, am, c["out_fused"], c["bias_kind"], bias, c["act"],
                         c["scale_d"], what, s_vals, c["beta"] if S is not None else 0.0)
            ran += 1
        except L.GemmError as e:
            assert e.status == L.GEMM_ERR_UNSUPPORTED, f"{what}: {e}"
            refused += 1
    print(f"seed {seed}: {ran} launches checked, {refused} refused as unsupported")
    assert ran >= CASES_PER_SEED // 2
