"""Launches at the planner's size limits, where the kernels' 32-bit buffer offsets come closest to
their ranges: N = 2^22 (the widest C the planner accepts: a wave's 127 output rows below it reach
2^31 - 16 bytes for fp32 elements) and, for one tile of each height, the deepest K whose operand
rows still fit a tile's 32-bit range (256 rows of 2K bytes just under 2^31 for bf16 on 256 x 256
tiles, 128 rows on 128 x 128).  Outputs are compared with the oracle on whole rows at the
sub-tile edges and on seeded random positions; every output must be finite (the canary gone)."""
import numpy as np
import pytest

import gemm_inputs as gi
import oracle
from dense_gemm_design_amd import _lib as L
from gpu_util import assert_within_tolerance, decode_output, oracle_dtype, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

N_MAX = 1 << 22


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()
    return torch.device("cuda:0")


def rows_of(op, rows):
    """The operand storage of A restricted to `rows` (row-major M x K)."""
    return np.ascontiguousarray(op.A.reshape(op.M, op.K)[rows]).reshape(-1)


def check_rows_and_samples(C, op, rows, n_samples, what):
    ref = oracle.gemm_ref(len(rows), op.N, op.K, oracle_dtype(op), rows_of(op, rows), op.B,
                          scale_a=op.scale_a, scale_b=op.scale_b)
    got = decode_output(C[torch.tensor(rows, device=C.device)], torch)
    sub = gi.Operands(len(rows), op.N, op.K, op.dtype, rows_of(op, rows), op.B, op.scale_a,
                      op.scale_b)
    assert_within_tolerance(got, ref, sub, f"{what} rows {rows}")
    rr, cc = gi.sample_positions(op.M, op.N, n_samples, seed=op.M + op.K)
    want = oracle.gemm_ref_sampled(op.M, op.N, op.K, oracle_dtype(op), op.A, op.B, rr, cc,
                                   scale_a=op.scale_a, scale_b=op.scale_b)
    got = C[torch.from_numpy(rr).to(C.device), torch.from_numpy(cc).to(C.device)]
    got = got.float().cpu().numpy().astype(np.float64)
    amax_a = oracle.max_abs_decoded(op.A, oracle_dtype(op), op.scale_a)
    amax_b = oracle.max_abs_decoded(op.B, oracle_dtype(op), op.scale_b)
    tol = oracle.tolerance(want, op.K, amax_a, amax_b)
    bad = np.abs(got - want) > tol
    assert not bad.any(), f"{what}: {int(bad.sum())} sampled outputs outside tolerance"


def launch(op, dev, out, tile, flags):
    A, B, sa, sb = to_device(op, torch, dev)
    plan = L.Plan(L.make_desc(op.M, op.N, op.K,
                              L.GEMM_BF16 if op.dtype == "bf16" else L.GEMM_FP8_E4M3,
                              L.GEMM_BF16 if out == "bf16" else L.GEMM_F32,
                              L.GEMM_MAP_LINEAR_N, 1, L.GEMM_SCHED_PERSISTENT, 0, tile, tile, 0,
                              flags))
    C = torch.full((op.M, op.N), float("nan"), device=dev,
                   dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    ws = (torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
          if plan.workspace_bytes else None)
    plan.run(A, B, C, sa, sb, ws)
    torch.cuda.synchronize()
    del A, B
    assert bool(torch.isfinite(C).all().item()), "outputs left unwritten or non-finite"
    return C, plan


@pytest.mark.parametrize("dt,out,tile,flags", [
    ("bf16", "f32", 256, L.GEMM_FLAG_WIDE),
    ("bf16", "bf16", 128, L.GEMM_FLAG_COOPERATIVE),
    ("e4m3", "bf16", 256, L.GEMM_FLAG_WIDE),
    ("e4m3", "f32", 128, L.GEMM_FLAG_COOPERATIVE),
])
def test_widest_output(dev, dt, out, tile, flags):
    M, K = 136, 16 if dt == "bf16" else 32
    print(f"N = 2^22: {M}x{N_MAX}x{K} {dt}->{out} tile {tile}", flush=True)
    dist = ("normal", 1.0) if dt == "e4m3" else ("uniform",)
    op = gi.make_operands(M, N_MAX, K, dt, dist, dist, seed=61)
    C, plan = launch(op, dev, out, tile, flags)
    assert (plan.info.bm, plan.info.nt) == (tile, N_MAX // tile)
    check_rows_and_samples(C, op, [0, 1, 127, 128, M - 1], 2000, f"N max {dt}->{out}")
    del C
    torch.cuda.empty_cache()
    # one more column is refused
    with pytest.raises(L.GemmError) as e:
        L.Plan(L.make_desc(M, N_MAX + 8, K, flags=flags, bm=tile, bn=tile))
    assert e.value.status == L.GEMM_ERR_UNSUPPORTED


@pytest.mark.parametrize("tile,flags", [(256, L.GEMM_FLAG_WIDE), (128, L.GEMM_FLAG_COOPERATIVE)])
def test_deepest_k(dev, tile, flags):
    # largest K (a multiple of 8: 16-byte rows) with tile * 2K below the 32-bit range limit
    K = ((0x7FFFFFF0 - 1) // (tile * 2)) // 8 * 8
    M, N = tile, 16
    print(f"deepest K: {M}x{N}x{K} bf16 tile {tile}", flush=True)
    op = gi.make_operands(M, N, K, "bf16", seed=62)
    C, plan = launch(op, dev, "f32", tile, flags)
    assert plan.info.kt == -(-K // plan.info.bk)
    ref = oracle.gemm_ref(M, N, K, oracle.BF16, op.A, op.B)
    assert_within_tolerance(decode_output(C, torch), ref, op, f"deepest K tile {tile}")
    del C
    torch.cuda.empty_cache()
    # eight more k are refused
    with pytest.raises(L.GemmError) as e:
        L.Plan(L.make_desc(M, N, K + 8, flags=flags, bm=tile, bn=tile))
    assert e.value.status == L.GEMM_ERR_UNSUPPORTED
