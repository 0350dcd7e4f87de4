"""Parity of the fused epilogue (source term, bias, activation, amax, e4m3 output) with the
oracle's (oracle/epilogue.py), through gemm_run_ex, on an MI355X.

Float outputs: |Y - Y_ref| within oracle.epilogue.tolerance.  e4m3 outputs: the stored code lies
between the codes of (Y_ref -+ tol) / scale_d -- and equals the oracle's code byte for byte
where the whole computation is exact (integer-valued products, representable biases, including
exact rounding midpoints).  amax: within [max(|Y_ref| - tol), max(|Y_ref| + tol)].
"""
import zlib

import numpy as np
import pytest

import gemm_inputs as gi
import oracle
from oracle import epilogue as E
from dense_gemm_design_amd import _lib as L
from gpu_util import decode_output, oracle_dtype, reference, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ACT_BITS = {None: 0, "relu": L.GEMM_EPI_RELU, "gelu": L.GEMM_EPI_GELU, "silu": L.GEMM_EPI_SILU}
OUT = {"f32": L.GEMM_F32, "bf16": L.GEMM_BF16, "e4m3": L.GEMM_FP8_E4M3}
E4M3_TABLE = np.array([oracle.decode_e4m3(c) for c in range(256)], dtype=np.float64)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()
    return torch.device("cuda:0")


def make_source(M, N, kind, seed):
    """A seeded M x N source matrix S of element type `kind` ("f32" or "bf16"): the torch tensor
    (on the CPU) and the values it holds exactly, as float64."""
    v = gi.make_vector(M * N, seed=seed, dist=("normal", 2.0)).reshape(M, N)
    if kind == "f32":
        t = torch.from_numpy(v.copy())
        return t, v.astype(np.float64)
    bits = gi.bf16_bits(torch.from_numpy(v))
    t = torch.from_numpy(bits.view(np.int16).reshape(M, N).copy()).view(torch.bfloat16)
    return t, t.float().numpy().astype(np.float64)


def run_epi(op, dev, out, bias_kind=None, bias=None, act=None, amax=True, scale_d=1.0,
            flags=0, sched=L.GEMM_SCHED_PERSISTENT, workers=3, tile=256, amax_init=0.0,
            mapping=L.GEMM_MAP_GROUPED_M, group=2, source=None, beta=0.0, in_place=False):
    """One fused GEMM through gemm_run_ex; returns (C as float64 or e4m3 codes, amax, plan).
    source: a CPU tensor from make_source (its type sets the GEMM_EPI_SOURCE_* bit), passed as
    S with factor beta -- or, in_place, copied into C and C passed as S."""
    A, B, sa, sb = to_device(op, torch, dev)
    epi = ACT_BITS[act] | (L.GEMM_EPI_AMAX if amax else 0)
    epi |= {None: 0, "row": L.GEMM_EPI_BIAS_ROW, "col": L.GEMM_EPI_BIAS_COL}[bias_kind]
    if source is not None:
        epi |= L.GEMM_EPI_SOURCE_F32 if source.dtype == torch.float32 else L.GEMM_EPI_SOURCE_BF16
    bm, bn = tile if isinstance(tile, tuple) else (tile, tile)
    desc = L.make_desc(op.M, op.N, op.K, L.GEMM_BF16 if op.dtype == "bf16" else L.GEMM_FP8_E4M3,
                       OUT[out], mapping, group, sched, workers, bm, bn, 0, flags,
                       epilogue=epi)
    plan = L.Plan(desc)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "e4m3": torch.uint8}[out]
    C = torch.empty((op.M, op.N), device=dev, dtype=dt)
    C.fill_(0x7F if out == "e4m3" else float("nan"))
    ws = None
    if plan.workspace_bytes:
        ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
    b = torch.from_numpy(np.asarray(bias, dtype=np.float32)).to(dev) if bias is not None else None
    am = torch.tensor([amax_init], dtype=torch.float32, device=dev)
    sd = torch.tensor([scale_d], dtype=torch.float32, device=dev)
    S = None
    if source is not None:
        if in_place:
            C.copy_(source.to(dev))
            S = C
        else:
            S = source.to(dev)
    plan.run(A, B, C, sa, sb, ws, bias=b, scale_d=sd if out == "e4m3" else None,
             amax=am if amax else None, source=S, beta=beta)
    torch.cuda.synchronize()
    got = C.cpu().numpy().copy() if out == "e4m3" else decode_output(C, torch)
    return got, float(am.cpu()[0]), plan


def expected(op, bias_kind, bias, act, src=None, beta=0.0):
    C = reference(op)
    kw = {"bias_row": bias} if bias_kind == "row" else (
        {"bias_col": bias} if bias_kind == "col" else {})
    z, y = E.apply(C, act=act, source=src, beta=beta,
                   **{k: np.asarray(v, dtype=np.float64) for k, v in kw.items()})
    return z, y


def check(op, got, am, out, bias_kind, bias, act, scale_d, what, src=None, beta=0.0):
    z, y = expected(op, bias_kind, bias, act, src, beta)
    ma = oracle.max_abs_decoded(op.A, oracle_dtype(op), op.scale_a)
    mb = oracle.max_abs_decoded(op.B, oracle_dtype(op), op.scale_b)
    s_ref = beta * src if src is not None else None
    tol = E.tolerance(y, z, op.K, ma, mb, out="f32", s_ref=s_ref)
    if out == "e4m3":
        lo, hi = E.quantized_bounds(y, tol, scale_d)
        v = E4M3_TABLE[got]
        bad = ~((v >= lo) & (v <= hi))
    else:
        full = E.tolerance(y, z, op.K, ma, mb, out=out, s_ref=s_ref)
        assert np.isfinite(got).all(), f"{what}: non-finite outputs"
        bad = np.abs(got - y) > full
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} elements outside the bound; first {i}: "
                             f"got {got[i]} want {y[i]} (scale_d {scale_d})")
    a_lo = float(np.max(np.abs(y) - tol, initial=0.0))
    a_hi = float(np.max(np.abs(y) + tol, initial=0.0))
    assert a_lo <= am <= a_hi, f"{what}: amax {am} outside [{a_lo}, {a_hi}]"
    return y


def operands(name, M, N, K, dt):
    # sigma = K^(-1/4) on both operands puts Z near N(0, 1), where the activations bend
    s = ("normal", float(K) ** -0.25)
    return gi.make_operands(M, N, K, dt, s, s, seed=zlib.crc32(name.encode()) % 10000)


# id, M, N, K, operand type, output, kernel flags, tile, sched, workers, bias, activation
CASES = [
    ("wide_bf16_bias_col_gelu", 520, 776, 1000, "bf16", "bf16", L.GEMM_FLAG_WIDE, 256,
     L.GEMM_SCHED_PERSISTENT, 3, "col", "gelu"),
    ("wide_bf16_f32_ragged_bias_row_silu", 300, 264, 104, "bf16", "f32", L.GEMM_FLAG_WIDE, 256,
     L.GEMM_SCHED_PERSISTENT, 2, "row", "silu"),
    ("wide_bf16_e4m3_out_relu", 776, 520, 1000, "bf16", "e4m3", L.GEMM_FLAG_WIDE, 256,
     L.GEMM_SCHED_PERSISTENT, 3, "col", "relu"),
    ("wide_fp8_bias_row_gelu", 520, 520, 1040, "e4m3", "bf16", L.GEMM_FLAG_WIDE, 256,
     L.GEMM_SCHED_STATIC, 0, "row", "gelu"),
    ("wide_fp8_e4m3_out_silu", 776, 520, 1040, "e4m3", "e4m3", L.GEMM_FLAG_WIDE, 256,
     L.GEMM_SCHED_PERSISTENT, 2, "col", "silu"),
    ("wide_fp8_f32_no_bias", 264, 520, 400, "e4m3", "f32", L.GEMM_FLAG_WIDE, 256,
     L.GEMM_SCHED_PERSISTENT, 2, None, "gelu"),
    ("coop256_bf16_bias_col_gelu", 520, 776, 1000, "bf16", "bf16", L.GEMM_FLAG_COOPERATIVE, 256,
     L.GEMM_SCHED_PERSISTENT, 3, "col", "gelu"),
    ("coop128_bf16_e4m3_ragged_relu", 300, 264, 104, "bf16", "e4m3", L.GEMM_FLAG_COOPERATIVE,
     128, L.GEMM_SCHED_STATIC, 0, "row", "relu"),
    ("coop128_fp8_f32_silu", 384, 264, 272, "e4m3", "f32", L.GEMM_FLAG_COOPERATIVE, 128,
     L.GEMM_SCHED_PERSISTENT, 4, "col", "silu"),
    ("wide128_fp8_bf16_gelu", 384, 264, 272, "e4m3", "bf16", 0, 128, L.GEMM_SCHED_PERSISTENT, 4,
     "row", "gelu"),
    ("wide128_bf16_e4m3_silu", 300, 264, 1000, "bf16", "e4m3", 0, 128, L.GEMM_SCHED_STATIC, 0,
     "col", "silu"),
    ("coop_streamk_sep_gelu", 256, 256, 8192, "bf16", "bf16", L.GEMM_FLAG_COOPERATIVE, 128,
     L.GEMM_SCHED_STREAMK, 8, "row", "gelu"),
    ("streamk_sep_bf16_f32_gelu", 256, 256, 8192, "bf16", "f32", 0, 128, L.GEMM_SCHED_STREAMK,
     8, "col", "gelu"),
    ("streamk_chain_bf16_bf16_silu", 256, 256, 8192, "bf16", "bf16", L.GEMM_FLAG_STREAMK_CHAIN,
     128, L.GEMM_SCHED_STREAMK, 8, "row", "silu"),
    ("streamk_fp8_e4m3_relu", 256, 256, 4096, "e4m3", "e4m3", 0, 128, L.GEMM_SCHED_STREAMK, 11,
     "col", "relu"),
    ("streamk_hybrid_ragged_gelu", 200, 136, 1000, "bf16", "bf16", 0, 128, L.GEMM_SCHED_STREAMK,
     9, "col", "gelu"),
    # Stream-K on the wide-wave kernel (256 x 256 tiles): the reduction applies the epilogue
    ("wide_streamk_bf16_gelu", 300, 520, 3000, "bf16", "bf16", L.GEMM_FLAG_WIDE, 256,
     L.GEMM_SCHED_STREAMK, 5, "col", "gelu"),
    ("wide_streamk_fp8_e4m3_silu", 512, 768, 8192, "e4m3", "e4m3", L.GEMM_FLAG_WIDE, 256,
     L.GEMM_SCHED_STREAMK, 4, "row", "silu"),
    # 256 x 224 tiles (wide-wave only): ragged edges, every output type, Stream-K
    ("wide224_bf16_bias_col_gelu", 520, 904, 1000, "bf16", "bf16", 0, (256, 224),
     L.GEMM_SCHED_PERSISTENT, 3, "col", "gelu"),
    ("wide224_fp8_e4m3_row_silu", 776, 688, 1040, "e4m3", "e4m3", 0, (256, 224),
     L.GEMM_SCHED_PERSISTENT, 4, "row", "silu"),
    ("wide224_streamk_bf16_f32_relu", 512, 448, 8192, "bf16", "f32", 0, (256, 224),
     L.GEMM_SCHED_STREAMK, 8, "col", "relu"),
    # 256 x 192 tiles (wide-wave only)
    ("wide192_bf16_bias_col_gelu", 520, 904, 1000, "bf16", "bf16", 0, (256, 192),
     L.GEMM_SCHED_PERSISTENT, 3, "col", "gelu"),
    ("wide192_fp8_e4m3_row_silu", 776, 688, 1040, "e4m3", "e4m3", 0, (256, 192),
     L.GEMM_SCHED_PERSISTENT, 4, "row", "silu"),
    ("wide192_streamk_fp8_f32_relu", 512, 384, 8192, "e4m3", "f32", 0, (256, 192),
     L.GEMM_SCHED_STREAMK, 8, "col", "relu"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fused_epilogue_parity(dev, case):
    name, M, N, K, dt, out, flags, tile, sched, workers, bias_kind, act = case
    op = operands(name, M, N, K, dt)
    n_bias = M if bias_kind == "row" else N
    bias = gi.make_vector(n_bias, seed=zlib.crc32(name.encode()) % 977) if bias_kind else None
    scale_d = 1.0
    if out == "e4m3":  # 80% of the largest |Y| lands on 448: the top of the range saturates
        _, y = expected(op, bias_kind, bias, act)
        scale_d = float(np.float32(E.amax(y) / 448.0 * 0.8))
    got, am, plan = run_epi(op, dev, out, bias_kind, bias, act, True, scale_d, flags, sched,
                            workers, tile)
    # the cooperative kernel when asked for, or for the Stream-K lock chain; else wide-wave
    coop = flags & (L.GEMM_FLAG_COOPERATIVE | L.GEMM_FLAG_STREAMK_CHAIN)
    assert plan.info.kernel == (0 if coop else 3)
    if sched == L.GEMM_SCHED_STREAMK:
        assert plan.info.sk_tiles > 0
    check(op, got, am, out, bias_kind, bias, act, scale_d, name)


# Z = alpha Acc + beta S on both kernel families and every epilogue path (wide-wave: staged bf16
# on 256 x 256 and 256 x 224, direct fp32 / e4m3 / bf16 on 64-wide sub-tiles, the Stream-K
# reduction; cooperative: whole tiles, lock chain, K = 0), S in fp32 or bf16, S = C (in place)
# id, M, N, K, operand type, output, source type, in place, beta, flags, tile, sched, workers,
# bias, activation
SRC_CASES = [
    ("src_f32_bias_col_gelu", 520, 776, 1000, "bf16", "f32", "f32", False, 0.75, 0, 256,
     L.GEMM_SCHED_PERSISTENT, 3, "col", "gelu"),
    ("src_f32_in_place_ragged_relu", 300, 264, 104, "bf16", "f32", "f32", True, -1.5, 0, 128,
     L.GEMM_SCHED_STATIC, 0, "row", "relu"),
    ("src_bf16_in_place_silu", 520, 520, 1000, "bf16", "bf16", "bf16", True, 2.0, 0, 256,
     L.GEMM_SCHED_PERSISTENT, 3, None, "silu"),
    ("src_bf16_fp8_e4m3_out", 384, 264, 272, "e4m3", "e4m3", "bf16", False, 0.5, 0, 128,
     L.GEMM_SCHED_PERSISTENT, 4, "row", "relu"),
    ("src_f32_fp8_256_bf16_out", 520, 776, 1040, "e4m3", "bf16", "f32", False, -0.25, 0, 256,
     L.GEMM_SCHED_PERSISTENT, 3, "col", None),
    ("src_f32_streamk_chain_in_place", 256, 256, 8192, "bf16", "f32", "f32", True, 1.0,
     L.GEMM_FLAG_STREAMK_CHAIN, 128, L.GEMM_SCHED_STREAMK, 8, "col", "gelu"),
    ("src_bf16_streamk_separate", 256, 256, 8192, "bf16", "bf16", "bf16", False, -1.0, 0, 128,
     L.GEMM_SCHED_STREAMK, 8, "row", None),
    ("src_f32_streamk_hybrid_ragged", 200, 136, 1000, "bf16", "f32", "f32", False, 3.0, 0, 128,
     L.GEMM_SCHED_STREAMK, 9, None, "silu"),
    ("src_f32_zero_depth", 130, 136, 0, "bf16", "f32", "f32", False, 0.5, 0, 128,
     L.GEMM_SCHED_PERSISTENT, 4, "col", "gelu"),
    ("src_coop256_f32_bias_col_gelu", 520, 776, 1000, "bf16", "f32", "f32", False, 0.75,
     L.GEMM_FLAG_COOPERATIVE, 256, L.GEMM_SCHED_PERSISTENT, 3, "col", "gelu"),
    ("src_coop128_bf16_in_place", 300, 264, 104, "bf16", "bf16", "bf16", True, -2.0,
     L.GEMM_FLAG_COOPERATIVE, 128, L.GEMM_SCHED_PERSISTENT, 4, "row", "silu"),
    ("src_wide224_bf16_in_place_gelu", 520, 904, 1000, "bf16", "bf16", "bf16", True, 1.5, 0,
     (256, 224), L.GEMM_SCHED_PERSISTENT, 3, "col", "gelu"),
    ("src_wide224_fp8_e4m3_f32_src", 776, 688, 1040, "e4m3", "e4m3", "f32", False, -0.75, 0,
     (256, 224), L.GEMM_SCHED_PERSISTENT, 4, "row", "relu"),
    ("src_wide192_bf16_in_place_silu", 520, 904, 1000, "bf16", "bf16", "bf16", True, 0.5, 0,
     (256, 192), L.GEMM_SCHED_PERSISTENT, 3, "row", "silu"),
    ("src_wide256_fp8_streamk_bf16_src", 512, 768, 8192, "e4m3", "bf16", "bf16", False, 0.5,
     L.GEMM_FLAG_WIDE, 256, L.GEMM_SCHED_STREAMK, 4, "row", "silu"),
    ("src_wide256_bf16_f32_in_place_ragged", 300, 520, 3000, "bf16", "f32", "f32", True, 1.0,
     L.GEMM_FLAG_WIDE, 256, L.GEMM_SCHED_PERSISTENT, 2, None, None),
]


@pytest.mark.parametrize("case", SRC_CASES, ids=[c[0] for c in SRC_CASES])
def test_source_term_parity(dev, case):
    (name, M, N, K, dt, out, src_kind, in_place, beta, flags, tile, sched, workers, bias_kind,
     act) = case
    print(f"source case {name}: {M}x{N}x{K} {dt}->{out} S {src_kind}", flush=True)
    op = operands(name, M, N, K, dt) if K else gi.make_operands(M, N, 0, dt, seed=3)
    n_bias = M if bias_kind == "row" else N
    bias = gi.make_vector(n_bias, seed=zlib.crc32(name.encode()) % 977) if bias_kind else None
    S, s_vals = make_source(M, N, src_kind, seed=zlib.crc32(name.encode()) % 991)
    scale_d = 1.0
    if out == "e4m3":
        _, y = expected(op, bias_kind, bias, act, s_vals, beta)
        scale_d = float(np.float32(E.amax(y) / 448.0 * 0.8))
    got, am, plan = run_epi(op, dev, out, bias_kind, bias, act, True, scale_d, flags, sched,
                            workers, tile, source=S, beta=beta, in_place=in_place)
    coop = K == 0 or flags & (L.GEMM_FLAG_COOPERATIVE | L.GEMM_FLAG_STREAMK_CHAIN)
    assert plan.info.kernel == (0 if coop else 3)
    if sched == L.GEMM_SCHED_STREAMK:
        assert plan.info.sk_tiles > 0
        assert plan.info.streamk_mode == (0 if flags & L.GEMM_FLAG_STREAMK_CHAIN else 1)
    check(op, got, am, out, bias_kind, bias, act, scale_d, name, s_vals, beta)


@pytest.mark.parametrize("flags", [0, L.GEMM_FLAG_COOPERATIVE])
def test_zero_beta_reads_no_source(dev, flags):
    """beta = 0: the source is not read, so NaNs in it do not reach C, and the bits equal those
    of the same plan run without a source."""
    M, N, K = 264, 520, 256
    op = operands("beta0", M, N, K, "bf16")
    bias = gi.make_vector(N, seed=23)
    S = torch.full((M, N), float("nan"), dtype=torch.float32)
    got, am, plan = run_epi(op, dev, "f32", "col", bias, "gelu", True, 1.0, flags, tile=128,
                            source=S, beta=0.0)
    plain, am2, plan2 = run_epi(op, dev, "f32", "col", bias, "gelu", True, 1.0, flags,
                                tile=128)
    assert plan.info.kernel == plan2.info.kernel == (0 if flags else 3)
    assert np.isfinite(got).all() and np.array_equal(got, plain) and am == am2


@pytest.mark.parametrize("tile", [256, (256, 224), 128])
def test_source_of_zero_keeps_the_bits(dev, tile):
    """A zero source with beta = 1 adds exact zeros: the wide-wave kernel's source instantiation
    must store the bits of its plain fused instantiation (same products, same bias and
    activation), on the staged and the direct paths."""
    M, N, K = 520, 904, 1000
    op = operands("zero_src", M, N, K, "bf16")
    bias = gi.make_vector(N, seed=29)
    for out in ("bf16", "f32"):
        S = torch.zeros((M, N), dtype=torch.float32)
        got, am, plan = run_epi(op, dev, out, "col", bias, "gelu", True, 1.0, 0, tile=tile,
                                source=S, beta=1.0)
        plain, am2, _ = run_epi(op, dev, out, "col", bias, "gelu", True, 1.0, 0, tile=tile)
        assert plan.info.kernel == 3
        assert np.array_equal(got, plain) and am == am2, (tile, out)


@pytest.mark.parametrize("out", ["f32", "bf16", "e4m3"])
def test_zero_depth_gives_activation_of_bias(dev, out):
    """K = 0: Z is the bias alone, so Y = act(bias) exactly up to the activation's rounding."""
    M, N = 130, 136
    op = gi.make_operands(M, N, 0, "bf16", seed=3)
    bias = gi.make_vector(N, seed=5, dist=("normal", 2.0))
    got, am, plan = run_epi(op, dev, out, "col", bias, "gelu", True, 0.01, tile=128, workers=4)
    assert plan.info.kernel == 0
    check(op, got, am, out, "col", bias, "gelu", 0.01, f"K=0 {out}")


@pytest.mark.parametrize("kern", [("wide", L.GEMM_FLAG_WIDE, 256), ("coop", 0, 128),
                                  ("streamk", 0, 128)])
@pytest.mark.parametrize("bias_kind", ["row", "col"])
def test_e4m3_output_codes_exact(dev, kern, bias_kind):
    """Integer-valued products (A[m,k] = ((m+k) mod 8)/8, B = 1, so C = 7K/16 exactly) plus biases
    on a 1/8 grid make every Z exact in fp32 and put many Y / scale_d exactly on rounding
    midpoints of the e4m3 grid: the codes must equal the oracle's byte for byte (nearest-even,
    saturating), and so must amax."""
    name, flags, tile = kern
    M, N, K = 272, 520, (64 if name != "streamk" else 4096)
    op = gi.rowsum_pattern(M, N, K, "bf16")
    n_bias = M if bias_kind == "row" else N
    bias = (np.arange(n_bias) % 512 - 256).astype(np.float32) / 4.0     # -64 .. 63.75
    sched = L.GEMM_SCHED_STREAMK if name == "streamk" else L.GEMM_SCHED_PERSISTENT
    workers = 7 if name == "streamk" else 3
    # powers of two, so Y / scale_d is exact; the last one saturates most of the output
    scales = (1.0, 0.5, 0.0625) if K == 64 else (8.0, 4.0, 0.5)
    for act, scale_d in zip((None, "relu", None), scales):
        got, am, plan = run_epi(op, dev, "e4m3", bias_kind, bias, act, True, scale_d, flags,
                                sched, workers, tile)
        _, y = expected(op, bias_kind, bias, act)
        want = E.quantize_e4m3(y, scale_d)
        assert np.array_equal(E4M3_TABLE[got], E4M3_TABLE[want]), (name, act, scale_d)
        assert am == E.amax(y), (name, act, scale_d)


@pytest.mark.parametrize("kern", [("wide", L.GEMM_FLAG_WIDE, 256), ("coop", 0, 128)])
def test_amax_combines_with_the_value_present(dev, kern):
    """amax is max-combined into the float the caller passes: a larger value stays, a smaller
    one is raised to this call's max |Y|, and two calls in a row give the same result."""
    name, flags, tile = kern
    op = operands("amax_" + name, 264, 520, 256, "bf16")
    bias = gi.make_vector(520, seed=17)
    _, first, _ = run_epi(op, dev, "bf16", "col", bias, "silu", True, 1.0, flags, tile=tile)
    _, again, _ = run_epi(op, dev, "bf16", "col", bias, "silu", True, 1.0, flags, tile=tile)
    assert first == again > 0
    _, big, _ = run_epi(op, dev, "bf16", "col", bias, "silu", True, 1.0, flags, tile=tile,
                        amax_init=1e30)
    assert big == np.float32(1e30)
    _, small, _ = run_epi(op, dev, "bf16", "col", bias, "silu", True, 1.0, flags, tile=tile,
                          amax_init=first / 2)
    assert small == first


@pytest.mark.parametrize("flags,tile", [(L.GEMM_FLAG_WIDE, 256), (L.GEMM_FLAG_COOPERATIVE, 256),
                                        (L.GEMM_FLAG_COOPERATIVE, 128)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_fused_path_keeps_the_products(dev, flags, tile, out):
    """The fused instantiation with only amax requested stores the same bits as the plain
    kernel (the MAC loop is shared; only the store differs), apart from the sign of exact zeros."""
    M, N, K = 520, 776, 1000
    op = operands("keep", M, N, K, "bf16")
    fused, am, _ = run_epi(op, dev, out, None, None, None, True, 1.0, flags, tile=tile)
    A, B, sa, sb = to_device(op, torch, dev)
    plan = L.Plan(L.make_desc(M, N, K, L.GEMM_BF16, OUT[out], L.GEMM_MAP_GROUPED_M, 2,
                              L.GEMM_SCHED_PERSISTENT, 3, tile, tile, 0, flags))
    C = torch.empty((M, N), device=dev, dtype=torch.float32 if out == "f32" else torch.bfloat16)
    plan.run(A, B, C)
    torch.cuda.synchronize()
    plain = decode_output(C, torch)
    assert np.array_equal(fused, plain)
    assert am == float(np.float32(np.abs(plain).max())) or out == "bf16"


@pytest.mark.parametrize("kern", [("wide", L.GEMM_FLAG_WIDE, 256), ("coop", L.GEMM_FLAG_COOPERATIVE, 128),
                                  ("wide", 0, 128), ("streamk", 0, 128), ("streamk", 0, 256),
                                  ("streamk", L.GEMM_FLAG_COOPERATIVE, 128)])
@pytest.mark.parametrize("out", ["bf16", "e4m3", "f32"])
@pytest.mark.parametrize("bias_kind", ["row", "col"])
def test_amax_ignores_positions_past_the_edge(dev, kern, out, bias_kind):
    """Ragged M and N: the tile positions past the edge of C have zero accumulators but still
    meet a bias (a row bias reaches columns past N, a column bias rows past M).  With every bias
    below -C, |Y| there would exceed every |Y| inside C, so amax must come from inside C only:
    exactly max |C + bias| for integer-exact products."""
    name, flags, tile = kern
    M, N, K = 300, 264, (64 if name != "streamk" else 4096)
    op = gi.rowsum_pattern(M, N, K, "bf16")                     # C = 7K/16 everywhere
    c = 7 * K / 16
    n_bias = M if bias_kind == "row" else N
    bias = (-c - 8.0 - (np.arange(n_bias) % 64) / 4.0).astype(np.float32)  # Z in [-23.75, -8]
    sched = L.GEMM_SCHED_STREAMK if name == "streamk" else L.GEMM_SCHED_PERSISTENT
    workers = (7 if tile == 128 else 16) if name == "streamk" else 3
    got, am, plan = run_epi(op, dev, out, bias_kind, bias, None, True, 0.125, flags, sched,
                            workers, tile)
    if name == "streamk":
        assert plan.info.sk_tiles > 0
    assert plan.info.kernel == (0 if flags & L.GEMM_FLAG_COOPERATIVE else 3)
    _, y = expected(op, bias_kind, bias, None)
    assert am == E.amax(y) == 23.75, (name, out, bias_kind, am)
    if out == "e4m3":
        assert np.array_equal(E4M3_TABLE[got], E4M3_TABLE[E.quantize_e4m3(y, 0.125)])
    else:
        assert np.array_equal(got, y)


@pytest.mark.parametrize("src_kind", ["f32", "bf16"])
def test_gemm_helper_with_source(dev, src_kind):
    """The package's one-call gemm() with a source, a column bias and ReLU, on the planner's own
    choices, against the oracle."""
    import dense_gemm_design_amd as dg
    M, N, K = 520, 776, 1000
    op = operands("helper_src_" + src_kind, M, N, K, "bf16")
    A, B, _, _ = to_device(op, torch, dev)
    bias = gi.make_vector(N, seed=31)
    S, s_vals = make_source(M, N, src_kind, seed=37)
    C = dg.gemm(A.view(torch.bfloat16), B.view(torch.bfloat16), out_dtype="f32",
                bias_col=torch.from_numpy(bias).to(dev), activation="relu",
                source=S.to(dev), beta=-0.5)
    torch.cuda.synchronize()
    z, y = expected(op, "col", bias, "relu", s_vals, -0.5)
    ma = oracle.max_abs_decoded(op.A, oracle_dtype(op), op.scale_a)
    mb = oracle.max_abs_decoded(op.B, oracle_dtype(op), op.scale_b)
    tol = E.tolerance(y, z, op.K, ma, mb, out="f32", s_ref=-0.5 * s_vals)
    got = decode_output(C, torch)
    assert np.isfinite(got).all() and (np.abs(got - y) <= tol).all()
