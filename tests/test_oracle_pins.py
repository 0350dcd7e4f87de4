"""Pins the CPU oracle's arithmetic to facts that do not come from the oracle itself.

Each check is chosen so that a plausible mistake in the oracle (a dropped term, a wrong sign,
a transposed operand, a wrong layout index, a bad decoder entry, a missing scale) fails it:
identity and all-ones operands, a closed-form row sum, exact rational brute force on small
shapes, the format facts printed by the pages, and library decoders/encoders (torch).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import gemm_inputs as gi
import oracle
from golden_util import load, ints


def dec_bf16(raw):
    return (raw.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def test_bf16_decoder_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=4000, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.decode_bf16(int(b)) for b in bits])
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_e4m3_decoder_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.decode_e4m3(c) for c in range(256)])
    for c in range(256):
        if np.isnan(ref[c]):
            assert np.isnan(got[c]), c
        else:
            assert got[c] == ref[c], (c, got[c], ref[c])
    # exactly two NaN codes (S.1111.111) and no infinities
    assert np.isnan(got).sum() == 2 and not np.isinf(got).any()


def test_e4m3_format_facts_from_pages():
    g = load("e4m3_format.txt")
    mx = float(g["max_finite"][0])
    vals = np.array([oracle.decode_e4m3(c) for c in range(256)])
    assert np.nanmax(vals) == mx and np.nanmin(vals) == -mx
    for s in g["saturate"]:
        x, want = (float(t) for t in s.split())
        assert oracle.decode_e4m3(oracle.encode_e4m3(x)) == want


def test_e4m3_encoder_matches_torch_nearest_even():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.normal(0, 100, 20000), rng.normal(0, 1, 20000), rng.uniform(-448, 448, 5000),
        rng.normal(0, 0.01, 5000),
    ]).astype(np.float32)
    # every exact midpoint between neighbouring codes: ties must go to the even mantissa
    finite = sorted({oracle.decode_e4m3(c) for c in range(0x7F)})
    mids = np.array([(a + b) / 2 for a, b in zip(finite, finite[1:])], dtype=np.float32)
    x = np.concatenate([x, mids, -mids]).clip(-448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.encode_e4m3(float(v)) for v in x], dtype=np.uint8)
    # +0 and -0 are both valid codes for a zero result; compare values, then codes elsewhere
    dv = lambda cs: np.array([oracle.decode_e4m3(int(c)) for c in cs])
    assert np.array_equal(dv(got), dv(ref))
    nz = dv(ref) != 0
    assert np.array_equal(got[nz], ref[nz])


def test_generator_fp8_bytes_match_oracle_encoder():
    """The generator's quantiser (torch) and the oracle's encoder (C) agree code for code."""
    M, N, K = 24, 16, 40
    op = gi.make_operands(M, N, K, "e4m3", ("normal", 1.0), ("normal", 1.0), seed=7)
    gen = torch.Generator(device="cpu")
    gen.manual_seed(7)
    a = torch.randn((M, K), generator=gen, dtype=torch.float32)
    b = torch.randn((N, K), generator=gen, dtype=torch.float32)
    for x, codes, scale in ((a, op.A, op.scale_a), (b, op.B, op.scale_b)):
        amax = float(x.abs().max())
        assert scale == float(np.float32(np.float32(amax) / np.float32(448.0)))
        y = (x / torch.tensor(scale, dtype=torch.float32)).numpy().astype(np.float32)
        want = np.array([oracle.encode_e4m3(float(v)) for v in y.reshape(-1)], dtype=np.uint8)
        dv = lambda cs: np.array([oracle.decode_e4m3(int(c)) for c in cs])
        assert np.array_equal(dv(codes.reshape(-1)), dv(want))
        # the largest-magnitude element lands on the format's maximum
        assert np.nanmax(np.abs(dv(codes.reshape(-1)))) == 448.0


@pytest.mark.parametrize("dtype", ["bf16", "e4m3"])
def test_closed_form_row_sums(dtype):
    """A[m,k] = ((m+k) mod 8)/8, B = 1, K multiple of 8: every C element is exactly 7K/16."""
    M, N, K = 24, 20, 64
    op = gi.rowsum_pattern(M, N, K, dtype)
    code = oracle.BF16 if dtype == "bf16" else oracle.E4M3
    C = oracle.gemm_ref(M, N, K, code, op.A, op.B)
    assert np.all(C == 7 * K / 16)


def test_identity_returns_b():
    M, N = 48, 40
    op = gi.identity_operands(M, N, seed=5)
    C = oracle.gemm_ref(M, N, M, oracle.BF16, op.A, op.B)
    # b(k, n) is stored at n*K + k, so C[m, n] = b(m, n) = storage[n, m]
    assert np.array_equal(C, dec_bf16(op.B).reshape(N, M).T)


def test_all_ones_b_gives_exact_row_sums():
    M, N, K = 16, 8, 96
    op = gi.make_operands(M, N, K, "bf16", seed=9)
    ones = gi.bf16_bits(torch.ones((N, K)))
    C = oracle.gemm_ref(M, N, K, oracle.BF16, op.A, ones)
    a = dec_bf16(op.A).reshape(M, K)
    for m in range(M):
        exact = sum(Fraction(v) for v in a[m])
        assert np.all(C[m] == float(exact))


def _brute(a, b, K, scale=Fraction(1)):
    """Exact rational C from decoded operand matrices a (M x K) and b (K x N)."""
    M, N = a.shape[0], b.shape[1]
    out = np.empty((M, N), dtype=object)
    for m in range(M):
        for n in range(N):
            out[m, n] = scale * sum(Fraction(a[m, k]) * Fraction(b[k, n]) for k in range(K))
    return out


@pytest.mark.parametrize("shape", [(16, 16, 16), (5, 7, 3), (9, 4, 33)])
def test_bf16_brute_force_rational(shape):
    M, N, K = shape
    op = gi.make_operands(M, N, K, "bf16", seed=11 + M)
    C = oracle.gemm_ref(M, N, K, oracle.BF16, op.A, op.B)
    a = dec_bf16(op.A).reshape(M, K)
    b = dec_bf16(op.B).reshape(N, K).T
    exact = _brute(a, b, K)
    bound = np.abs(a) @ np.abs(b) * K * 2.0 ** -52 + 1e-300
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(C[m, n]) - exact[m, n]) <= Fraction(bound[m, n])


def test_e4m3_brute_force_rational_with_scales():
    M, N, K = 16, 16, 16
    op = gi.make_operands(M, N, K, "e4m3", ("normal", 1.0), ("normal", 1.0), seed=21)
    C = oracle.gemm_ref(M, N, K, oracle.E4M3, op.A, op.B, scale_a=op.scale_a, scale_b=op.scale_b)
    dv = np.vectorize(lambda c: oracle.decode_e4m3(int(c)))
    qa = dv(op.A).reshape(M, K)
    qb = dv(op.B).reshape(N, K).T
    scale = Fraction(op.scale_a) * Fraction(op.scale_b)
    exact = _brute(qa, qb, K, scale)
    for m in range(M):
        for n in range(N):
            # integer-grid products of e4m3 values sum exactly in fp64; one rounding for the scale
            assert abs(Fraction(C[m, n]) - exact[m, n]) <= abs(exact[m, n]) * Fraction(2) ** -52


def test_layouts_are_transposes():
    """Row-major A and its column-major copy give the same C; same for B."""
    M, N, K = 12, 10, 14
    op = gi.make_operands(M, N, K, "bf16", seed=31)
    C = oracle.gemm_ref(M, N, K, oracle.BF16, op.A, op.B, oracle.ROW, oracle.COL)
    a_col = np.ascontiguousarray(op.A.reshape(M, K).T)      # K x M storage: (m,k) at k*M+m
    b_row = np.ascontiguousarray(op.B.reshape(N, K).T)      # K x N storage: (k,n) at k*N+n
    C2 = oracle.gemm_ref(M, N, K, oracle.BF16, a_col, b_row, oracle.COL, oracle.ROW)
    assert np.array_equal(C, C2)
    # and the product is not symmetric in its operands: swapping them changes the answer
    C3 = oracle.gemm_ref(N, M, K, oracle.BF16, op.B, op.A, oracle.ROW, oracle.COL)
    assert np.array_equal(C3, C.T)


def test_sampled_equals_full():
    M, N, K = 40, 36, 72
    op = gi.make_operands(M, N, K, "bf16", seed=41)
    C = oracle.gemm_ref(M, N, K, oracle.BF16, op.A, op.B)
    rows, cols = gi.sample_positions(M, N, 200, seed=1, BM=16, BN=16)
    s = oracle.gemm_ref_sampled(M, N, K, oracle.BF16, op.A, op.B, rows, cols)
    assert np.array_equal(s, C[rows, cols])


def test_tolerance_formula_values():
    # |C - C_ref| <= 4e-3 |C_ref| + 1e-3 sqrt(K) max|a| max|b|
    t = oracle.tolerance(np.array([0.0, 10.0, -10.0]), 4096, 1.0, 1.0)
    assert np.allclose(t, [0.064, 0.104, 0.104])
    t = oracle.tolerance(np.array([2.0]), 65536, 0.5, 2.0)
    assert np.allclose(t, [4e-3 * 2 + 1e-3 * 256])


def test_max_abs_decoded():
    op = gi.rowsum_pattern(8, 8, 16, "e4m3")
    assert oracle.max_abs_decoded(op.A, oracle.E4M3, 2.0) == 7 / 8 * 2.0
    op = gi.rowsum_pattern(8, 8, 16, "bf16")
    assert oracle.max_abs_decoded(op.A, oracle.BF16) == 7 / 8
