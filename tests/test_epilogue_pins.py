"""Pins the oracle's fused epilogue (oracle/epilogue.py) to facts that do not come from it.

Textbook values of the standard normal distribution function and of the logistic function,
the odd-part identities act(z) - act(-z) = z that GELU and SiLU share, closed forms of the
epilogue on all-ones operands (which fix the bias orientation, the bias-before-activation order
and amax), the e4m3 grid near rounding midpoints, and torch's own e4m3 cast.
"""
import math

import numpy as np
import pytest
import torch

import gemm_inputs as gi
import oracle
from oracle import epilogue as epi


# Standard normal distribution function Phi(z), four decimals, as printed in statistical tables.
PHI_TABLE = {0.5: 0.6915, 1.0: 0.8413, 1.5: 0.9332, 2.0: 0.9772, 2.5: 0.9938, 3.0: 0.9987}


def test_gelu_is_z_times_normal_cdf():
    for z, phi in PHI_TABLE.items():
        assert abs(epi.gelu(z) / z - phi) < 5e-5, z
        # Phi(-z) = 1 - Phi(z)
        assert abs(epi.gelu(-z) / -z - (1.0 - phi)) < 5e-5, z
    assert epi.gelu(0.0) == 0.0
    assert epi.gelu(10.0) == pytest.approx(10.0, rel=1e-15)
    assert abs(epi.gelu(-10.0)) < 1e-20


@pytest.mark.parametrize("fn", ["gelu", "silu"])
def test_odd_part_is_identity(fn):
    """GELU(z) - GELU(-z) = z and SiLU(z) - SiLU(-z) = z, since Phi(z) + Phi(-z) = 1 and
    sigmoid(z) + sigmoid(-z) = 1."""
    z = np.random.default_rng(3).normal(0, 3, 1000)
    f = getattr(epi, fn)
    assert np.allclose(f(z) - f(-z), z, rtol=1e-13, atol=1e-13)


def test_silu_closed_forms():
    assert epi.silu(0.0) == 0.0
    assert epi.silu(1.0) == pytest.approx(math.e / (1.0 + math.e), rel=1e-15)
    # sigmoid(ln 3) = 1 / (1 + 1/3) = 3/4
    assert epi.silu(math.log(3.0)) == pytest.approx(0.75 * math.log(3.0), rel=1e-15)
    assert epi.silu(-800.0) == 0.0 and epi.silu(800.0) == 800.0   # no overflow at the ends


def test_relu_values():
    assert np.array_equal(epi.relu(np.array([-2.0, -1e-300, 0.0, 3.5])), [0.0, 0.0, 0.0, 3.5])


def _ones(M, N, K):
    """C = A x B for all-ones operands: every element is exactly K."""
    one = gi.bf16_bits(torch.ones(1))[0]
    A = np.full(M * K, one, dtype=np.uint16)
    B = np.full(N * K, one, dtype=np.uint16)
    return oracle.gemm_ref(M, N, K, oracle.BF16, A, B)


def test_bias_orientation():
    """Column bias varies along n, row bias along m (M != N, so a transposed bias cannot fit)."""
    M, N, K = 3, 5, 16
    C = _ones(M, N, K)
    _, y = epi.apply(C, bias_col=np.arange(N, dtype=np.float64))
    assert np.array_equal(y, K + np.arange(N)[None, :] + np.zeros((M, 1)))
    _, y = epi.apply(C, bias_row=np.arange(M, dtype=np.float64) * 10)
    assert np.array_equal(y, K + 10 * np.arange(M)[:, None] + np.zeros((1, N)))
    with pytest.raises(ValueError):
        epi.apply(C, bias_col=np.zeros(M))
    with pytest.raises(ValueError):
        epi.apply(C, bias_row=np.zeros(M), bias_col=np.zeros(N))


def test_bias_is_added_before_the_activation():
    M, N, K = 4, 8, 32
    C = _ones(M, N, K)
    _, y = epi.apply(C, bias_col=np.full(N, -(K + 0.5)), act="relu")
    assert np.all(y == 0.0)            # relu(K - K - 0.5); relu first would leave -0.5
    _, y = epi.apply(C, bias_col=np.full(N, -(K - 0.5)), act="relu")
    assert np.all(y == 0.5)
    _, y = epi.apply(C, bias_row=np.full(M, -float(K)), act="gelu")
    assert np.all(y == 0.0)            # gelu(0) = 0
    z, y = epi.apply(C, bias_col=np.full(N, 1.0 - K), act="silu")
    assert np.all(z == 1.0) and np.allclose(y, math.e / (1.0 + math.e), rtol=1e-15)


def test_source_term_hand_worked():
    """Z = alpha Acc + beta S, then the bias, then the activation, worked by hand on all-ones
    operands (Acc = K = 16): with S = [[3, 1], [-40, 0]], beta = 0.5 and a column bias
    (0.25, -17), Z = [[16 + 1.5 + 0.25, 16 + 0.5 - 17], [16 - 20 + 0.25, 16 + 0 - 17]]
    = [[17.75, -0.5], [-3.75, -1]]; ReLU keeps 17.75 alone."""
    C = _ones(2, 2, 16)
    S = np.array([[3.0, 1.0], [-40.0, 0.0]])
    z, y = epi.apply(C, bias_col=np.array([0.25, -17.0]), act="relu", source=S, beta=0.5)
    assert np.array_equal(z, [[17.75, -0.5], [-3.75, -1.0]])
    assert np.array_equal(y, [[17.75, 0.0], [0.0, 0.0]])
    # beta = 0 is the product alone; beta = -1 with S = C cancels it: Z is the bias
    assert np.array_equal(epi.apply(C, source=S, beta=0.0)[0], C)
    z, y = epi.apply(C, bias_row=np.array([1.0, -1.0]), act="gelu", source=C, beta=-1.0)
    assert np.array_equal(z, [[1.0, 1.0], [-1.0, -1.0]])
    assert abs(y[0, 0] - PHI_TABLE[1.0]) < 5e-5 and abs(y[1, 0] + (1 - PHI_TABLE[1.0])) < 5e-5
    with pytest.raises(ValueError):
        epi.apply(C, source=np.zeros((2, 3)), beta=1.0)


def test_amax_closed_form():
    M, N, K = 2, 8, 16
    C = _ones(M, N, K)
    bias = np.arange(N, dtype=np.float64) - 3 * K      # Z[m, n] = n - 2K, all negative
    _, y = epi.apply(C, bias_col=bias)
    assert epi.amax(y) == 2 * K
    _, y = epi.apply(C, bias_col=bias, act="relu")
    assert epi.amax(y) == 0.0
    assert epi.amax(np.zeros((0, 4))) == 0.0


def test_e4m3_output_codes():
    M, N, K = 2, 8, 64
    C = _ones(M, N, K)
    _, y = epi.apply(C)
    assert np.all(epi.quantize_e4m3(y, 0.5) == 0x70)     # 128 = 2^7: exponent field 14
    assert np.all(epi.quantize_e4m3(-y, 0.5) == 0xF0)
    assert np.all(epi.quantize_e4m3(y, 0.125) == 0x7E)   # 512 saturates to 448
    assert np.all(epi.quantize_e4m3(-y, 0.125) == 0xFE)
    # 16 and 18 are neighbours on the grid: 17 is a tie (even mantissa: 16), anything above it
    # goes to 18 -- at float64 precision, where a binary32 rounding would land on the tie
    assert oracle.encode_e4m3_f64(17.0) == 0x58
    assert oracle.encode_e4m3_f64(17.0 + 1e-9) == 0x59
    assert oracle.encode_e4m3(17.0 + 1e-9) == 0x58
    assert oracle.encode_e4m3_f64(19.0) == 0x5A                # tie between 18 and 20 -> 20


def test_e4m3_array_encoder_matches_torch():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.normal(0, 50, 20000), rng.normal(0, 0.02, 5000)]).astype(np.float32)
    x = x.clip(-448, 448).astype(np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.encode_e4m3_array(x)
    table = np.array([oracle.decode_e4m3(c) for c in range(256)])
    assert np.array_equal(table[got], table[ref])


def test_quantized_bounds_bracket_the_code():
    y = np.random.default_rng(6).normal(0, 100, 2000)
    table = np.array([oracle.decode_e4m3(c) for c in range(256)])
    q = table[epi.quantize_e4m3(y, 0.5)]
    lo, hi = epi.quantized_bounds(y, 0.0, 0.5)
    assert np.array_equal(lo, q) and np.array_equal(hi, q)
    lo, hi = epi.quantized_bounds(y, 3.0, 0.5)
    assert np.all(lo <= q) and np.all(q <= hi) and np.any(lo < hi)


def test_epilogue_tolerance_values():
    # 1.2 (1e-3 sqrt(K) max|a| max|b| + 2e-6 |Z|) + 1e-6 |Z|  (+ 4e-3 |Y| for bf16 output)
    t = epi.tolerance(np.array([2.0]), np.array([1.0]), 4096, 1.0, 0.5, out="f32")
    assert np.allclose(t, [1.2 * (1e-3 * 64 * 0.5 + 2e-6) + 1e-6])
    t = epi.tolerance(np.array([2.0]), np.array([1.0]), 4096, 1.0, 0.5, out="bf16")
    assert np.allclose(t, [1.2 * (1e-3 * 64 * 0.5 + 2e-6) + 1e-6 + 8e-3])
    # a source term beta S adds 1.2 * 2e-6 |beta S|
    t = epi.tolerance(np.array([2.0]), np.array([1.0]), 4096, 1.0, 0.5, out="f32",
                      s_ref=np.array([-100.0]))
    assert np.allclose(t, [1.2 * (1e-3 * 64 * 0.5 + 2e-6) + 1e-6 + 1.2 * 2e-4])
