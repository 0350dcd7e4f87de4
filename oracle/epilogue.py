"""Fused-epilogue reference -- TEST INFRASTRUCTURE ONLY.

Part of the oracle package: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg
may use it, and the HIP library never does.  Everything here is float64 numpy on the output of
oracle.gemm_ref, in the order of the forward template of the "H100 Kernel Design" lesson,
section 12 (12.2 steps 2-5 and 12.3 template 1):

    Z = alpha * Acc           gemm_ref's result (alpha = s_a * s_b for e4m3 operands, else 1)
    Z = Z + beta * S          an optional source matrix S (M x N), 12.1 item 1, 12.2 step 2
    Z = Z + bias              one value per row (length M) or one per column (length N)
    Y = act(Z)                ReLU, GELU or SiLU (12.1 item 3)
    amax = max |Y|            collected at the output-scaling step (12.2 step 5, 12.1 item 8)
    D = cast(Y)               f32 or bf16, or the e4m3 code of Y / scale_d (12.2 steps 5 and 7)

Readings where the page leaves a step open:
  * GELU is the exact form z * Phi(z), Phi the standard normal distribution function, written
    0.5 * (1 + erf(z / sqrt(2)));  SiLU is z * sigmoid(z);  ReLU is max(z, 0).
  * amax is the largest |Y| in full precision, before the output scale and the cast.
  * scale_d is a dequantisation scale like the operands' per-tensor scales ("WGMMA part 2"
    lesson, section 11): an e4m3 output code q stands for scale_d * q, so q is Y / scale_d
    rounded to nearest-even on the e4m3 grid and saturated to +-448 (sections 10 and 13).
"""
import math

import numpy as np
from scipy.special import erf, expit

ACTIVATIONS = (None, "relu", "gelu", "silu")


def relu(z):
    """max(z, 0)."""
    z = np.asarray(z, dtype=np.float64)
    return np.where(z < 0.0, 0.0, z)


def gelu(z):
    """z * Phi(z) with Phi(z) = 0.5 * (1 + erf(z / sqrt 2)), the standard normal CDF."""
    z = np.asarray(z, dtype=np.float64)
    return z * 0.5 * (1.0 + erf(z / math.sqrt(2.0)))


def silu(z):
    """z * sigmoid(z), sigmoid(z) = 1 / (1 + exp(-z)) (scipy's expit)."""
    z = np.asarray(z, dtype=np.float64)
    return z * expit(z)


def activation(z, act):
    if act is None:
        return np.asarray(z, dtype=np.float64)
    return {"relu": relu, "gelu": gelu, "silu": silu}[act](z)


def apply(c, bias_row=None, bias_col=None, act=None, source=None, beta=0.0):
    """Y = act(C + beta * S + bias) for C = alpha * Acc (M x N float64); returns (Z, Y).

    source: M x N values S (taken exactly, as float64), scaled by beta -- the linear combination
    alpha * Acc + beta * C of section 12.1 item 1, formed first (section 12.2 step 2);
    bias_row: length-M vector added to every column (Z[m, n] += bias_row[m]);
    bias_col: length-N vector added to every row (Z[m, n] += bias_col[n]).
    """
    z = np.array(c, dtype=np.float64, copy=True)
    if source is not None:
        s = np.asarray(source, dtype=np.float64)
        if s.shape != z.shape:
            raise ValueError("the source must be M x N")
        z = z + float(beta) * s
    if bias_row is not None and bias_col is not None:
        raise ValueError("one bias vector at most")
    if bias_row is not None:
        b = np.asarray(bias_row, dtype=np.float64)
        if b.shape != (z.shape[0],):
            raise ValueError("row bias must have length M")
        z = z + b[:, None]
    if bias_col is not None:
        b = np.asarray(bias_col, dtype=np.float64)
        if b.shape != (z.shape[1],):
            raise ValueError("column bias must have length N")
        z = z + b[None, :]
    return z, activation(z, act)


def amax(y):
    """max |Y| over every element (0 for an empty output)."""
    y = np.asarray(y, dtype=np.float64)
    return float(np.abs(y).max(initial=0.0))


def quantize_e4m3(y, scale_d):
    """e4m3 codes of Y / scale_d (nearest-even, saturating), computed in float64."""
    from . import encode_e4m3_array
    return encode_e4m3_array(np.asarray(y, dtype=np.float64) / float(scale_d))


def tolerance(y_ref, z_ref, k, max_abs_a, max_abs_b, out="bf16", s_ref=None):
    """Per-element bound on |Y_gpu - Y_ref| before any output rounding, plus the output cast.

    The accumulation error of Z is bounded as in oracle.tolerance (1e-3 sqrt(K) max|a| max|b|)
    with a 2e-6 |Z| allowance for the rounded additions of alpha and the bias, and 2e-6 |beta S|
    more for the source term s_ref = beta * S (its rounded product and sum); the activations
    are Lipschitz with constant below 1.2 (ReLU 1, SiLU 1.1, GELU 1.13) and are evaluated to a
    few fp32 ulps.  A bf16 output adds its own rounding, 4e-3 |Y_ref|; f32 output adds nothing
    more, and an e4m3 output is checked on the code grid instead (quantized_bounds).
    """
    z = np.abs(np.asarray(z_ref, dtype=np.float64))
    base = 1.2 * (1e-3 * math.sqrt(k) * float(max_abs_a) * float(max_abs_b) + 2e-6 * z) + 1e-6 * z
    if s_ref is not None:
        base = base + 1.2 * 2e-6 * np.abs(np.asarray(s_ref, dtype=np.float64))
    if out == "bf16":
        return base + 4e-3 * np.abs(np.asarray(y_ref, dtype=np.float64))
    return base


def quantized_bounds(y_ref, tol, scale_d):
    """Lowest and highest e4m3 value (as float64, in units of scale_d) a correct kernel may
    store: the codes of (Y_ref -+ tol) / scale_d, since nearest-even rounding never decreases."""
    from . import decode_e4m3
    table = np.array([decode_e4m3(c) for c in range(256)], dtype=np.float64)
    lo = table[quantize_e4m3(np.asarray(y_ref) - tol, scale_d)]
    hi = table[quantize_e4m3(np.asarray(y_ref) + tol, scale_d)]
    return lo, hi
