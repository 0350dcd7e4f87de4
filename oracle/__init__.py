"""Reference CPU oracle for the tiled dense GEMM -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this package.
The HIP library never imports it, and it imports nothing from the HIP library: the two share
only the seeded input generators in gemm_inputs/, which hold none of the GEMM's arithmetic.

Contents
  gemm_ref / gemm_ref_sampled   fp64 C = A x B over the raw operand bytes (gemm_oracle.c)
  decode_bf16 / decode_e4m3     exact operand decoders (gemm_oracle.c)
  encode_e4m3 / _f64 / _array   nearest-even, saturating e4m3 encoder (checks the generator,
                                expected codes of an e4m3 output)
  epilogue                      the fused epilogue: bias, activation, amax, output quantisation
                                (oracle/epilogue.py)
  tolerance                     the per-element acceptance bound
  schedule                      CPU enumeration of the tile mapping, worker assignment and
                                Stream-K splits (oracle/schedule.py)
"""
import ctypes
import math
import os

import numpy as np

from . import schedule  # noqa: F401  (re-exported)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

BF16 = 0
E4M3 = 1
ROW = 0
COL = 1


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(os.path.join(_HERE, "gemm_oracle.c"))):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
    lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
    lib.oracle_decode_bf16.restype = dbl
    lib.oracle_decode_e4m3.argtypes = [ctypes.c_uint8]
    lib.oracle_decode_e4m3.restype = dbl
    lib.oracle_encode_e4m3.argtypes = [ctypes.c_float]
    lib.oracle_encode_e4m3.restype = ctypes.c_uint8
    lib.oracle_encode_e4m3_f64.argtypes = [dbl]
    lib.oracle_encode_e4m3_f64.restype = ctypes.c_uint8
    lib.oracle_encode_e4m3_array.argtypes = [vp, vp, i64]
    lib.oracle_encode_e4m3_array.restype = None
    lib.oracle_gemm.argtypes = [i64, i64, i64, i32, vp, i32, vp, i32, dbl, dbl, vp, i32]
    lib.oracle_gemm.restype = i32
    lib.oracle_gemm_sampled.argtypes = [i64, i64, i64, i32, vp, i32, vp, i32, dbl, dbl,
                                        vp, vp, i64, vp, i32]
    lib.oracle_gemm_sampled.restype = i32
    _lib = lib
    return lib


def default_threads() -> int:
    n = os.cpu_count() or 1
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        pass
    return max(1, min(n, 16))


def decode_bf16(bits: int) -> float:
    return _load().oracle_decode_bf16(int(bits) & 0xFFFF)


def decode_e4m3(code: int) -> float:
    return _load().oracle_decode_e4m3(int(code) & 0xFF)


def encode_e4m3(x: float) -> int:
    """e4m3 code of x rounded to binary32 first (the generator's fp32 quantisation)."""
    return int(_load().oracle_encode_e4m3(float(x)))


def encode_e4m3_f64(x: float) -> int:
    """e4m3 code of x at full double precision."""
    return int(_load().oracle_encode_e4m3_f64(float(x)))


def encode_e4m3_array(x) -> np.ndarray:
    """e4m3 codes (uint8, same shape) of an array of doubles, each at full double precision."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    _load().oracle_encode_e4m3_array(x.ctypes.data, out.ctypes.data, x.size)
    return out


def _raw(arr, dtype):
    """Contiguous numpy view of the operand's storage bytes (uint16 for bf16, uint8 for e4m3)."""
    want = np.uint16 if dtype == BF16 else np.uint8
    a = np.ascontiguousarray(arr)
    if a.dtype != want:
        raise TypeError(f"operand storage must be {want}, got {a.dtype}")
    return a


def gemm_ref(M, N, K, dtype, A, B, layout_a=ROW, layout_b=COL, scale_a=1.0, scale_b=1.0,
             threads=None):
    """fp64 C (M x N, row-major) from the operands' raw storage (numpy uint16 / uint8 arrays)."""
    A = _raw(A, dtype)
    B = _raw(B, dtype)
    if A.size != M * K or B.size != K * N:
        raise ValueError("operand sizes do not match M, N, K")
    C = np.zeros((M, N), dtype=np.float64)
    rc = _load().oracle_gemm(M, N, K, dtype, A.ctypes.data, layout_a, B.ctypes.data, layout_b,
                             float(scale_a), float(scale_b), C.ctypes.data,
                             threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_gemm failed ({rc})")
    return C


def gemm_ref_sampled(M, N, K, dtype, A, B, rows, cols, layout_a=ROW, layout_b=COL,
                     scale_a=1.0, scale_b=1.0, threads=None):
    """fp64 C[rows[i], cols[i]] for each i, computed one element at a time."""
    A = _raw(A, dtype)
    B = _raw(B, dtype)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    out = np.zeros(rows.shape, dtype=np.float64)
    rc = _load().oracle_gemm_sampled(M, N, K, dtype, A.ctypes.data, layout_a, B.ctypes.data,
                                     layout_b, float(scale_a), float(scale_b), rows.ctypes.data,
                                     cols.ctypes.data, rows.size, out.ctypes.data,
                                     threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_sampled failed ({rc})")
    return out


def tolerance(c_ref, K, max_abs_a, max_abs_b):
    """Per-element bound |C - C_ref| <= 4e-3 |C_ref| + 1e-3 sqrt(K) max|a| max|b|.

    A relative term for the output rounding (a bf16 result carries 2^-9 relative error) plus an
    absolute term that grows like the square root of the reduction length, for fp32-class
    accumulation error.  For FP8 operands max|a| and max|b| are taken over the dequantised
    values s * q.
    """
    return 4e-3 * np.abs(c_ref) + 1e-3 * math.sqrt(K) * float(max_abs_a) * float(max_abs_b)


def max_abs_decoded(raw, dtype, scale=1.0):
    """max |decoded value| of an operand's storage, times its scale (exact lookup per code)."""
    raw = np.ascontiguousarray(raw)
    if dtype == E4M3:
        table = np.array([abs(decode_e4m3(c)) for c in range(256)], dtype=np.float64)
        table[np.isnan(table)] = 0.0
        present = np.bincount(raw.reshape(-1), minlength=256) > 0
        return float(table[present].max(initial=0.0)) * float(scale)
    bits = raw.reshape(-1).astype(np.uint32) << np.uint32(16)
    vals = np.abs(bits.view(np.float32).astype(np.float64))
    return float(vals.max(initial=0.0)) * float(scale)


from . import epilogue  # noqa: E402,F401  (re-exported; uses the encoders above)
