"""Seeded synthetic operands for the dense GEMM workloads.

This module only draws numbers and stores them; it holds none of the GEMM's arithmetic.  Both
the HIP path's tests/benchmark and the CPU oracle read the bytes it produces, so the two sides see
identical inputs.

Operand storage (K-major for both operands, as FP8 requires and BF16 prefers):
  A: M x K, row-major          -> element (m, k) at m*K + k
  B: K x N, column-major       -> element (k, n) at n*K + k, i.e. stored as an N x K array

Draw order: A first, then B, each in storage order, from torch.Generator('cpu') seeded per
workload.  uniform[-1, 1] is 2*rand - 1 in fp32; N(0, s) is s*randn in fp32; both are then
rounded to bf16 (nearest-even).  FP8 operands are drawn N(0, 1) in fp32 and quantised per tensor
(quantize_e4m3_per_tensor below).
"""
from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dtype: str            # "bf16" or "e4m3"
    out: str              # "f32" or "bf16"
    dist_a: tuple         # ("uniform",) | ("normal", sigma)
    dist_b: tuple
    mapping: str          # "linear_n" | "linear_m" | "grouped_m" | "grouped_n"
    group: int
    sched: str            # "static" | "persistent" | "streamk"
    seed: int
    notes: str = ""
    extra: dict = field(default_factory=dict)


# The five workloads the benchmark and the parity suite are built around.
WORKLOADS = {
    "bf16_256": Workload("bf16_256", 256, 256, 256, "bf16", "f32", ("uniform",), ("uniform",),
                         "linear_n", 1, "static", 1001,
                         "small parity case, A row / B column major, fp32 out"),
    "bf16_4096": Workload("bf16_4096", 4096, 4096, 4096, "bf16", "bf16", ("uniform",),
                          ("uniform",), "grouped_m", 8, "persistent", 1002,
                          "square 4096^3, bf16 out, linear vs grouped-M(8), persistent"),
    "bf16_mlp_up": Workload("bf16_mlp_up", 4096, 14336, 4096, "bf16", "bf16", ("normal", 1.0),
                            ("normal", 0.02), "grouped_m", 8, "persistent", 1003,
                            "transformer MLP up-projection shape"),
    "fp8_8192": Workload("fp8_8192", 8192, 8192, 8192, "e4m3", "bf16", ("normal", 1.0),
                         ("normal", 1.0), "grouped_m", 16, "persistent", 1004,
                         "per-tensor scales amax/448, fused scale + bf16 epilogue"),
    "bf16_streamk": Workload("bf16_streamk", 512, 512, 65536, "bf16", "f32", ("uniform",),
                             ("uniform",), "linear_n", 1, "streamk", 1005,
                             "16 output tiles, K = 65536, split-K fixup"),
}


def _draw(gen, shape, dist):
    if dist[0] == "uniform":
        return torch.rand(shape, generator=gen, dtype=torch.float32) * 2.0 - 1.0
    if dist[0] == "normal":
        return torch.randn(shape, generator=gen, dtype=torch.float32) * float(dist[1])
    if dist[0] == "smallint":           # integers in [lo, hi], exact in every format used here
        lo, hi = dist[1], dist[2]
        return torch.randint(lo, hi + 1, shape, generator=gen, dtype=torch.int64).to(torch.float32)
    raise ValueError(f"unknown distribution {dist}")


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    """fp32 tensor -> bf16 (nearest-even) -> the raw 16-bit storage as a numpy uint16 array."""
    return x.to(torch.bfloat16).contiguous().view(torch.int16).numpy().view(np.uint16)


def quantize_e4m3_per_tensor(x: torch.Tensor):
    """Per-tensor FP8 quantisation of an fp32 tensor.

    scale = fp32(amax) / 448 in fp32; q = e4m3(clamp(x / scale, -448, 448)) with nearest-even
    rounding (the clamp first, because torch's cast to float8_e4m3fn does not saturate).
    Returns (codes as numpy uint8, scale as a Python float holding an fp32 value).
    """
    amax = x.abs().max().to(torch.float32)
    scale = (amax / torch.tensor(448.0, dtype=torch.float32)).to(torch.float32)
    if float(scale) == 0.0:
        scale = torch.tensor(1.0, dtype=torch.float32)
    q = torch.clamp(x / scale, -448.0, 448.0).to(torch.float8_e4m3fn)
    return q.contiguous().view(torch.uint8).numpy().copy(), float(scale)


@dataclass
class Operands:
    M: int
    N: int
    K: int
    dtype: str
    A: np.ndarray         # storage of A (M x K row-major): uint16 for bf16, uint8 for e4m3
    B: np.ndarray         # storage of B (N x K, i.e. K x N column-major)
    scale_a: float = 1.0
    scale_b: float = 1.0


def make_operands(M, N, K, dtype="bf16", dist_a=("uniform",), dist_b=("uniform",), seed=0):
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(seed))
    a = _draw(gen, (M, K), dist_a)
    b = _draw(gen, (N, K), dist_b)
    if dtype == "bf16":
        return Operands(M, N, K, dtype, bf16_bits(a), bf16_bits(b))
    if dtype == "e4m3":
        qa, sa = quantize_e4m3_per_tensor(a)
        qb, sb = quantize_e4m3_per_tensor(b)
        return Operands(M, N, K, dtype, qa, qb, sa, sb)
    raise ValueError(f"unknown dtype {dtype}")


def make_vector(n, seed, dist=("normal", 1.0)):
    """A seeded fp32 vector of length n (a bias), as a numpy float32 array."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(seed))
    return _draw(gen, (int(n),), dist).numpy().copy()


def make_workload(name_or_wl):
    wl = WORKLOADS[name_or_wl] if isinstance(name_or_wl, str) else name_or_wl
    return make_operands(wl.M, wl.N, wl.K, wl.dtype, wl.dist_a, wl.dist_b, wl.seed)


def rowsum_pattern(M, N, K, dtype="bf16"):
    """A[m, k] = ((m + k) mod 8) / 8 and B = 1: every value is exact in bf16 and in e4m3."""
    m = torch.arange(M).view(M, 1)
    k = torch.arange(K).view(1, K)
    a = ((m + k) % 8).to(torch.float32) / 8.0
    b = torch.ones((N, K), dtype=torch.float32)
    if dtype == "bf16":
        return Operands(M, N, K, dtype, bf16_bits(a), bf16_bits(b))
    codes_a = a.to(torch.float8_e4m3fn).contiguous().view(torch.uint8).numpy().copy()
    codes_b = b.to(torch.float8_e4m3fn).contiguous().view(torch.uint8).numpy().copy()
    return Operands(M, N, K, dtype, codes_a, codes_b, 1.0, 1.0)


def identity_operands(M, N, dtype="bf16", seed=0):
    """A = I (M x M, so K = M) and B uniform[-1, 1]."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(seed))
    a = torch.eye(M, dtype=torch.float32)
    b = _draw(gen, (N, M), ("uniform",))
    return Operands(M, N, M, dtype, bf16_bits(a), bf16_bits(b))


def sample_positions(M, N, count, seed, BM=256, BN=256):
    """Output positions for sampled checks: tile corners and edges plus seeded random points."""
    rng = np.random.default_rng(int(seed))
    rows = [0, M - 1, min(BM, M - 1), min(BM - 1, M - 1), M // 2]
    cols = [0, N - 1, min(BN, N - 1), min(BN - 1, N - 1), N // 2]
    pts = [(r, c) for r in rows for c in cols]
    r = rng.integers(0, M, size=max(0, count - len(pts)))
    c = rng.integers(0, N, size=max(0, count - len(pts)))
    pts += list(zip(r.tolist(), c.tolist()))
    rr = np.array([p[0] for p in pts], dtype=np.int64)
    cc = np.array([p[1] for p in pts], dtype=np.int64)
    return rr, cc
