"""fp64 reference outputs of the full-size workloads, for the full-size parity tests.

Each reference is oracle.gemm_ref over the workload's seeded operands (gemm_inputs), so every
value in it comes from the oracle alone.  It is cached per (workload, shape, dtype, seed) in
memory for the test session and on disk under tests/.cref_cache/ (git-ignored), keyed also by a
hash of the oracle's and the generator's sources, so a change to either recomputes it.  The disk
copy is read with numpy.load's default allow_pickle=False.
"""
import hashlib
import os

import numpy as np

import gemm_inputs as gi
import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CACHE_DIR = os.path.join(HERE, ".cref_cache")

_mem = {}


def _sources_hash():
    h = hashlib.sha256()
    for rel in ("oracle/gemm_oracle.c", "oracle/__init__.py", "gemm_inputs/__init__.py"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(rel.encode() + f.read())
    return h.hexdigest()[:12]


def key_of(name):
    wl = gi.WORKLOADS[name]
    return f"{name}_{wl.M}x{wl.N}x{wl.K}_{wl.dtype}_seed{wl.seed}_{_sources_hash()}"


def cref(name, op=None):
    """C_ref (M x N float64) of workload `name`: alpha * sum_k a(m,k) b(k,n) by the oracle."""
    key = key_of(name)
    if key in _mem:
        return _mem[key]
    path = os.path.join(CACHE_DIR, key + ".npy")
    ref = None
    if os.path.exists(path):
        try:
            ref = np.load(path)
        except (OSError, ValueError):
            ref = None
    if ref is None:
        if op is None:
            op = gi.make_workload(name)
        code = oracle.BF16 if op.dtype == "bf16" else oracle.E4M3
        ref = oracle.gemm_ref(op.M, op.N, op.K, code, op.A, op.B, scale_a=op.scale_a,
                              scale_b=op.scale_b)
        try:
            os.makedirs(CACHE_DIR, exist_ok=True)
            tmp = path + f".tmp{os.getpid()}.npy"
            np.save(tmp, ref)
            os.replace(tmp, path)
        except OSError:
            pass  # a read-only tree: the in-memory copy still serves this session
    _mem.clear()  # one full-size reference at a time (the largest is 512 MiB)
    _mem[key] = ref
    return ref
