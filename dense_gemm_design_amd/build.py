"""Builds the HIP library libdgemm.so in-tree for gfx950 with hipcc.

Each translation unit compiles to an object of its own, all at once (the wide-wave kernels that
read a source matrix sit in gemm_src_*.hip for this), and the objects are linked into the
shared library."""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdgemm.so")
SOURCES = [os.path.join(CSRC, name)
           for name in ("gemm.hip", "gemm_src_bf16.hip", "gemm_src_fp8.hip")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC",
    # keep the compiler from forming packed-FP32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False, extra=()) -> str:
    with tempfile.TemporaryDirectory(prefix="dgemm_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(src) + ".o") for src in SOURCES]
        cmds = [[HIPCC, *FLAGS, *extra, "-c", "-o", obj, src] for src, obj in zip(SOURCES, objs)]
        for cmd in cmds:
            if verbose:
                print(" ".join(cmd), flush=True)
        with ThreadPoolExecutor(max_workers=len(cmds)) as pool:
            results = list(pool.map(lambda c: subprocess.run(c), cmds))
        for cmd, res in zip(cmds, results):
            if res.returncode != 0:
                raise subprocess.CalledProcessError(res.returncode, cmd)
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp", *objs]
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.run(link, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, extra=[a for a in sys.argv[1:] if a != "-v"]))
