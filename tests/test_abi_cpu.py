"""The C-ABI library loads, exports what include/gemm.h declares, and rejects bad input before
enqueueing anything.  No compute call is made here: these run without a GPU."""
import ctypes
import os
import re

import pytest

import dense_gemm_design_amd as dg
from dense_gemm_design_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "gemm.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|int)\s*(gemm_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    lib = L.load()
    names = header_functions()
    assert names, "no declarations found"
    assert set(names) == set(L.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name


def test_struct_layouts_match_c_compiler(tmp_path):
    """sizeof and every field offset of the ctypes mirrors equal what a C compiler sees."""
    import subprocess
    structs = {"gemm_desc": L.GemmDesc, "gemm_work_item": L.GemmWorkItem,
               "gemm_plan_info": L.GemmPlanInfo, "gemm_config_score": L.GemmConfigScore,
               "gemm_epilogue_args": L.GemmEpilogueArgs}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "gemm.h"', 'int main(void){']
    for cname, py in structs.items():
        lines.append(f'printf("{cname} %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'printf("{cname}.{fname} %zu\\n", offsetof({cname}, {fname}));')
    lines.append("return 0;}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), "-o", str(exe), str(src)],
                   check=True)
    out = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True,
                                                        text=True, check=True).stdout.splitlines())
    for cname, py in structs.items():
        assert int(out[cname]) == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert int(out[f"{cname}.{fname}"]) == getattr(py, fname).offset, (cname, fname)


def test_status_strings():
    lib = L.load()
    for st in (0, -1, -2, -3, -4, -5, -6, -7):
        assert lib.gemm_status_string(st).decode() not in ("", "unknown status")
    assert lib.gemm_status_string(12345).decode() == "unknown status"


def create(**kw):
    base = dict(M=512, N=512, K=512, sched=L.GEMM_SCHED_PERSISTENT, num_workers=8)
    base.update(kw)
    lib = L.load()
    h = ctypes.c_void_p()
    st = lib.gemm_create(ctypes.byref(L.make_desc(**base)), ctypes.byref(h))
    if st == 0:
        lib.gemm_destroy(h)
    return st


@pytest.mark.parametrize("kw,want", [
    (dict(M=-1), L.GEMM_ERR_INVALID_ARG),
    (dict(N=-8), L.GEMM_ERR_INVALID_ARG),
    (dict(K=-16), L.GEMM_ERR_INVALID_ARG),
    (dict(M=0), L.GEMM_OK),
    (dict(N=0), L.GEMM_OK),
    (dict(K=0), L.GEMM_OK),
    (dict(dtype_ab=7), L.GEMM_ERR_INVALID_ARG),
    (dict(dtype_ab=L.GEMM_F32), L.GEMM_ERR_INVALID_ARG),
    (dict(dtype_c=9), L.GEMM_ERR_INVALID_ARG),
    (dict(mapping=6), L.GEMM_ERR_INVALID_ARG),
    (dict(mapping=L.GEMM_MAP_BLOCKED), L.GEMM_OK),                    # the planner picks the box
    (dict(mapping=L.GEMM_MAP_BLOCKED, group=2, group_n=3), L.GEMM_OK),
    (dict(mapping=L.GEMM_MAP_BLOCKED, group_n=-1), L.GEMM_ERR_INVALID_ARG),
    (dict(mapping=L.GEMM_MAP_BLOCKED, group=-1), L.GEMM_ERR_INVALID_ARG),
    (dict(mapping=L.GEMM_MAP_MORTON), L.GEMM_OK),
    (dict(mapping=L.GEMM_MAP_GROUPED_M, group=-1), L.GEMM_ERR_INVALID_ARG),
    (dict(mapping=L.GEMM_MAP_GROUPED_M, group=0), L.GEMM_OK),       # the planner picks G
    (dict(sched=9), L.GEMM_ERR_INVALID_ARG),
    (dict(num_workers=-1), L.GEMM_ERR_INVALID_ARG),
    (dict(flags=0x80), L.GEMM_ERR_INVALID_ARG),
    (dict(layout_a=3), L.GEMM_ERR_INVALID_ARG),
    (dict(layout_a=L.GEMM_COL_MAJOR), L.GEMM_ERR_UNSUPPORTED),
    (dict(layout_b=L.GEMM_ROW_MAJOR), L.GEMM_ERR_UNSUPPORTED),
    (dict(K=100), L.GEMM_ERR_UNSUPPORTED),            # 200-byte rows: not a multiple of 16
    (dict(N=100), L.GEMM_ERR_UNSUPPORTED),            # output rows must be 8-element multiples
    (dict(N=(1 << 22) + 8), L.GEMM_ERR_UNSUPPORTED),  # beyond 32-bit offsets inside a tile
    (dict(bm=64, bn=64), L.GEMM_ERR_UNSUPPORTED),     # no such tile kernel
    (dict(bm=256, bn=256, bk=16), L.GEMM_ERR_UNSUPPORTED),
    (dict(dtype_ab=L.GEMM_FP8_E4M3, K=8), L.GEMM_ERR_UNSUPPORTED),
    (dict(), L.GEMM_OK),
    (dict(K=104), L.GEMM_OK),                         # ragged K (multiple of 8 bf16 elements)
    (dict(M=300, N=264), L.GEMM_OK),                  # ragged M and N
    (dict(dtype_ab=L.GEMM_FP8_E4M3, K=272, bm=128, bn=128), L.GEMM_OK),
    (dict(flags=L.GEMM_FLAG_PINGPONG), L.GEMM_OK),   # ping-pong picks 256 x 256 tiles
    (dict(flags=L.GEMM_FLAG_PINGPONG, dtype_ab=L.GEMM_FP8_E4M3), L.GEMM_OK),
    (dict(flags=L.GEMM_FLAG_PINGPONG, sched=L.GEMM_SCHED_STATIC, M=300, K=104), L.GEMM_OK),
    (dict(flags=L.GEMM_FLAG_PINGPONG, K=0), L.GEMM_ERR_UNSUPPORTED),
    (dict(flags=L.GEMM_FLAG_PINGPONG, bm=128, bn=128), L.GEMM_ERR_UNSUPPORTED),
    (dict(flags=L.GEMM_FLAG_PINGPONG, sched=L.GEMM_SCHED_STREAMK), L.GEMM_ERR_UNSUPPORTED),
    (dict(flags=L.GEMM_FLAG_COOPERATIVE), L.GEMM_OK),
    (dict(flags=L.GEMM_FLAG_COOPERATIVE | L.GEMM_FLAG_PINGPONG), L.GEMM_ERR_INVALID_ARG),
    (dict(flags=L.GEMM_FLAG_WIDE | L.GEMM_FLAG_PINGPONG), L.GEMM_ERR_INVALID_ARG),
    (dict(flags=0x20), L.GEMM_ERR_INVALID_ARG),  # the retired register-staged kernel's flag
    (dict(flags=L.GEMM_FLAG_WIDE), L.GEMM_OK),
    (dict(flags=L.GEMM_FLAG_WIDE, dtype_ab=L.GEMM_FP8_E4M3, K=400, M=300), L.GEMM_OK),
    (dict(flags=L.GEMM_FLAG_WIDE, bk=32), L.GEMM_ERR_UNSUPPORTED),  # its bf16 k-tile is 64 deep
    (dict(flags=L.GEMM_FLAG_WIDE, sched=L.GEMM_SCHED_STREAMK), L.GEMM_OK),  # separate fixup
    (dict(flags=L.GEMM_FLAG_WIDE | L.GEMM_FLAG_STREAMK_CHAIN, sched=L.GEMM_SCHED_STREAMK),
     L.GEMM_ERR_UNSUPPORTED),                                       # it has no lock chain
    (dict(flags=L.GEMM_FLAG_WIDE, sched=L.GEMM_SCHED_STREAMK, K=64, num_workers=256),
     L.GEMM_ERR_UNSUPPORTED),                                       # band < P: chain needed
    (dict(flags=L.GEMM_FLAG_WIDE, K=0), L.GEMM_ERR_UNSUPPORTED),
    (dict(flags=L.GEMM_FLAG_WIDE | L.GEMM_FLAG_COOPERATIVE), L.GEMM_ERR_INVALID_ARG),
    # fused epilogue
    (dict(epilogue=0x100), L.GEMM_ERR_INVALID_ARG),                      # unknown bit
    (dict(epilogue=L.GEMM_EPI_SOURCE_F32 | L.GEMM_EPI_SOURCE_BF16), L.GEMM_ERR_INVALID_ARG),
    (dict(epilogue=L.GEMM_EPI_SOURCE_F32), L.GEMM_OK),
    (dict(epilogue=L.GEMM_EPI_SOURCE_BF16 | L.GEMM_EPI_GELU, sched=L.GEMM_SCHED_STREAMK),
     L.GEMM_OK),
    (dict(epilogue=L.GEMM_EPI_SOURCE_F32, K=0), L.GEMM_OK),
    (dict(epilogue=L.GEMM_EPI_SOURCE_F32, flags=L.GEMM_FLAG_WIDE), L.GEMM_OK),
    (dict(epilogue=L.GEMM_EPI_SOURCE_F32, flags=L.GEMM_FLAG_PINGPONG), L.GEMM_ERR_UNSUPPORTED),
    (dict(epilogue=L.GEMM_EPI_SOURCE_F32, bm=256, bn=224), L.GEMM_OK),
    (dict(epilogue=L.GEMM_EPI_BIAS_ROW | L.GEMM_EPI_BIAS_COL), L.GEMM_ERR_INVALID_ARG),
    (dict(epilogue=L.GEMM_EPI_RELU | L.GEMM_EPI_GELU), L.GEMM_ERR_INVALID_ARG),
    (dict(epilogue=L.GEMM_EPI_SILU | L.GEMM_EPI_GELU), L.GEMM_ERR_INVALID_ARG),
    (dict(epilogue=0x3F & ~(L.GEMM_EPI_BIAS_ROW | L.GEMM_EPI_RELU | L.GEMM_EPI_SILU)), L.GEMM_OK),
    (dict(epilogue=L.GEMM_EPI_BIAS_ROW | L.GEMM_EPI_SILU | L.GEMM_EPI_AMAX), L.GEMM_OK),
    (dict(dtype_c=L.GEMM_FP8_E4M3), L.GEMM_OK),
    (dict(dtype_c=L.GEMM_FP8_E4M3, dtype_ab=L.GEMM_FP8_E4M3), L.GEMM_OK),
    (dict(epilogue=L.GEMM_EPI_RELU, K=0), L.GEMM_OK),                    # Z = bias: cooperative
    (dict(epilogue=L.GEMM_EPI_RELU, sched=L.GEMM_SCHED_STREAMK, bm=128, bn=128), L.GEMM_OK),
    (dict(epilogue=L.GEMM_EPI_RELU, flags=L.GEMM_FLAG_WIDE), L.GEMM_OK),
    (dict(epilogue=L.GEMM_EPI_RELU, flags=L.GEMM_FLAG_COOPERATIVE), L.GEMM_OK),
    (dict(epilogue=L.GEMM_EPI_RELU, flags=L.GEMM_FLAG_PINGPONG), L.GEMM_ERR_UNSUPPORTED),
    (dict(dtype_c=L.GEMM_FP8_E4M3, flags=L.GEMM_FLAG_PINGPONG), L.GEMM_ERR_UNSUPPORTED),
])
def test_create_validation(kw, want):
    assert create(**kw) == want


def test_null_arguments():
    lib = L.load()
    h = ctypes.c_void_p()
    assert lib.gemm_create(None, ctypes.byref(h)) == L.GEMM_ERR_INVALID_ARG
    assert lib.gemm_create(ctypes.byref(L.make_desc(64, 64, 64, num_workers=1)), None) \
        == L.GEMM_ERR_INVALID_ARG
    assert lib.gemm_destroy(None) == L.GEMM_ERR_INVALID_ARG
    n = ctypes.c_size_t()
    assert lib.gemm_workspace_bytes(None, ctypes.byref(n)) == L.GEMM_ERR_INVALID_ARG
    assert lib.gemm_schedule_enumerate(None, None, 0, ctypes.byref(n)) == L.GEMM_ERR_INVALID_ARG


def test_plan_info_and_workspace():
    p = L.Plan(L.make_desc(512, 512, 65536, sched=L.GEMM_SCHED_STREAMK, num_workers=256,
                           bm=128, bn=128))
    i = p.info
    assert (i.bm, i.bn, i.bk, i.mt, i.nt, i.kt) == (128, 128, 64, 4, 4, 1024)
    assert (i.dp_tiles, i.sk_tiles, i.grid, i.sched) == (0, 16, 256, L.GEMM_SCHED_STREAMK)
    # 16 partial tiles of 128 x 128 fp32, then 16 locks, then the error word
    assert p.workspace_bytes >= 16 * 128 * 128 * 4 + 16 * 4 + 4
    assert i.error_offset >= 16 * 128 * 128 * 4 + 16 * 4
    q = L.Plan(L.make_desc(4096, 4096, 4096, sched=L.GEMM_SCHED_PERSISTENT, num_workers=256,
                           mapping=L.GEMM_MAP_GROUPED_M, group=8))
    assert q.workspace_bytes == 0 and q.info.bm == 256 and q.info.grid == 256
    assert i.kernel == 3 and q.info.kernel == 3     # Stream-K and 256^2 DP: wide-wave
    assert q.info.lds_bytes == 160 * 1024
    r = L.Plan(L.make_desc(4096, 4096, 4096, sched=L.GEMM_SCHED_PERSISTENT, num_workers=256,
                           flags=L.GEMM_FLAG_COOPERATIVE))
    assert r.info.kernel == 0 and r.info.lds_bytes == 128 * 1024
    w = L.Plan(L.make_desc(4096, 4096, 4096, sched=L.GEMM_SCHED_PERSISTENT, num_workers=256,
                           flags=L.GEMM_FLAG_WIDE))
    assert (w.info.kernel, w.info.threads, w.info.bk, w.info.kt) == (3, 256, 64, 64)
    assert w.info.lds_bytes == 160 * 1024 and w.info.stages == 2
    w8 = L.Plan(L.make_desc(8192, 8192, 8192, dtype_ab=L.GEMM_FP8_E4M3, num_workers=256,
                            sched=L.GEMM_SCHED_PERSISTENT, flags=L.GEMM_FLAG_WIDE))
    assert (w8.info.kernel, w8.info.bk, w8.info.kt) == (3, 128, 64)
    s = L.Plan(L.make_desc(256, 256, 256, sched=L.GEMM_SCHED_STATIC, bm=128, bn=128))
    assert s.info.grid == 4 and s.info.sched == L.GEMM_SCHED_STATIC


@pytest.mark.skipif(__import__("torch").cuda.is_available(),
                    reason="validation-only test; on a GPU machine the parity suite covers runs")
def test_run_validation_before_enqueue():
    p = L.Plan(L.make_desc(512, 512, 65536, sched=L.GEMM_SCHED_STREAMK, num_workers=256,
                           bm=128, bn=128))
    ok = 1 << 20  # an aligned address; never dereferenced because every call below fails first
    assert p.run_raw(0, ok, ok) == L.GEMM_ERR_INVALID_ARG
    assert p.run_raw(ok + 8, ok, ok, 0, 0, ok, p.workspace_bytes) == L.GEMM_ERR_ALIGNMENT
    assert p.run_raw(ok, ok, ok) == L.GEMM_ERR_WORKSPACE
    assert p.run_raw(ok, ok, ok, 0, 0, ok, p.workspace_bytes - 1) == L.GEMM_ERR_WORKSPACE
    assert p.run_raw(ok, ok, ok, 0, 0, ok + 4, p.workspace_bytes) == L.GEMM_ERR_ALIGNMENT
    f = L.Plan(L.make_desc(512, 512, 512, dtype_ab=L.GEMM_FP8_E4M3, num_workers=4))
    assert f.run_raw(ok, ok, ok) == L.GEMM_ERR_INVALID_ARG          # FP8 needs both scales
    assert f.run_raw(ok, ok, ok, ok, 0) == L.GEMM_ERR_INVALID_ARG
    assert f.run_raw(ok, ok, ok, ok + 2, ok) == L.GEMM_ERR_ALIGNMENT
    # everything valid but no device in this container: the launch itself reports the failure
    b = L.Plan(L.make_desc(256, 256, 256, num_workers=4))
    assert b.run_raw(ok, ok, ok) == L.GEMM_ERR_HIP
    # an empty output is a no-op that needs no pointers at all
    e = L.Plan(L.make_desc(0, 256, 256, num_workers=4))
    assert e.info.grid == 0 and e.run_raw(0, 0, 0) == L.GEMM_OK


def test_fused_epilogue_plans():
    """Epilogue plans run on the wide-wave kernel for data-parallel 256 x 256 work and on the
    cooperative kernel otherwise; without epilogue bits nothing changes."""
    kw = dict(sched=L.GEMM_SCHED_PERSISTENT, num_workers=256)
    dp = L.Plan(L.make_desc(4096, 4096, 4096, epilogue=L.GEMM_EPI_GELU | L.GEMM_EPI_BIAS_COL,
                            **kw))
    assert (dp.info.kernel, dp.info.bm) == (3, 256)
    q = L.Plan(L.make_desc(4096, 4096, 4096, dtype_ab=L.GEMM_FP8_E4M3, dtype_c=L.GEMM_FP8_E4M3,
                           **kw))
    assert (q.info.kernel, q.info.bk) == (3, 128)
    sk = L.Plan(L.make_desc(512, 512, 65536, sched=L.GEMM_SCHED_STREAMK, num_workers=256, bm=128,
                            bn=128, epilogue=L.GEMM_EPI_AMAX))
    assert sk.info.kernel == 3 and sk.info.sk_tiles > 0
    z = L.Plan(L.make_desc(256, 256, 0, epilogue=L.GEMM_EPI_BIAS_ROW, num_workers=4))
    assert z.info.kernel == 0
    # the planner's own choice (everything auto) takes a kernel that has the fused epilogue
    for M, N, K in ((4096, 4096, 4096), (512, 512, 65536), (2048, 2048, 2048), (256, 512, 4096)):
        a = L.Plan(L.make_desc(M, N, K, sched=L.GEMM_SCHED_AUTO, num_workers=256,
                               epilogue=L.GEMM_EPI_SILU))
        assert a.info.kernel in (0, 3), (M, N, K)


def test_source_plans_take_the_plain_plans_kernel():
    """A source matrix is read by the wide-wave and the cooperative kernels alike: a plan with one
    runs the kernel the same plan without it runs (and the kernel asked for by a flag).  The cost
    model adds the source's bytes to every candidate and ranks one more for such plans,
    cooperative 256 x 256 data-parallel, which plans without a source never see."""
    for M, N, K, sched in ((4096, 4096, 4096, L.GEMM_SCHED_AUTO),
                           (4096, 4096, 4096, L.GEMM_SCHED_PERSISTENT),
                           (4096, 14336, 4096, L.GEMM_SCHED_AUTO),
                           (512, 512, 65536, L.GEMM_SCHED_STREAMK),
                           (300, 264, 0, L.GEMM_SCHED_STATIC)):
        for src in (L.GEMM_EPI_SOURCE_F32, L.GEMM_EPI_SOURCE_BF16):
            for flags in (0, L.GEMM_FLAG_COOPERATIVE):
                p = L.Plan(L.make_desc(M, N, K, sched=sched, num_workers=256, flags=flags,
                                       epilogue=src | L.GEMM_EPI_GELU))
                plain = L.Plan(L.make_desc(M, N, K, sched=sched, num_workers=256, flags=flags,
                                           epilogue=L.GEMM_EPI_GELU))
                want = 0 if (K == 0 or flags) else 3
                assert p.info.kernel == plain.info.kernel == want, (M, N, K, sched, flags)
    ranked = L.rank_configs(L.make_desc(4096, 4096, 4096, sched=L.GEMM_SCHED_AUTO,
                                        num_workers=256, epilogue=L.GEMM_EPI_SOURCE_BF16))
    plain = L.rank_configs(L.make_desc(4096, 4096, 4096, sched=L.GEMM_SCHED_AUTO,
                                       num_workers=256))
    extra = lambda rs: [r for r in rs if r.kernel == 0 and r.bm == 256 and
                        r.sched == L.GEMM_SCHED_PERSISTENT]
    assert len(ranked) == len(plain) + 1 and len(extra(ranked)) == 1 and not extra(plain)
    # the source's bytes raise every candidate's L2 clocks
    key = lambda r: (r.kernel, r.bm, r.bn, r.sched)
    base = {key(r): r.cycles_l2 for r in plain}
    assert all(r.cycles_l2 > base[key(r)] for r in ranked if key(r) in base)


@pytest.mark.skipif(__import__("torch").cuda.is_available(),
                    reason="validation-only test; on a GPU machine the parity suite covers runs")
def test_run_ex_validation_before_enqueue():
    ok = 1 << 20
    epi = L.GEMM_EPI_BIAS_COL | L.GEMM_EPI_RELU | L.GEMM_EPI_AMAX
    p = L.Plan(L.make_desc(256, 256, 256, num_workers=4, epilogue=epi,
                           dtype_c=L.GEMM_FP8_E4M3))
    full = dict(bias=ok, scale_d=ok, amax=ok)
    assert p.run_ex_raw(ok, ok, ok, epi_null=True) == L.GEMM_ERR_INVALID_ARG
    for missing in full:
        assert p.run_ex_raw(ok, ok, ok, **{**full, missing: 0}) == L.GEMM_ERR_INVALID_ARG, missing
    assert p.run_ex_raw(ok, ok, ok, **{**full, "bias": ok + 4}) == L.GEMM_ERR_ALIGNMENT
    assert p.run_ex_raw(ok, ok, ok, **{**full, "amax": ok + 2}) == L.GEMM_ERR_ALIGNMENT
    assert p.run_ex_raw(ok, ok, ok, **{**full, "scale_d": ok + 1}) == L.GEMM_ERR_ALIGNMENT
    assert p.run_ex_raw(ok, ok, ok, **{**full, "amax": ok + 4}) == L.GEMM_ERR_HIP  # 4 B is enough
    # gemm_run is gemm_run_ex without epilogue operands
    assert p.run_raw(ok, ok, ok) == L.GEMM_ERR_INVALID_ARG
    # a plan that needs no epilogue operand accepts a NULL epi and ignores the pointers
    b = L.Plan(L.make_desc(256, 256, 256, num_workers=4, epilogue=L.GEMM_EPI_GELU))
    assert b.run_ex_raw(ok, ok, ok, epi_null=True) == L.GEMM_ERR_HIP
    assert b.run_ex_raw(ok, ok, ok, bias=3, amax=5) == L.GEMM_ERR_HIP
    # a source matrix: beta != 0 needs it, aligned for its element type; beta == 0 reads none
    s = L.Plan(L.make_desc(256, 256, 256, num_workers=4, epilogue=L.GEMM_EPI_SOURCE_F32))
    assert s.run_ex_raw(ok, ok, ok, epi_null=True) == L.GEMM_ERR_INVALID_ARG
    assert s.run_ex_raw(ok, ok, ok, beta=0.5) == L.GEMM_ERR_INVALID_ARG
    assert s.run_ex_raw(ok, ok, ok, beta=0.5, source=ok + 8) == L.GEMM_ERR_ALIGNMENT
    assert s.run_ex_raw(ok, ok, ok, beta=0.5, source=ok) == L.GEMM_ERR_HIP
    assert s.run_ex_raw(ok, ok, ok, beta=0.0) == L.GEMM_ERR_HIP
    h = L.Plan(L.make_desc(256, 256, 256, num_workers=4, epilogue=L.GEMM_EPI_SOURCE_BF16))
    assert h.run_ex_raw(ok, ok, ok, beta=-1.0, source=ok + 4) == L.GEMM_ERR_ALIGNMENT
    assert h.run_ex_raw(ok, ok, ok, beta=-1.0, source=ok + 8) == L.GEMM_ERR_HIP  # 8 B is enough
    # an empty output checks the epilogue operands, then does nothing
    e = L.Plan(L.make_desc(0, 256, 256, num_workers=4, epilogue=L.GEMM_EPI_AMAX))
    assert e.run_ex_raw(0, 0, 0, epi_null=True) == L.GEMM_ERR_INVALID_ARG
    assert e.run_ex_raw(0, 0, 0, amax=ok) == L.GEMM_OK


def test_package_has_no_cpu_fallback():
    """The product path neither imports the oracle nor computes a product any other way."""
    pkg = os.path.join(ROOT, "dense_gemm_design_amd")
    for name in os.listdir(pkg):
        if not name.endswith(".py"):
            continue
        src = open(os.path.join(pkg, name)).read()
        assert not re.search(r"^\s*(import|from)\s+oracle", src, re.M), name
        for pat in ("matmul", "torch.mm(", "einsum", "bmm(", "np.dot", " @ "):
            assert pat not in src, (name, pat)


@pytest.mark.parametrize("bn", [224, 192])
def test_wide_only_tile_plans(bn):
    """256 x 224 and 256 x 192 tiles exist only on the wide-wave kernel: data-parallel and
    separate-reduction Stream-K plans are built; K = 0, the lock chain and the other kernels are
    refused."""
    import ctypes
    lib = L.load()
    h = ctypes.c_void_p()

    N = 2 * bn  # 2 x 2 tiles: a Stream-K band over 8 workers

    def status(K, sched=L.GEMM_SCHED_PERSISTENT, flags=0, P=8):
        d = L.make_desc(512, N, K, L.GEMM_BF16, L.GEMM_F32, L.GEMM_MAP_LINEAR_N, 1, sched, P,
                        256, bn, 0, flags)
        st = lib.gemm_create(ctypes.byref(d), ctypes.byref(h))
        if st == L.GEMM_OK:
            info = L.GemmPlanInfo()
            lib.gemm_plan_get(h, ctypes.byref(info))
            lib.gemm_destroy(h)
            return st, info.kernel
        return st, None
    assert status(1024) == (L.GEMM_OK, 3)
    assert status(1024, flags=L.GEMM_FLAG_WIDE) == (L.GEMM_OK, 3)
    assert status(16384, sched=L.GEMM_SCHED_STREAMK) == (L.GEMM_OK, 3)
    assert status(0)[0] == L.GEMM_ERR_UNSUPPORTED
    assert status(0, flags=L.GEMM_FLAG_WIDE)[0] == L.GEMM_ERR_UNSUPPORTED
    assert status(1024, flags=L.GEMM_FLAG_COOPERATIVE)[0] == L.GEMM_ERR_UNSUPPORTED
    assert status(1024, flags=L.GEMM_FLAG_PINGPONG)[0] == L.GEMM_ERR_UNSUPPORTED
    assert status(16384, sched=L.GEMM_SCHED_STREAMK,
                  flags=L.GEMM_FLAG_STREAMK_CHAIN)[0] == L.GEMM_ERR_UNSUPPORTED


def test_noalloc_rejects_plans_beyond_the_scratch_before_any_device_call():
    """A Stream-K plan whose workspace exceeds the no-allocation entry point's scratch returns
    GEMM_ERR_SCRATCH_LIMIT at once (no GPU is needed to reach that answer)."""
    plan = L.Plan(L.make_desc(1024, 1024, 65536, L.GEMM_BF16, L.GEMM_F32, L.GEMM_MAP_LINEAR_N,
                              1, L.GEMM_SCHED_STREAMK, 1024, 128, 128))
    assert plan.workspace_bytes > L.GEMM_NOALLOC_SCRATCH_BYTES
    st = plan.run_noalloc_raw(16, 16, 16)
    assert st == L.GEMM_ERR_SCRATCH_LIMIT
    assert "scratch" in L.load().gemm_status_string(st).decode()
    assert plan.run_noalloc_raw(16, 16, 16, epi_null=True) == L.GEMM_ERR_SCRATCH_LIMIT
    assert L.load().gemm_run_noalloc(None, None, None, None, None, None, None, None) == \
        L.GEMM_ERR_INVALID_ARG
