"""ctypes binding of the C ABI in include/gemm.h (argument marshalling only).

Every step of the GEMM runs in the HIP library libdgemm.so; this module only mirrors its structs,
loads it, and turns torch tensors into device pointers and torch's current stream into a
hipStream_t.  If the library is missing the import of the entry points fails loudly; there is no
CPU fallback.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdgemm.so")

# enums (gemm.h)
GEMM_OK, GEMM_ERR_INVALID_ARG, GEMM_ERR_UNSUPPORTED = 0, -1, -2
GEMM_ERR_ALIGNMENT, GEMM_ERR_WORKSPACE, GEMM_ERR_HIP, GEMM_ERR_CAPACITY = -3, -4, -5, -6
GEMM_BF16, GEMM_FP8_E4M3, GEMM_F32 = 0, 1, 2
GEMM_ROW_MAJOR, GEMM_COL_MAJOR = 0, 1
GEMM_MAP_LINEAR_N, GEMM_MAP_LINEAR_M, GEMM_MAP_GROUPED_M, GEMM_MAP_GROUPED_N = 0, 1, 2, 3
GEMM_MAP_BLOCKED, GEMM_MAP_MORTON = 4, 5
GEMM_SCHED_STATIC, GEMM_SCHED_PERSISTENT, GEMM_SCHED_STREAMK, GEMM_SCHED_AUTO = 0, 1, 2, 3
GEMM_FLAG_TRACE = 0x1
GEMM_FLAG_NO_XCD_REMAP = 0x2
GEMM_FLAG_STREAMK_CHAIN = 0x4
GEMM_FLAG_PINGPONG = 0x8
GEMM_FLAG_COOPERATIVE = 0x10
GEMM_FLAG_REGSTAGED = 0x20
GEMM_FLAG_WIDE = 0x40
GEMM_FLAG_TEST_SKIP_PUBLISH = 0x100
GEMM_DEVICE_OK, GEMM_DEVICE_ERR_SPIN = 0, 1
GEMM_EPI_BIAS_ROW = 0x1
GEMM_EPI_BIAS_COL = 0x2
GEMM_EPI_RELU = 0x4
GEMM_EPI_GELU = 0x8
GEMM_EPI_SILU = 0x10
GEMM_EPI_AMAX = 0x20

EXPORTS = ("gemm_create", "gemm_workspace_bytes", "gemm_plan_get", "gemm_run", "gemm_run_ex",
           "gemm_destroy", "gemm_schedule_enumerate", "gemm_rank_configs", "gemm_status_string")


class GemmDesc(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("dtype_ab", ctypes.c_int32), ("dtype_c", ctypes.c_int32),
                ("layout_a", ctypes.c_int32), ("layout_b", ctypes.c_int32),
                ("mapping", ctypes.c_int32), ("group", ctypes.c_int32),
                ("sched", ctypes.c_int32), ("num_workers", ctypes.c_int32),
                ("bm", ctypes.c_int32), ("bn", ctypes.c_int32), ("bk", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("epilogue", ctypes.c_uint32),
                ("group_n", ctypes.c_int32), ("sk_groups", ctypes.c_int32)]


class GemmEpilogueArgs(ctypes.Structure):
    _fields_ = [("bias", ctypes.c_void_p), ("scale_d", ctypes.c_void_p),
                ("amax", ctypes.c_void_p)]


class GemmWorkItem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("worker", "seq", "tile", "tile_m", "tile_n", "k_begin", "k_end", "role")]


class GemmPlanInfo(ctypes.Structure):
    _fields_ = [("bm", ctypes.c_int32), ("bn", ctypes.c_int32), ("bk", ctypes.c_int32),
                ("stages", ctypes.c_int32), ("threads", ctypes.c_int32), ("grid", ctypes.c_int32),
                ("mt", ctypes.c_int32), ("nt", ctypes.c_int32), ("kt", ctypes.c_int32),
                ("sched", ctypes.c_int32), ("xcds", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
                ("dp_tiles", ctypes.c_int64), ("sk_tiles", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_int64), ("trace_offset", ctypes.c_int64),
                ("trace_capacity", ctypes.c_int32), ("error_offset", ctypes.c_int32),
                ("streamk_mode", ctypes.c_int32), ("kernel", ctypes.c_int32),
                ("group", ctypes.c_int32), ("group_n", ctypes.c_int32),
                ("sk_groups", ctypes.c_int32)]


class GemmConfigScore(ctypes.Structure):
    _fields_ = [("bm", ctypes.c_int32), ("bn", ctypes.c_int32), ("bk", ctypes.c_int32),
                ("kernel", ctypes.c_int32), ("sched", ctypes.c_int32),
                ("workers", ctypes.c_int32), ("group", ctypes.c_int32), ("group_n", ctypes.c_int32),
                ("cycles_mfma", ctypes.c_double), ("cycles_l2", ctypes.c_double),
                ("cycles_local", ctypes.c_double), ("wave_efficiency", ctypes.c_double),
                ("cycles_fixed", ctypes.c_double), ("score", ctypes.c_double)]


_lib = None


def load():
    """Loads libdgemm.so (built by dense_gemm_design_amd/build.py); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run dense_gemm_design_amd/build.py "
                           "(or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.gemm_create.argtypes = [ctypes.POINTER(GemmDesc), ctypes.POINTER(vp)]
    lib.gemm_workspace_bytes.argtypes = [vp, ctypes.POINTER(sz)]
    lib.gemm_plan_get.argtypes = [vp, ctypes.POINTER(GemmPlanInfo)]
    lib.gemm_run.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gemm_run_ex.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.POINTER(GemmEpilogueArgs), vp, sz,
                                vp]
    lib.gemm_destroy.argtypes = [vp]
    lib.gemm_schedule_enumerate.argtypes = [vp, ctypes.POINTER(GemmWorkItem), sz,
                                            ctypes.POINTER(sz)]
    lib.gemm_rank_configs.argtypes = [ctypes.POINTER(GemmDesc), ctypes.POINTER(GemmConfigScore),
                                      sz, ctypes.POINTER(sz)]
    lib.gemm_status_string.argtypes = [ctypes.c_int]
    lib.gemm_status_string.restype = ctypes.c_char_p
    for name in EXPORTS:
        if name != "gemm_status_string":
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


class GemmError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = load().gemm_status_string(status).decode()
        super().__init__(f"{where}: {msg} ({status})")


def _check(status, where):
    if status != GEMM_OK:
        raise GemmError(status, where)


def make_desc(M, N, K, dtype_ab=GEMM_BF16, dtype_c=GEMM_F32, mapping=GEMM_MAP_LINEAR_N, group=1,
              sched=GEMM_SCHED_PERSISTENT, num_workers=0, bm=0, bn=0, bk=0, flags=0,
              layout_a=GEMM_ROW_MAJOR, layout_b=GEMM_COL_MAJOR, epilogue=0, group_n=0,
              sk_groups=0):
    return GemmDesc(M, N, K, dtype_ab, dtype_c, layout_a, layout_b, mapping, group, sched,
                    num_workers, bm, bn, bk, flags, epilogue, group_n, sk_groups)


def rank_configs(desc):
    """The planner's cost-model ranking for `desc` (a GemmDesc), best first."""
    lib = load()
    n = ctypes.c_size_t()
    st = lib.gemm_rank_configs(ctypes.byref(desc), None, 0, ctypes.byref(n))
    if st not in (GEMM_OK, GEMM_ERR_CAPACITY):
        _check(st, "gemm_rank_configs")
    arr = (GemmConfigScore * max(n.value, 1))()
    _check(lib.gemm_rank_configs(ctypes.byref(desc), arr, n.value, ctypes.byref(n)),
           "gemm_rank_configs")
    return list(arr[:n.value])


class Plan:
    """Owns a gemm_handle.  run() takes torch device tensors and enqueues on the current stream."""

    def __init__(self, desc: GemmDesc):
        lib = load()
        h = ctypes.c_void_p()
        _check(lib.gemm_create(ctypes.byref(desc), ctypes.byref(h)), "gemm_create")
        self.handle = h
        self.desc = desc
        info = GemmPlanInfo()
        _check(lib.gemm_plan_get(h, ctypes.byref(info)), "gemm_plan_get")
        self.info = info

    def close(self):
        if self.handle:
            load().gemm_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def workspace_bytes(self):
        n = ctypes.c_size_t()
        _check(load().gemm_workspace_bytes(self.handle, ctypes.byref(n)), "gemm_workspace_bytes")
        return n.value

    def schedule(self):
        """CPU replay of the schedule as a list of (worker, seq, tile, m, n, kb, ke, role)."""
        lib = load()
        n = ctypes.c_size_t()
        st = lib.gemm_schedule_enumerate(self.handle, None, 0, ctypes.byref(n))
        if st not in (GEMM_OK, GEMM_ERR_CAPACITY):
            _check(st, "gemm_schedule_enumerate")
        arr = (GemmWorkItem * max(1, n.value))()
        _check(lib.gemm_schedule_enumerate(self.handle, arr, n.value, ctypes.byref(n)),
               "gemm_schedule_enumerate")
        return [(it.worker, it.seq, it.tile, it.tile_m, it.tile_n, it.k_begin, it.k_end, it.role)
                for it in arr[:n.value]]

    def run_raw(self, A, B, C, scale_a=0, scale_b=0, workspace=0, workspace_bytes=0, stream=0):
        """Enqueues with raw integer device pointers; returns the gemm_status."""
        return load().gemm_run(self.handle, A, B, C, scale_a or None, scale_b or None,
                               workspace or None, workspace_bytes, stream or None)

    def run_ex_raw(self, A, B, C, scale_a=0, scale_b=0, bias=0, scale_d=0, amax=0, workspace=0,
                   workspace_bytes=0, stream=0, epi_null=False):
        """gemm_run_ex with raw integer device pointers (epi_null passes a NULL epilogue-args
        pointer); returns the gemm_status."""
        epi = None if epi_null else ctypes.byref(
            GemmEpilogueArgs(bias or None, scale_d or None, amax or None))
        return load().gemm_run_ex(self.handle, A, B, C, scale_a or None, scale_b or None, epi,
                                  workspace or None, workspace_bytes, stream or None)

    def run(self, A, B, C, scale_a=None, scale_b=None, workspace=None, stream=None, bias=None,
            scale_d=None, amax=None):
        """A, B, C, scales, workspace, bias, amax: torch tensors on the GPU; stream:
        torch.cuda.Stream.  bias / scale_d / amax feed the fused epilogue (gemm_run_ex)."""
        import torch
        if stream is None:
            stream = torch.cuda.current_stream()
        ptr = lambda t: t.data_ptr() if t is not None else 0
        ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
        st = self.run_ex_raw(ptr(A), ptr(B), ptr(C), ptr(scale_a), ptr(scale_b), ptr(bias),
                             ptr(scale_d), ptr(amax), ptr(workspace), ws_len, stream.cuda_stream)
        _check(st, "gemm_run_ex")
