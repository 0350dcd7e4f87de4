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
GEMM_ERR_SCRATCH_LIMIT = -7
GEMM_NOALLOC_SCRATCH_BYTES = 32 << 20
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
GEMM_FLAG_WIDE = 0x40
GEMM_FLAG_TEST_SKIP_PUBLISH = 0x100
GEMM_DEVICE_OK, GEMM_DEVICE_ERR_SPIN = 0, 1
GEMM_EPI_BIAS_ROW = 0x1
GEMM_EPI_BIAS_COL = 0x2
GEMM_EPI_RELU = 0x4
GEMM_EPI_GELU = 0x8
GEMM_EPI_SILU = 0x10
GEMM_EPI_AMAX = 0x20
GEMM_EPI_SOURCE_F32 = 0x40
GEMM_EPI_SOURCE_BF16 = 0x80

EXPORTS = ("gemm_create", "gemm_workspace_bytes", "gemm_plan_get", "gemm_run", "gemm_run_ex",
           "gemm_run_noalloc", "gemm_destroy", "gemm_schedule_enumerate", "gemm_rank_configs", "gemm_status_string")


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
                ("amax", ctypes.c_void_p), ("source", ctypes.c_void_p), ("beta", ctypes.c_float)]


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
                ("sk_groups", ctypes.c_int32), ("xcd_box_r", ctypes.c_int32),
                ("xcd_box_c", ctypes.c_int32)]


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
    # PyTorch-ROCm carries its own HIP runtime; importing torch first makes the library bind to
    # that same runtime, so torch's device pointers and streams are valid in it (loading the
    # library first would bring in a second runtime, in which torch's allocations do not exist).
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.gemm_create.argtypes = [ctypes.POINTER(GemmDesc), ctypes.POINTER(vp)]
    lib.gemm_workspace_bytes.argtypes = [vp, ctypes.POINTER(sz)]
    lib.gemm_plan_get.argtypes = [vp, ctypes.POINTER(GemmPlanInfo)]
    lib.gemm_run.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gemm_run_ex.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.POINTER(GemmEpilogueArgs), vp, sz,
                                vp]
    lib.gemm_run_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.POINTER(GemmEpilogueArgs),
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
                   workspace_bytes=0, stream=0, epi_null=False, source=0, beta=0.0):
        """gemm_run_ex with raw integer device pointers (epi_null passes a NULL epilogue-args
        pointer); returns the gemm_status."""
        epi = None if epi_null else ctypes.byref(
            GemmEpilogueArgs(bias or None, scale_d or None, amax or None, source or None,
                             float(beta)))
        return load().gemm_run_ex(self.handle, A, B, C, scale_a or None, scale_b or None, epi,
                                  workspace or None, workspace_bytes, stream or None)

    def validate(self, A, B, C, scale_a=None, scale_b=None, workspace=None, bias=None,
                 scale_d=None, amax=None, source=None, beta=0.0):
        """Checks torch tensors against the plan before any pointer reaches the library: the
        kernels size their buffer ranges from M, N, K, not from the tensors, so a tensor that is
        too small, strided or of the wrong element type would be read or written past its end.
        Raises ValueError naming the first problem; returns None."""
        validate_operands(self.desc, A, B, C, scale_a, scale_b, workspace, bias, scale_d, amax,
                          self.workspace_bytes, source, beta)

    def run_noalloc_raw(self, A, B, C, scale_a=0, scale_b=0, bias=0, scale_d=0, amax=0,
                        stream=0, epi_null=False, source=0, beta=0.0):
        """gemm_run_noalloc with raw integer device pointers; returns the gemm_status."""
        epi = None if epi_null else ctypes.byref(
            GemmEpilogueArgs(bias or None, scale_d or None, amax or None, source or None,
                             float(beta)))
        return load().gemm_run_noalloc(self.handle, A, B, C, scale_a or None, scale_b or None,
                                       epi, stream or None)

    def run_noalloc(self, A, B, C, scale_a=None, scale_b=None, stream=None, bias=None,
                    scale_d=None, amax=None, source=None, beta=0.0):
        """gemm_run_noalloc on torch tensors: as run(), with the library's own scratch as the
        workspace (nothing is allocated).  The tensors are checked first (ValueError)."""
        import torch
        validate_operands(self.desc, A, B, C, scale_a, scale_b, None, bias, scale_d, amax, 0,
                          source, beta)
        if stream is None:
            stream = torch.cuda.current_stream()
        ptr = lambda t: t.data_ptr() if t is not None else 0
        st = self.run_noalloc_raw(ptr(A), ptr(B), ptr(C), ptr(scale_a), ptr(scale_b), ptr(bias),
                                  ptr(scale_d), ptr(amax), stream.cuda_stream,
                                  source=ptr(source), beta=beta)
        _check(st, "gemm_run_noalloc")

    def run(self, A, B, C, scale_a=None, scale_b=None, workspace=None, stream=None, bias=None,
            scale_d=None, amax=None, source=None, beta=0.0):
        """A, B, C, scales, workspace, bias, amax, source: torch tensors on the GPU; stream:
        torch.cuda.Stream.  bias / scale_d / amax / source and beta feed the fused epilogue
        (gemm_run_ex); source may be C itself.  The tensors are checked first (validate); a
        mismatch raises ValueError."""
        import torch
        self.validate(A, B, C, scale_a, scale_b, workspace, bias, scale_d, amax, source, beta)
        if stream is None:
            stream = torch.cuda.current_stream()
        ptr = lambda t: t.data_ptr() if t is not None else 0
        ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
        st = self.run_ex_raw(ptr(A), ptr(B), ptr(C), ptr(scale_a), ptr(scale_b), ptr(bias),
                             ptr(scale_d), ptr(amax), ptr(workspace), ws_len, stream.cuda_stream,
                             source=ptr(source), beta=beta)
        _check(st, "gemm_run_ex")


def _dtype_names(torch):
    return {GEMM_BF16: (torch.bfloat16, torch.int16),
            GEMM_FP8_E4M3: (torch.uint8, torch.float8_e4m3fn),
            GEMM_F32: (torch.float32,)}


def validate_operands(desc, A, B, C, scale_a=None, scale_b=None, workspace=None, bias=None,
                      scale_d=None, amax=None, workspace_bytes=0, source=None, beta=0.0):
    """The checks of Plan.validate for a GemmDesc: shapes, element types and contiguity first
    (so they can be exercised on CPU tensors), then that every tensor is on one GPU."""
    import torch
    M, N, K = desc.M, desc.N, desc.K
    kinds = _dtype_names(torch)
    used = []

    def need(t, what, dtypes, numel=None, shape=None, at_least=False):
        if t is None:
            raise ValueError(f"{what} is required for this plan")
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{what} must be a torch tensor")
        if t.dtype not in dtypes:
            raise ValueError(f"{what} has dtype {t.dtype}; expected one of "
                             f"{[str(d) for d in dtypes]}")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{what} has shape {tuple(t.shape)}; expected {tuple(shape)}")
        if numel is not None and (t.numel() < numel if at_least else t.numel() != numel):
            raise ValueError(f"{what} has {t.numel()} elements; expected "
                             f"{'at least ' if at_least else ''}{numel}")
        if not t.is_contiguous():
            raise ValueError(f"{what} must be contiguous (the library takes packed rows)")
        used.append((what, t))

    if M > 0 and N > 0:
        if K > 0:
            need(A, "A", kinds[desc.dtype_ab], shape=(M, K))
            need(B, "B (the K x N operand stored as N rows of K)", kinds[desc.dtype_ab],
                 shape=(N, K))
        need(C, "C", kinds[desc.dtype_c], numel=M * N, at_least=True)
        if desc.dtype_ab == GEMM_FP8_E4M3:
            need(scale_a, "scale_a", (torch.float32,), numel=1)
            need(scale_b, "scale_b", (torch.float32,), numel=1)
        if desc.epilogue & (GEMM_EPI_BIAS_ROW | GEMM_EPI_BIAS_COL):
            n = M if desc.epilogue & GEMM_EPI_BIAS_ROW else N
            need(bias, "bias", (torch.float32,), numel=n)
        if desc.dtype_c == GEMM_FP8_E4M3:
            need(scale_d, "scale_d", (torch.float32,), numel=1)
        if desc.epilogue & GEMM_EPI_AMAX:
            need(amax, "amax", (torch.float32,), numel=1)
        if desc.epilogue & (GEMM_EPI_SOURCE_F32 | GEMM_EPI_SOURCE_BF16) and float(beta) != 0.0:
            f32 = desc.epilogue & GEMM_EPI_SOURCE_F32
            need(source, "source", (torch.float32,) if f32 else (torch.bfloat16, torch.int16),
                 numel=M * N, at_least=True)   # like C, which it may be
        if workspace_bytes:
            if workspace is None:
                raise ValueError(f"this plan needs a workspace of {workspace_bytes} bytes")
            if not workspace.is_contiguous():
                raise ValueError("workspace must be contiguous")
            have = workspace.numel() * workspace.element_size()
            if have < workspace_bytes:
                raise ValueError(f"workspace has {have} bytes; the plan needs {workspace_bytes}")
            used.append(("workspace", workspace))
    devices = {(t.device.type, t.device.index) for _, t in used}
    for what, t in used:
        if t.device.type != "cuda":
            raise ValueError(f"{what} is on {t.device}; every operand must be on the GPU")
    if len(devices) > 1:
        raise ValueError(f"operands are on different devices: {sorted(devices)}")
