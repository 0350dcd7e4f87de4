"""The Python binding's checks on torch tensors (Plan.validate, gemm()), run on CPU tensors: a
tensor of the wrong shape, element type, length or layout must be refused with ValueError before
any pointer reaches the library, because the kernels size their buffer ranges from M, N and K,
not from the tensors.  With every check passed, CPU tensors are refused for not being on the GPU.
Also the planner: when the cost model picks the cooperative kernel, the plan runs it."""
import pytest

torch = pytest.importorskip("torch")

import dense_gemm_design_amd as dg  # noqa: E402
from dense_gemm_design_amd import _lib as L  # noqa: E402

M, N, K = 256, 128, 64


def plan_of(dtype_ab=L.GEMM_BF16, dtype_c=L.GEMM_F32, epilogue=0, sched=L.GEMM_SCHED_PERSISTENT,
            workers=4, tile=128):
    return L.Plan(L.make_desc(M, N, K, dtype_ab, dtype_c, L.GEMM_MAP_LINEAR_N, 1, sched, workers,
                              tile, tile, 0, 0, epilogue=epilogue))


def good_bf16():
    return (torch.zeros((M, K), dtype=torch.bfloat16), torch.zeros((N, K), dtype=torch.bfloat16),
            torch.zeros((M, N), dtype=torch.float32))


def refused(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_shapes_and_types_are_checked_first():
    p = plan_of()
    A, B, C = good_bf16()
    refused(r"A has shape", p.validate, A[:, :32], B, C)
    refused(r"B .* has shape", p.validate, A, torch.zeros((K, N), dtype=torch.bfloat16), C)
    refused(r"A has dtype", p.validate, A.float(), B, C)
    refused(r"C has dtype", p.validate, A, B, C.to(torch.bfloat16))
    refused(r"C has \d+ elements; expected at least", p.validate, A, B, C[: M - 1])
    refused(r"A must be contiguous", p.validate,
            torch.zeros((K, M), dtype=torch.bfloat16).t(), B, C)
    refused(r"A is required", p.validate, None, B, C)
    # int16 bit patterns are accepted for bf16 operands
    refused(r"is on cpu", p.validate, A.view(torch.int16), B.view(torch.int16), C)


def test_source_operand():
    """A source bit with beta != 0 needs an M x N source of the bit's type; beta == 0 none."""
    A, B, C = good_bf16()
    p = plan_of(epilogue=L.GEMM_EPI_SOURCE_F32)
    refused(r"source is required", p.validate, A, B, C, source=None, beta=0.5)
    refused(r"source has dtype", p.validate, A, B, C, source=C.to(torch.bfloat16), beta=0.5)
    refused(r"source has 32640 elements; expected at least 32768", p.validate, A, B, C,
            source=C[: M - 1], beta=0.5)
    refused(r"is on cpu", p.validate, A, B, C, source=C, beta=0.5)      # C itself: accepted
    refused(r"is on cpu", p.validate, A, B, C, source=None, beta=0.0)   # nothing read
    q = plan_of(dtype_c=L.GEMM_BF16, epilogue=L.GEMM_EPI_SOURCE_BF16)
    Cb = C.to(torch.bfloat16)
    refused(r"source has dtype", q.validate, A, B, Cb, source=C, beta=1.0)
    refused(r"is on cpu", q.validate, A, B, Cb, source=Cb.view(torch.int16), beta=1.0)


def test_fp8_scales_and_epilogue_operands():
    p = plan_of(L.GEMM_FP8_E4M3, L.GEMM_FP8_E4M3, L.GEMM_EPI_BIAS_ROW | L.GEMM_EPI_AMAX)
    A = torch.zeros((M, K), dtype=torch.uint8)
    B = torch.zeros((N, K), dtype=torch.float8_e4m3fn)
    C = torch.zeros((M, N), dtype=torch.uint8)
    one = torch.ones(1, dtype=torch.float32)
    bias = torch.zeros(M, dtype=torch.float32)
    refused(r"scale_a is required", p.validate, A, B, C, None, one, bias=bias, scale_d=one,
            amax=one)
    refused(r"scale_b has 2 elements", p.validate, A, B, C, one, torch.ones(2), bias=bias,
            scale_d=one, amax=one)
    refused(r"bias has 128 elements; expected 256", p.validate, A, B, C, one, one,
            bias=torch.zeros(N), scale_d=one, amax=one)
    refused(r"bias has dtype", p.validate, A, B, C, one, one, bias=bias.double(), scale_d=one,
            amax=one)
    refused(r"scale_d is required", p.validate, A, B, C, one, one, bias=bias, amax=one)
    refused(r"amax is required", p.validate, A, B, C, one, one, bias=bias, scale_d=one)
    refused(r"is on cpu", p.validate, A, B, C, one, one, bias=bias, scale_d=one, amax=one)


def test_workspace_size_is_checked():
    p = plan_of(sched=L.GEMM_SCHED_STREAMK, workers=8)
    need = p.workspace_bytes
    assert need > 0
    A, B, C = good_bf16()
    refused(r"needs a workspace", p.validate, A, B, C)
    refused(r"workspace has \d+ bytes", p.validate, A, B, C,
            workspace=torch.zeros(need - 1, dtype=torch.uint8))
    refused(r"is on cpu", p.validate, A, B, C, workspace=torch.zeros(need, dtype=torch.uint8))


def test_empty_output_needs_nothing():
    p = L.Plan(L.make_desc(0, N, K, num_workers=4))
    assert p.validate(None, None, None) is None


def test_gemm_helper_checks_before_planning():
    A, B, _ = good_bf16()
    refused(r"must be 2-D", dg.gemm, A.reshape(-1), B)
    refused(r"B must be \(N, K\)", dg.gemm, A, torch.zeros((N, K + 16), dtype=torch.bfloat16))
    refused(r"both be bf16 or both e4m3", dg.gemm, A, B.view(torch.int16).to(torch.uint8))
    refused(r"out_dtype", dg.gemm, A, B, out_dtype="f16")
    refused(r"one bias at most", dg.gemm, A, B, bias_row=torch.zeros(M), bias_col=torch.zeros(N))


def test_model_pick_of_the_cooperative_kernel_is_the_kernel_that_runs():
    """A shape the cost model gives to the cooperative kernel (one 128 x 128 tile, one k-tile):
    the plan runs that kernel, on the grid the planner sized for it."""
    d = L.make_desc(128, 128, 64, L.GEMM_BF16, L.GEMM_F32, L.GEMM_MAP_GROUPED_M, 0,
                    L.GEMM_SCHED_AUTO, 256)
    ranked = L.rank_configs(d)
    assert ranked[0].kernel == 0, "the model no longer picks the cooperative kernel here"
    p = L.Plan(d)
    assert (p.info.kernel, p.info.bm, p.info.bn) == (0, ranked[0].bm, ranked[0].bn)
    assert p.info.sched == ranked[0].sched
