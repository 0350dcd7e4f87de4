"""Parity of the HIP path with the CPU oracle, through the C ABI, on an MI355X.

Tolerance per element: |C - C_ref| <= 4e-3 |C_ref| + 1e-3 sqrt(K) max|a| max|b|.  Integer and
schedule results are compared exactly: the closed-form row sums and small-integer products are
exact in FP32 whatever the summation order, and the device trace of work items must equal the CPU
enumeration.
"""
import zlib

import numpy as np
import pytest

import gemm_inputs as gi
import oracle
from oracle import schedule as S
from dense_gemm_design_amd import _lib as L
from gpu_util import assert_within_tolerance, reference, run_gpu, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()
    return torch.device("cuda:0")


def test_bf16_256_static_linear_full(dev):
    """256^3 bf16, A row / B column major, uniform[-1,1], fp32 out, linear N-fast, static."""
    op = gi.make_workload("bf16_256")
    C, plan, _ = run_gpu(op, torch, dev, "f32", L.GEMM_MAP_LINEAR_N, 1, L.GEMM_SCHED_STATIC,
                         tile=128)
    assert plan.info.grid == 4 and plan.info.bm == 128
    assert_within_tolerance(C, reference(op), op, "bf16_256")


SMALL = [
    # id, M, N, K, dtype, out, tile, mapping, G, sched, workers
    ("bf16_t256_grouped_persist", 512, 768, 1024, "bf16", "bf16", 256, L.GEMM_MAP_GROUPED_M, 2,
     L.GEMM_SCHED_PERSISTENT, 3),
    ("bf16_t128_linear_m", 640, 512, 384, "bf16", "f32", 128, L.GEMM_MAP_LINEAR_M, 1,
     L.GEMM_SCHED_PERSISTENT, 5),
    ("bf16_ragged_t128", 300, 264, 104, "bf16", "f32", 128, L.GEMM_MAP_GROUPED_N, 2,
     L.GEMM_SCHED_STATIC, 0),
    ("bf16_ragged_t256", 300, 264, 104, "bf16", "bf16", 256, L.GEMM_MAP_LINEAR_N, 1,
     L.GEMM_SCHED_PERSISTENT, 2),
    ("bf16_tiny", 1, 8, 8, "bf16", "f32", 128, L.GEMM_MAP_LINEAR_N, 1, L.GEMM_SCHED_STATIC, 0),
    ("fp8_t256", 512, 512, 1024, "e4m3", "bf16", 256, L.GEMM_MAP_GROUPED_M, 16,
     L.GEMM_SCHED_PERSISTENT, 2),
    ("fp8_ragged_t128", 384, 264, 272, "e4m3", "f32", 128, L.GEMM_MAP_LINEAR_N, 1,
     L.GEMM_SCHED_PERSISTENT, 4),
    ("bf16_streamk", 256, 256, 8192, "bf16", "f32", 128, L.GEMM_MAP_LINEAR_N, 1,
     L.GEMM_SCHED_STREAMK, 8),
    ("bf16_streamk_hybrid", 640, 640, 2048, "bf16", "f32", 128, L.GEMM_MAP_GROUPED_M, 2,
     L.GEMM_SCHED_STREAMK, 20),
    ("fp8_streamk", 256, 256, 4096, "e4m3", "bf16", 128, L.GEMM_MAP_LINEAR_N, 1,
     L.GEMM_SCHED_STREAMK, 11),
    ("bf16_streamk_ragged", 200, 136, 1000, "bf16", "f32", 128, L.GEMM_MAP_LINEAR_N, 1,
     L.GEMM_SCHED_STREAMK, 9),
]


SK_MODES = {"separate": 0, "chain": L.GEMM_FLAG_STREAMK_CHAIN}
# data-parallel 256 x 256 plans default to the wide-wave kernel; "coop" forces the cooperative one
MODES = dict(SK_MODES, coop=L.GEMM_FLAG_COOPERATIVE)


def modes_of(case):
    if case[9] == L.GEMM_SCHED_STREAMK:
        return list(SK_MODES) + ["coop"]
    return ["separate", "coop"]


CASES = [(c, m) for c in SMALL for m in modes_of(c)]


@pytest.mark.parametrize("case,mode", CASES, ids=[f"{c[0]}-{m}" for c, m in CASES])
def test_small_parity(dev, case, mode):
    name, M, N, K, dt, out, tile, mapping, G, sched, workers = case
    dist = ("normal", 1.0) if dt == "e4m3" else ("uniform",)
    op = gi.make_operands(M, N, K, dt, dist, dist, seed=zlib.crc32(name.encode()) % 10000)
    C, plan, _ = run_gpu(op, torch, dev, out, mapping, G, sched, workers, tile,
                         flags=MODES[mode])
    # wide-wave unless the cooperative kernel is asked for or the lock chain is needed
    assert plan.info.kernel == (0 if mode == "coop" or plan.info.streamk_mode == 0 and
                                plan.info.sk_tiles else 3)
    if plan.info.sk_tiles and mode != "coop":
        assert plan.info.streamk_mode == (0 if mode == "chain" else 1)
    if sched == L.GEMM_SCHED_STREAMK and name != "bf16_streamk_hybrid":
        assert plan.info.sk_tiles > 0
    if name == "bf16_streamk_hybrid":
        assert plan.info.dp_tiles == 20 and plan.info.sk_tiles == 5
    assert_within_tolerance(C, reference(op), op, name)


PINGPONG = [
    # id, M, N, K, dtype, out, mapping, G, sched, workers
    ("pp_bf16_persist", 512, 768, 1024, "bf16", "bf16", L.GEMM_MAP_GROUPED_M, 2,
     L.GEMM_SCHED_PERSISTENT, 3),
    ("pp_bf16_ragged", 300, 264, 104, "bf16", "bf16", L.GEMM_MAP_LINEAR_N, 1,
     L.GEMM_SCHED_PERSISTENT, 1),
    ("pp_bf16_one_kstep_many_items", 768, 512, 64, "bf16", "bf16", L.GEMM_MAP_GROUPED_M, 2,
     L.GEMM_SCHED_PERSISTENT, 2),
    ("pp_bf16_f32_static", 512, 512, 200, "bf16", "f32", L.GEMM_MAP_LINEAR_M, 1,
     L.GEMM_SCHED_STATIC, 0),
    ("pp_bf16_short_k", 264, 520, 8, "bf16", "bf16", L.GEMM_MAP_LINEAR_N, 1,
     L.GEMM_SCHED_PERSISTENT, 2),
    ("pp_fp8_persist", 512, 512, 1024, "e4m3", "bf16", L.GEMM_MAP_GROUPED_M, 16,
     L.GEMM_SCHED_PERSISTENT, 2),
    ("pp_fp8_ragged", 520, 264, 400, "e4m3", "bf16", L.GEMM_MAP_GROUPED_N, 2,
     L.GEMM_SCHED_PERSISTENT, 3),
]


# data-parallel kernels for 256 x 256 tiles: flag, plan_info.kernel, threads
DP_KERNELS = {"pingpong": (L.GEMM_FLAG_PINGPONG, 1, 512),
              "wide": (L.GEMM_FLAG_WIDE, 3, 256)}


@pytest.mark.parametrize("kern", list(DP_KERNELS))
@pytest.mark.parametrize("case", PINGPONG, ids=[c[0] for c in PINGPONG])
def test_pingpong_parity(dev, case, kern):
    """The data-parallel kernels (ping-pong, wide-wave): several items per
    worker, ragged M/N/K, one k-step per item, fp32 and bf16 outputs."""
    name, M, N, K, dt, out, mapping, G, sched, workers = case
    flag, kind, threads = DP_KERNELS[kern]
    dist = ("normal", 1.0) if dt == "e4m3" else ("uniform",)
    op = gi.make_operands(M, N, K, dt, dist, dist, seed=zlib.crc32(name.encode()) % 10000)
    C, plan, _ = run_gpu(op, torch, dev, out, mapping, G, sched, workers, 256, flags=flag)
    assert plan.info.bm == 256 and plan.info.threads == threads and plan.info.kernel == kind
    assert_within_tolerance(C, reference(op), op, name)


@pytest.mark.parametrize("kern", list(DP_KERNELS))
@pytest.mark.parametrize("dt", ["bf16", "e4m3"])
def test_pingpong_closed_form_exact(dev, dt, kern):
    M, N, K = 640, 520, 2048
    op = gi.rowsum_pattern(M, N, K, dt)
    C, plan, _ = run_gpu(op, torch, dev, "f32", L.GEMM_MAP_GROUPED_M, 2, L.GEMM_SCHED_PERSISTENT,
                         2, 256, flags=DP_KERNELS[kern][0])
    assert np.all(C == 7 * K / 16)


@pytest.mark.parametrize("dt", ["bf16", "e4m3"])
@pytest.mark.parametrize("tile,sched,workers", [(128, L.GEMM_SCHED_STATIC, 0),
                                                 (256, L.GEMM_SCHED_PERSISTENT, 3),
                                                 (128, L.GEMM_SCHED_STREAMK, 9)])
def test_closed_form_row_sums_exact(dev, dt, tile, sched, workers):
    """A[m,k] = ((m+k) mod 8)/8, B = 1: every output is exactly 7K/16 in FP32 (256 x 256
    data-parallel plans: both kernels)."""
    M, N, K = 384, 264, 2048
    op = gi.rowsum_pattern(M, N, K, dt)
    for flags in ([0, L.GEMM_FLAG_COOPERATIVE] if tile == 256 else [0]):
        C, plan, _ = run_gpu(op, torch, dev, "f32", L.GEMM_MAP_GROUPED_M, 2, sched, workers, tile,
                             flags=flags)
        assert np.all(C == 7 * K / 16)


@pytest.mark.parametrize("mode", list(SK_MODES))
def test_streamk_small_integers_bit_exact(dev, mode):
    """|a|, |b| <= 2 integers: every partial sum is exact in FP32, so the Stream-K fixup must
    reproduce the oracle bit for bit (a lost or doubled k-tile would show)."""
    M, N, K = 256, 128, 16384
    op = gi.make_operands(M, N, K, "bf16", ("smallint", -2, 2), ("smallint", -2, 2), seed=77)
    C, plan, _ = run_gpu(op, torch, dev, "f32", L.GEMM_MAP_LINEAR_N, 1, L.GEMM_SCHED_STREAMK,
                         24, 128, flags=SK_MODES[mode])
    assert plan.info.sk_tiles == 2
    assert np.array_equal(C, reference(op))


def test_streamk_modes_deterministic_and_identical(dev):
    """Both fixups sum the splits of a tile left to right in K, so on one kernel (the cooperative
    one runs both) they agree bit for bit with each other and with themselves across runs; the
    wide-wave kernel's separate reduction is deterministic too."""
    op = gi.make_operands(256, 256, 8192, "bf16", seed=5)
    coop = L.GEMM_FLAG_COOPERATIVE
    C1, plan, _ = run_gpu(op, torch, dev, "f32", L.GEMM_MAP_LINEAR_N, 1, L.GEMM_SCHED_STREAMK,
                          16, 128, flags=coop)
    C2, _, _ = run_gpu(op, torch, dev, "f32", plan=plan)
    C3, plan3, _ = run_gpu(op, torch, dev, "f32", L.GEMM_MAP_LINEAR_N, 1, L.GEMM_SCHED_STREAMK,
                           16, 128, flags=coop | L.GEMM_FLAG_STREAMK_CHAIN)
    assert plan.info.streamk_mode == 1 and plan3.info.streamk_mode == 0
    assert np.array_equal(C1, C2)
    assert np.array_equal(C1, C3)
    W1, wplan, _ = run_gpu(op, torch, dev, "f32", L.GEMM_MAP_LINEAR_N, 1, L.GEMM_SCHED_STREAMK,
                           16, 128)
    W2, _, _ = run_gpu(op, torch, dev, "f32", plan=wplan)
    assert wplan.info.kernel == 3 and np.array_equal(W1, W2)
    assert_within_tolerance(W1, reference(op), op, "wide Stream-K")


@pytest.mark.parametrize("sched,workers,tile,mapping,G,W", [
    (L.GEMM_SCHED_STREAMK, 20, 128, L.GEMM_MAP_GROUPED_M, 2, 0),
    (L.GEMM_SCHED_PERSISTENT, 8, 256, L.GEMM_MAP_GROUPED_N, 3, 0),
    (L.GEMM_SCHED_STATIC, 0, 128, L.GEMM_MAP_LINEAR_M, 1, 0),
    (L.GEMM_SCHED_STREAMK, 20, 128, L.GEMM_MAP_BLOCKED, 2, 3),
    (L.GEMM_SCHED_PERSISTENT, 2, 256, L.GEMM_MAP_BLOCKED, 2, 2),
    (L.GEMM_SCHED_STATIC, 0, 128, L.GEMM_MAP_MORTON, 1, 0),
    (L.GEMM_SCHED_PERSISTENT, 3, 256, L.GEMM_MAP_MORTON, 1, 0),
    (L.GEMM_SCHED_STREAMK, 6, 256, L.GEMM_MAP_GROUPED_M, 2, 0),     # wide-wave Stream-K
])
def test_device_trace_matches_enumeration(dev, sched, workers, tile, mapping, G, W):
    """Work items recorded by the kernel equal the CPU replay and the oracle's enumeration."""
    M, N, K = 640, 640, 2048
    op = gi.make_operands(M, N, K, "bf16", seed=3)
    C, plan, ws = run_gpu(op, torch, dev, "f32", mapping, G, sched, workers, tile,
                          flags=L.GEMM_FLAG_TRACE, group_n=W)
    info = plan.info
    raw = ws.cpu().numpy()[info.trace_offset:].view(np.int32)[: info.grid * info.trace_capacity * 8]
    rec = raw.reshape(info.grid, info.trace_capacity, 8)
    got = []
    for w in range(info.grid):
        for r in rec[w]:
            if r[0] == w and (r[6] > 0):
                got.append(tuple(int(x) for x in r))
    want = plan.schedule()
    assert got == want
    MAP = {0: S.LINEAR_N, 1: S.LINEAR_M, 2: S.GROUPED_M, 3: S.GROUPED_N, 4: S.BLOCKED,
           5: S.MORTON}
    SCH = {0: S.STATIC, 1: S.PERSISTENT, 2: S.STREAMK}
    ora = S.enumerate_schedule(M, N, K, tile, tile, info.bk, MAP[mapping], G, SCH[sched],
                               P=None if sched == L.GEMM_SCHED_STATIC else info.grid,
                               W=info.group_n, sk_groups=info.sk_groups)
    assert got == [(w.worker, w.seq, w.tile, w.m, w.n, w.k_begin, w.k_end, w.role) for w in ora]
    assert_within_tolerance(C, reference(op), op, "trace run")


@pytest.mark.parametrize("mapping", [L.GEMM_MAP_GROUPED_M, L.GEMM_MAP_GROUPED_N])
def test_device_trace_xcd_box(dev, mapping):
    """A plan on the XCD box remap (Grouped-M/N(8) on 16 x 8 tiles of 128, 64 workers: every
    wave is an 8 x 8 block, each XCD takes a 2 x 4 box of it): the kernel's recorded work items
    equal the CPU replay and the oracle's enumeration, and the product is within tolerance."""
    M, N, K = (2048, 1024, 256) if mapping == L.GEMM_MAP_GROUPED_M else (1024, 2048, 256)
    op = gi.make_operands(M, N, K, "bf16", seed=31)
    C, plan, ws = run_gpu(op, torch, dev, "f32", mapping, 8, L.GEMM_SCHED_PERSISTENT, 64, 128,
                          flags=L.GEMM_FLAG_TRACE)
    info = plan.info
    assert (info.xcd_box_r, info.xcd_box_c) == (2, 4)
    raw = ws.cpu().numpy()[info.trace_offset:].view(np.int32)[: info.grid * info.trace_capacity * 8]
    rec = raw.reshape(info.grid, info.trace_capacity, 8)
    got = [tuple(int(x) for x in r) for w in range(info.grid) for r in rec[w]
           if r[0] == w and r[6] > 0]
    assert got == plan.schedule()
    ora = S.enumerate_schedule(M, N, K, 128, 128, info.bk,
                               S.GROUPED_M if mapping == L.GEMM_MAP_GROUPED_M else S.GROUPED_N,
                               8, S.PERSISTENT, P=info.grid)
    assert got == [(w.worker, w.seq, w.tile, w.m, w.n, w.k_begin, w.k_end, w.role) for w in ora]
    assert_within_tolerance(C, reference(op), op, "box trace run")


@pytest.mark.parametrize("mode", list(SK_MODES))
def test_spin_watchdog_reports_instead_of_hanging(dev, mode):
    """The first split of band tile 0 withholds its lock / arrival (test flag); the bounded waits
    on it expire, the kernel still finishes, and the device error word says so."""
    op = gi.make_operands(256, 256, 4096, "bf16", seed=9)
    C, plan, ws = run_gpu(op, torch, dev, "f32", L.GEMM_MAP_LINEAR_N, 1, L.GEMM_SCHED_STREAMK, 8,
                          128, flags=L.GEMM_FLAG_TEST_SKIP_PUBLISH | SK_MODES[mode])
    err = int(ws.cpu().numpy()[plan.info.error_offset:plan.info.error_offset + 4].view(np.int32)[0])
    assert err == L.GEMM_DEVICE_ERR_SPIN
    # and a normal run of the same plan shape reports no error
    C, plan, ws = run_gpu(op, torch, dev, "f32", L.GEMM_MAP_LINEAR_N, 1, L.GEMM_SCHED_STREAMK, 8,
                          128)
    err = int(ws.cpu().numpy()[plan.info.error_offset:plan.info.error_offset + 4].view(np.int32)[0])
    assert err == L.GEMM_DEVICE_OK


@pytest.mark.parametrize("tile", [128, 256])
def test_every_mapping_gives_identical_bits(dev, tile):
    """The mapping only reorders whole tiles; each tile's arithmetic is unchanged: linear,
    grouped, blocked and Morton orders give the same bits (ragged grid, several items per
    worker)."""
    op = gi.make_operands(1160, 1288, 512, "bf16", seed=12)
    C1, _, _ = run_gpu(op, torch, dev, "bf16", L.GEMM_MAP_LINEAR_N, 1, L.GEMM_SCHED_PERSISTENT,
                       7, tile)
    assert_within_tolerance(C1, reference(op), op, "linear")
    for mapping, G, W in ((L.GEMM_MAP_GROUPED_M, 8, 0), (L.GEMM_MAP_GROUPED_N, 3, 0),
                          (L.GEMM_MAP_BLOCKED, 2, 3), (L.GEMM_MAP_BLOCKED, 0, 0),
                          (L.GEMM_MAP_MORTON, 1, 0)):
        C2, _, _ = run_gpu(op, torch, dev, "bf16", mapping, G, L.GEMM_SCHED_PERSISTENT, 7, tile,
                           group_n=W)
        assert np.array_equal(C1, C2), (mapping, G, W)


@pytest.mark.parametrize("M,N,K", [(0, 64, 64), (64, 0, 64), (64, 64, 0), (130, 136, 0)])
def test_empty_and_zero_depth(dev, M, N, K):
    """M or N = 0: nothing is written.  K = 0: C is the empty sum, all zeros."""
    op = gi.make_operands(M, N, K, "bf16", seed=1)
    if M == 0 or N == 0:
        A, B, sa, sb = to_device(op, torch, dev)
        plan = L.Plan(L.make_desc(M, N, K, num_workers=4))
        C = torch.empty((M, N), device=dev)
        plan.run(A, B, C)
        torch.cuda.synchronize()
        assert C.numel() == 0
        return
    for sched, workers in ((L.GEMM_SCHED_PERSISTENT, 3), (L.GEMM_SCHED_STREAMK, 8),
                           (L.GEMM_SCHED_STATIC, 0)):
        C, plan, _ = run_gpu(op, torch, dev, "f32", sched=sched, workers=workers, tile=128)
        assert np.array_equal(C, np.zeros((M, N)))


# kernels whose MFMA is the 16 x 16 form (a different summation order inside each MFMA than the
# 32 x 32 form the other kernels use), per operand type
MFMA16 = {("wide", "bf16"), ("wide", "e4m3"), ("wide128", "bf16"), ("wide128", "e4m3")}


@pytest.mark.parametrize("dt,out", [("bf16", "f32"), ("bf16", "bf16"), ("e4m3", "bf16"),
                                    ("e4m3", "f32")])
def test_data_parallel_kernels_bit_identical(dev, dt, out):
    """Every data-parallel kernel with the same MFMA shape sums each output over K in the same
    order with the same instruction (k-tile depth only groups the MFMAs), so kernels of one
    shape -- cooperative (128 and 256 tiles), ping-pong, wide-wave -- must agree
    bit for bit, across tile shapes, ragged M/N/K and several items per worker; every kernel is
    within tolerance of the oracle."""
    M, N, K = 776, 520, 1000 if dt == "bf16" else 1040
    dist = ("normal", 1.0) if dt == "e4m3" else ("uniform",)
    op = gi.make_operands(M, N, K, dt, dist, dist, seed=4242)
    ref = reference(op)
    runs = {}
    for name, tile, flags in (("coop128", 128, L.GEMM_FLAG_COOPERATIVE),
                              ("coop256", 256, L.GEMM_FLAG_COOPERATIVE),
                              ("pingpong", 256, L.GEMM_FLAG_PINGPONG),
                              ("wide", 256, L.GEMM_FLAG_WIDE),
                              ("wide128", 128, L.GEMM_FLAG_WIDE)):
        C, plan, _ = run_gpu(op, torch, dev, out, L.GEMM_MAP_GROUPED_M, 2,
                             L.GEMM_SCHED_PERSISTENT, 3, tile, flags=flags)
        assert_within_tolerance(C, ref, op, f"dp kernel {name}")
        runs[name] = C
    families = {}
    for name, C in runs.items():
        families.setdefault((name, dt) in MFMA16, []).append((name, C))
    for members in families.values():
        first, C0 = members[0]
        for name, C in members[1:]:
            assert np.array_equal(C, C0), f"{name} differs from {first} (same MFMA shape)"


@pytest.mark.parametrize("M,N,K", [(776, 520, 1000), (300, 264, 104), (1, 8, 64), (520, 776, 200)])
def test_no_writes_past_c(dev, M, N, K):
    """C is the front of a larger buffer whose tail holds a canary pattern: after every kernel
    and output type (edge tiles whose waves lie wholly past M or N included) the canary is
    untouched, and C matches the oracle."""
    op = gi.make_operands(M, N, K, "bf16", ("uniform",), ("uniform",), seed=M + N + K)
    ref = reference(op)
    A, B, sa, sb = to_device(op, torch, dev)
    for out in ("bf16", "f32"):
        eb = 2 if out == "bf16" else 4
        canary_bytes = 4 << 20
        buf = torch.empty(M * N * eb + canary_bytes, dtype=torch.uint8, device=dev)
        for tile, flags in ((128, L.GEMM_FLAG_COOPERATIVE), (256, L.GEMM_FLAG_COOPERATIVE),
                            (256, L.GEMM_FLAG_PINGPONG),
                            (256, L.GEMM_FLAG_WIDE), (128, L.GEMM_FLAG_WIDE)):
            buf.fill_(0xA5)
            plan = L.Plan(L.make_desc(M, N, K, L.GEMM_BF16,
                                      L.GEMM_BF16 if out == "bf16" else L.GEMM_F32,
                                      L.GEMM_MAP_GROUPED_M, 2, L.GEMM_SCHED_PERSISTENT, 2,
                                      tile, tile, 0, flags))
            st = plan.run_raw(A.data_ptr(), B.data_ptr(), buf.data_ptr())
            assert st == L.GEMM_OK
            torch.cuda.synchronize()
            tail = buf[M * N * eb:]
            assert bool((tail == 0xA5).all()), f"tile {tile} flags {flags:#x} {out}: wrote past C"
            C = buf[:M * N * eb].view(torch.bfloat16 if out == "bf16" else torch.float32)
            got = C.float().cpu().numpy().astype(np.float64).reshape(M, N)
            assert_within_tolerance(got, ref, op, f"canary {M}x{N}x{K} {out} {flags:#x}")


@pytest.mark.parametrize("M,N,K", [(776, 520, 1040), (300, 264, 128), (1, 8, 64), (520, 776, 256)])
def test_fp8_wide_staged_output(dev, M, N, K):
    """The e4m3 wide-wave kernel on 256 x 256 tiles writes a tile's bf16 output during the
    worker's next item's first k-step (the worker's last tile after its own k-loop).  Over ragged
    edges (waves wholly past M or N), one-k-step items (K <= 128) and several items per worker:
    nothing is written past C, both outputs are within tolerance of the oracle, and every bf16
    output is the round-to-nearest-even bf16 of the same launch's f32 output (alpha * Acc in both:
    the same accumulators, scaled the same way) bit for bit."""
    op = gi.make_operands(M, N, K, "e4m3", ("normal", 1.0), ("normal", 1.0), seed=7 * M + N + K)
    ref = reference(op)
    A, B, sa, sb = to_device(op, torch, dev)
    canary_bytes = 4 << 20
    got = {}
    for out in ("f32", "bf16"):
        eb = 2 if out == "bf16" else 4
        buf = torch.empty(M * N * eb + canary_bytes, dtype=torch.uint8, device=dev)
        buf.fill_(0xA5)
        plan = L.Plan(L.make_desc(M, N, K, L.GEMM_FP8_E4M3,
                                  L.GEMM_BF16 if out == "bf16" else L.GEMM_F32,
                                  L.GEMM_MAP_GROUPED_M, 2, L.GEMM_SCHED_PERSISTENT, 2,
                                  256, 256, 0, L.GEMM_FLAG_WIDE))
        assert plan.info.kernel == 3 and plan.info.bm == 256 and plan.info.bk == 128
        st = plan.run_raw(A.data_ptr(), B.data_ptr(), buf.data_ptr(), sa.data_ptr(), sb.data_ptr())
        assert st == L.GEMM_OK
        torch.cuda.synchronize()
        assert bool((buf[M * N * eb:] == 0xA5).all()), f"{out}: wrote past C"
        C = buf[:M * N * eb].view(torch.bfloat16 if out == "bf16" else torch.float32)
        got[out] = C.reshape(M, N).clone()
        assert_within_tolerance(C.float().cpu().numpy().astype(np.float64).reshape(M, N), ref, op,
                                f"fp8 wide {M}x{N}x{K} {out}")
    want = got["f32"].to(torch.bfloat16).view(torch.int16)
    diff = int((got["bf16"].view(torch.int16) != want).sum())
    assert diff == 0, f"{diff} bf16 outputs differ from the bf16 rounding of the f32 outputs"


WIDE_SK = [
    # id, M, N, K, dtype, out, workers, mapping, G; 256 x 256 tiles, Stream-K
    ("bf16_all_split", 512, 512, 16384, "bf16", "f32", 8, L.GEMM_MAP_LINEAR_N, 1),
    ("bf16_hybrid_ragged", 300, 520, 3000, "bf16", "bf16", 5, L.GEMM_MAP_GROUPED_M, 2),
    ("fp8_hybrid", 512, 768, 8192, "e4m3", "bf16", 4, L.GEMM_MAP_GROUPED_N, 2),
    ("fp8_all_split_f32", 256, 520, 16384, "e4m3", "f32", 16, L.GEMM_MAP_BLOCKED, 1),
]


@pytest.mark.parametrize("forced", [True, False])
@pytest.mark.parametrize("case", WIDE_SK, ids=[c[0] for c in WIDE_SK])
def test_wide_streamk_parity(dev, case, forced):
    """Stream-K plans on 256 x 256 tiles run on the wide-wave kernel (by default, or forced):
    splits store row-major partials, every unit reduces its share after its MAC work."""
    name, M, N, K, dt, out, workers, mapping, G = case
    dist = ("normal", 1.0) if dt == "e4m3" else ("uniform",)
    op = gi.make_operands(M, N, K, dt, dist, dist, seed=zlib.crc32(name.encode()) % 10000)
    C, plan, ws = run_gpu(op, torch, dev, out, mapping, G, L.GEMM_SCHED_STREAMK, workers, 256,
                          flags=L.GEMM_FLAG_WIDE if forced else 0)
    info = plan.info
    assert info.kernel == 3 and info.sk_tiles > 0 and info.streamk_mode == 1
    err = int(ws.cpu().numpy()[info.error_offset:info.error_offset + 4].view(np.int32)[0])
    assert err == L.GEMM_DEVICE_OK
    assert_within_tolerance(C, reference(op), op, name)


def test_wide_streamk_small_integers_bit_exact(dev):
    """Small-integer operands: every partial and every sum is exact in fp32, so the wide-wave
    Stream-K result equals the oracle bit for bit (and the cooperative kernel's)."""
    M, N, K = 512, 512, 32768
    op = gi.make_operands(M, N, K, "bf16", ("smallint", -2, 2), ("smallint", -2, 2), seed=77)
    ref = reference(op)
    C, plan, _ = run_gpu(op, torch, dev, "f32", L.GEMM_MAP_LINEAR_N, 1, L.GEMM_SCHED_STREAMK, 24,
                         256)
    assert plan.info.kernel == 3 and plan.info.sk_tiles == 4
    assert np.array_equal(C, ref)
    C2, plan2, _ = run_gpu(op, torch, dev, "f32", L.GEMM_MAP_LINEAR_N, 1, L.GEMM_SCHED_STREAMK,
                           24, 256, flags=L.GEMM_FLAG_COOPERATIVE)
    assert plan2.info.kernel == 0 and np.array_equal(C2, ref)


def test_wide_streamk_watchdog(dev):
    """The first split of band tile 0 withholds its arrival (test flag): the bounded wait on it
    expires, the kernel finishes, and the device error word says so; a normal run reports OK."""
    op = gi.make_operands(512, 512, 8192, "bf16", seed=9)
    C, plan, ws = run_gpu(op, torch, dev, "f32", L.GEMM_MAP_LINEAR_N, 1, L.GEMM_SCHED_STREAMK, 8,
                          256, flags=L.GEMM_FLAG_TEST_SKIP_PUBLISH)
    assert plan.info.kernel == 3
    err = int(ws.cpu().numpy()[plan.info.error_offset:plan.info.error_offset + 4].view(np.int32)[0])
    assert err == L.GEMM_DEVICE_ERR_SPIN
    C, plan, ws = run_gpu(op, torch, dev, "f32", L.GEMM_MAP_LINEAR_N, 1, L.GEMM_SCHED_STREAMK, 8,
                          256)
    err = int(ws.cpu().numpy()[plan.info.error_offset:plan.info.error_offset + 4].view(np.int32)[0])
    assert err == L.GEMM_DEVICE_OK


# ---- Stream-K groups ---------------------------------------------------------------------------

SKG_KERNELS = {"wide": (0, 3, 1), "coop_separate": (L.GEMM_FLAG_COOPERATIVE, 0, 1),
               "coop_chain": (L.GEMM_FLAG_COOPERATIVE | L.GEMM_FLAG_STREAMK_CHAIN, 0, 0)}
SKG_CASES = [
    # id, M, N, K, dtype, out, workers, tile, mapping, G, requested groups -> planned groups
    ("all_split_g4", 512, 512, 16384, "bf16", "f32", 64, 128, L.GEMM_MAP_LINEAR_N, 1, 4, 4),
    ("hybrid_g5", 1280, 640, 2048, "bf16", "bf16", 40, 128, L.GEMM_MAP_GROUPED_M, 4, 5, 5),
    ("hybrid_g8_ragged", 1256, 632, 1000, "bf16", "f32", 40, 128, L.GEMM_MAP_LINEAR_N, 1, 8, 8),
    ("fp8_256_g3", 768, 1280, 4096, "e4m3", "bf16", 12, 256, L.GEMM_MAP_GROUPED_N, 2, 3, 3),
]


@pytest.mark.parametrize("kern", list(SKG_KERNELS))
@pytest.mark.parametrize("case", SKG_CASES, ids=[c[0] for c in SKG_CASES])
def test_streamk_groups_parity(dev, case, kern):
    """Stream-K groups on both kernels and both fixups: within tolerance of the oracle, the
    device error word clear, the plan as asked."""
    name, M, N, K, dt, out, workers, tile, mapping, G, req, planned = case
    flags, kind, mode = SKG_KERNELS[kern]
    dist = ("normal", 1.0) if dt == "e4m3" else ("uniform",)
    op = gi.make_operands(M, N, K, dt, dist, dist, seed=zlib.crc32(name.encode()) % 10000)
    C, plan, ws = run_gpu(op, torch, dev, out, mapping, G, L.GEMM_SCHED_STREAMK, workers, tile,
                          flags=flags, sk_groups=req)
    info = plan.info
    assert info.sk_tiles > 0 and info.sk_groups == planned
    assert info.kernel == kind and info.streamk_mode == mode
    err = int(ws.cpu().numpy()[info.error_offset:info.error_offset + 4].view(np.int32)[0])
    assert err == L.GEMM_DEVICE_OK
    assert_within_tolerance(C, reference(op), op, f"{name} {kern}")


@pytest.mark.parametrize("kern", list(SKG_KERNELS))
def test_streamk_groups_small_integers_bit_exact(dev, kern):
    """Exact partial sums: every group count gives the oracle's result bit for bit (a k-tile lost
    or doubled by the group split would show)."""
    flags = SKG_KERNELS[kern][0]
    M, N, K = 1280, 640, 4096
    op = gi.make_operands(M, N, K, "bf16", ("smallint", -2, 2), ("smallint", -2, 2), seed=91)
    ref = reference(op)
    for req in (1, 2, 5, 8):
        C, plan, _ = run_gpu(op, torch, dev, "f32", L.GEMM_MAP_GROUPED_M, 4, L.GEMM_SCHED_STREAMK,
                             40, 128, flags=flags, sk_groups=req)
        assert plan.info.sk_groups == req and plan.info.sk_tiles == 10
        assert np.array_equal(C, ref), f"{kern} groups {req}"


@pytest.mark.parametrize("tile,workers,req,flags", [(128, 40, 5, 0), (128, 40, 8, 0),
                                                    (256, 12, 3, 0),
                                                    (128, 40, 4, L.GEMM_FLAG_COOPERATIVE),
                                                    (128, 40, 2, L.GEMM_FLAG_STREAMK_CHAIN)])
def test_device_trace_streamk_groups(dev, tile, workers, req, flags):
    """Work items the kernel records under Stream-K groups equal the CPU replay and the oracle."""
    M, N, K = 1280, 640, 2048
    if tile == 256:
        M, N = 768, 1280
    op = gi.make_operands(M, N, K, "bf16", seed=13)
    C, plan, ws = run_gpu(op, torch, dev, "f32", L.GEMM_MAP_GROUPED_M, 2, L.GEMM_SCHED_STREAMK,
                          workers, tile, flags=flags | L.GEMM_FLAG_TRACE, sk_groups=req)
    info = plan.info
    assert info.sk_groups == req and info.sk_tiles > 0
    raw = ws.cpu().numpy()[info.trace_offset:].view(np.int32)[: info.grid * info.trace_capacity * 8]
    rec = raw.reshape(info.grid, info.trace_capacity, 8)
    got = [tuple(int(x) for x in r) for w in range(info.grid) for r in rec[w]
           if r[0] == w and r[6] > 0]
    assert got == plan.schedule()
    ora = S.enumerate_schedule(M, N, K, tile, tile, info.bk, S.GROUPED_M, 2, S.STREAMK,
                               P=info.grid, sk_groups=req)
    assert got == [(w.worker, w.seq, w.tile, w.m, w.n, w.k_begin, w.k_end, w.role) for w in ora]
    assert_within_tolerance(C, reference(op), op, "groups trace run")


# ---- 256 x 224 and 256 x 192 tiles ---------------------------------------------------------------

T224 = [
    # id, M, N, K, dtype, out, sched, workers, mapping, G
    ("bf16_ragged", 520, 904, 1000, "bf16", "bf16", L.GEMM_SCHED_PERSISTENT, 3,
     L.GEMM_MAP_GROUPED_M, 2),
    ("bf16_f32_static", 512, 672, 512, "bf16", "f32", L.GEMM_SCHED_STATIC, 0,
     L.GEMM_MAP_LINEAR_N, 1),
    ("fp8_ragged", 776, 688, 1040, "e4m3", "bf16", L.GEMM_SCHED_PERSISTENT, 4,
     L.GEMM_MAP_BLOCKED, 0),
    ("bf16_streamk", 512, 448, 16384, "bf16", "f32", L.GEMM_SCHED_STREAMK, 8,
     L.GEMM_MAP_LINEAR_N, 1),
    ("fp8_streamk_hybrid", 768, 1344, 4096, "e4m3", "bf16", L.GEMM_SCHED_STREAMK, 12,
     L.GEMM_MAP_GROUPED_N, 2),
]


@pytest.mark.parametrize("bn", [224, 192])
@pytest.mark.parametrize("case", T224, ids=[c[0] for c in T224])
def test_tile_256_narrow_parity(dev, case, bn):
    """256 x 224 and 256 x 192 tiles run on the wide-wave kernel only (waves of 128 x 112 and
    128 x 96): within tolerance of the oracle for data-parallel and Stream-K plans, ragged edges
    included."""
    name, M, N, K, dt, out, sched, workers, mapping, G = case
    if sched == L.GEMM_SCHED_STREAMK:
        N = N * bn // 224  # the same tile count, so the tail still makes a Stream-K band
    dist = ("normal", 1.0) if dt == "e4m3" else ("uniform",)
    op = gi.make_operands(M, N, K, dt, dist, dist, seed=zlib.crc32(name.encode()) % 10000)
    C, plan, ws = run_gpu(op, torch, dev, out, mapping, G, sched, workers, 256, bn=bn)
    info = plan.info
    assert info.kernel == 3 and (info.bm, info.bn) == (256, bn)
    if sched == L.GEMM_SCHED_STREAMK:
        assert info.sk_tiles > 0
        err = int(ws.cpu().numpy()[info.error_offset:info.error_offset + 4].view(np.int32)[0])
        assert err == L.GEMM_DEVICE_OK
    assert_within_tolerance(C, reference(op), op, name)


@pytest.mark.parametrize("bn", [224, 192])
def test_tile_256_narrow_small_integers_bit_exact(dev, bn):
    """Exact partial sums: the 256 x 224 and 256 x 192 kernels equal the oracle bit for bit,
    data-parallel and Stream-K, and equal the 256 x 256 kernel (same MFMA, same k order)."""
    M, N, K = 512, 896, 8192
    op = gi.make_operands(M, N, K, "bf16", ("smallint", -2, 2), ("smallint", -2, 2), seed=33)
    ref = reference(op)
    C1, p1, _ = run_gpu(op, torch, dev, "f32", L.GEMM_MAP_LINEAR_N, 1, L.GEMM_SCHED_PERSISTENT, 8,
                        256, bn=bn)
    C2, p2, _ = run_gpu(op, torch, dev, "f32", L.GEMM_MAP_LINEAR_N, 1, L.GEMM_SCHED_STREAMK, 24,
                        256, bn=bn)
    C3, _, _ = run_gpu(op, torch, dev, "f32", L.GEMM_MAP_LINEAR_N, 1, L.GEMM_SCHED_PERSISTENT, 8,
                       256)
    assert p1.info.bn == bn and p2.info.sk_tiles > 0
    assert np.array_equal(C1, ref) and np.array_equal(C2, ref) and np.array_equal(C3, ref)


def test_python_gemm_wrapper_tiles_and_groups(dev):
    """dg.gemm(): (bm, bn) tiles and Stream-K groups reach the plan; results within tolerance."""
    import dense_gemm_design_amd as dg
    op = gi.make_operands(512, 896, 8192, "bf16", seed=41)
    A, B, _, _ = to_device(op, torch, dev)
    ref = reference(op)
    C = dg.gemm(A, B, out_dtype="f32", mapping="linear_n", group=1, sched="persistent",
                tile=(256, 224))
    torch.cuda.synchronize()
    assert_within_tolerance(C.cpu().numpy().astype(np.float64), ref, op, "gemm() 256 x 224")
    C = dg.gemm(A, B, out_dtype="f32", mapping="linear_n", group=1, sched="streamk", tile=128,
                sk_groups=4)
    torch.cuda.synchronize()
    assert_within_tolerance(C.cpu().numpy().astype(np.float64), ref, op, "gemm() Stream-K groups")
