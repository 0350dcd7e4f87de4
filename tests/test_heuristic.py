"""The planner's kernel-configuration heuristic (gemm_rank_configs): the cost model of "DeepGEMM
on SM90" (section "Kernel Configuration Heuristic") re-fitted to gfx950.  CPU tests check the
model's arithmetic and its choices on the workloads whose best configuration was measured; the
GPU test times every candidate the model ranks and checks that its pick is close to the fastest."""
import math
import os
import sys
import time

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from dense_gemm_design_amd import _lib as L  # noqa: E402

P = 256


def desc(M, N, K, dt=L.GEMM_BF16, out=L.GEMM_BF16, mapping=L.GEMM_MAP_GROUPED_M, group=0, P=P):
    return L.make_desc(M, N, K, dt, out, mapping, group, L.GEMM_SCHED_AUTO, P)


def test_scores_are_the_models_formula():
    for d in (desc(4096, 4096, 4096), desc(4096, 14336, 4096), desc(512, 512, 65536, out=L.GEMM_F32),
              desc(8192, 8192, 8192, dt=L.GEMM_FP8_E4M3)):
        ranked = L.rank_configs(d)
        assert ranked, "at least one feasible candidate"
        assert [c.score for c in ranked] == sorted(c.score for c in ranked)
        for c in ranked:
            worst = max(c.cycles_mfma, c.cycles_l2, c.cycles_local)
            factor = 1.03 if c.sched == L.GEMM_SCHED_STREAMK else 1.0
            assert c.score == pytest.approx((worst / c.wave_efficiency + c.cycles_fixed) * factor,
                                            rel=1e-12)
            assert c.cycles_fixed > 0
            assert 0 < c.wave_efficiency <= 1


def test_wave_efficiency_of_a_partial_last_wave():
    # 4096 x 14336 on 256 x 256 tiles: 16 x 56 = 896 tiles, 3.5 waves of 256; the half-busy last
    # wave runs at a higher clock (power limit) and costs max(0.5^0.39, 1/1.3) of a full one
    ranked = L.rank_configs(desc(4096, 14336, 4096))
    dp = [c for c in ranked if (c.bm, c.bn) == (256, 256) and c.sched == L.GEMM_SCHED_PERSISTENT][0]
    assert dp.wave_efficiency == pytest.approx(3.5 / (3 + max(0.5 ** 0.39, 1 / 1.3)))
    # 3072 x 3072 on 256 x 256 tiles: 144 tiles, one wave with 56 % of the CUs busy
    d256 = [c for c in L.rank_configs(desc(3072, 3072, 4096))
            if (c.bm, c.bn) == (256, 256) and c.sched == L.GEMM_SCHED_PERSISTENT][0]
    assert d256.wave_efficiency == pytest.approx((144 / 256) / (144 / 256) ** 0.39)
    # one partial wave of the narrower tiles gains less from the headroom: f^0.2 (256 x 192: 12 x 16
    # = 192 tiles; 256 x 224: 12 x 14 = 168), while their partial last waves of longer launches
    # keep f^0.39 (4096 x 14336 on 256 x 192: 16 x 75 = 1200 tiles, 4.6875 waves)
    one = L.rank_configs(desc(3072, 3072, 4096))
    d192 = [c for c in one if (c.bm, c.bn) == (256, 192)][0]
    assert d192.wave_efficiency == pytest.approx(0.75 / 0.75 ** 0.2)
    d224s = [c for c in one if (c.bm, c.bn) == (256, 224)][0]
    assert d224s.wave_efficiency == pytest.approx((168 / 256) / (168 / 256) ** 0.2)
    m192 = [c for c in ranked if (c.bm, c.bn) == (256, 192)][0]
    assert m192.wave_efficiency == pytest.approx(4.6875 / (4 + max(0.6875 ** 0.39, 1 / 1.3)))
    # a nearly empty wave costs no less than the clock headroom allows (1 / 1.3 of a full one):
    # 512 x 512 on 128 x 128 tiles is 16 tiles on 256 CUs
    small = [c for c in L.rank_configs(desc(512, 512, 65536, out=L.GEMM_F32))
             if c.bm == 128 and c.sched == L.GEMM_SCHED_PERSISTENT][0]
    assert small.wave_efficiency == pytest.approx((16 / 256) * 1.3)
    # 256 x 224 tiles: 16 x 64 = 1024 tiles, four whole waves
    d224 = [c for c in ranked if (c.bm, c.bn) == (256, 224)][0]
    assert d224.wave_efficiency == pytest.approx(1.0)
    # the cooperative 128 x 128 candidate has 3584 tiles = 14 whole waves
    c128 = [c for c in ranked if c.bm == 128 and c.sched == L.GEMM_SCHED_PERSISTENT][0]
    assert c128.wave_efficiency == pytest.approx(1.0)


def test_data_movement_terms():
    # bf16 4096^3, 256 x 256 wide-wave: per tile K (BM + BN) 2 bytes of A/B plus BM BN 2 of C
    # through L2, at 57 B/clk/CU on 256 CUs
    c = [c for c in L.rank_configs(desc(4096, 4096, 4096)) if c.kernel == 3][0]
    tiles = 16 * 16
    l2_bytes = tiles * (4096 * 512 * 2 + 256 * 256 * 2)
    assert c.cycles_l2 == pytest.approx(l2_bytes / (P * 57.0))
    # LDS: fills plus fragment reads (each A row read by 2 waves, each B row by 2) plus C staging
    lds_bytes = tiles * (4096 * 512 * 2 + 4096 * (256 * 2 + 256 * 2) * 2 + 256 * 256 * 2)
    assert c.cycles_local == pytest.approx(lds_bytes / (P * 256.0))
    # MFMA: 2 M N K / (4096 FLOP per clock per CU x 256 CUs x the kernel's measured efficiency)
    eff = 2 * 4096 ** 3 / (P * 4096.0) / c.cycles_mfma
    assert 0.5 < eff < 1.0


@pytest.mark.parametrize("shape,dt,out,want", [
    ((4096, 4096, 4096), L.GEMM_BF16, L.GEMM_BF16, (256, 3, L.GEMM_SCHED_PERSISTENT)),
    ((8192, 8192, 8192), L.GEMM_FP8_E4M3, L.GEMM_BF16, (256, 3, L.GEMM_SCHED_PERSISTENT)),
    # 896 tiles of 256 x 256 = 3.5 waves; 256 x 224 tiles fill four whole waves (measured 4 %
    # faster than 256 x 256, with or without a Stream-K tail)
    ((4096, 14336, 4096), L.GEMM_BF16, L.GEMM_BF16, ((256, 224), 3, L.GEMM_SCHED_PERSISTENT)),
    ((4096, 14336, 4096), L.GEMM_FP8_E4M3, L.GEMM_BF16, ((256, 224), 3, L.GEMM_SCHED_PERSISTENT)),
    # 1792 tiles of 256 x 256 = 7 whole waves: the wider tile stays
    ((8192, 14336, 4096), L.GEMM_BF16, L.GEMM_BF16, ((256, 256), 3, L.GEMM_SCHED_PERSISTENT)),
    # one partial wave of big tiles (192 of 256 CUs, at a higher clock) beats 128 x 128 tiles
    # with a Stream-K tail (measured 69 against 83 us); of the big tiles 256 x 192 measured
    # fastest (65.0 us, 256 x 224 70.9, 256 x 256 83.4)
    ((3072, 3072, 4096), L.GEMM_BF16, L.GEMM_BF16, ((256, 192), 3, L.GEMM_SCHED_PERSISTENT)),
    # N a multiple of 6,144: 256 x 192 tiles fill whole waves (measured 148.6 against 161.5 us
    # for 256 x 224 and 181.7 for 256 x 256 in bf16, 79.6 / 85.3 / 98.2 in e4m3; 6144^2 x 4096
    # bf16 219.0 / 239.5 / 266.6)
    ((4096, 6144, 4096), L.GEMM_BF16, L.GEMM_BF16, ((256, 192), 3, L.GEMM_SCHED_PERSISTENT)),
    ((4096, 6144, 4096), L.GEMM_FP8_E4M3, L.GEMM_BF16, ((256, 192), 3, L.GEMM_SCHED_PERSISTENT)),
    ((6144, 6144, 4096), L.GEMM_BF16, L.GEMM_BF16, ((256, 192), 3, L.GEMM_SCHED_PERSISTENT)),
    # 344 tiles of 256 x 256 (1.34 waves): the Stream-K tail measured no faster than the plain
    # second wave (324 against 328 us); 256 x 192 tiles (1.81 waves) measured 268 us
    ((2048, 11008, 8192), L.GEMM_BF16, L.GEMM_BF16, ((256, 192), 3, L.GEMM_SCHED_PERSISTENT)),
    # 1.34 waves of 256 x 256 in e4m3: data-parallel 504 us, with the Stream-K tail 546
    ((8192, 11008, 8192), L.GEMM_FP8_E4M3, L.GEMM_BF16, ((256, 256), 3, L.GEMM_SCHED_PERSISTENT)),
    # one partial wave (0.67) of 256 x 192 tiles against two whole waves of 128 x 128 tiles: the
    # latter measured 63 against 72 us
    ((1024, 8192, 4096), L.GEMM_BF16, L.GEMM_BF16, (128, 3, L.GEMM_SCHED_PERSISTENT)),
    # a band of 2 k-steps per unit: data-parallel 128 x 128 tiles measured 19 against 29 us (bf16
    # 256 x 256 x 4096, one k-step per unit on 64-step tiles, keeps Stream-K: 25 against 29; the
    # timed test checks it, with the device's own occupancy for the cooperative candidates)
    ((512, 512, 4096), L.GEMM_FP8_E4M3, L.GEMM_BF16, (128, 3, L.GEMM_SCHED_PERSISTENT)),
    ((512, 512, 65536), L.GEMM_BF16, L.GEMM_F32, (128, 3, L.GEMM_SCHED_STREAMK)),
    ((256, 256, 256), L.GEMM_BF16, L.GEMM_F32, (128, 3, L.GEMM_SCHED_PERSISTENT)),
])
def test_choices_on_measured_workloads(shape, dt, out, want):
    d = desc(*shape, dt=dt, out=out)
    best = L.rank_configs(d)[0]
    bm, kernel, sched = want
    assert (best.kernel, best.sched) == (kernel, sched)
    if isinstance(bm, tuple):
        assert (best.bm, best.bn) == bm
    elif bm is not None:
        assert best.bm == bm
    # gemm_create with everything left to the planner takes the best candidate
    info = L.Plan(d).info
    assert (info.bm, info.bn, info.kernel, info.sched) == (best.bm, best.bn, best.kernel, best.sched)


def test_stream_k_fixup_costs():
    # a band of few k-steps per unit pays for the burst of partials: 20,000 clocks at one k-step,
    # falling linearly to none at 16 (16 tiles x 32 k-steps of e4m3 over 256 units: 2 each, so
    # 17,500); the separate reduction's traffic comes on top
    ranked = L.rank_configs(desc(512, 512, 4096, dt=L.GEMM_FP8_E4M3))
    assert ranked[0].sched == L.GEMM_SCHED_PERSISTENT
    sk = [c for c in ranked if c.sched == L.GEMM_SCHED_STREAMK and c.kernel == 3][0]
    traffic = 2.0 * 16 * 16 * 128 * 128 * 4 / 2600 + 2000
    assert sk.cycles_fixed >= 17500 + traffic
    # 64 k-steps per unit (512 x 512 x 65536): no burst term
    sk64 = [c for c in L.rank_configs(desc(512, 512, 65536, out=L.GEMM_F32))
            if c.sched == L.GEMM_SCHED_STREAMK and c.kernel == 3 and c.bm == 128][0]
    assert sk64.cycles_fixed < 17500 + traffic
    # the lock chain: a tile's non-empty splits hand the lock on one after another, each hop
    # 13,000 clocks plus the tile's partial read and written at 96 B/clk (16 tiles, 256 units:
    # 16 splits per tile)
    d = L.make_desc(512, 512, 65536, L.GEMM_BF16, L.GEMM_F32, L.GEMM_MAP_GROUPED_M, 0,
                    L.GEMM_SCHED_AUTO, P, flags=L.GEMM_FLAG_STREAMK_CHAIN)
    sk = [c for c in L.rank_configs(d) if c.sched == L.GEMM_SCHED_STREAMK and c.bm == 128]
    assert sk and all(c.kernel == 0 for c in sk)  # the wide-wave kernel has no chain
    assert sk[0].cycles_fixed >= 16 * (13000 + 2 * 128 * 128 * 4 / 96)


def test_zero_depth_keeps_to_the_kernel_that_runs_it():
    ranked = L.rank_configs(desc(512, 512, 0, out=L.GEMM_F32))
    assert ranked and all(c.kernel == 0 for c in ranked)


def test_group_choice_minimises_operand_strips():
    # each XCD runs 32 consecutive tiles: G x 32/G block -> G + 32/G strips, least at G = 4 or 8;
    # the larger wins the tie
    info = L.Plan(desc(4096, 4096, 4096)).info
    assert info.group == 8
    assert L.rank_configs(desc(4096, 4096, 4096))[0].group == 8
    # few tile rows: G never exceeds them
    few = L.Plan(desc(512, 8192, 4096)).info
    assert few.group <= few.mt
    # an explicit G is kept
    assert L.Plan(desc(4096, 4096, 4096, group=16)).info.group == 16
    for G in (1, 2, 4, 8, 16, 32):
        strips = min(G, 16) + math.ceil(32 / min(G, 16))
        assert strips >= 12


def test_rank_validation():
    lib = L.load()
    import ctypes
    n = ctypes.c_size_t()
    assert lib.gemm_rank_configs(None, None, 0, ctypes.byref(n)) == L.GEMM_ERR_INVALID_ARG
    d = desc(4096, 4096, 4096)
    assert lib.gemm_rank_configs(ctypes.byref(d), None, 0, ctypes.byref(n)) == L.GEMM_ERR_CAPACITY
    assert n.value >= 2
    bad = desc(-1, 4, 4)
    assert lib.gemm_rank_configs(ctypes.byref(bad), None, 0, ctypes.byref(n)) == \
        L.GEMM_ERR_INVALID_ARG


@pytest.mark.gpu
@pytest.mark.parametrize("shape,dt,out", [
    ((4096, 4096, 4096), L.GEMM_BF16, L.GEMM_BF16),
    ((4096, 14336, 4096), L.GEMM_BF16, L.GEMM_BF16),
    ((4096, 14336, 4096), L.GEMM_FP8_E4M3, L.GEMM_BF16),
    ((512, 512, 65536), L.GEMM_BF16, L.GEMM_F32),
    ((2048, 2048, 2048), L.GEMM_BF16, L.GEMM_BF16),
    ((1024, 1024, 16384), L.GEMM_FP8_E4M3, L.GEMM_BF16),
    ((8192, 14336, 4096), L.GEMM_BF16, L.GEMM_BF16),
    ((3072, 3072, 4096), L.GEMM_BF16, L.GEMM_BF16),
    ((1280, 1280, 32768), L.GEMM_BF16, L.GEMM_BF16),
    ((6144, 6144, 6144), L.GEMM_FP8_E4M3, L.GEMM_BF16),
    ((4096, 6144, 4096), L.GEMM_BF16, L.GEMM_BF16),
    # from the 184-shape sweep the 256 x 192 efficiency and the Stream-K factor were refit to
    ((2048, 11008, 8192), L.GEMM_BF16, L.GEMM_BF16),
    ((8192, 11008, 8192), L.GEMM_FP8_E4M3, L.GEMM_BF16),
    ((1536, 5120, 6144), L.GEMM_FP8_E4M3, L.GEMM_BF16),
    ((1024, 8192, 4096), L.GEMM_BF16, L.GEMM_BF16),
    ((512, 512, 4096), L.GEMM_FP8_E4M3, L.GEMM_BF16),
    ((256, 256, 4096), L.GEMM_BF16, L.GEMM_BF16),
    # shapes the model's constants were not fitted to
    ((768, 18432, 3072), L.GEMM_BF16, L.GEMM_BF16),
    ((2560, 9216, 5120), L.GEMM_FP8_E4M3, L.GEMM_BF16),
    ((2048, 12288, 4096), L.GEMM_BF16, L.GEMM_BF16),
    ((5120, 5120, 5120), L.GEMM_BF16, L.GEMM_BF16),
    ((4096, 11008, 4096), L.GEMM_BF16, L.GEMM_BF16),
    ((4096, 28672, 8192), L.GEMM_FP8_E4M3, L.GEMM_BF16),
])
def test_pick_is_close_to_the_fastest_candidate(shape, dt, out):
    """Each candidate the model ranks runs as a forced plan; the model's pick must be within 15 %
    of the fastest measured (the model ignores launch and fixup latencies)."""
    import torch
    dev = torch.device("cuda:0")
    M, N, K = shape
    # operands like the workloads' (uniform[-1, 1] bf16, or N(0, 1) e4m3): the clock the board
    # holds, and so the time, depends on the data
    gen = torch.Generator(device=dev)
    gen.manual_seed(1)
    if dt == L.GEMM_BF16:
        A = (torch.rand((M, K), device=dev, generator=gen) * 2 - 1).to(torch.bfloat16)
        B = (torch.rand((N, K), device=dev, generator=gen) * 2 - 1).to(torch.bfloat16)
    else:
        A = torch.randn((M, K), device=dev, generator=gen).to(torch.float8_e4m3fn).view(torch.uint8)
        B = torch.randn((N, K), device=dev, generator=gen).to(torch.float8_e4m3fn).view(torch.uint8)
    C = torch.empty((M, N), dtype=torch.bfloat16 if out == L.GEMM_BF16 else torch.float32,
                    device=dev)
    sa = torch.ones(1, dtype=torch.float32, device=dev)
    d = L.make_desc(M, N, K, dt, out, L.GEMM_MAP_GROUPED_M, 0, L.GEMM_SCHED_AUTO, 0)
    ranked = L.rank_configs(d)
    times = []
    for c in ranked:
        flags = L.GEMM_FLAG_COOPERATIVE if c.kernel == 0 else 0
        plan = L.Plan(L.make_desc(M, N, K, dt, out, L.GEMM_MAP_GROUPED_M, c.group, c.sched, 0,
                                  c.bm, c.bn, c.bk, flags))
        ws = torch.empty(max(plan.workspace_bytes, 1), dtype=torch.uint8, device=dev)
        run = lambda: plan.run(A, B, C, sa, sa, ws if plan.workspace_bytes else None)
        # the clock climbs for a few hundred ms under load: settle, then take the better of two
        # timed batches
        t0 = time.time()
        while time.time() - t0 < 0.5:
            run()
            torch.cuda.synchronize()
        best = float("inf")
        for _ in range(2):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(20):
                run()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) / 20)
        times.append(best)
    print(f"{shape}: " + ", ".join(f"{c.bm}x{c.bn}/{c.kernel}/{c.sched}: {t * 1e3:.1f} us"
                                   for c, t in zip(ranked, times)), flush=True)
    assert times[0] <= 1.15 * min(times), "the model's pick is much slower than the fastest"
