"""The library's schedule (gemm_schedule_enumerate, the same code the kernel runs) matches the
oracle's independent CPU enumeration bit for bit."""
import pytest

from dense_gemm_design_amd import _lib as L
from oracle import schedule as S

MAP = {L.GEMM_MAP_LINEAR_N: S.LINEAR_N, L.GEMM_MAP_LINEAR_M: S.LINEAR_M,
       L.GEMM_MAP_GROUPED_M: S.GROUPED_M, L.GEMM_MAP_GROUPED_N: S.GROUPED_N,
       L.GEMM_MAP_BLOCKED: S.BLOCKED, L.GEMM_MAP_MORTON: S.MORTON}
SCHED = {L.GEMM_SCHED_STATIC: S.STATIC, L.GEMM_SCHED_PERSISTENT: S.PERSISTENT,
         L.GEMM_SCHED_STREAMK: S.STREAMK}

CASES = [
    # M, N, K, dtype, tile, mapping, G, sched, P, remap
    (256, 256, 256, L.GEMM_BF16, 128, L.GEMM_MAP_LINEAR_N, 1, L.GEMM_SCHED_STATIC, 0, True),
    (4096, 4096, 4096, L.GEMM_BF16, 128, L.GEMM_MAP_LINEAR_N, 1, L.GEMM_SCHED_PERSISTENT, 256, True),
    (4096, 4096, 4096, L.GEMM_BF16, 128, L.GEMM_MAP_GROUPED_M, 8, L.GEMM_SCHED_PERSISTENT, 256, True),
    (4096, 4096, 4096, L.GEMM_BF16, 256, L.GEMM_MAP_GROUPED_M, 8, L.GEMM_SCHED_PERSISTENT, 256, True),
    (4096, 14336, 4096, L.GEMM_BF16, 256, L.GEMM_MAP_GROUPED_M, 8, L.GEMM_SCHED_PERSISTENT, 256, True),
    (8192, 8192, 8192, L.GEMM_FP8_E4M3, 256, L.GEMM_MAP_GROUPED_M, 16, L.GEMM_SCHED_PERSISTENT, 256, True),
    (512, 512, 65536, L.GEMM_BF16, 128, L.GEMM_MAP_LINEAR_N, 1, L.GEMM_SCHED_STREAMK, 256, True),
    (1000, 1000, 512, L.GEMM_BF16, 128, L.GEMM_MAP_GROUPED_N, 3, L.GEMM_SCHED_PERSISTENT, 24, True),
    (1000, 1000, 512, L.GEMM_BF16, 128, L.GEMM_MAP_LINEAR_M, 1, L.GEMM_SCHED_STATIC, 0, False),
    (1280, 640, 1024, L.GEMM_BF16, 128, L.GEMM_MAP_GROUPED_M, 4, L.GEMM_SCHED_STREAMK, 40, True),
    (1280, 640, 1024, L.GEMM_BF16, 128, L.GEMM_MAP_GROUPED_M, 4, L.GEMM_SCHED_STREAMK, 40, False),
    (384, 256, 448, L.GEMM_BF16, 128, L.GEMM_MAP_LINEAR_N, 1, L.GEMM_SCHED_STREAMK, 5, True),
    (300, 264, 104, L.GEMM_BF16, 128, L.GEMM_MAP_GROUPED_M, 2, L.GEMM_SCHED_STREAMK, 3, True),
    (2048, 2048, 2048, L.GEMM_FP8_E4M3, 128, L.GEMM_MAP_GROUPED_N, 8, L.GEMM_SCHED_STREAMK, 300, True),
    # 2D blocking (G = box height, the box width in the last field) and Morton
    (8192, 8192, 8192, L.GEMM_FP8_E4M3, 256, L.GEMM_MAP_BLOCKED, 4, L.GEMM_SCHED_PERSISTENT, 256, True, 8),
    (4096, 14336, 4096, L.GEMM_BF16, 256, L.GEMM_MAP_BLOCKED, 4, L.GEMM_SCHED_PERSISTENT, 256, True, 8),
    (1000, 3000, 512, L.GEMM_BF16, 128, L.GEMM_MAP_BLOCKED, 3, L.GEMM_SCHED_PERSISTENT, 24, True, 5),
    (1000, 3000, 512, L.GEMM_BF16, 128, L.GEMM_MAP_BLOCKED, 3, L.GEMM_SCHED_STATIC, 0, True, 5),
    (1280, 640, 1024, L.GEMM_BF16, 128, L.GEMM_MAP_BLOCKED, 2, L.GEMM_SCHED_STREAMK, 40, True, 3),
    (4096, 4096, 4096, L.GEMM_BF16, 256, L.GEMM_MAP_MORTON, 1, L.GEMM_SCHED_PERSISTENT, 256, True),
    (1000, 3000, 512, L.GEMM_BF16, 128, L.GEMM_MAP_MORTON, 1, L.GEMM_SCHED_PERSISTENT, 24, True),
    (4096, 14336, 4096, L.GEMM_BF16, 256, L.GEMM_MAP_MORTON, 1, L.GEMM_SCHED_STATIC, 0, True),
    (1280, 640, 1024, L.GEMM_BF16, 128, L.GEMM_MAP_MORTON, 1, L.GEMM_SCHED_STREAMK, 40, True),
    # XCD box remap: waves that are whole G x P/G blocks of one strip (G = 8, P = 64: 2 x 4
    # boxes per XCD instead of 8 x 1 columns); the fp8 8192^3 case above takes 4 x 8 boxes
    (4096, 2048, 256, L.GEMM_BF16, 256, L.GEMM_MAP_GROUPED_M, 8, L.GEMM_SCHED_PERSISTENT, 64, True),
    (2048, 4096, 256, L.GEMM_BF16, 256, L.GEMM_MAP_GROUPED_N, 8, L.GEMM_SCHED_PERSISTENT, 64, True),
    (4096, 2048, 256, L.GEMM_BF16, 256, L.GEMM_MAP_GROUPED_M, 8, L.GEMM_SCHED_PERSISTENT, 64, False),
    # grouped plans whose waves span several strips (keep the contiguous runs): two strips of
    # 8 x 4 tiles per wave of 64, and a Stream-K wave of four 2 x 5 strips
    (2048, 512, 256, L.GEMM_BF16, 128, L.GEMM_MAP_GROUPED_M, 8, L.GEMM_SCHED_PERSISTENT, 64, True),
    (512, 2048, 256, L.GEMM_BF16, 128, L.GEMM_MAP_GROUPED_N, 8, L.GEMM_SCHED_PERSISTENT, 64, True),
    (1280, 640, 2048, L.GEMM_BF16, 128, L.GEMM_MAP_GROUPED_M, 2, L.GEMM_SCHED_STREAMK, 40, True),
]


@pytest.mark.parametrize("mapping", [L.GEMM_MAP_GROUPED_M, L.GEMM_MAP_GROUPED_N])
def test_grouped_remap_sweep_matches_oracle(mapping):
    """Every small grouped plan (tile grids up to 16 x 16, G up to 8, waves of 8 to 128 workers,
    persistent and Stream-K) enumerates exactly the oracle's schedule, whichever remap applies."""
    n_box = 0
    for mt in (2, 4, 6, 8, 16):
        for nt in (2, 4, 5, 8, 16):
            for G in (1, 2, 3, 4, 8):
                for P in (8, 16, 24, 40, 64, 128):
                    for sched in (L.GEMM_SCHED_PERSISTENT, L.GEMM_SCHED_STREAMK):
                        M, N = mt * 128, nt * 128
                        plan = L.Plan(L.make_desc(M, N, 512, mapping=mapping, group=G,
                                                  sched=sched, num_workers=P, bm=128, bn=128))
                        info = plan.info
                        n_box += info.xcd_box_r > 0
                        want = S.enumerate_schedule(M, N, 512, 128, 128, info.bk, MAP[mapping],
                                                    G, SCHED[sched], P=info.grid,
                                                    sk_groups=info.sk_groups)
                        assert plan.schedule() == [
                            (w.worker, w.seq, w.tile, w.m, w.n, w.k_begin, w.k_end, w.role)
                            for w in want], (mt, nt, G, P, sched)
    assert n_box > 0


@pytest.mark.parametrize("case", CASES)
def test_enumeration_matches_oracle(case):
    M, N, K, dt, tile, mapping, G, sched, P, remap = case[:10]
    W = case[10] if len(case) > 10 else 0
    flags = 0 if remap else L.GEMM_FLAG_NO_XCD_REMAP
    plan = L.Plan(L.make_desc(M, N, K, dtype_ab=dt, mapping=mapping, group=G, sched=sched,
                              num_workers=P, bm=tile, bn=tile, flags=flags, group_n=W))
    if mapping == L.GEMM_MAP_BLOCKED:
        assert (plan.info.group, plan.info.group_n) == (G, W)
    got = plan.schedule()
    bk = plan.info.bk
    Pw = plan.info.grid if sched != L.GEMM_SCHED_STATIC else None
    want = S.enumerate_schedule(M, N, K, tile, tile, bk, MAP[mapping], G, SCHED[sched],
                                P=P if sched != L.GEMM_SCHED_STATIC else None,
                                xcd_remap=remap, W=max(W, 1), sk_groups=plan.info.sk_groups)
    want = [(w.worker, w.seq, w.tile, w.m, w.n, w.k_begin, w.k_end, w.role) for w in want]
    if sched == L.GEMM_SCHED_PERSISTENT:
        # the planner caps P at the tile count; the oracle is asked with the same P
        want = [(w.worker, w.seq, w.tile, w.m, w.n, w.k_begin, w.k_end, w.role) for w in
                S.enumerate_schedule(M, N, K, tile, tile, bk, MAP[mapping], G, SCHED[sched],
                                     P=Pw, xcd_remap=remap, W=max(W, 1),
                                     sk_groups=plan.info.sk_groups)]
    assert got == want


def test_enumerate_capacity_reporting():
    plan = L.Plan(L.make_desc(1024, 1024, 1024, sched=L.GEMM_SCHED_PERSISTENT, num_workers=7,
                              bm=128, bn=128))
    import ctypes
    lib = L.load()
    n = ctypes.c_size_t()
    arr = (L.GemmWorkItem * 3)()
    assert lib.gemm_schedule_enumerate(plan.handle, arr, 3, ctypes.byref(n)) == L.GEMM_ERR_CAPACITY
    assert n.value == 64
    assert (arr[0].worker, arr[0].seq) == (0, 0)


def test_blocked_planner_box():
    """group = group_n = 0: the planner fills a box with the tiles one XCD runs at a time
    (P / 8), choosing the fewest operand strips H + W, the wider box on a tie; one given side
    fixes the other."""
    def box(M, N, P, G=0, W=0):
        p = L.Plan(L.make_desc(M, N, 4096, mapping=L.GEMM_MAP_BLOCKED, group=G, group_n=W,
                               sched=L.GEMM_SCHED_PERSISTENT, num_workers=P, bm=256, bn=256))
        return p.info.group, p.info.group_n
    assert box(8192, 8192, 256) == (4, 8)            # 32 tiles per XCD: 4 + 8 strips
    assert box(4096, 14336, 256) == (4, 8)
    assert box(8192, 8192, 256, G=2) == (2, 16)
    assert box(8192, 8192, 256, W=2) == (16, 2)
    assert box(512, 8192, 256) == (2, 4)             # 64 tiles: P = 64, 8 per XCD
    # Morton and the linear mappings report 1 x 1
    p = L.Plan(L.make_desc(1024, 1024, 1024, mapping=L.GEMM_MAP_MORTON, num_workers=8, bm=128,
                           bn=128))
    assert (p.info.group, p.info.group_n) == (1, 1)


SK_GROUP_CASES = [
    # M, N, K, dtype, tile, mapping, G (mapping), P, requested groups, planned groups
    (512, 512, 65536, L.GEMM_BF16, 128, L.GEMM_MAP_LINEAR_N, 1, 256, 4, 4),
    (512, 512, 65536, L.GEMM_BF16, 128, L.GEMM_MAP_LINEAR_N, 1, 256, 8, 8),
    (3072, 3072, 4096, L.GEMM_BF16, 128, L.GEMM_MAP_GROUPED_M, 8, 256, 8, 8),
    (3072, 3072, 4096, L.GEMM_BF16, 256, L.GEMM_MAP_LINEAR_N, 1, 64, 8, 8),
    (1280, 640, 1024, L.GEMM_BF16, 128, L.GEMM_MAP_GROUPED_M, 4, 40, 8, 8),
    (1280, 640, 1024, L.GEMM_BF16, 128, L.GEMM_MAP_GROUPED_M, 4, 40, 7, 5),   # 7, 6 do not divide 40
    (1280, 640, 1024, L.GEMM_BF16, 128, L.GEMM_MAP_GROUPED_M, 4, 40, 3, 2),
    (384, 256, 448, L.GEMM_BF16, 128, L.GEMM_MAP_LINEAR_N, 1, 5, 4, 1),       # a band of 1 tile
    (2048, 2048, 2048, L.GEMM_FP8_E4M3, 128, L.GEMM_MAP_GROUPED_N, 8, 768, 6, 6),
    (1280, 640, 1024, L.GEMM_BF16, 128, L.GEMM_MAP_BLOCKED, 2, 40, 4, 4),
]


@pytest.mark.parametrize("case", SK_GROUP_CASES)
def test_streamk_groups_enumeration_matches_oracle(case):
    """Stream-K groups: the planned count follows the lowering rule (largest count <= the request
    that divides P and leaves every group a tile), and the schedule equals the oracle's."""
    M, N, K, dt, tile, mapping, G, P, req, planned = case
    W = 3 if mapping == L.GEMM_MAP_BLOCKED else 0
    plan = L.Plan(L.make_desc(M, N, K, dtype_ab=dt, mapping=mapping, group=G,
                              sched=L.GEMM_SCHED_STREAMK, num_workers=P, bm=tile, bn=tile,
                              group_n=W, sk_groups=req))
    info = plan.info
    assert info.sk_tiles > 0 and info.sk_groups == planned
    want = S.enumerate_schedule(M, N, K, tile, tile, info.bk, MAP[mapping], G, S.STREAMK,
                                P=info.grid, W=max(W, 1), sk_groups=planned)
    assert plan.schedule() == [(w.worker, w.seq, w.tile, w.m, w.n, w.k_begin, w.k_end, w.role)
                               for w in want]


def test_streamk_groups_validation_and_reporting():
    lib = L.load()
    import ctypes
    h = ctypes.c_void_p()
    for bad in (-1, 9):
        d = L.make_desc(512, 512, 65536, sched=L.GEMM_SCHED_STREAMK, num_workers=256, bm=128,
                        bn=128, sk_groups=bad)
        assert lib.gemm_create(ctypes.byref(d), ctypes.byref(h)) == L.GEMM_ERR_INVALID_ARG
    # no band: reported as one group, whatever was asked
    p = L.Plan(L.make_desc(1024, 1024, 1024, sched=L.GEMM_SCHED_PERSISTENT, num_workers=8,
                           bm=128, bn=128, sk_groups=4))
    assert p.info.sk_groups == 1
    p = L.Plan(L.make_desc(512, 512, 65536, sched=L.GEMM_SCHED_STREAMK, num_workers=256, bm=128,
                           bn=128, sk_groups=1))
    assert p.info.sk_groups == 1


def test_streamk_groups_planner_choice():
    """sk_groups = 0: the largest count up to 8 that divides P, leaves P / G a multiple of the 8
    XCDs, gives every group a tile, and keeps the fixup mode one pool would have."""
    def planned(M, N, K, P, tile=128):
        i = L.Plan(L.make_desc(M, N, K, sched=L.GEMM_SCHED_STREAMK, num_workers=P, bm=tile,
                               bn=tile)).info
        return i.sk_tiles, i.sk_groups, i.streamk_mode
    assert planned(512, 512, 65536, 256) == (16, 8, 1)
    assert planned(1280, 1280, 32768, 256) == (100, 8, 1)
    assert planned(1280, 640, 1024, 40) == (10, 5, 1)           # 40 / 8 = 5 units: not on one XCD
    assert planned(768, 1280, 4096, 12, 256) == (3, 1, 1)       # 12 / 3 = 4 units
    # 12 band tiles of 22 k-tiles on 256 units: 8 groups would leave groups of one tile (22
    # iterations) for 32 units -> the chain; 4 groups (3 tiles, 66 iterations, 64 units) do not
    assert planned(512, 67 * 128, 22 * 64, 256) == (12, 4, 1)
    # no XCD-compatible count at all
    assert planned(1280, 640, 1024, 36)[1] == 1


def test_streamk_groups_fixup_mode_and_workspace():
    """The separate reduction needs every unit of every group to own an iteration; the partial
    area holds G (P/G + ceil(sk_tiles/G)) tiles."""
    d = dict(sched=L.GEMM_SCHED_STREAMK, num_workers=256, bm=128, bn=128)
    one = L.Plan(L.make_desc(512, 512, 65536, sk_groups=1, **d)).info
    eight = L.Plan(L.make_desc(512, 512, 65536, sk_groups=8, **d)).info
    assert one.streamk_mode == eight.streamk_mode == 1
    slot = 128 * 128 * 4
    assert eight.workspace_bytes - one.workspace_bytes == (8 * (32 + 2) - (256 + 16)) * slot
    # 10 band tiles of 4 k-tiles over 40 units: one pool gives every unit an iteration; in 8
    # groups of 5 units the smallest group has one tile (4 iterations) -> the lock chain
    d = dict(sched=L.GEMM_SCHED_STREAMK, num_workers=40, bm=128, bn=128,
             mapping=L.GEMM_MAP_GROUPED_M, group=4)
    p1 = L.Plan(L.make_desc(1280, 640, 256, sk_groups=1, **d)).info
    p8 = L.Plan(L.make_desc(1280, 640, 256, sk_groups=8, **d)).info
    assert p1.sk_tiles == p8.sk_tiles == 10 and p8.sk_groups == 8
    assert p1.streamk_mode == 1 and p8.streamk_mode == 0


@pytest.mark.parametrize("M,N,K,dt,G,P,sched,box", [
    # 16 x 2 runs -> 4 x 8 boxes
    (8192, 8192, 8192, L.GEMM_FP8_E4M3, 16, 256, L.GEMM_SCHED_PERSISTENT, (4, 8)),
    (4096, 2048, 256, L.GEMM_BF16, 8, 64, L.GEMM_SCHED_PERSISTENT, (2, 4)),
    # 256 x 256 tiles: 16 x 56, strips of 448 tasks are no multiple of the 256-task wave
    (4096, 14336, 4096, L.GEMM_BF16, 8, 256, L.GEMM_SCHED_PERSISTENT, (0, 0)),
    # 256 x 224 tiles: 16 x 64; runs of 32 are 8 x 4 slabs, no box needs fewer strips
    (4096, 14336, 4096, L.GEMM_BF16, 8, 256, L.GEMM_SCHED_AUTO, (0, 0)),
    # a wave spans two strips
    (4096, 4096, 4096, L.GEMM_BF16, 8, 256, L.GEMM_SCHED_PERSISTENT, (0, 0)),
    # 2 x 20 tiles, Grouped-M(2), 40 workers: runs of 5 tasks are neither a slab nor a column
    (256, 2560, 256, L.GEMM_BF16, 2, 40, L.GEMM_SCHED_PERSISTENT, (0, 0)),
])
def test_planner_xcd_box(M, N, K, dt, G, P, sched, box):
    """The plan reports the box the oracle's rule picks, and none where it does not apply."""
    bm = 128 if P == 40 else 0
    plan = L.Plan(L.make_desc(M, N, K, dtype_ab=dt, mapping=L.GEMM_MAP_GROUPED_M, group=G,
                              sched=sched, num_workers=P, bm=bm, bn=bm))
    info = plan.info
    assert (info.xcd_box_r, info.xcd_box_c) == box
    ids = S.xcd_box_assignment(S.GROUPED_M, info.mt, info.nt, G, info.grid)
    assert (ids is None) == (box == (0, 0))
    if ids is not None:   # and the planner's first wave is the oracle's
        first = [(w[0], w[2]) for w in plan.schedule() if w[1] == 0]
        assert sorted(first) == list(enumerate(ids))
