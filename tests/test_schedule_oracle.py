"""Pins the oracle's CPU enumeration of the tile mapping, assignment and Stream-K splits to the
pages' worked examples and to invariants that hold for any correct schedule."""
from collections import Counter

import pytest

from oracle import schedule as S
from golden_util import load, ints


def test_streamk_worked_example():
    g = load("streamk_worked_example.txt")
    tiles, kt, units = int(g["tiles"][0]), int(g["k_tiles_per_tile"][0]), int(g["units"][0])
    plan = S.streamk_units(tiles, kt, units)
    for s in g["split"]:
        u, t, k_idx, count, final = ints(s)
        assert (t, k_idx, count, bool(final)) in plan[u]
    u, nsplits = ints(g["unit_split_count"][0])
    assert len(plan[u]) == nsplits


def test_wave_quantization_example():
    g = load("wave_quantization.txt")
    ctas, sms = int(g["ctas"][0]), int(g["num_sms"][0])
    assert -(-ctas // sms) == int(g["waves"][0])
    assert round(100 * S.wave_efficiency(ctas, sms), 1) == float(g["efficiency_percent"][0])


def test_mapping_working_set_example():
    g = load("mapping_working_set.txt")
    mt, nt = ints(g["grid"][0])
    BM, BN, K = int(g["BM"][0]), int(g["BN"][0]), int(g["K"][0])
    esz, conc, G = int(g["bytes_per_element"][0]), int(g["concurrent"][0]), int(g["group"][0])
    first = S.tile_order(S.GROUPED_M, mt, nt, G)[:conc]
    a_bands = {m for m, _ in first}
    b_bands = {n for _, n in first}
    assert len(a_bands) == int(g["unique_a_bands"][0])
    assert len(b_bands) == int(g["unique_b_bands"][0])
    mib = 1 << 20
    a_bytes = len(a_bands) * BM * K * esz
    b_bytes = len(b_bands) * BN * K * esz
    assert a_bytes == int(g["a_mib"][0]) * mib and b_bytes == int(g["b_mib"][0]) * mib
    assert a_bytes + b_bytes == int(g["working_set_mib"][0]) * mib
    # linear N-fast over the same grid touches 1 A band and 8 B bands instead
    lin = S.tile_order(S.LINEAR_N, mt, nt)[:conc]
    assert len({m for m, _ in lin}) == 1 and len({n for _, n in lin}) == 8


@pytest.mark.parametrize("mode", [S.LINEAR_N, S.LINEAR_M, S.GROUPED_M, S.GROUPED_N, S.BLOCKED,
                                  S.MORTON])
@pytest.mark.parametrize("Mt,Nt,G", [(1, 1, 1), (7, 5, 3), (32, 32, 8), (4, 112, 8), (9, 2, 4)])
def test_mapping_is_a_bijection(mode, Mt, Nt, G):
    order = S.tile_order(mode, Mt, Nt, G, W=3)
    assert len(order) == Mt * Nt
    assert set(order) == {(m, n) for m in range(Mt) for n in range(Nt)}


def test_mapping_equivalences_from_table():
    # Grouped-M with G = 1 is Linear N-fast; a strip covering all rows is Linear M-fast
    for Mt, Nt in [(5, 7), (8, 8), (1, 9)]:
        assert S.tile_order(S.GROUPED_M, Mt, Nt, 1) == S.tile_order(S.LINEAR_N, Mt, Nt)
        assert S.tile_order(S.GROUPED_M, Mt, Nt, Mt) == S.tile_order(S.LINEAR_M, Mt, Nt)
        assert S.tile_order(S.GROUPED_N, Mt, Nt, 1) == S.tile_order(S.LINEAR_M, Mt, Nt)
        assert S.tile_order(S.GROUPED_N, Mt, Nt, Nt) == S.tile_order(S.LINEAR_N, Mt, Nt)
        # Grouped-N is Grouped-M of the transposed grid
        for G in (2, 3):
            gn = S.tile_order(S.GROUPED_N, Mt, Nt, G)
            gm_t = [(m, n) for (n, m) in S.tile_order(S.GROUPED_M, Nt, Mt, G)]
            assert gn == gm_t


def test_blocking_working_set_example():
    """The page's working-set example (8 concurrent tiles on a 16 x 16 grid, 6 MiB) with a 4 x 2
    box: the first 8 tiles are one 4 x 2 rectangle, 4 A bands and 2 B bands."""
    g = load("mapping_working_set.txt")
    mt, nt = ints(g["grid"][0])
    BM, BN, K = int(g["BM"][0]), int(g["BN"][0]), int(g["K"][0])
    esz, conc = int(g["bytes_per_element"][0]), int(g["concurrent"][0])
    first = S.tile_order(S.BLOCKED, mt, nt, 4, W=2)[:conc]
    assert set(first) == {(m, n) for m in range(4) for n in range(2)}
    a_bytes = len({m for m, _ in first}) * BM * K * esz
    b_bytes = len({n for _, n in first}) * BN * K * esz
    assert a_bytes + b_bytes == int(g["working_set_mib"][0]) << 20


def test_blocking_equivalences():
    """A box as wide as the grid is a Grouped-M strip; one-row boxes are Linear N-fast; a box of
    all rows and one column is Linear M-fast."""
    for Mt, Nt in [(5, 7), (8, 8), (1, 9), (12, 20)]:
        for G in (1, 2, 3, 4):
            assert S.tile_order(S.BLOCKED, Mt, Nt, G, W=Nt) == S.tile_order(S.GROUPED_M, Mt, Nt, G)
        for W in (1, 2, 5):
            assert S.tile_order(S.BLOCKED, Mt, Nt, 1, W=W) == S.tile_order(S.LINEAR_N, Mt, Nt)
        assert S.tile_order(S.BLOCKED, Mt, Nt, Mt, W=1) == S.tile_order(S.LINEAR_M, Mt, Nt)


def test_blocking_boxes_are_rectangles():
    """Every run of H * W consecutive tiles that starts at a box boundary fills one H x W box,
    and the boxes of a box row follow each other along N; edge boxes hold what is left."""
    Mt, Nt, H, W = 10, 13, 4, 3
    order = S.tile_order(S.BLOCKED, Mt, Nt, H, W=W)
    i = 0
    for r0 in range(0, Mt, H):
        for c0 in range(0, Nt, W):
            h, w = min(H, Mt - r0), min(W, Nt - c0)
            box = order[i:i + h * w]
            assert set(box) == {(m, n) for m in range(r0, r0 + h) for n in range(c0, c0 + w)}
            assert box[:h] == [(m, c0) for m in range(r0, r0 + h)]   # M-fast inside
            i += h * w
    assert i == Mt * Nt


def test_morton_textbook_order():
    """The Z-order curve of a 4 x 4 grid (n in the even bits, m in the odd ones)."""
    z = [(0, 0), (0, 1), (1, 0), (1, 1), (0, 2), (0, 3), (1, 2), (1, 3),
         (2, 0), (2, 1), (3, 0), (3, 1), (2, 2), (2, 3), (3, 2), (3, 3)]
    assert S.tile_order(S.MORTON, 4, 4) == z
    assert [S.morton_code(m, n) for m, n in z] == list(range(16))
    # bit interleaving by hand: m = 0b101, n = 0b011 -> code bits m2 n2 m1 n1 m0 n0 = 100111
    assert S.morton_code(5, 3) == 0b100111


@pytest.mark.parametrize("Mt,Nt", [(3, 5), (7, 2), (16, 56), (1, 6), (9, 9)])
def test_morton_on_a_partial_grid_keeps_the_square_order(Mt, Nt):
    """On a grid that is not a power-of-two square the order is the enclosing square's Z-order
    with the tiles outside the grid left out."""
    side = 1
    while side < max(Mt, Nt):
        side *= 2
    full = S.tile_order(S.MORTON, side, side)
    assert S.tile_order(S.MORTON, Mt, Nt) == [(m, n) for m, n in full if m < Mt and n < Nt]


def test_grouped_m_inside_a_strip_is_m_fast():
    order = S.tile_order(S.GROUPED_M, 10, 3, 4)
    assert order[:5] == [(0, 0), (1, 0), (2, 0), (3, 0), (0, 1)]
    # the short last strip (rows 8, 9) still runs M-fast
    assert order[-4:] == [(8, 1), (9, 1), (8, 2), (9, 2)]


def test_persistent_stride():
    items = S.enumerate_schedule(1024, 1024, 256, 128, 128, 64, S.LINEAR_N, 1, S.PERSISTENT,
                                 P=24, xcd_remap=False)
    by_worker = {}
    for it in items:
        by_worker.setdefault(it.worker, []).append(it.tile)
    for p, tiles in by_worker.items():
        assert tiles == list(range(p, 64, 24))
    assert sorted(t for ts in by_worker.values() for t in ts) == list(range(64))


def test_xcd_remap_contiguous_per_xcd():
    ids = S.xcd_worker_ids(256, 8)
    assert sorted(ids) == list(range(256))
    for x in range(8):
        got = sorted(ids[b] for b in range(256) if b % 8 == x)
        assert got == list(range(32 * x, 32 * x + 32))
    assert S.xcd_worker_ids(100, 8) == list(range(100))


def _coverage(items, Kt):
    cnt = Counter()
    for it in items:
        for k in range(it.k_begin, it.k_end):
            cnt[(it.tile, k)] += 1
    return cnt


@pytest.mark.parametrize("M,N,K,P", [(512, 512, 65536, 256), (512, 384, 4096, 8),
                                     (1024, 1024, 1024, 40), (384, 256, 7 * 64, 5)])
def test_streamk_covers_every_k_tile_once(M, N, K, P):
    BM = BN = 128
    BK = 64
    Mt, Nt, Kt = S.tile_counts(M, N, K, BM, BN, BK)
    items = S.enumerate_schedule(M, N, K, BM, BN, BK, S.LINEAR_N, 1, S.STREAMK, P=P)
    cnt = _coverage(items, Kt)
    assert set(cnt) == {(t, k) for t in range(Mt * Nt) for k in range(Kt)}
    assert set(cnt.values()) == {1}
    # exactly one split per tile ends the tile, and it is the final (or whole-tile) role
    for t in range(Mt * Nt):
        ends = [it for it in items if it.tile == t and it.k_end == Kt]
        assert len(ends) == 1 and ends[0].role in (S.ROLE_WHOLE, S.ROLE_LAST)
        starts = [it for it in items if it.tile == t and it.k_begin == 0]
        assert len(starts) == 1 and starts[0].role in (S.ROLE_WHOLE, S.ROLE_FIRST)


def test_streamk_config_band_shape():
    """512 x 512 x 65536 with 128 x 128 x 64 tiles on 256 workers: 16 tiles, 16 splits each."""
    items = S.enumerate_schedule(512, 512, 65536, 128, 128, 64, S.LINEAR_N, 1, S.STREAMK, P=256)
    assert len(items) == 256
    per_tile = Counter(it.tile for it in items)
    assert set(per_tile.values()) == {16}
    roles = Counter(it.role for it in items)
    assert roles == {S.ROLE_FIRST: 16, S.ROLE_MIDDLE: 224, S.ROLE_LAST: 16}
    assert all(it.k_end - it.k_begin == 64 for it in items)


def test_streamk_fifty_percent_rule():
    assert S.streamk_split_plan(16, 256) == (0, 16)       # tail far below half: Stream-K
    assert S.streamk_split_plan(256 + 100, 256) == (256, 100)
    assert S.streamk_split_plan(256 + 128, 256) == (256, 128)   # exactly half: still Stream-K
    assert S.streamk_split_plan(256 + 129, 256) == (385, 0)     # more than half full: DP
    assert S.streamk_split_plan(512, 256) == (512, 0)           # no tail


def test_streamk_backward_tile_order_and_roles():
    items = S.enumerate_schedule(384, 256, 7 * 64, 128, 128, 64, S.LINEAR_N, 1, S.STREAMK, P=5)
    by_worker = {}
    for it in items:
        by_worker.setdefault(it.worker, []).append(it)
    for its in by_worker.values():
        sk = [it for it in its if it.role != S.ROLE_WHOLE or it.k_end - it.k_begin != 7]
        tiles = [it.tile for it in sk]
        assert tiles == sorted(tiles, reverse=True)
    for it in items:
        first = it.k_begin == 0
        final = it.k_end == 7
        want = {(True, True): S.ROLE_WHOLE, (True, False): S.ROLE_FIRST,
                (False, False): S.ROLE_MIDDLE, (False, True): S.ROLE_LAST}[(first, final)]
        assert it.role == want


# ---- Stream-K groups ("H100 Stream-K" lesson, section 7) -------------------------------------

def test_streamk_groups_hand_example():
    """4 band tiles of 4 k-tiles, 8 units, 2 groups: group 0 holds tiles 0 and 2 and units 0-3,
    group 1 tiles 1 and 3 and units 4-7; each group splits its 8 iterations 2 per unit."""
    plan = S.streamk_units(4, 4, 8, groups=2)
    want = [[(0, 0, 2, False)], [(0, 2, 2, True)], [(2, 0, 2, False)], [(2, 2, 2, True)],
            [(1, 0, 2, False)], [(1, 2, 2, True)], [(3, 0, 2, False)], [(3, 2, 2, True)]]
    assert plan == want


@pytest.mark.parametrize("sk_tiles,Kt,P,G", [(16, 1024, 256, 4), (16, 1024, 256, 8), (5, 7, 6, 2),
                                            (64, 32, 256, 8), (10, 16, 40, 5), (3, 9, 12, 3),
                                            (100, 64, 256, 8), (7, 5, 8, 4)])
def test_streamk_groups_partition_and_interleave(sk_tiles, Kt, P, G):
    """Every (tile, k-tile) of the band is done exactly once; a tile's splits all come from one
    group's units, a contiguous block in K order; band tile j is in group j mod G at position
    j div G (tile id = id in group * G + group index); each group's units share its iterations
    equally (within one)."""
    first = 37
    plan = S.streamk_units(sk_tiles, Kt, P, first_tile=first, groups=G)
    U = P // G
    cnt = Counter()
    owners = {}
    for u, splits in enumerate(plan):
        g = u // U
        for (tile, k_idx, count, final) in splits:
            j = tile - first
            assert 0 <= j < sk_tiles and j % G == g
            assert final == (k_idx + count == Kt)
            for k in range(k_idx, k_idx + count):
                cnt[(j, k)] += 1
            owners.setdefault(j, []).append((k_idx, u))
    assert set(cnt) == {(j, k) for j in range(sk_tiles) for k in range(Kt)}
    assert set(cnt.values()) == {1}
    for j, ks in owners.items():
        ks.sort()
        units = [u for _, u in ks]
        assert units == list(range(units[0], units[0] + len(units)))
    for g in range(G):
        tiles_g = len(range(g, sk_tiles, G))
        work = [sum(c for (_, _, c, _) in plan[u]) for u in range(g * U, (g + 1) * U)]
        assert sum(work) == tiles_g * Kt and max(work) - min(work) <= 1


@pytest.mark.parametrize("sk_tiles,Kt,P,G", [(16, 1024, 256, 4), (64, 32, 256, 8), (6, 7, 9, 3)])
def test_streamk_groups_same_k_range_across_groups(sk_tiles, Kt, P, G):
    """With equal groups, the v-th unit of every group works the same K ranges, on the tiles that
    sit next to each other in the band (the same wave of the data-parallel raster order)."""
    plan = S.streamk_units(sk_tiles, Kt, P, groups=G)
    U = P // G
    for v in range(U):
        base = plan[v]
        for g in range(1, G):
            other = plan[g * U + v]
            assert [(t - g, k, c, f) for (t, k, c, f) in other] == base


def test_streamk_one_group_is_the_single_pool():
    """G = 1 is the plain Stream-K split (the lesson's worked example holds for it)."""
    for args in [(16, 1024, 256), (7, 5, 8), (100, 64, 256)]:
        assert S.streamk_units(*args, groups=1) == S.streamk_units(*args)
    g = load("streamk_worked_example.txt")
    tiles, kt, units = int(g["tiles"][0]), int(g["k_tiles_per_tile"][0]), int(g["units"][0])
    plan = S.streamk_units(tiles, kt, units, groups=1)
    for s in g["split"]:
        u, t, k_idx, count, final = ints(s)
        assert (t, k_idx, count, bool(final)) in plan[u]


def test_streamk_groups_rejected_shapes():
    with pytest.raises(ValueError):
        S.streamk_units(16, 64, 256, groups=3)      # 3 does not divide 256
    with pytest.raises(ValueError):
        S.streamk_units(2, 64, 256, groups=4)       # more groups than band tiles


def test_streamk_groups_in_the_launch_enumeration():
    """enumerate_schedule passes the group count through: 3072^2 on 128 x 128 tiles and 256
    workers leaves a band of 64 tiles after two data-parallel waves; with 8 groups the band's
    tile j is split only among workers 32 (j mod 8) ... 32 (j mod 8) + 31."""
    items = S.enumerate_schedule(3072, 3072, 4096, 128, 128, 64, S.LINEAR_N, 1, S.STREAMK,
                                 P=256, sk_groups=8)
    dp = [it for it in items if it.tile < 512]
    sk = [it for it in items if it.tile >= 512]
    assert all(it.k_begin == 0 and it.k_end == 64 for it in dp) and len(dp) == 512
    for it in sk:
        assert it.worker // 32 == (it.tile - 512) % 8
    assert Counter(it.tile for it in sk) == {t: 4 for t in range(512, 576)}


def test_xcd_box_hand_worked():
    """8 x 8 tiles, Grouped-M(4), 16 workers on 4 XCDs: a wave is the 4 x 4 block of strip 0
    (in-strip task t = column * 4 + row).  Runs of 4 tasks would be 4 x 1 columns (5 strips);
    2 x 2 boxes need 4.  XCD x = b mod 4 takes box (x mod 2, x div 2), its k-th workgroup
    (k = b div 4) the tile at (k mod 2, k div 2) inside it -- worked out by hand."""
    ids = S.xcd_box_assignment(S.GROUPED_M, 8, 8, 4, 16, X=4)
    assert ids == [0, 2, 8, 10, 1, 3, 9, 11, 4, 6, 12, 14, 5, 7, 13, 15]


def test_xcd_box_geometry_fp8_8192():
    """fp8 8192^3 on 256 x 256 tiles, Grouped-M(16), 256 workers: in every wave each XCD's 32
    tiles form a 4 x 8 box (12 operand strips, against 18 for runs of 32 tasks; 8 x 4 ties and
    loses to the wider box), and every task is taken exactly once."""
    Mt = Nt = 32
    items = S.enumerate_schedule(8192, 8192, 8192, 256, 256, 128, S.GROUPED_M, 16, S.PERSISTENT,
                                 P=256)
    assert sorted(w.tile for w in items) == list(range(Mt * Nt))
    for wave in range(4):
        for x in range(8):
            mine = [(w.m, w.n) for w in items if w.worker % 8 == x and w.seq == wave]
            ms, ns = {m for m, _ in mine}, {n for _, n in mine}
            assert len(mine) == 32 and len(ms) == 4 and len(ns) == 8
            assert max(ms) - min(ms) == 3 and max(ns) - min(ns) == 7   # a rectangle
    contiguous = S.enumerate_schedule(8192, 8192, 8192, 256, 256, 128, S.GROUPED_M, 16,
                                      S.PERSISTENT, P=256, xcd_box=False)
    for x in range(8):
        mine = [(w.m, w.n) for w in contiguous if w.worker % 8 == x and w.seq == 0]
        assert len({m for m, _ in mine}) + len({n for _, n in mine}) == 18


def test_xcd_box_not_used_without_gain_or_outside_whole_blocks():
    # runs of 32 tasks under Grouped-M(8) on 16 x 64 tiles are already 8 x 4 (12 strips)
    assert S.xcd_box_assignment(S.GROUPED_M, 16, 64, 8, 256) is None
    # a wave of 256 tasks spans two Grouped-M(8) strips of 16 x 16 tiles
    assert S.xcd_box_assignment(S.GROUPED_M, 16, 16, 8, 256) is None
    # a short last strip (Mt not a multiple of G)
    assert S.xcd_box_assignment(S.GROUPED_M, 20, 32, 16, 256) is None
    # the linear mappings keep contiguous runs
    assert S.xcd_box_assignment(S.LINEAR_N, 32, 32, 1, 256) is None
