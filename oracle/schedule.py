"""CPU enumeration of the tile mapping, the worker assignment and the Stream-K splits.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Written from the pages' prose, as
orderings produced by walking the tile grid, not as the closed-form index arithmetic that the
HIP library uses, so that the two are independent descriptions of the same schedule.

Sources
  * "DeepGEMM on SM90" page, CTA <-> output tile section and its mapping-family table:
    the mapping F(i) -> (m, n) assigns the i-th linear task an output tile; Linear N-fast visits
    C00, C01, ... then C10; Linear M-fast visits C00, C10, ... then C01; Grouped-M cuts M into
    strips of G tile-rows and runs M-fast inside a strip; Grouped-N cuts N into strips of G
    tile-columns and runs N-fast inside; 2D blocking packs the tiles that run together into a
    box (a local rectangle) and then moves the box; Morton is the Z-order of the bit-interleaved
    tile coordinates.  Static assignment gives CTA i the tile F(i);
    persistent workers take i = p, p + P, p + 2P, ...
  * Same page, Kernel Configuration Heuristic: CTA count = ceil(M/BM) * ceil(N/BN),
    waves = ceil(CTAs / num_sms), wave efficiency = CTAs / (waves * num_sms).
  * "H100 Kernel Design" lesson, section 10.3, and "H100 Stream-K" lesson, sections 2-6:
    Stream-K treats the whole product as one band of MMA iterations split equally across the
    workers; only the tail wave is split when it is at most half full (otherwise plain data
    parallel); a split is one worker's share of one output tile, tracked by
    (K_idx, k_tile_count, is_final = K_idx + k_tile_count == k-tiles per tile); the worker walks
    its tiles backwards; the lock counts the cumulative k-tiles reduced so far.

Readings where the pages are open:
  * a short last strip in the grouped mappings holds the remaining tile rows (columns);
  * blocking: boxes of H tile-rows x W tile-columns; the boxes of a box row are visited along N,
    box rows along M; inside a box M runs fastest (as in a Grouped-M strip); boxes at the bottom
    and right edges hold what is left;
  * Morton: n supplies the even bits of the code and m the odd ones (a 2 x 2 square is visited
    (0,0), (0,1), (1,0), (1,1)); tiles are taken in increasing code order, so codes that fall
    outside a grid which is not a power-of-two square are simply absent;
  * the Stream-K unit u owns iterations [floor(u T / P), floor((u+1) T / P));
  * Stream-K groups: group g holds the units g P/G' ... (g+1) P/G' - 1 (G' groups, G' | P) and
    the band tiles j with j mod G' = g; a group's unit v owns [floor(v T_g / (P/G')),
    floor((v+1) T_g / (P/G'))) of the group's own T_g iterations;
  * roles: K_idx == 0 and final -> whole tile; K_idx == 0 only -> first; final only -> last;
    neither -> middle;
  * the data-parallel tiles run first, then the Stream-K tail.

The XCD remap is the library's own MI355X design, not the pages': with X L2 domains (XCDs) and
workgroups dealt to them round-robin, the worker id that workgroup b runs under is chosen so that
every XCD owns a contiguous run of worker ids.  It is enumerated here from that statement.  For a
grouped mapping whose data-parallel waves are whole G x (P/G) blocks of one strip, the planner
instead gives each XCD a box of every wave's block (the analogue, inside one launch, of the
"DeepGEMM on SM90" page's 2D blocking), when a box needs fewer operand strips than a contiguous
run; xcd_box_assignment enumerates that from its statement, by geometry.
"""
from dataclasses import dataclass

LINEAR_N, LINEAR_M, GROUPED_M, GROUPED_N, BLOCKED, MORTON = 0, 1, 2, 3, 4, 5
STATIC, PERSISTENT, STREAMK = 0, 1, 2
ROLE_WHOLE, ROLE_FIRST, ROLE_MIDDLE, ROLE_LAST = 0, 1, 2, 3


def tile_counts(M, N, K, BM, BN, BK):
    """Tiles along M, along N, and k-tiles along K (ceilings)."""
    cdiv = lambda a, b: -(-a // b)
    return cdiv(M, BM), cdiv(N, BN), cdiv(K, BK)


def morton_code(m, n):
    """Interleave the bits of n (even positions) and m (odd positions)."""
    code, bit = 0, 0
    while (m >> bit) or (n >> bit):
        code |= ((n >> bit) & 1) << (2 * bit)
        code |= ((m >> bit) & 1) << (2 * bit + 1)
        bit += 1
    return code


def tile_order(mode, Mt, Nt, G=1, W=1):
    """The list F(0), F(1), ... of (m, n) tile coordinates, built by walking the grid.
    G: strip width (grouped) or box height (blocked); W: box width (blocked)."""
    order = []
    if mode == LINEAR_N:
        for m in range(Mt):
            for n in range(Nt):
                order.append((m, n))
    elif mode == LINEAR_M:
        for n in range(Nt):
            for m in range(Mt):
                order.append((m, n))
    elif mode == GROUPED_M:
        if G < 1:
            raise ValueError("G must be >= 1")
        for strip_start in range(0, Mt, G):
            rows = range(strip_start, min(strip_start + G, Mt))
            for n in range(Nt):           # the strip advances along N ...
                for m in rows:            # ... and runs M-fast inside
                    order.append((m, n))
    elif mode == GROUPED_N:
        if G < 1:
            raise ValueError("G must be >= 1")
        for strip_start in range(0, Nt, G):
            cols = range(strip_start, min(strip_start + G, Nt))
            for m in range(Mt):
                for n in cols:
                    order.append((m, n))
    elif mode == BLOCKED:
        if G < 1 or W < 1:
            raise ValueError("box sides must be >= 1")
        for row_start in range(0, Mt, G):             # box rows, along M
            rows = range(row_start, min(row_start + G, Mt))
            for col_start in range(0, Nt, W):         # boxes of the row, along N
                for n in range(col_start, min(col_start + W, Nt)):
                    for m in rows:                    # M-fast inside the box
                        order.append((m, n))
    elif mode == MORTON:
        order = sorted(((m, n) for m in range(Mt) for n in range(Nt)),
                       key=lambda t: morton_code(*t))
    else:
        raise ValueError(f"unknown mapping {mode}")
    return order


def xcd_worker_ids(P, X=8):
    """worker id of each workgroup b < P when workgroups are dealt to X XCDs round-robin.

    XCD x receives workgroups x, x + X, x + 2X, ... in that order; it is given the worker ids
    x * P/X, x * P/X + 1, ... in the same order.  Only defined when X divides P; otherwise every
    workgroup keeps its own index.
    """
    if P % X != 0:
        return list(range(P))
    per = P // X
    ids = [None] * P
    for x in range(X):
        dealt = [b for b in range(P) if b % X == x]
        for rank, b in enumerate(dealt):
            ids[b] = x * per + rank
    return ids


def xcd_box_assignment(mode, Mt, Nt, G, P, X=8):
    """The first-wave task of each workgroup b under the XCD box remap, or None where it does not
    apply (then xcd_worker_ids holds).

    It applies to the grouped mappings when every strip holds G tile rows (columns), every wave of
    P consecutive tasks lies inside one strip (so it is a G x P/G block: G across the strip, P/G
    along it), X divides P, and the P/X tasks an XCD runs per wave divide G or are a multiple of
    it.  The box is r across x c along with r | G, c | P/G, r c = P/X, r + c smallest (the wider
    box, smaller r, on a tie); it is used only when r + c is below the number of operand strips (distinct
    rows plus distinct columns) of a contiguous run of P/X tasks.  XCD x (the workgroups b with
    b mod X = x, the k-th of them being b = x + k X) takes the box at block position
    (x mod (G/r), x div (G/r)) -- counted in boxes across, then along -- and its k-th workgroup
    the task at (k mod r, k div r) inside that box: in every wave, so later waves add P.
    """
    if mode not in (GROUPED_M, GROUPED_N) or X <= 1 or G < 1 or P < X or P % X or P % G:
        return None
    n_across, n_along = (Mt, Nt) if mode == GROUPED_M else (Nt, Mt)
    per = P // X
    if n_across % G or (G * n_along) % P or not (per % G == 0 or G % per == 0):
        return None
    wave = tile_order(mode, Mt, Nt, G)[:P]

    def across_along(t):
        m, n = wave[t]
        return (m, n) if mode == GROUPED_M else (n, m)

    first = [across_along(t) for t in range(per)]
    contiguous = len({a for a, _ in first}) + len({b for _, b in first})
    boxes = [(r + per // r, r) for r in range(1, G + 1)
             if G % r == 0 and per % r == 0 and (P // G) % (per // r) == 0]
    if not boxes:
        return None
    strips, r = min(boxes)
    c = per // r
    if strips >= contiguous:
        return None
    task_at = {across_along(t): t for t in range(P)}
    ids = [None] * P
    for b in range(P):
        x, k = b % X, b // X
        a0 = (x % (G // r)) * r
        l0 = (x // (G // r)) * c
        ids[b] = task_at[(a0 + k % r, l0 + k // r)]
    return ids


def wave_efficiency(ctas, num_sms):
    waves = -(-ctas // num_sms)
    return ctas / (waves * num_sms)


@dataclass(frozen=True)
class WorkItem:
    worker: int      # workgroup index b
    seq: int         # position in that workgroup's processing order
    tile: int        # linear task index i (F(i) gives m, n)
    m: int
    n: int
    k_begin: int     # first k-tile (K_idx)
    k_end: int       # one past the last k-tile (K_idx + k_tile_count)
    role: int


def streamk_split_plan(tiles, P):
    """(data-parallel tile count, Stream-K tile count) under the hybrid rule."""
    full, tail = divmod(tiles, P)
    if tail == 0 or tail * 2 > P:
        return tiles, 0
    return full * P, tail


def streamk_units(sk_tiles, Kt, P, first_tile=0, groups=1):
    """For each unit u, its splits [(tile, K_idx, count, final)] in forward k order.

    With `groups` > 1 ("H100 Stream-K" lesson, section 7) the units form that many independent
    groups and so do the band's tiles: band tile j belongs to group j mod groups as that group's
    (j div groups)-th tile (tile id = id in group * groups + group index), and each group splits
    the iterations of its own tiles equally over its own units.  Reading: the units of a group are
    a contiguous block of P / groups unit ids (group g = u div (P / groups)), so that units with
    the same index in every group -- which work the same K range of neighbouring tiles -- are
    P / groups apart.
    """
    if groups < 1 or P % groups != 0:
        raise ValueError("the group count must divide P")
    if groups > max(sk_tiles, 1):
        raise ValueError("more Stream-K groups than Stream-K tiles")
    per_group = P // groups
    # the tiles of each group, in the group's own order
    group_tiles = [[j for j in range(sk_tiles) if j % groups == g] for g in range(groups)]
    units = []
    for u in range(P):
        g, v = divmod(u, per_group)
        mine = group_tiles[g]
        T = len(mine) * Kt
        lo, hi = (v * T) // per_group, ((v + 1) * T) // per_group
        splits = []
        it = lo
        while it < hi:
            t = it // Kt                      # position of the tile in the group's list
            tile_first_iter = t * Kt
            end = min(hi, tile_first_iter + Kt)
            k_idx = it - tile_first_iter
            count = end - it
            splits.append((first_tile + mine[t], k_idx, count, k_idx + count == Kt))
            it = end
        units.append(splits)
    return units


def role_of(k_idx, final):
    if k_idx == 0:
        return ROLE_WHOLE if final else ROLE_FIRST
    return ROLE_LAST if final else ROLE_MIDDLE


def enumerate_schedule(M, N, K, BM, BN, BK, mapping, G, sched, P=None, X=8, xcd_remap=True,
                       W=1, sk_groups=1, xcd_box=True):
    """Every work item of the launch, grouped by workgroup, in each workgroup's order."""
    Mt, Nt, Kt = tile_counts(M, N, K, BM, BN, BK)
    order = tile_order(mapping, Mt, Nt, G, W)
    tiles = Mt * Nt
    items = []
    if sched == STATIC:
        ids = xcd_worker_ids(tiles, X) if xcd_remap else list(range(tiles))
        for b in range(tiles):
            i = ids[b]
            m, n = order[i]
            items.append(WorkItem(b, 0, i, m, n, 0, Kt, ROLE_WHOLE))
        return items
    if P is None or P < 1:
        raise ValueError("persistent and Stream-K schedules need P >= 1 workers")
    if sched == PERSISTENT:
        dp_tiles, sk_tiles = tiles, 0
    elif sched == STREAMK:
        dp_tiles, sk_tiles = streamk_split_plan(tiles, P)
        if Kt == 0:                       # an empty reduction has nothing to split
            dp_tiles, sk_tiles = tiles, 0
    else:
        raise ValueError(f"unknown scheduler {sched}")
    ids = xcd_worker_ids(P, X) if xcd_remap else list(range(P))
    if xcd_remap and xcd_box:
        box = xcd_box_assignment(mapping, Mt, Nt, G, P, X)
        if box is not None:
            ids = box
    units = (streamk_units(sk_tiles, Kt, P, first_tile=dp_tiles, groups=sk_groups)
             if sk_tiles else None)
    for b in range(P):
        seq = 0
        for i in range(ids[b], dp_tiles, P):
            m, n = order[i]
            items.append(WorkItem(b, seq, i, m, n, 0, Kt, ROLE_WHOLE))
            seq += 1
        if units:
            for (i, k_idx, count, final) in reversed(units[b]):
                m, n = order[i]
                items.append(WorkItem(b, seq, i, m, n, k_idx, k_idx + count,
                                      role_of(k_idx, final)))
                seq += 1
    return items
