// Tile scheduler of the dense GEMM: the mapping F(i) -> (m, n), the assignment of linear tasks to
// workgroups (static, persistent, Stream-K hybrid) and the MI355X XCD remap.  Compiled for host
// and device: the kernel walks its work with it, and gemm_schedule_enumerate() replays the same
// code on the CPU.
//
// Sources:
//  * "DeepGEMM on SM90" page, CTA <-> output tile section and its mapping-family table: F(i) names
//    the output tile of the i-th linear task; Linear N-fast, Linear M-fast, Grouped-M strip
//    (M cut into strips of G tile-rows, M-fast inside), Grouped-N strip (the transpose), 2D
//    blocking (the tiles that run together packed into a box, then the box moves) and Morton
//    (Z-order: the bits of m and n interleaved).
//    Persistence is not a mapping: a persistent worker p takes i = p, p + P, p + 2P, ...
//  * "H100 Kernel Design" lesson, sections 9-10 (persistent grid-stride loop, Stream-K hybrid:
//    data-parallel full waves, Stream-K only for a tail wave at most half full, backward tile
//    iteration) and "H100 Stream-K" lesson, sections 2-6 (a unit's share of one tile is a split
//    tracked by K_idx, k_tile_count and is_final = K_idx + k_tile_count == k-tiles per tile).
#pragma once
#include <stdint.h>

#if defined(__HIPCC__) || defined(__HIP__)
#define DG_HD __host__ __device__ __forceinline__
#else
#define DG_HD inline
#endif

namespace dg {

enum Mapping {
  MAP_LINEAR_N = 0,
  MAP_LINEAR_M = 1,
  MAP_GROUPED_M = 2,
  MAP_GROUPED_N = 3,
  MAP_BLOCKED = 4,
  MAP_MORTON = 5
};
enum Role { ROLE_WHOLE = 0, ROLE_FIRST = 1, ROLE_MIDDLE = 2, ROLE_LAST = 3 };

// Division of a non-negative 31-bit value by a fixed positive divisor as a multiply-high, add
// and shift (Granlund and Montgomery, "Division by invariant integers using multiplication",
// PLDI 1994): with l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1, n / d equals
// (mulhi(m, n) + n) >> l for 0 <= n < 2^31.  Uniform operands stay on the scalar unit.
struct FastDiv {
  uint32_t d, m, l;
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t l = 0;
  while (l < 32 && ((uint64_t)1 << l) < d) ++l;
  f.l = l;
  f.m = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d + 1);
  return f;
}

DG_HD uint32_t umulhi32(uint32_t a, uint32_t b) { return (uint32_t)(((uint64_t)a * b) >> 32); }

DG_HD int32_t fdiv(int32_t n, const FastDiv &f) {
  return (int32_t)((umulhi32(f.m, (uint32_t)n) + (uint32_t)n) >> f.l);
}

struct SchedParams {
  int32_t Mt, Nt, Kt;      // tiles along M and N, k-tiles along K
  int32_t mapping, G;      // F(i) family and strip width (blocked: box height in tile rows)
  int32_t P;               // workgroups in the launch (workers)
  int32_t X;               // XCDs the workgroups are dealt to round-robin (1 = no remap)
  int32_t G2;              // blocked: box width in tile columns
  int32_t dp_tiles;        // tasks i < dp_tiles run whole (data parallel)
  int32_t sk_tiles;        // the next sk_tiles tasks are split along K (Stream-K band)
  int32_t sk_groups;       // Stream-K groups (divides P, at most sk_tiles; 1 = one pool)
  int32_t sk_gunits;       // units per group, P / sk_groups
  int32_t sk_gtiles;       // band tiles of the largest group, ceil(sk_tiles / sk_groups)
  // divisors of the mapping and of the Stream-K band (filled by sched_prepare)
  FastDiv div_major;       // Nt (linear N), Mt (linear M), G*Nt (grouped M), G*Mt (grouped N)
  FastDiv div_g;           // G (grouped), unused otherwise
  FastDiv div_g_last;      // width of the short last strip (grouped), else = div_g
  FastDiv div_kt;          // Kt (Stream-K band), 1 when Kt == 0
  FastDiv div_skg;         // sk_groups
  FastDiv div_box;         // blocked: G * G2 tiles of a full-height box
  FastDiv div_box_last;    // blocked: (height of the short last box row) * G2
  int32_t full_strips;     // strips (blocked: box rows) of exactly G
  int32_t morton_size;     // Morton: the smallest power of two >= max(Mt, Nt)
  int32_t xbox_r, xbox_c;  // XCD box remap (grouped mappings): each XCD's P/X tasks of a wave
                           // form an xbox_r (across the strip) x xbox_c (along it) box; 0 = the
                           // contiguous remap (xcd_worker)
};

// Fills the divisor fields from Mt, Nt, Kt, mapping, G and G2.
inline void sched_prepare(SchedParams &sp) {
  const int32_t G = sp.G < 1 ? 1 : sp.G;
  const int32_t G2 = sp.G2 < 1 ? 1 : sp.G2;
  switch (sp.mapping) {
    case MAP_LINEAR_N: sp.div_major = make_fastdiv(sp.Nt > 0 ? sp.Nt : 1); break;
    case MAP_LINEAR_M: sp.div_major = make_fastdiv(sp.Mt > 0 ? sp.Mt : 1); break;
    case MAP_GROUPED_N: sp.div_major = make_fastdiv((uint32_t)(G * (sp.Mt > 0 ? sp.Mt : 1))); break;
    default: sp.div_major = make_fastdiv((uint32_t)(G * (sp.Nt > 0 ? sp.Nt : 1))); break;
  }
  const int32_t rows = sp.mapping == MAP_GROUPED_N ? sp.Nt : sp.Mt;
  sp.full_strips = rows / G;
  const int32_t last = rows - sp.full_strips * G;
  sp.div_g = make_fastdiv((uint32_t)G);
  sp.div_g_last = make_fastdiv((uint32_t)(last > 0 ? last : G));
  sp.div_box = make_fastdiv((uint32_t)(G * G2));
  sp.div_box_last = make_fastdiv((uint32_t)((last > 0 ? last : G) * G2));
  sp.div_kt = make_fastdiv((uint32_t)(sp.Kt > 0 ? sp.Kt : 1));
  if (sp.sk_groups < 1) sp.sk_groups = 1;
  sp.sk_gunits = sp.P / sp.sk_groups;
  sp.sk_gtiles = (sp.sk_tiles + sp.sk_groups - 1) / sp.sk_groups;
  sp.div_skg = make_fastdiv((uint32_t)sp.sk_groups);
  int32_t size = 1;
  while (size < sp.Mt || size < sp.Nt) size *= 2;
  sp.morton_size = size;
}

struct WorkItem {
  int32_t tile;            // linear task i
  int32_t m, n;            // F(i)
  int32_t kb, ke;          // k-tiles [kb, ke) of the tile
  int32_t role;
  int32_t sk_slot;         // i - dp_tiles for a split tile (workspace slot), else -1
};

struct TileMN {
  int32_t m, n;
};

// Morton (Z-order) F(i): the i-th tile of the grid in the order of its interleaved code -- bit b
// of n at code bit 2b, bit b of m at 2b + 1, so a 2 x 2 square goes (0,0) (0,1) (1,0) (1,1).  On a
// grid that is not a power-of-two square the codes outside the grid are skipped: descend the
// quadtree of the enclosing 2^k square, skipping whole quadrants by their count of grid tiles.
DG_HD TileMN morton_tile(const SchedParams &sp, int32_t i) {
  int32_t m0 = 0, n0 = 0;
  for (int32_t half = sp.morton_size / 2; half >= 1; half /= 2) {
#pragma unroll
    for (int32_t q = 0; q < 4; ++q) {
      const int32_t qm = m0 + (q >> 1) * half, qn = n0 + (q & 1) * half;
      const int32_t rows = sp.Mt - qm < 0 ? 0 : (sp.Mt - qm < half ? sp.Mt - qm : half);
      const int32_t cols = sp.Nt - qn < 0 ? 0 : (sp.Nt - qn < half ? sp.Nt - qn : half);
      const int32_t cnt = rows * cols;
      if (i < cnt || q == 3) {
        m0 = qm;
        n0 = qn;
        break;
      }
      i -= cnt;
    }
  }
  return TileMN{m0, n0};
}

// F(i) -> (m, n).  Grouped-M: a strip holds G tile-rows (fewer in a short last strip) and is
// walked column by column, M-fast inside: i = strip * (G * Nt) + n * g + (m - strip * G).
// Blocked: box rows of G tile-rows (fewer in the last), each cut into boxes of G2 tile-columns
// (fewer in the last) walked along N; inside a box of g rows, M-fast:
// i = boxrow * (G * Nt) + box * (g * G2) + (n - box * G2) * g + (m - boxrow * G).  G2 = Nt is
// Grouped-M(G).  Task indices fit in 32 bits (the planner rejects larger grids).
DG_HD TileMN map_tile(const SchedParams &sp, int32_t i) {
  TileMN t;
  if (sp.mapping == MAP_MORTON) return morton_tile(sp, i);
  const int32_t q = fdiv(i, sp.div_major);
  const int32_t r = i - q * (int32_t)sp.div_major.d;
  if (sp.mapping == MAP_LINEAR_N) {
    t.m = q;
    t.n = r;
  } else if (sp.mapping == MAP_LINEAR_M) {
    t.n = q;
    t.m = r;
  } else if (sp.mapping == MAP_BLOCKED) {
    // box row q (g rows), position r inside it: box b, position u inside the box
    const bool last = q >= sp.full_strips;
    const FastDiv &dbox = last ? sp.div_box_last : sp.div_box;
    const FastDiv &dg = last ? sp.div_g_last : sp.div_g;
    const int32_t b = fdiv(r, dbox);
    const int32_t u = r - b * (int32_t)dbox.d;
    const int32_t col = fdiv(u, dg);
    t.m = q * sp.G + (u - col * (int32_t)dg.d);
    t.n = b * sp.G2 + col;
  } else {
    // strip q, position r inside it; the strip is g wide (G, or less for the last one)
    const bool last = q >= sp.full_strips;
    const FastDiv &dg = last ? sp.div_g_last : sp.div_g;
    const int32_t along = fdiv(r, dg);            // tile index along the strip's length
    const int32_t across = r - along * (int32_t)dg.d;
    const int32_t first = q * sp.G + across;      // tile index across the strip
    if (sp.mapping == MAP_GROUPED_M) {
      t.m = first;
      t.n = along;
    } else {
      t.n = first;
      t.m = along;
    }
  }
  return t;
}

// Worker id of workgroup b.  Workgroups are dealt to the X XCDs round-robin (b mod X), each XCD
// with its own L2; giving XCD x the worker ids x*P/X ... x*P/X + P/X - 1 keeps the tiles that
// consecutive ids take -- which share A and B bands under a grouped mapping -- on one L2.
DG_HD int32_t xcd_worker(int32_t b, int32_t P, int32_t X) {
  if (X <= 1 || P % X != 0) return b;
  return (b % X) * (P / X) + b / X;
}

// XCD box remap of a grouped mapping.  When every wave of P consecutive tasks is a whole G x (P/G)
// block of one strip (G tile-rows across the strip, P/G positions along it, in-strip task
// t = along * G + across), contiguous runs of P/X tasks give each XCD a G x (P/(X G)) slab, which
// needs G + P/(X G) operand strips per k-step in that XCD's L2.  Cutting the block into X boxes of
// r x c tasks (r | G, c | P/G, r c = P/X) with r + c smallest needs only r + c: for G = 16 and
// 32 tasks per XCD, 8 x 4 boxes need 12 strips where 16 x 2 slabs need 18.  Workgroup b runs on
// XCD x = b mod X as its k-th workgroup, k = b div X; XCD x takes box (x mod (G/r), x div (G/r))
// and its k-th workgroup the task at (k mod r, k div r) inside the box, in every wave.  Returns the
// workgroup's task in the first wave (later waves add P).
DG_HD int32_t xcd_box_task(const SchedParams &sp, int32_t b) {
  const int32_t x = b % sp.X, k = b / sp.X;
  const int32_t across_boxes = sp.G / sp.xbox_r;
  const int32_t across = (x % across_boxes) * sp.xbox_r + k % sp.xbox_r;
  const int32_t along = (x / across_boxes) * sp.xbox_c + k / sp.xbox_r;
  return along * sp.G + across;
}

// Cursor over one workgroup's work: its data-parallel tiles first, then its Stream-K splits from
// the last tile it touches back to the first.
struct Cursor {
  int32_t next_dp;         // next data-parallel task
  int32_t sk_lo, sk_hi;    // remaining Stream-K iterations [sk_lo, sk_hi) of the unit's group,
                           // consumed from the top
  int32_t sk_group;        // the unit's Stream-K group
};

// Stream-K groups: unit u is unit v = u mod (P/G) of group g = u div (P/G); band tile t is tile
// t div G of group t mod G.  Group g has ceil((sk_tiles - g) / G) tiles and T_g = tiles * Kt
// iterations, of which its unit v owns [floor(v T_g / (P/G)), floor((v+1) T_g / (P/G))).  With
// G = 1 this is the single pool: unit b owns [floor(b T / P), floor((b+1) T / P)).
DG_HD int64_t sk_group_iters(const SchedParams &sp, int32_t g) {
  return (int64_t)((sp.sk_tiles - g + sp.sk_groups - 1) / sp.sk_groups) * sp.Kt;
}

DG_HD void cursor_init(const SchedParams &sp, int32_t b, Cursor &c) {
  c.next_dp = sp.xbox_r > 0 ? xcd_box_task(sp, b) : xcd_worker(b, sp.P, sp.X);
  c.sk_group = 0;
  if (sp.sk_tiles > 0) {
    const int32_t g = b / sp.sk_gunits, v = b - g * sp.sk_gunits;
    const int64_t T = sk_group_iters(sp, g);
    c.sk_group = g;
    c.sk_lo = (int32_t)((int64_t)v * T / sp.sk_gunits);
    c.sk_hi = (int32_t)((int64_t)(v + 1) * T / sp.sk_gunits);
  } else {
    c.sk_lo = c.sk_hi = 0;
  }
}

DG_HD bool cursor_next(const SchedParams &sp, Cursor &c, WorkItem &w) {
  if (c.next_dp < sp.dp_tiles) {
    w.tile = c.next_dp;
    c.next_dp += sp.P;
    w.kb = 0;
    w.ke = sp.Kt;
    w.role = ROLE_WHOLE;
    w.sk_slot = -1;
  } else if (c.sk_hi > c.sk_lo) {
    const int32_t last = c.sk_hi - 1;
    const int32_t tg = fdiv(last, sp.div_kt);       // the group's tile of the top iteration
    const int32_t t_first = tg * sp.Kt;
    const int32_t start = c.sk_lo > t_first ? c.sk_lo : t_first;
    const int32_t t = tg * sp.sk_groups + c.sk_group;  // band-local tile
    w.tile = sp.dp_tiles + t;
    w.kb = start - t_first;
    w.ke = c.sk_hi - t_first;
    c.sk_hi = start;
    const bool first = w.kb == 0, final = w.ke == sp.Kt;
    w.role = first ? (final ? ROLE_WHOLE : ROLE_FIRST) : (final ? ROLE_LAST : ROLE_MIDDLE);
    w.sk_slot = t;
  } else {
    return false;
  }
  const TileMN mn = map_tile(sp, w.tile);
  w.m = mn.m;
  w.n = mn.n;
  return true;
}

// Stream-K units that share band-local tile t: in its group g, unit v covers iterations
// [floor(v T_g / U), floor((v+1) T_g / U)) (U = P/G units per group), so the unit holding
// iteration x is the largest v with floor(v T_g / U) <= x, i.e. floor(((x + 1) U - 1) / T_g).
// Tile t is the group's tile t div G and spans its iterations [(t div G) Kt, (t div G + 1) Kt);
// its units are u0 .. u1 (unit ids g U + v), consecutive, in increasing K order.
DG_HD void sk_tile_units(const SchedParams &sp, int32_t t, int32_t &u0, int32_t &u1) {
  const int32_t tg = fdiv(t, sp.div_skg), g = t - tg * sp.sk_groups;
  const int64_t T = sk_group_iters(sp, g), U = sp.sk_gunits;
  const int64_t x0 = (int64_t)tg * sp.Kt, x1 = x0 + sp.Kt - 1;
  u0 = g * sp.sk_gunits + (int32_t)(((x0 + 1) * U - 1) / T);
  u1 = g * sp.sk_gunits + (int32_t)(((x1 + 1) * U - 1) / T);
}

// Separate-reduction partial slot of unit u's split of band tile t.  Within a group, unit v and
// the group's tile tg give v + tg, which no other split of the group shares (a later unit only
// touches the same or later tiles, so v' > v and tg' < tg never meet); groups take disjoint
// ranges of U + sk_gtiles slots, and the units of one tile have consecutive slots.
DG_HD int64_t sk_partial_slot(const SchedParams &sp, int32_t u, int32_t t) {
  const int32_t tg = fdiv(t, sp.div_skg), g = t - tg * sp.sk_groups;
  const int32_t v = u - g * sp.sk_gunits;
  return (int64_t)g * (sp.sk_gunits + sp.sk_gtiles) + v + tg;
}
DG_HD int64_t sk_partial_slots(const SchedParams &sp) {
  return (int64_t)sp.sk_groups * (sp.sk_gunits + sp.sk_gtiles);
}

// Hybrid rule: with P workers and `tiles` tasks, the full waves stay data parallel; the tail
// wave goes to Stream-K only when it is at most half full, otherwise everything is data parallel.
DG_HD void streamk_plan(int64_t tiles, int32_t P, int32_t &dp_tiles, int32_t &sk_tiles) {
  const int64_t full = tiles / P, tail = tiles % P;
  if (tail == 0 || tail * 2 > P) {
    dp_tiles = (int32_t)tiles;
    sk_tiles = 0;
  } else {
    dp_tiles = (int32_t)(full * P);
    sk_tiles = (int32_t)tail;
  }
}

}  // namespace dg
