// C ABI of the MI355X dense GEMM: planner, launcher and CPU schedule replay (include/gemm.h).
//
// The planner turns a gemm_desc into a plan: the tile shape and its kernel, the tile grid
// (CTA count = ceil(M/BM) * ceil(N/BN), "DeepGEMM on SM90" page, Kernel Configuration Heuristic),
// the scheduler's parameters (sched.h) and the workspace size for the Stream-K fixup ("H100
// Stream-K" lesson, section 6: one FP32 partial tile per split output tile, followed by one int
// lock per tile in the same allocation, all locks zero at launch).
#include <hip/hip_runtime.h>

#include <new>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

#include "../../include/gemm.h"
#include "gemm_kernel.h"
#include "launch.h"
#include "sched.h"

namespace {

using namespace dg;

// Zeroes the Stream-K locks, the error word and the trace area of a workspace before a run.
__global__ void clear_ints_kernel(int *p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

typedef hipError_t (*launch_fn)(const KernelArgs &, int grid, bool ragged_k, hipStream_t);
typedef const void *(*kernel_fn)();

// A plan with a fused epilogue (EPI_* bits or an e4m3 output) launches the kernels' FUSED
// instantiation; all others the plain one.
bool fused_args(const KernelArgs &a) { return a.epi != 0 || a.out_fp8; }

template <class CFG>
hipError_t launch_cfg(const KernelArgs &a, int grid, bool ragged_k, hipStream_t s) {
  const dim3 g(grid), t(CFG::THREADS);
  if (fused_args(a)) {
    if (ragged_k)
      hipLaunchKernelGGL((gemm_kernel<CFG, true, true>), g, t, 0, s, a);
    else
      hipLaunchKernelGGL((gemm_kernel<CFG, false, true>), g, t, 0, s, a);
  } else if (ragged_k) {
    hipLaunchKernelGGL((gemm_kernel<CFG, true>), g, t, 0, s, a);
  } else {
    hipLaunchKernelGGL((gemm_kernel<CFG, false>), g, t, 0, s, a);
  }
  return hipGetLastError();
}
template <class CFG>
const void *kernel_of() {
  return (const void *)&gemm_kernel<CFG, false>;
}
template <class CFG>
hipError_t launch_pp(const KernelArgs &a, int grid, bool ragged_k, hipStream_t s) {
  if (ragged_k)
    hipLaunchKernelGGL((gemm_kernel_pp<CFG, true>), dim3(grid), dim3(CFG::THREADS), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_kernel_pp<CFG, false>), dim3(grid), dim3(CFG::THREADS), 0, s, a);
  return hipGetLastError();
}
template <class CFG>
const void *kernel_of_pp() {
  return (const void *)&gemm_kernel_pp<CFG, false>;
}
template <class CFG>
hipError_t launch_wide(const KernelArgs &a, int grid, bool ragged_k, hipStream_t s) {
  if (!fused_args(a))
    launch_wide_as<CFG, FUSE_OFF>(a, grid, ragged_k, s);
  else if (a.epi & (EPI_SRC_F32 | EPI_SRC_BF16))  // reads a source matrix: its own kernels
    return launch_wide_src<CFG>(a, grid, ragged_k, s);
  else
    launch_wide_act<CFG, 0>(a, grid, ragged_k, s);
  return hipGetLastError();
}
template <class CFG>
const void *kernel_of_wide() {
  return (const void *)wide_kernel<CFG, false>();
}

// kind: KIND_COOP runs every plan; the others run data-parallel work only (no Stream-K splits,
// K > 0)
// (value 2 belonged to a register-staged kernel that is no longer built)
enum { KIND_COOP = 0, KIND_PP = 1, KIND_WIDE = 3, KIND_COUNT = 4 };
struct KernelEntry {
  int dt, bm, bn, bk, threads, stages, lds, kind;
  launch_fn launch;
  kernel_fn kernel;
};

template <class CFG>
constexpr KernelEntry entry() {
  return KernelEntry{CFG::DT, CFG::BM, CFG::BN, CFG::BK, CFG::THREADS, CFG::STAGES,
                     CFG::LDS_BYTES, KIND_COOP, &launch_cfg<CFG>, &kernel_of<CFG>};
}
template <class CFG>
constexpr KernelEntry entry_pp() {
  return KernelEntry{CFG::DT, CFG::BM, CFG::BN, CFG::BK, CFG::THREADS, CFG::STAGES,
                     pp_lds_bytes<CFG>(), KIND_PP, &launch_pp<CFG>, &kernel_of_pp<CFG>};
}
template <class CFG>
constexpr KernelEntry entry_wide() {
  return KernelEntry{CFG::DT, CFG::BM, CFG::BN, CFG::BK, CFG::THREADS, CFG::STAGES,
                     wide_lds_bytes<CFG>(), KIND_WIDE, &launch_wide<CFG>, &kernel_of_wide<CFG>};
}

// The first entry that matches (dtype, bm, bn[, bk]) is the default for that tile shape.
const KernelEntry kKernels[] = {
    entry<CfgBf16_256>(),
    entry_pp<CfgBf16_256pp>(),
    entry<CfgBf16_128>(),
    entry<CfgFp8_256>(),
    entry_pp<CfgFp8_256pp>(),
    entry_wide<CfgBf16_256w>(),
    entry_wide<CfgFp8_256w>(),
    entry_wide<CfgBf16_128w>(),
    entry_wide<CfgFp8_128w>(),
    entry_wide<CfgBf16_224w>(),
    entry_wide<CfgFp8_224w>(),
    entry_wide<CfgBf16_192w>(),
    entry_wide<CfgFp8_192w>(),
    entry<CfgFp8_128>(),
};

constexpr int kXcds = 8;           // MI355X: 8 accelerator complex dies, one L2 each
constexpr int kMaxSkGroups = 8;    // Stream-K groups: at most 8 ("H100 Stream-K" lesson, sec. 7)

// Stream-K group count of a requested count (>= 1): lowered to the largest count that divides the
// P units evenly and leaves every group at least one band tile.
int32_t streamk_groups(int32_t requested, int32_t P, int32_t sk_tiles) {
  if (sk_tiles <= 0 || requested <= 1) return 1;
  for (int32_t g = requested; g > 1; --g)
    if (P % g == 0 && g <= sk_tiles) return g;
  return 1;
}

// The planner's count (request 0).  Workgroup b runs on XCD b mod X, so when the P / G units of a
// group are a multiple of X, the units with the same index in every group -- which work the same
// K range of neighbouring band tiles at the same time -- share one XCD and its L2.  Measured on
// all-split bands of 100 - 128 tiles over 256 units: G = 8 runs 1.1 - 1.8x faster than one pool
// when the band's iterations do not fall on tile boundaries, and within a few % when they do.
// The largest such count up to 8 is taken, unless it would leave a unit of the smallest group
// without an iteration (forcing the lock chain) where one pool would not.
int32_t streamk_auto_groups(int32_t P, int32_t sk_tiles, int64_t Kt, int32_t X) {
  if (sk_tiles <= 0) return 1;
  const bool separate1 = (int64_t)sk_tiles * Kt >= P;
  for (int32_t g = kMaxSkGroups; g > 1; --g) {
    if (P % g != 0 || g > sk_tiles || (P / g) % X != 0) continue;
    if (separate1 && (int64_t)(sk_tiles / g) * Kt < P / g) continue;
    return g;
  }
  return 1;
}
constexpr int kDefaultSpin = 1 << 24;
constexpr int kTestSpin = 4096;
constexpr int kTraceCap = 64;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t align_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

constexpr uint32_t kEpiSource = GEMM_EPI_SOURCE_F32 | GEMM_EPI_SOURCE_BF16;

// Known GEMM_EPI_* bits, at most one source, one bias vector and one activation.
bool epilogue_valid(uint32_t e) {
  const uint32_t all = GEMM_EPI_BIAS_ROW | GEMM_EPI_BIAS_COL | GEMM_EPI_RELU | GEMM_EPI_GELU |
                       GEMM_EPI_SILU | GEMM_EPI_AMAX | kEpiSource;
  if (e & ~all) return false;
  if (__builtin_popcount(e & kEpiSource) > 1) return false;
  if (__builtin_popcount(e & (GEMM_EPI_BIAS_ROW | GEMM_EPI_BIAS_COL)) > 1) return false;
  return __builtin_popcount(e & (GEMM_EPI_RELU | GEMM_EPI_GELU | GEMM_EPI_SILU)) <= 1;
}
static_assert(GEMM_EPI_BIAS_ROW == EPI_BIAS_ROW && GEMM_EPI_BIAS_COL == EPI_BIAS_COL &&
                  GEMM_EPI_RELU == EPI_RELU && GEMM_EPI_GELU == EPI_GELU &&
                  GEMM_EPI_SILU == EPI_SILU && GEMM_EPI_AMAX == EPI_AMAX &&
                  GEMM_EPI_SOURCE_F32 == EPI_SRC_F32 && GEMM_EPI_SOURCE_BF16 == EPI_SRC_BF16,
              "epilogue bits shared with the kernels");

// ---- kernel-configuration heuristic -----------------------------------------------------------
// The cost model of "DeepGEMM on SM90" (section "Kernel Configuration Heuristic"), re-fitted to
// gfx950.  Per candidate, whole-GEMM clocks on three sides:
//   cycles_l2    = bytes from L2 to the CUs (A/B k-tiles, C, Stream-K partials) / L2->CU bandwidth
//   cycles_local = bytes through LDS (A/B fills, MFMA fragment reads, C staging) / LDS bandwidth
//   cycles_mfma  = FLOPs / (matrix-core FLOP per clock x the kernel's measured efficiency)
// and score = max of the three / wave_efficiency + cycles_fixed, the minimum winning.  The page's
// SM-side term counts the Tensor Core operand bytes; on gfx950 the fragment reads are those
// bytes and the matrix cores get their own term, because a kernel's schedule -- not only its
// bytes -- sets how close it comes to peak.  cycles_fixed adds what does not overlap the MAC
// loop: a worker's first stage of loads, each item's epilogue, and for Stream-K the partial sums,
// which go to device memory (coherent accesses past the XCD's L2) after the MAC work.  The
// constants are measurements on MI355X (all CUs busy):
constexpr double kL2BytesPerClk = 57.0;      // global->LDS loads per CU
constexpr double kLdsBytesPerClk = 256.0;    // ds_read_b128 per CU
constexpr double kDeviceBytesPerClk = 2600;  // Stream-K partials, whole device (128 MiB in 25 us)
// Lock chain: a hop reads and writes a tile's partial from one CU and hands the lock on; fit to
// 64 chained splits per tile taking 462 us on 128 x 128 tiles and 590 us on 256 x 256 tiles
// (256 x 256 x 4096 bf16, cooperative kernel, 512 units)
constexpr double kChainBytesPerClk = 96;
constexpr double kChainHopClk = 13000;
constexpr double kLatencyClk = 2000;         // first load or store round trip of a phase
// A partial last wave: the board is held at its power limit, so with a fraction f of the CUs busy
// the busy ones clock higher (144 of 256 CUs finish a 256 x 256 x 4096 bf16 tile in 75 us, all
// 256 in 95), up to the clock's headroom (2.4 GHz against the 1.9 held under full load).  Such a
// wave is costed f^0.39 of a full one (fit to that pair), and no less than 1 / 1.3.
constexpr double kPartialWaveExp = 0.39;
constexpr double kMinPartialWave = 1.0 / 1.3;
// ... except a launch that is one partial wave of 256 x 224 or 256 x 192 tiles: their k-step is
// shorter for the same load latency, so the clock headroom buys them less (measured time over
// score 4-6 % above their classes' medians in such launches, 2 % for 256 x 256)
constexpr double kPartialWaveExpNarrow = 0.2;
// Stream-K plans ran about 3 % slower per costed cycle than data-parallel ones over the same 184
// shapes (the waits and the fixup's latency, beyond its bytes): their score is scaled by this
constexpr double kStreamKFactor = 1.03;
// ... and a band that gives each unit only a few k-steps: all units then store and reduce their
// partials at once, a burst the reduction waits on.  Costed kSkBurstClk at one k-step per unit,
// falling linearly to none at kSkBurstSteps (fit to small outputs: e4m3 512 x 512 x 4096, 2
// k-steps per unit, ran 29 us on Stream-K against 19 data-parallel; bf16 256 x 256 x 4096, 1
// k-step per unit, 25 against 29)
constexpr double kSkBurstClk = 20000;
constexpr double kSkBurstSteps = 16;
// MFMA efficiency of whole launches at the held clock (bench workloads, profiles/)
double kernel_efficiency(int kind, int bm, int bn, int dt) {
  if (kind == KIND_WIDE && bm == 128) return dt == DT_BF16 ? 0.56 : 0.55;
  // 256 x 224: 2 % below 256 x 256 at whole waves (8192 x 14336 x 4096 bf16, one board: 1,367
  // against 1,397 TFLOP/s) -- 12.5 % fewer MACs per operand byte
  if (kind == KIND_WIDE && bn == 224) return dt == DT_BF16 ? 0.74 : 0.77;
  // 256 x 192: 25 % fewer MACs per operand byte than 256 x 256; refit with the Stream-K factor
  // below against every candidate timed on 184 shapes (M 1,024-8,192, N 2,560-28,672, K
  // 2,048-8,192, both operand types): the pick's time over the fastest averages 1.0038 there
  if (kind == KIND_WIDE && bn == 192) return dt == DT_BF16 ? 0.71 : 0.74;
  if (kind == KIND_WIDE) return dt == DT_BF16 ? 0.76 : 0.79;
  if (kind == KIND_PP) return 0.66;
  if (bm == 256) return dt == DT_BF16 ? 0.60 : 0.70;
  return dt == DT_BF16 ? 0.35 : 0.25;
}
double flop_per_clk_per_cu(int dt) { return dt == DT_BF16 ? 4096.0 : 8192.0; }

// G for a grouped mapping: each XCD runs `chunk` consecutive tiles of F(i) at a time (the XCD
// remap gives it a contiguous run of workers); under grouped-M(G) they form a G x (chunk / G)
// block, which reads G + chunk / G operand strips per k-step.  The fewest strips win, the larger
// G on a tie.
int choose_group(int mapping, int64_t Mt, int64_t Nt, int64_t chunk) {
  const int64_t span = mapping == GEMM_MAP_GROUPED_M ? Mt : Nt;
  const int64_t other = mapping == GEMM_MAP_GROUPED_M ? Nt : Mt;
  int best = 1;
  int64_t best_strips = INT64_MAX;
  for (int G = 1; G <= 32; G *= 2) {
    const int64_t g = G < span ? G : (span > 0 ? span : 1);
    int64_t cols = cdiv(chunk, g);
    if (cols > other) cols = other;
    const int64_t strips = g + cols;
    if (strips <= best_strips) {
      best_strips = strips;
      best = G;
    }
    if (G >= span) break;
  }
  return best;
}

// Box of the blocked mapping for the same `chunk` tiles: H x W = chunk tile rows x columns (a
// given H or W kept, the other one derived), reading H + W operand strips per k-step.  The
// fewest strips win, the wider box on a tie.
// XCD box remap of a grouped mapping (sched.h, xcd_box_task): used when every data-parallel wave
// of P tasks is a whole G x (P/G) block of one strip (all strips full, strip length a multiple
// of P, the P/X tasks an XCD runs per wave a multiple or a divisor of G) and an r x c box per
// XCD (r | G, c | P/G, r c = P/X, r + c smallest, the wider box on a
// tie: fewer rows across the strip, measured 0.5 % faster on fp8 8192^3, 4 x 8 against 8 x 4)
// needs fewer operand strips than the contiguous runs of P/X tasks do.
void choose_xcd_box(SchedParams &sp) {
  sp.xbox_r = sp.xbox_c = 0;
  const int32_t X = sp.X, P = sp.P, G = sp.G;
  if (sp.mapping != MAP_GROUPED_M && sp.mapping != MAP_GROUPED_N) return;
  if (X <= 1 || P < X || P % X != 0 || G < 1 || P % G != 0) return;
  const int32_t across = sp.mapping == MAP_GROUPED_M ? sp.Mt : sp.Nt;
  const int32_t along = sp.mapping == MAP_GROUPED_M ? sp.Nt : sp.Mt;
  if (across % G != 0 || ((int64_t)G * along) % P != 0) return;
  const int32_t per = P / X, len = P / G;
  if (per % G != 0 && G % per != 0) return;  // runs of `per` tasks are no slab or column
  int32_t best_r = 0, best_c = 0;
  for (int32_t r = G; r >= 1; --r) {
    if (G % r != 0 || per % r != 0 || len % (per / r) != 0) continue;
    const int32_t c = per / r;
    if (best_r == 0 || r + c <= best_r + best_c) {  // r falls: a tie goes to the wider box
      best_r = r;
      best_c = c;
    }
  }
  // a contiguous run of `per` tasks is a G x per/G slab (or a per x 1 column when G > per)
  const int32_t contiguous = per % G == 0 ? G + per / G : per + 1;
  if (best_r > 0 && best_r + best_c < contiguous) {
    sp.xbox_r = best_r;
    sp.xbox_c = best_c;
  }
}

void choose_box(int64_t Mt, int64_t Nt, int64_t chunk, int32_t &H, int32_t &W) {
  if (H > 0 && W > 0) return;
  if (H > 0) {
    W = (int32_t)std::min<int64_t>(std::max<int64_t>(cdiv(chunk, H), 1), std::max<int64_t>(Nt, 1));
    return;
  }
  if (W > 0) {
    H = (int32_t)std::min<int64_t>(std::max<int64_t>(cdiv(chunk, W), 1), std::max<int64_t>(Mt, 1));
    return;
  }
  int64_t best = INT64_MAX;
  for (int64_t h = 1; h <= 64; h *= 2) {
    const int64_t hh = std::min<int64_t>(h, std::max<int64_t>(Mt, 1));
    const int64_t ww = std::min<int64_t>(std::max<int64_t>(cdiv(chunk, hh), 1), std::max<int64_t>(Nt, 1));
    const int64_t strips = hh + ww;
    if (strips < best || (strips == best && ww > W)) {
      best = strips;
      H = (int32_t)hh;
      W = (int32_t)ww;
    }
    if (h >= Mt) break;
  }
}

struct ModelCand {
  int kind, bm, bn, sched;
};

// Scores every feasible candidate for `d` (already validated), best first.  cus / occupancy come
// from the device when num_workers == 0.
int rank_configs(const gemm_desc &d, std::vector<gemm_config_score> &out) {
  const int dt = d.dtype_ab == GEMM_BF16 ? DT_BF16 : DT_FP8;
  const double eb = dt == DT_BF16 ? 2.0 : 1.0, ec = d.dtype_c == GEMM_BF16       ? 2.0
                                                    : d.dtype_c == GEMM_FP8_E4M3 ? 1.0
                                                                                 : 4.0;
  const ModelCand cands[] = {{KIND_WIDE, 256, 256, GEMM_SCHED_PERSISTENT},
                             {KIND_WIDE, 256, 224, GEMM_SCHED_PERSISTENT},
                             {KIND_WIDE, 256, 192, GEMM_SCHED_PERSISTENT},
                             {KIND_WIDE, 128, 128, GEMM_SCHED_PERSISTENT},
                             {KIND_COOP, 128, 128, GEMM_SCHED_PERSISTENT},
                             {KIND_WIDE, 128, 128, GEMM_SCHED_STREAMK},
                             {KIND_COOP, 128, 128, GEMM_SCHED_STREAMK},
                             {KIND_WIDE, 256, 256, GEMM_SCHED_STREAMK},
                             {KIND_COOP, 256, 256, GEMM_SCHED_STREAMK},
                             {KIND_COOP, 256, 256, GEMM_SCHED_PERSISTENT}};
  // a source matrix (Z = alpha Acc + beta S) adds its bytes to every candidate's output traffic;
  // the last candidate is ranked for plans with a source only (the others keep their set)
  const bool source = (d.epilogue & kEpiSource) != 0;
  const double es = !source ? 0.0 : (d.epilogue & GEMM_EPI_SOURCE_F32) ? 4.0 : 2.0;
  int cus = 0, dev = 0;
  if (d.num_workers == 0) {
    if (hipGetDevice(&dev) != hipSuccess) return GEMM_ERR_HIP;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return GEMM_ERR_HIP;
  }
  const bool grouped = d.mapping == GEMM_MAP_GROUPED_M || d.mapping == GEMM_MAP_GROUPED_N;
  const bool blocked = d.mapping == GEMM_MAP_BLOCKED;
  out.clear();
  for (const ModelCand &c : cands) {
    if (!source && &c == &cands[std::size(cands) - 1]) continue;
    if (c.kind != KIND_COOP && d.K == 0) continue;  // the data-parallel kernels need K > 0
    const KernelEntry *e = nullptr;
    for (const KernelEntry &k : kKernels)
      if (k.dt == dt && k.bm == c.bm && k.bn == c.bn && k.kind == c.kind) {
        e = &k;
        break;
      }
    if (!e) continue;
    int occ = 1;
    int P = d.num_workers;
    if (P == 0) {
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, e->kernel(), e->threads, 0) !=
          hipSuccess)
        return GEMM_ERR_HIP;
      if (occ < 1 || e->kind == KIND_WIDE) occ = 1;  // wide-wave: one wave per SIMD by design
      P = cus * occ;
    }
    // without a device: one worker per CU
    const double ncu = d.num_workers == 0 ? (double)cus : (double)P;
    const int64_t Mt = cdiv(d.M, c.bm), Nt = cdiv(d.N, c.bn), tiles = Mt * Nt;
    const int64_t Kt = cdiv(d.K, e->bk), Keff = Kt * e->bk;
    int32_t dp = (int32_t)tiles, sk = 0;
    if (c.sched == GEMM_SCHED_STREAMK) {
      if (tiles > INT32_MAX) continue;
      streamk_plan(tiles, P, dp, sk);
      if (sk == 0 || Kt == 0) continue;  // no tail to balance: the data-parallel candidate covers it
      // the wide-wave kernel's separate reduction needs a band of at least P iterations
      if (c.kind == KIND_WIDE && ((int64_t)sk * Kt < P || (d.flags & GEMM_FLAG_STREAMK_CHAIN)))
        continue;
    }
    const int wgm = 2, wgn = e->threads / 64 / 2;  // waves along M and N
    const double t = (double)tiles, bm = c.bm, bn = c.bn, kk = (double)Keff;
    gemm_config_score r;
    memset(&r, 0, sizeof r);
    r.bm = c.bm;
    r.bn = c.bn;
    r.bk = e->bk;
    r.kernel = c.kind;
    r.sched = c.sched;
    r.workers = P;
    const int X = P % 8 == 0 ? 8 : 1;
    r.group = grouped ? (d.group > 0 ? d.group : choose_group(d.mapping, Mt, Nt, P / X)) : 1;
    r.group_n = 1;
    if (blocked) {
      r.group = d.group;
      r.group_n = d.group_n;
      choose_box(Mt, Nt, P / X, r.group, r.group_n);
    }
    const double bytes_l2 = t * (kk * (bm + bn) * eb + bm * bn * (ec + es));
    const double bytes_local = t * (kk * (bm + bn) * eb + kk * (bm * wgn + bn * wgm) * eb + bm * bn * ec);
    r.cycles_l2 = bytes_l2 / (ncu * kL2BytesPerClk);
    r.cycles_local = bytes_local / (ncu * kLdsBytesPerClk);
    r.cycles_mfma = 2.0 * bm * bn * kk * t /
                    (ncu * flop_per_clk_per_cu(dt) * kernel_efficiency(c.kind, c.bm, c.bn, dt));
    // wave efficiency over the CUs (a CU that runs fewer resident workgroups runs each faster)
    double items;  // items per worker, for the epilogues
    if (c.sched == GEMM_SCHED_STREAMK) {
      const double iters = t * (double)Kt;
      r.wave_efficiency = iters / (std::ceil(iters / P) * P);
      items = std::ceil((double)dp / P) + 2.0;  // data-parallel tiles and about two splits
    } else {
      const double waves = t / ncu, full = std::floor(waves), frac = waves - full;
      const bool narrow_single = full == 0 && c.kind == KIND_WIDE && (c.bn == 224 || c.bn == 192);
      const double e = narrow_single ? kPartialWaveExpNarrow : kPartialWaveExp;
      const double last = frac > 0 ? std::max(std::pow(frac, e), kMinPartialWave) : 0.0;
      r.wave_efficiency = tiles > 0 ? waves / (full + last) : 1.0;
      items = std::ceil(t / ncu);
    }
    const double stage_bytes = (bm + bn) * e->bk * eb;
    r.cycles_fixed = stage_bytes * (e->stages - 1) / kL2BytesPerClk + kLatencyClk +
                     items * (bm * bn * (ec + es) / kL2BytesPerClk + kLatencyClk / 2);
    if (sk > 0) {
      const double units_per_tile = std::ceil((double)P / sk);
      if ((d.flags & GEMM_FLAG_STREAMK_CHAIN) || (int64_t)sk * Kt < P) {
        // lock chain (a band with fewer iterations than units): a tile's non-empty splits add
        // into its workspace one after another
        const double splits = std::min(units_per_tile, (double)Kt);
        r.cycles_fixed += splits * (2.0 * bm * bn * 4.0 / kChainBytesPerClk + kChainHopClk);
      } else {  // separate reduction: every split writes its partial, the reduction reads it
        r.cycles_fixed +=
            2.0 * sk * units_per_tile * bm * bn * 4.0 / kDeviceBytesPerClk + kLatencyClk;
      }
      const double steps = (double)sk * (double)Kt / P;  // band k-steps per unit
      r.cycles_fixed += kSkBurstClk * std::max(0.0, 1.0 - steps / kSkBurstSteps);
    }
    const double worst = std::max(r.cycles_mfma, std::max(r.cycles_l2, r.cycles_local));
    r.score = worst / r.wave_efficiency + r.cycles_fixed;
    if (c.sched == GEMM_SCHED_STREAMK) r.score *= kStreamKFactor;
    out.push_back(r);
  }
  std::stable_sort(out.begin(), out.end(), [](const gemm_config_score &a,
                                              const gemm_config_score &b) { return a.score < b.score; });
  return out.empty() ? GEMM_ERR_UNSUPPORTED : GEMM_OK;
}

}  // namespace

struct gemm_plan {
  gemm_desc d;
  const KernelEntry *k;
  KernelArgs proto;     // everything but the pointers
  gemm_plan_info info;
  int64_t partial_off, lock_off, error_off, trace_off, ws_bytes;
};

// Workspace of gemm_run_noalloc: one array per GPU, allocated when the code object is loaded on
// that GPU and held until the process ends.  In host code `scratch` names a host-side stand-in
// for the symbol, not a device address: the kernels get the address hipGetSymbolAddress reports
// for the current device, looked up once per device and kept in scratch_addr.
static __device__ __align__(256) char scratch[GEMM_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_addr[kMaxDevices];

int scratch_of_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GEMM_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return GEMM_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_addr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GEMM_ERR_HIP;
    scratch_addr[dev] = p;
  }
  *out = scratch_addr[dev];
  return GEMM_OK;
}
}  // namespace

extern "C" {

const char *gemm_status_string(int status) {
  switch (status) {
    case GEMM_OK: return "ok";
    case GEMM_ERR_INVALID_ARG: return "invalid argument";
    case GEMM_ERR_UNSUPPORTED: return "unsupported problem or configuration";
    case GEMM_ERR_ALIGNMENT: return "device pointer misaligned";
    case GEMM_ERR_WORKSPACE: return "workspace missing or too small";
    case GEMM_ERR_HIP: return "HIP runtime error";
    case GEMM_ERR_CAPACITY: return "output buffer too small";
    case GEMM_ERR_SCRATCH_LIMIT:
      return "plan needs more workspace than the no-allocation entry point's scratch holds";
    default: return "unknown status";
  }
}

int gemm_create(const gemm_desc *desc, gemm_handle *out) {
  if (!desc || !out) return GEMM_ERR_INVALID_ARG;
  *out = nullptr;
  const gemm_desc d = *desc;
  if (d.M < 0 || d.N < 0 || d.K < 0) return GEMM_ERR_INVALID_ARG;
  if (d.dtype_ab != GEMM_BF16 && d.dtype_ab != GEMM_FP8_E4M3) return GEMM_ERR_INVALID_ARG;
  if (d.dtype_c != GEMM_F32 && d.dtype_c != GEMM_BF16 && d.dtype_c != GEMM_FP8_E4M3)
    return GEMM_ERR_INVALID_ARG;
  if (!epilogue_valid(d.epilogue)) return GEMM_ERR_INVALID_ARG;
  if ((d.layout_a != GEMM_ROW_MAJOR && d.layout_a != GEMM_COL_MAJOR) ||
      (d.layout_b != GEMM_ROW_MAJOR && d.layout_b != GEMM_COL_MAJOR))
    return GEMM_ERR_INVALID_ARG;
  if (d.mapping < GEMM_MAP_LINEAR_N || d.mapping > GEMM_MAP_MORTON) return GEMM_ERR_INVALID_ARG;
  const bool blocked = d.mapping == GEMM_MAP_BLOCKED;
  const bool grouped = d.mapping == GEMM_MAP_GROUPED_M || d.mapping == GEMM_MAP_GROUPED_N || blocked;
  if (grouped && d.group < 0) return GEMM_ERR_INVALID_ARG;  // 0: the planner picks G
  if (blocked && d.group_n < 0) return GEMM_ERR_INVALID_ARG;
  if (d.sk_groups < 0 || d.sk_groups > kMaxSkGroups) return GEMM_ERR_INVALID_ARG;
  if (d.sched < GEMM_SCHED_STATIC || d.sched > GEMM_SCHED_AUTO) return GEMM_ERR_INVALID_ARG;
  if (d.num_workers < 0 || d.bm < 0 || d.bn < 0 || d.bk < 0) return GEMM_ERR_INVALID_ARG;
  const uint32_t kind_flags =
      GEMM_FLAG_PINGPONG | GEMM_FLAG_COOPERATIVE | GEMM_FLAG_WIDE;
  if (d.flags & ~(GEMM_FLAG_TRACE | GEMM_FLAG_NO_XCD_REMAP | GEMM_FLAG_STREAMK_CHAIN | kind_flags |
                  GEMM_FLAG_TEST_SKIP_PUBLISH))
    return GEMM_ERR_INVALID_ARG;
  if (__builtin_popcount(d.flags & kind_flags) > 1) return GEMM_ERR_INVALID_ARG;

  // Well-formed; now what the kernels implement.
  if (d.layout_a != GEMM_ROW_MAJOR || d.layout_b != GEMM_COL_MAJOR) return GEMM_ERR_UNSUPPORTED;
  const int eb = d.dtype_ab == GEMM_BF16 ? 2 : 1;
  if ((d.K * eb) % 16 != 0) return GEMM_ERR_UNSUPPORTED;   // 16-byte rows for the LDS loads
  if (d.N % 8 != 0) return GEMM_ERR_UNSUPPORTED;           // 16-byte output rows
  // the buffer stores of C address a wave's output sub-tile with 32-bit byte offsets from its
  // origin: its last element (127 rows of up to 4-byte elements down: under 2^31 - 16 bytes
  // here) stays inside the buffer range, and an out-of-range offset (0x80000000 plus a row
  // offset) stays below 2^32
  if (d.N > ((int64_t)1 << 22)) return GEMM_ERR_UNSUPPORTED;
  if (d.K * eb > (int64_t)1 << 30) return GEMM_ERR_UNSUPPORTED;

  // the ping-pong and wide-wave kernels run data-parallel work only, on
  // 256 x 256 tiles
  const int force_kind = (d.flags & GEMM_FLAG_PINGPONG)      ? KIND_PP
                         : (d.flags & GEMM_FLAG_WIDE)        ? KIND_WIDE
                         : (d.flags & GEMM_FLAG_COOPERATIVE) ? KIND_COOP
                                                             : -1;
  // (the wide-wave kernel also runs Stream-K plans, with the separate-reduction fixup)
  const bool force_dp = force_kind == KIND_PP || force_kind == KIND_WIDE;
  const bool dp_only = force_kind == KIND_PP;
  if (force_dp && (d.K == 0 || (dp_only && (d.sched == GEMM_SCHED_STREAMK ||
                                            d.sched == GEMM_SCHED_AUTO))))
    return GEMM_ERR_UNSUPPORTED;
  // the fused epilogue runs on the wide-wave and cooperative kernels
  const bool fused = d.epilogue != 0 || d.dtype_c == GEMM_FP8_E4M3;
  if (fused && force_kind == KIND_PP) return GEMM_ERR_UNSUPPORTED;

  // Tile shape and scheduler: the cost model when everything is left to the planner, else
  // 256 x 256 unless asked otherwise or the problem has too few big tiles.
  int bm = d.bm, bn = d.bn;
  int model_sched = -1, model_kind = -1;
  if (bm == 0 && bn == 0 && d.bk == 0 && d.sched == GEMM_SCHED_AUTO && force_kind < 0) {
    std::vector<gemm_config_score> ranked;
    const int st = rank_configs(d, ranked);
    if (st != GEMM_OK) return st;
    bm = ranked[0].bm;
    bn = ranked[0].bn;
    model_sched = ranked[0].sched;
    model_kind = ranked[0].kernel;
  } else if (bm == 0 && bn == 0) {
    const int64_t big = cdiv(d.M, 256) * cdiv(d.N, 256);  // 0 for an empty output
    const bool streamk = d.sched == GEMM_SCHED_STREAMK;
    bm = bn = ((big >= 128 && !streamk) || force_dp) ? 256 : 128;
  } else if (bm == 0 || bn == 0) {
    bm = bn = (bm ? bm : bn);
  }
  const int want_dt = d.dtype_ab == GEMM_BF16 ? DT_BF16 : DT_FP8;
  const KernelEntry *by_kind[KIND_COUNT] = {};
  for (const KernelEntry &e : kKernels)
    if (e.dt == want_dt && e.bm == bm && e.bn == bn && (d.bk == 0 || d.bk == e.bk) &&
        !by_kind[e.kind])
      by_kind[e.kind] = &e;
  const KernelEntry *k = by_kind[force_kind >= 0 ? force_kind : KIND_COOP];
  // tile shapes only the wide-wave kernel has (which needs K > 0, like every data-parallel kernel)
  if (!k && force_kind < 0 && d.K > 0) k = by_kind[KIND_WIDE];
  if (!k) return GEMM_ERR_UNSUPPORTED;  // the schedule is planned with this one
  // rows of one tile must stay addressable by 32-bit buffer offsets
  if ((int64_t)bm * d.K * eb >= 0x7FFFFFF0ll || (int64_t)bn * d.K * eb >= 0x7FFFFFF0ll)
    return GEMM_ERR_UNSUPPORTED;

  const int64_t Mt = cdiv(d.M, bm), Nt = cdiv(d.N, bn);
  const int64_t tiles = Mt * Nt;
  if (Mt > INT32_MAX || Nt > INT32_MAX || tiles > INT32_MAX) return GEMM_ERR_UNSUPPORTED;

  int sched = model_sched >= 0 ? model_sched : d.sched;
  int workers = d.num_workers;
  if (sched != GEMM_SCHED_STATIC && workers == 0) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GEMM_ERR_HIP;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return GEMM_ERR_HIP;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k->kernel(), k->threads, 0) !=
        hipSuccess)
      return GEMM_ERR_HIP;
    if (per_cu < 1) per_cu = 1;
    // the wide-wave kernels, which take every plan with K > 0 unless another kernel is asked
    // for, run one workgroup -- one wave per SIMD -- per CU (two measured no faster for
    // data-parallel 128 x 128 tiles and 30 % slower for Stream-K)
    const bool wide_next = force_kind == KIND_WIDE ||
                           (force_kind < 0 && d.K > 0 && by_kind[KIND_WIDE] &&
                            model_kind != KIND_COOP);
    if (wide_next) per_cu = 1;
    workers = cus * per_cu;
  }
  if (sched == GEMM_SCHED_AUTO) {
    int32_t dp, sk;
    streamk_plan(tiles, workers, dp, sk);
    sched = sk > 0 ? GEMM_SCHED_STREAMK : GEMM_SCHED_PERSISTENT;
  }
  // Data-parallel work runs on the wide-wave kernel unless a kernel is asked for, or the cost
  // model picked another one (its grid was sized for that kernel above); so does Stream-K work,
  // unless it needs the lock chain (checked below, once the band is known).
  if (force_kind < 0 && d.K > 0 && (sched == GEMM_SCHED_STATIC || sched == GEMM_SCHED_PERSISTENT) &&
      (model_kind < 0 || model_kind == KIND_WIDE)) {
    if (by_kind[KIND_WIDE])
      k = by_kind[KIND_WIDE];
    else if (by_kind[KIND_PP] && !fused)
      k = by_kind[KIND_PP];
  } else if (force_kind < 0 && d.K > 0 && sched == GEMM_SCHED_STREAMK && by_kind[KIND_WIDE] &&
             !(d.flags & GEMM_FLAG_STREAMK_CHAIN) && (model_kind < 0 || model_kind == KIND_WIDE)) {
    k = by_kind[KIND_WIDE];
  }
  const int64_t Kt = cdiv(d.K, k->bk);  // the kernel's own k-tile depth
  if (Kt > INT32_MAX) return GEMM_ERR_UNSUPPORTED;

  SchedParams sp;
  memset(&sp, 0, sizeof sp);
  sp.Mt = (int32_t)Mt;
  sp.Nt = (int32_t)Nt;
  sp.Kt = (int32_t)Kt;
  sp.mapping = d.mapping;
  sp.G = grouped ? d.group : 1;
  sp.G2 = blocked ? d.group_n : 1;
  if (sched == GEMM_SCHED_STATIC) {
    sp.P = (int32_t)tiles;
    sp.dp_tiles = (int32_t)tiles;
    sp.sk_tiles = 0;
  } else if (sched == GEMM_SCHED_PERSISTENT || tiles == 0) {
    sched = sched == GEMM_SCHED_STREAMK ? sched : GEMM_SCHED_PERSISTENT;
    sp.P = (int32_t)(workers < tiles ? workers : tiles);
    sp.dp_tiles = (int32_t)tiles;
    sp.sk_tiles = 0;
  } else {
    sp.P = workers;
    streamk_plan(tiles, workers, sp.dp_tiles, sp.sk_tiles);
    if (Kt == 0) {  // nothing to split: every tile is written (with zeros) data-parallel
      sp.dp_tiles = (int32_t)tiles;
      sp.sk_tiles = 0;
    }
    if ((int64_t)sp.sk_tiles * Kt > INT32_MAX) return GEMM_ERR_UNSUPPORTED;
  }
  sp.X = (d.flags & GEMM_FLAG_NO_XCD_REMAP) ? 1 : kXcds;
  sp.sk_groups = d.sk_groups == 0 ? streamk_auto_groups(sp.P, sp.sk_tiles, Kt, kXcds)
                                  : streamk_groups(d.sk_groups, sp.P, sp.sk_tiles);
  if (blocked) {  // the planner's box: fewest operand strips per XCD's run of tiles
    choose_box(Mt, Nt, sp.P % sp.X == 0 ? sp.P / sp.X : sp.P, sp.G, sp.G2);
  } else if (grouped && d.group == 0)  // likewise for the strip width G
    sp.G = choose_group(d.mapping, Mt, Nt, sp.P % sp.X == 0 ? sp.P / sp.X : sp.P);
  if (sched != GEMM_SCHED_STATIC) choose_xcd_box(sp);
  sched_prepare(sp);

  gemm_plan *p = new (std::nothrow) gemm_plan;
  if (!p) return GEMM_ERR_INVALID_ARG;
  memset(p, 0, sizeof *p);
  p->d = d;
  p->k = k;

  // Stream-K fixup mode: the separate reduction needs every unit to own at least one iteration
  // (each group's band of T_g >= P / G iterations; the smallest group holds floor(sk_tiles / G)
  // tiles); otherwise, or when asked, the lock chain.
  const bool chain = (d.flags & GEMM_FLAG_STREAMK_CHAIN) ||
                     (int64_t)(sp.sk_tiles / sp.sk_groups) * Kt < sp.sk_gunits;
  const int sk_mode = chain ? SK_CHAIN : SK_SEPARATE;
  if (chain && sp.sk_tiles > 0 && k->kind == KIND_WIDE) {  // the wide-wave kernel has no chain
    if (force_kind == KIND_WIDE || !by_kind[KIND_COOP]) {
      delete p;
      return GEMM_ERR_UNSUPPORTED;
    }
    k = by_kind[KIND_COOP];
    p->k = k;
  }
  // partial tiles: one per split tile (chain), or one per (unit, tile) pair (separate: per group,
  // unit + the group's tile, P / G + ceil(sk_tiles / G) of them)
  const int64_t partial_slots = sp.sk_tiles == 0 ? 0 : (chain ? sp.sk_tiles : sk_partial_slots(sp));
  // the kernels address the partial area with 32-bit buffer offsets
  if (partial_slots * (int64_t)bm * bn * 4 > 0x7FFFFFF0ll) {
    delete p;
    return GEMM_ERR_UNSUPPORTED;
  }

  // Workspace: [partials][locks or counters: sk_tiles int][error word][trace]
  int64_t off = 0;
  p->partial_off = p->lock_off = p->error_off = p->trace_off = -1;
  if (sp.sk_tiles > 0 || (d.flags & GEMM_FLAG_TRACE)) {
    p->partial_off = 0;
    off = partial_slots * (int64_t)bm * bn * 4;
    p->lock_off = off;
    off = align_up(off + sp.sk_tiles * 4, 256);
    p->error_off = off;
    off += 256;
    if (d.flags & GEMM_FLAG_TRACE) {
      p->trace_off = off;
      off += (int64_t)sp.P * kTraceCap * 8 * 4;
    }
  }
  p->ws_bytes = off;

  KernelArgs &a = p->proto;
  memset(&a, 0, sizeof a);
  a.M = d.M;
  a.N = d.N;
  a.K = d.K;
  a.lda_bytes = d.K * eb;
  a.ldb_bytes = d.K * eb;
  a.ldc = d.N;
  a.sp = sp;
  a.out_bf16 = d.dtype_c == GEMM_BF16;
  a.out_fp8 = d.dtype_c == GEMM_FP8_E4M3;
  a.epi = d.epilogue;
  a.flags = d.flags;
  a.trace_cap = kTraceCap;
  a.max_spin = (d.flags & GEMM_FLAG_TEST_SKIP_PUBLISH) ? kTestSpin : kDefaultSpin;
  a.sk_mode = sk_mode;

  gemm_plan_info &in = p->info;
  in.bm = k->bm;
  in.bn = k->bn;
  in.bk = k->bk;
  in.stages = k->stages;
  in.threads = k->threads;
  in.grid = sp.P;
  in.mt = sp.Mt;
  in.nt = sp.Nt;
  in.kt = sp.Kt;
  in.sched = sched;
  in.xcds = sp.X;
  in.lds_bytes = k->lds;
  in.dp_tiles = sp.dp_tiles;
  in.sk_tiles = sp.sk_tiles;
  in.workspace_bytes = p->ws_bytes;
  in.trace_offset = p->trace_off;
  in.trace_capacity = (d.flags & GEMM_FLAG_TRACE) ? kTraceCap : 0;
  in.error_offset = (int32_t)p->error_off;
  in.streamk_mode = sk_mode;
  in.kernel = k->kind;
  in.group = sp.G;
  in.group_n = sp.G2;
  in.sk_groups = sp.sk_groups;
  in.xcd_box_r = sp.xbox_r;
  in.xcd_box_c = sp.xbox_c;
  *out = p;
  return GEMM_OK;
}

int gemm_rank_configs(const gemm_desc *desc, gemm_config_score *items, size_t cap,
                      size_t *n_out) {
  if (!desc || !n_out || (cap && !items)) return GEMM_ERR_INVALID_ARG;
  *n_out = 0;
  const gemm_desc d = *desc;
  if (d.M < 0 || d.N < 0 || d.K < 0 || d.num_workers < 0 || d.group < 0) return GEMM_ERR_INVALID_ARG;
  if (d.dtype_ab != GEMM_BF16 && d.dtype_ab != GEMM_FP8_E4M3) return GEMM_ERR_INVALID_ARG;
  if (d.dtype_c != GEMM_F32 && d.dtype_c != GEMM_BF16 && d.dtype_c != GEMM_FP8_E4M3)
    return GEMM_ERR_INVALID_ARG;
  if (!epilogue_valid(d.epilogue)) return GEMM_ERR_INVALID_ARG;
  if (d.mapping < GEMM_MAP_LINEAR_N || d.mapping > GEMM_MAP_MORTON) return GEMM_ERR_INVALID_ARG;
  if (d.mapping == GEMM_MAP_BLOCKED && d.group_n < 0) return GEMM_ERR_INVALID_ARG;
  if (d.sk_groups < 0 || d.sk_groups > kMaxSkGroups) return GEMM_ERR_INVALID_ARG;
  std::vector<gemm_config_score> ranked;
  const int st = rank_configs(d, ranked);
  if (st != GEMM_OK) return st;
  *n_out = ranked.size();
  if (cap < ranked.size()) return GEMM_ERR_CAPACITY;
  for (size_t i = 0; i < ranked.size(); ++i) items[i] = ranked[i];
  return GEMM_OK;
}

int gemm_workspace_bytes(gemm_handle h, size_t *bytes) {
  if (!h || !bytes) return GEMM_ERR_INVALID_ARG;
  *bytes = (size_t)h->ws_bytes;
  return GEMM_OK;
}

int gemm_plan_get(gemm_handle h, gemm_plan_info *info) {
  if (!h || !info) return GEMM_ERR_INVALID_ARG;
  *info = h->info;
  return GEMM_OK;
}

int gemm_run(gemm_handle h, const void *A, const void *B, void *C, const float *scale_a,
             const float *scale_b, void *workspace, size_t workspace_bytes, void *stream) {
  return gemm_run_ex(h, A, B, C, scale_a, scale_b, nullptr, workspace, workspace_bytes, stream);
}

int gemm_run_ex(gemm_handle h, const void *A, const void *B, void *C, const float *scale_a,
                const float *scale_b, const gemm_epilogue_args *epi, void *workspace,
                size_t workspace_bytes, void *stream) {
  if (!h) return GEMM_ERR_INVALID_ARG;
  // epilogue operands: checked before the empty-output return, so a bad call fails alike
  const uint32_t ebits = h->d.epilogue;
  const bool need_bias = ebits & (GEMM_EPI_BIAS_ROW | GEMM_EPI_BIAS_COL);
  const bool need_amax = ebits & GEMM_EPI_AMAX;
  const bool out_fp8 = h->d.dtype_c == GEMM_FP8_E4M3;
  if ((need_bias || need_amax || out_fp8) && !epi) return GEMM_ERR_INVALID_ARG;
  if ((need_bias && !epi->bias) || (need_amax && !epi->amax) || (out_fp8 && !epi->scale_d))
    return GEMM_ERR_INVALID_ARG;
  // a source bit needs beta; with beta == 0 no source is read
  const uint32_t src_bit = ebits & kEpiSource;
  if (src_bit && !epi) return GEMM_ERR_INVALID_ARG;
  const bool need_source = src_bit && epi->beta != 0.0f;
  if (need_source && !epi->source) return GEMM_ERR_INVALID_ARG;
  if (need_source && ((uintptr_t)epi->source & (src_bit == GEMM_EPI_SOURCE_F32 ? 15 : 7)))
    return GEMM_ERR_ALIGNMENT;
  if ((need_bias && ((uintptr_t)epi->bias & 15)) || (need_amax && ((uintptr_t)epi->amax & 3)) ||
      (out_fp8 && ((uintptr_t)epi->scale_d & 3)))
    return GEMM_ERR_ALIGNMENT;
  if (h->info.grid == 0) return GEMM_OK;  // empty output: nothing to compute
  if (!C || (h->d.K > 0 && (!A || !B))) return GEMM_ERR_INVALID_ARG;  // K == 0 reads no operand
  const bool fp8 = h->d.dtype_ab == GEMM_FP8_E4M3;
  if (fp8 && (!scale_a || !scale_b)) return GEMM_ERR_INVALID_ARG;
  if (((uintptr_t)A | (uintptr_t)B | (uintptr_t)C) & 15) return GEMM_ERR_ALIGNMENT;
  if (h->d.K == 0) A = B = C;  // never dereferenced; keeps the kernel's resource bases non-null
  if (fp8 && (((uintptr_t)scale_a | (uintptr_t)scale_b) & 3)) return GEMM_ERR_ALIGNMENT;
  if (h->ws_bytes > 0) {
    if (!workspace || workspace_bytes < (size_t)h->ws_bytes) return GEMM_ERR_WORKSPACE;
    if ((uintptr_t)workspace & 15) return GEMM_ERR_ALIGNMENT;
  }
  hipStream_t s = (hipStream_t)stream;
  KernelArgs a = h->proto;
  a.A = (const char *)A;
  a.B = (const char *)B;
  a.C = (char *)C;
  a.scale_a = scale_a;
  a.scale_b = scale_b;
  if (need_source) {
    a.src = (const char *)epi->source;
    a.beta = epi->beta;
  } else {
    a.epi &= ~kEpiSource;  // beta == 0: Z = alpha Acc, and nothing is read
  }
  if (need_bias) a.bias = epi->bias;
  if (need_amax) a.amax = epi->amax;
  if (out_fp8) a.scale_d = epi->scale_d;
  if (h->ws_bytes > 0) {
    char *ws = (char *)workspace;
    a.partials = (float *)(ws + h->partial_off);
    a.locks = (int *)(ws + h->lock_off);
    a.error_word = (int *)(ws + h->error_off);
    a.trace = h->trace_off >= 0 ? (int *)(ws + h->trace_off) : nullptr;
    // zero the locks (and the error word and trace, which follow them)
    const int64_t first = h->lock_off;
    const int64_t n_ints = (h->ws_bytes - first) / 4;
    const int threads = 256;
    const int blocks = (int)cdiv(n_ints, threads);
    hipLaunchKernelGGL(clear_ints_kernel, dim3(blocks), dim3(threads), 0, s,
                       (int *)(ws + first), (int)n_ints);
    if (hipGetLastError() != hipSuccess) return GEMM_ERR_HIP;
  }
  const bool ragged_k = h->d.K % h->k->bk != 0;
  if (h->k->launch(a, h->info.grid, ragged_k, s) != hipSuccess) return GEMM_ERR_HIP;
  return GEMM_OK;
}

int gemm_run_noalloc(gemm_handle h, const void *A, const void *B, void *C, const float *scale_a,
                     const float *scale_b, const gemm_epilogue_args *epi, void *stream) {
  if (!h) return GEMM_ERR_INVALID_ARG;
  if (h->ws_bytes > (int64_t)GEMM_NOALLOC_SCRATCH_BYTES) return GEMM_ERR_SCRATCH_LIMIT;
  void *ws = nullptr;
  if (h->ws_bytes > 0 && h->info.grid > 0) {
    const int st = scratch_of_current_device(&ws);
    if (st != GEMM_OK) return st;
  }
  return gemm_run_ex(h, A, B, C, scale_a, scale_b, epi, ws, ws ? (size_t)h->ws_bytes : 0, stream);
}

int gemm_destroy(gemm_handle h) {
  if (!h) return GEMM_ERR_INVALID_ARG;
  delete h;
  return GEMM_OK;
}

int gemm_schedule_enumerate(gemm_handle h, gemm_work_item *items, size_t cap, size_t *n_out) {
  if (!h || !n_out || (cap > 0 && !items)) return GEMM_ERR_INVALID_ARG;
  const SchedParams &sp = h->proto.sp;
  size_t n = 0;
  for (int32_t b = 0; b < sp.P; ++b) {
    Cursor c;
    cursor_init(sp, b, c);
    WorkItem w;
    int32_t seq = 0;
    while (cursor_next(sp, c, w)) {
      if (n < cap) {
        gemm_work_item &it = items[n];
        it.worker = b;
        it.seq = seq;
        it.tile = (int32_t)w.tile;
        it.tile_m = w.m;
        it.tile_n = w.n;
        it.k_begin = w.kb;
        it.k_end = w.ke;
        it.role = w.role;
      }
      ++n;
      ++seq;
    }
  }
  *n_out = n;
  return n > cap ? GEMM_ERR_CAPACITY : GEMM_OK;
}

}  // extern "C"
