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

#include "../../include/gemm.h"
#include "gemm_kernel.h"
#include "sched.h"

namespace {

using namespace dg;

// Tile configurations: TileCfg<dtype, BM, BN, BK, wave rows, wave columns, stages, swizzle>.
// SWZ spreads the 16 rows one 16-lane LDS read phase touches over 16 distinct 16-byte bank groups
// (1 for 128-byte rows, 2 for 64-byte rows).  Defaults (first match per tile shape): 8 waves of
// 128 x 64 sub-tiles with 2 stages of 64 KiB -- two waves per SIMD hide each other's LDS waits.
// The ping-pong kernel (GEMM_FLAG_PINGPONG) runs the same 256 x 256 tiles with two wave groups.
using CfgBf16_256pp = TileCfg<DT_BF16, 256, 256, 64, 2, 4, 2, 1>;
using CfgBf16_256 = TileCfg<DT_BF16, 256, 256, 64, 2, 4, 2, 1>;
using CfgBf16_128 = TileCfg<DT_BF16, 128, 128, 64, 2, 2, 2, 1>;
using CfgFp8_256pp = TileCfg<DT_FP8, 256, 256, 128, 2, 4, 2, 1>;
using CfgBf16_256vs = TileCfg<DT_BF16, 256, 256, 64, 2, 2, 2, 1>;
using CfgFp8_256vs = TileCfg<DT_FP8, 256, 256, 128, 2, 2, 2, 1>;
using CfgFp8_256 = TileCfg<DT_FP8, 256, 256, 128, 2, 4, 2, 1>;
using CfgFp8_128 = TileCfg<DT_FP8, 128, 128, 128, 2, 2, 2, 1>;
// The wide-wave kernel (GEMM_FLAG_WIDE): four waves of 128 x 128, two stages.
using CfgBf16_256w = TileCfg<DT_BF16, 256, 256, 64, 2, 2, 2, 1, 16>;  // 16 x 16 x 32 MFMAs
using CfgFp8_256w = TileCfg<DT_FP8, 256, 256, 128, 2, 2, 2, 1, 16>;  // 16 x 16 x 128 MFMAs

typedef hipError_t (*launch_fn)(const KernelArgs &, int grid, bool ragged_k, hipStream_t);
typedef const void *(*kernel_fn)();

template <class CFG>
hipError_t launch_cfg(const KernelArgs &a, int grid, bool ragged_k, hipStream_t s) {
  if (ragged_k)
    hipLaunchKernelGGL((gemm_kernel<CFG, true>), dim3(grid), dim3(CFG::THREADS), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_kernel<CFG, false>), dim3(grid), dim3(CFG::THREADS), 0, s, a);
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
hipError_t launch_vs(const KernelArgs &a, int grid, bool ragged_k, hipStream_t s) {
  if (ragged_k)
    hipLaunchKernelGGL((gemm_kernel_vs<CFG, true>), dim3(grid), dim3(CFG::THREADS), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_kernel_vs<CFG, false>), dim3(grid), dim3(CFG::THREADS), 0, s, a);
  return hipGetLastError();
}
template <class CFG>
const void *kernel_of_vs() {
  return (const void *)&gemm_kernel_vs<CFG, false>;
}

// k-tiles one MFMA deep (e4m3 16 x 16 x 128) take the single-A-buffer form of the schedule
template <class CFG, bool RAGGED_K>
constexpr auto wide_kernel() {
  if constexpr (CFG::KSUB == 1)
    return &gemm_kernel_wide1<CFG, RAGGED_K>;
  else
    return &gemm_kernel_wide<CFG, RAGGED_K>;
}
template <class CFG>
hipError_t launch_wide(const KernelArgs &a, int grid, bool ragged_k, hipStream_t s) {
  if (ragged_k)
    hipLaunchKernelGGL((wide_kernel<CFG, true>()), dim3(grid), dim3(CFG::THREADS), 0, s, a);
  else
    hipLaunchKernelGGL((wide_kernel<CFG, false>()), dim3(grid), dim3(CFG::THREADS), 0, s, a);
  return hipGetLastError();
}
template <class CFG>
const void *kernel_of_wide() {
  return (const void *)wide_kernel<CFG, false>();
}

// kind: KIND_COOP runs every plan; the others run data-parallel work only (no Stream-K splits,
// K > 0)
enum { KIND_COOP = 0, KIND_PP = 1, KIND_VS = 2, KIND_WIDE = 3, KIND_COUNT = 4 };
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
constexpr KernelEntry entry_vs() {
  return KernelEntry{CFG::DT, CFG::BM, CFG::BN, CFG::BK, CFG::THREADS, CFG::STAGES,
                     CFG::LDS_BYTES, KIND_VS, &launch_vs<CFG>, &kernel_of_vs<CFG>};
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
    entry_vs<CfgBf16_256vs>(),
    entry_vs<CfgFp8_256vs>(),
    entry_wide<CfgBf16_256w>(),
    entry_wide<CfgFp8_256w>(),
    entry<CfgFp8_128>(),
};

constexpr int kXcds = 8;           // MI355X: 8 accelerator complex dies, one L2 each
constexpr int kDefaultSpin = 1 << 24;
constexpr int kTestSpin = 4096;
constexpr int kTraceCap = 64;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t align_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

}  // namespace

struct gemm_plan {
  gemm_desc d;
  const KernelEntry *k;
  KernelArgs proto;     // everything but the pointers
  gemm_plan_info info;
  int64_t partial_off, lock_off, error_off, trace_off, ws_bytes;
};

extern "C" {

const char *gemm_status_string(int status) {
  switch (status) {
    case GEMM_OK: return "ok";
    case GEMM_ERR_INVALID_ARG: return "invalid argument";
    case GEMM_ERR_UNSUPPORTED: return "unsupported problem or configuration";
    case GEMM_ERR_ALIGNMENT: return "device pointer not 16-byte aligned";
    case GEMM_ERR_WORKSPACE: return "workspace missing or too small";
    case GEMM_ERR_HIP: return "HIP runtime error";
    case GEMM_ERR_CAPACITY: return "output buffer too small";
    default: return "unknown status";
  }
}

int gemm_create(const gemm_desc *desc, gemm_handle *out) {
  if (!desc || !out) return GEMM_ERR_INVALID_ARG;
  *out = nullptr;
  const gemm_desc d = *desc;
  if (d.M < 0 || d.N < 0 || d.K < 0) return GEMM_ERR_INVALID_ARG;
  if (d.dtype_ab != GEMM_BF16 && d.dtype_ab != GEMM_FP8_E4M3) return GEMM_ERR_INVALID_ARG;
  if (d.dtype_c != GEMM_F32 && d.dtype_c != GEMM_BF16) return GEMM_ERR_INVALID_ARG;
  if ((d.layout_a != GEMM_ROW_MAJOR && d.layout_a != GEMM_COL_MAJOR) ||
      (d.layout_b != GEMM_ROW_MAJOR && d.layout_b != GEMM_COL_MAJOR))
    return GEMM_ERR_INVALID_ARG;
  if (d.mapping < GEMM_MAP_LINEAR_N || d.mapping > GEMM_MAP_GROUPED_N) return GEMM_ERR_INVALID_ARG;
  const bool grouped = d.mapping == GEMM_MAP_GROUPED_M || d.mapping == GEMM_MAP_GROUPED_N;
  if (grouped && d.group < 1) return GEMM_ERR_INVALID_ARG;
  if (d.sched < GEMM_SCHED_STATIC || d.sched > GEMM_SCHED_AUTO) return GEMM_ERR_INVALID_ARG;
  if (d.num_workers < 0 || d.bm < 0 || d.bn < 0 || d.bk < 0) return GEMM_ERR_INVALID_ARG;
  const uint32_t kind_flags =
      GEMM_FLAG_PINGPONG | GEMM_FLAG_COOPERATIVE | GEMM_FLAG_REGSTAGED | GEMM_FLAG_WIDE;
  if (d.flags & ~(GEMM_FLAG_TRACE | GEMM_FLAG_NO_XCD_REMAP | GEMM_FLAG_STREAMK_CHAIN | kind_flags |
                  GEMM_FLAG_TEST_SKIP_PUBLISH))
    return GEMM_ERR_INVALID_ARG;
  if (__builtin_popcount(d.flags & kind_flags) > 1) return GEMM_ERR_INVALID_ARG;

  // Well-formed; now what the kernels implement.
  if (d.layout_a != GEMM_ROW_MAJOR || d.layout_b != GEMM_COL_MAJOR) return GEMM_ERR_UNSUPPORTED;
  const int eb = d.dtype_ab == GEMM_BF16 ? 2 : 1;
  if ((d.K * eb) % 16 != 0) return GEMM_ERR_UNSUPPORTED;   // 16-byte rows for the LDS loads
  if (d.N % 8 != 0) return GEMM_ERR_UNSUPPORTED;           // 16-byte output rows
  if (d.K * eb > (int64_t)1 << 30) return GEMM_ERR_UNSUPPORTED;

  // the ping-pong, register-staged and wide-wave kernels run data-parallel work only, on
  // 256 x 256 tiles
  const int force_kind = (d.flags & GEMM_FLAG_PINGPONG)      ? KIND_PP
                         : (d.flags & GEMM_FLAG_REGSTAGED)   ? KIND_VS
                         : (d.flags & GEMM_FLAG_WIDE)        ? KIND_WIDE
                         : (d.flags & GEMM_FLAG_COOPERATIVE) ? KIND_COOP
                                                             : -1;
  const bool force_dp = force_kind == KIND_PP || force_kind == KIND_VS || force_kind == KIND_WIDE;
  if (force_dp && (d.K == 0 || d.sched == GEMM_SCHED_STREAMK || d.sched == GEMM_SCHED_AUTO))
    return GEMM_ERR_UNSUPPORTED;

  // Tile shape: 256 x 256 unless asked otherwise or the problem has too few big tiles.
  int bm = d.bm, bn = d.bn;
  if (bm == 0 && bn == 0) {
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
  if (!k) return GEMM_ERR_UNSUPPORTED;  // the schedule is planned with this one
  // rows of one tile must stay addressable by 32-bit buffer offsets
  if ((int64_t)bm * d.K * eb >= 0x7FFFFFF0ll || (int64_t)bn * d.K * eb >= 0x7FFFFFF0ll)
    return GEMM_ERR_UNSUPPORTED;

  const int64_t Mt = cdiv(d.M, bm), Nt = cdiv(d.N, bn);
  const int64_t tiles = Mt * Nt;
  if (Mt > INT32_MAX || Nt > INT32_MAX || tiles > INT32_MAX) return GEMM_ERR_UNSUPPORTED;

  int sched = d.sched;
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
    workers = cus * per_cu;
  }
  if (sched == GEMM_SCHED_AUTO) {
    int32_t dp, sk;
    streamk_plan(tiles, workers, dp, sk);
    sched = sk > 0 ? GEMM_SCHED_STREAMK : GEMM_SCHED_PERSISTENT;
  }
  // Data-parallel work on 256 x 256 tiles runs on the wide-wave kernel unless a kernel is asked
  // for (all of them hold one workgroup per CU, so the worker count stays).
  if (force_kind < 0 && d.K > 0 && (sched == GEMM_SCHED_STATIC || sched == GEMM_SCHED_PERSISTENT)) {
    if (by_kind[KIND_WIDE])
      k = by_kind[KIND_WIDE];
    else if (by_kind[KIND_PP])
      k = by_kind[KIND_PP];
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
  sched_prepare(sp);

  gemm_plan *p = new (std::nothrow) gemm_plan;
  if (!p) return GEMM_ERR_INVALID_ARG;
  memset(p, 0, sizeof *p);
  p->d = d;
  p->k = k;

  // Stream-K fixup mode: the separate reduction needs every unit to own at least one iteration
  // (band of T >= P iterations); otherwise, or when asked, the lock chain.
  const bool chain = (d.flags & GEMM_FLAG_STREAMK_CHAIN) || (int64_t)sp.sk_tiles * Kt < sp.P;
  const int sk_mode = chain ? SK_CHAIN : SK_SEPARATE;
  // partial tiles: one per split tile (chain), or one per (unit, tile) pair, indexed unit + tile,
  // at most P + sk_tiles of them (separate)
  const int64_t partial_slots = sp.sk_tiles == 0 ? 0 : (chain ? sp.sk_tiles : sp.P + sp.sk_tiles);
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
  *out = p;
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
  if (!h) return GEMM_ERR_INVALID_ARG;
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
