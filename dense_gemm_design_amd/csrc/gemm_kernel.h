// Persistent tiled GEMM kernel for gfx950 (MI355X): C = alpha * A x B with MFMA, FP32 accumulate.
//
// One workgroup of WGM x WGN waves owns a BM x BN output tile at a time; each wave owns a
// (BM/WGM) x (BN/WGN) sub-tile of 32 x 32 MFMA blocks held in accumulator registers.  The work
// list of a workgroup (data-parallel tiles, then Stream-K splits) comes from sched.h.
//
// K-loop: an S-stage ring of LDS buffers ("H100 Kernel Design" lesson, sections 4-6).  Stage
// s = c mod S holds the A and B k-tiles of the workgroup's c-th k-step; the ring runs across
// work items, so the next tile's first k-tiles are in flight while the current tile finishes.
//  * Producer phase: every wave issues its share of the stage's 1 KiB buffer loads that write
//    LDS directly (buffer_load_dwordx4 ... lds), S-1 k-steps ahead of the MFMA.  These play the
//    part of the pages' TMA copies; lanes whose element lies outside A or B are pointed past the
//    buffer's end and fill zeros, which handles ragged M, N and K edges.
//  * FULL(c): each wave waits until its own loads of step c have landed (s_waitcnt vmcnt(n),
//    n = loads it issued after step c), then all waves meet at s_barrier.  After the barrier every
//    wave's bytes of step c are in LDS.
//  * EMPTY(c-1): the same barrier is also the release of stage (c-1) mod S: each wave reached it
//    only after its MFMAs of step c-1 consumed their ds_read results, so the producer may refill
//    that stage with step c+S-1 right after the barrier.  The ring position (stage, phase =
//    floor(c / S) & 1, count = c) lives in scalar registers; the phase is implicit in c.
//  * Consumer phase: ds_read_b128 of the A and B fragments of the wave's sub-tile, MFMA chain.
// With one wave per SIMD a burst of memory instructions stalls the only instruction stream that
// feeds the MFMA pipe, so each k-step is software-pipelined at the instruction level: the MFMAs of
// a sub-step are issued one by one and the LDS reads of the next sub-step's fragments and the
// producer's loads are placed between them (a fixed per-slot plan, below); the handshake sits a
// quarter of the way into the last sub-step, so the MFMA pipe still has queued work across it.
// LDS rows are XOR-swizzled in 16-byte chunks (chunk' = chunk ^ f(row)), the gfx950 counterpart
// of the pages' 128-byte swizzle ("H100 cuTensorMap" lesson, section 11; "H100 WGMMA part 1",
// section 11), so that the 32 rows one MFMA operand read touches spread over all LDS banks.
//
// Epilogue ("H100 Kernel Design" lesson, section 12): Z = alpha * Acc, cast to the output type,
// store -- or, for a Stream-K split, the fixup of "H100 Stream-K" lesson section 6: partial sums
// go through a per-tile FP32 workspace slot guarded by a lock counting the k-tiles already
// reduced; each split waits until the lock equals its K_idx (deterministic left-to-right order),
// the final split adds the slot to its accumulators and runs the epilogue.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "sched.h"

namespace dg {

typedef __attribute__((address_space(3))) char lds_t;
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

enum { DT_BF16 = 0, DT_FP8 = 1 };

// Flags shared with the C ABI (gemm.h).
enum : uint32_t { KF_TRACE = 0x1u, KF_TEST_SKIP_PUBLISH = 0x100u };

// Stream-K fixup modes.
enum { SK_CHAIN = 0, SK_SEPARATE = 1 };

struct KernelArgs {
  const char *A;           // M x K, row pitch lda_bytes
  const char *B;           // N x K (K x N column-major), row pitch ldb_bytes
  char *C;                 // M x N row-major, ldc elements per row
  const float *scale_a;    // FP8 only
  const float *scale_b;
  float *partials;         // Stream-K partial tiles, BM*BN floats each
  int *locks;              // per split tile: lock (chain mode) or arrival counter (separate)
  int *error_word;
  int *trace;              // 8 ints per record, trace_cap records per workgroup
  int64_t M, N, K;
  int64_t lda_bytes, ldb_bytes, ldc;
  SchedParams sp;
  int32_t out_bf16;
  uint32_t flags;
  int32_t trace_cap;
  int32_t max_spin;
  int32_t sk_mode;         // SK_CHAIN or SK_SEPARATE
  uint32_t epi;            // fused epilogue: EPI_* bits (0 = alpha and the cast only)
  const float *bias;       // EPI_BIAS_ROW: M floats, EPI_BIAS_COL: N floats
  const float *scale_d;    // e4m3 output: its dequantisation scale (a code q stands for s_d * q)
  float *amax;             // EPI_AMAX: max |Y| is folded in (atomic max on the float's bits)
  int32_t out_fp8;         // C holds e4m3 codes
  float beta;              // EPI_SRC_*: the source's factor
  const char *src;         // EPI_SRC_*: S, M x N row-major, ldc elements per row (may be C)
};

template <int DT_, int BM_, int BN_, int BK_, int WGM_, int WGN_, int STAGES_, int SWZ_,
          int MI_ = 32>
struct TileCfg {
  static constexpr int DT = DT_, BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_;
  static constexpr int STAGES = STAGES_, SWZ = SWZ_;
  // MFMA block edge: 32 (32 x 32 blocks, two k-groups of lanes) or 16 (16 x 16, four k-groups)
  static constexpr int MI = MI_, KG = 64 / MI_;
  static constexpr int WAVES = WGM * WGN, THREADS = WAVES * 64;
  // waves of this workgroup per SIMD (4 SIMDs per CU); with two, each wave gets half the
  // register file and the other wave of the SIMD issues MFMAs while this one waits on LDS
  static constexpr int WAVES_PER_SIMD = (WAVES + 3) / 4;
  static constexpr int WM = BM / WGM, WN = BN / WGN;     // wave sub-tile
  static constexpr int FM = WM / MI, FN = WN / MI;       // MI x MI MFMA blocks per wave
  static constexpr int EB = DT == DT_BF16 ? 2 : 1;       // bytes per element
  static constexpr int ROWB = BK * EB;                   // bytes of one tile row in LDS
  static constexpr int CH = ROWB / 16;                   // 16-byte chunks per row
  static constexpr int RPL = 1024 / ROWB;                // rows per wave-wide 1 KiB load
  static constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static constexpr int LA = A_BYTES / 1024 / WAVES;      // loads per wave per stage (A)
  static constexpr int LB = B_BYTES / 1024 / WAVES;
  // reduction depth of one MFMA: 32x32x16 / 16x16x32 bf16, 32x32x64 / 16x16x128 e4m3
  static constexpr int KMFMA = (DT == DT_BF16 ? 16 : 64) * (MI == 16 ? 2 : 1);
  static constexpr int KSUB = BK / KMFMA;                // MFMAs along K per k-tile
  static constexpr int CPL = KMFMA * EB / (KG * 16);     // 16-byte chunks per lane per operand
  static_assert(ROWB == 64 || ROWB == 128, "tile rows must be 64 or 128 bytes");
  static_assert(A_BYTES % (1024 * WAVES) == 0 && B_BYTES % (1024 * WAVES) == 0, "load split");
  static_assert(MI == 32 || MI == 16, "MFMA block edge");
  static_assert(WM % MI == 0 && WN % MI == 0, "wave tile must be whole MFMA blocks");
  static_assert(BK % KMFMA == 0, "k-tile must hold whole MFMAs");
  static_assert(LA + LB <= 63, "vmcnt range");
  static_assert(LDS_BYTES <= 160 * 1024, "gfx950 LDS per workgroup");
  static_assert((MI >> SWZ) % CH == 0, "swizzle must not depend on the MFMA row block");
};

// ---- small device helpers ------------------------------------------------------------------

__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until this wave's loads of a k-step have landed, given that `steps_after` later k-steps
// (L loads each) were issued after it: s_waitcnt vmcnt(min(63, steps_after * L)).  Vector memory
// operations of one wave complete in issue order, so at most that many can still be pending.
template <int L>
__device__ __forceinline__ void wait_loads_after(int steps_after) {
  if (steps_after <= 0) wait_vmcnt<0>();
  else if (steps_after == 1) wait_vmcnt<L>();
  else if (steps_after == 2) wait_vmcnt<(2 * L > 63 ? 63 : 2 * L)>();
  else if (steps_after == 3) wait_vmcnt<(3 * L > 63 ? 63 : 3 * L)>();
  else wait_vmcnt<(4 * L > 63 ? 63 : 4 * L)>();
}

// A buffer resource over [base, base + bytes): every access at or past the end reads zero or is
// dropped.  bytes <= 0 (a region that starts past the end of its matrix) gives an empty range.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char *base, int64_t bytes) {
  const int32_t n = bytes <= 0 ? 0 : bytes > 0x7FFFFFF0ll ? 0x7FFFFFF0 : (int32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, n, 0x00020000);
}

constexpr uint32_t kOOB = 0x80000000u;  // any offset >= num_records reads as zero

// Stream-K partial sums move between workgroups on different XCDs, each with its own L2.  They
// are written and read with device-coherent buffer accesses (cache-policy bit sc1: the line is
// not served from or left dirty in a non-coherent L2), and ordered by s_waitcnt vmcnt(0) plus the
// workgroup barrier before the flag store -- instead of agent-scope fences, which write back and
// invalidate the whole L2 of the XCD.  The accesses are compiler builtins, so the compiler itself
// places the waits before each use of a loaded value.  Offsets are bytes from the start of the
// partial-tile area, which the planner keeps below 2 GiB.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kCachePolicySC1 = 16;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t partial_rsrc(const float *partials) {
  return __builtin_amdgcn_make_buffer_rsrc((void *)partials, (short)0, 0x7FFFFFF0, 0x00020000);
}
__device__ __forceinline__ void store_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kCachePolicySC1);
}
__device__ __forceinline__ f32x4 load_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCachePolicySC1));
}

// Two floats to bf16 (round to nearest even), lo in the low half.  Converted as one two-element
// vector, so that the compiler emits one v_cvt_pk_bf16_f32 for both; element by element it emits
// one per value plus a shift and an or to combine them.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// One MFMA operand fragment of a lane: 8 bf16 (one 16-byte chunk) or 32 e4m3 (two chunks).
template <int DT>
struct FragT;
template <>
struct FragT<DT_BF16> {
  typedef bf16x8 type;
};
template <>
struct FragT<DT_FP8> {
  typedef i32x8 type;
};

template <int DT>
__device__ __forceinline__ typename FragT<DT>::type lds_frag(const lds_t *p0, const lds_t *p1) {
  typedef const i32x4 __attribute__((address_space(3))) *ptr;
  if constexpr (DT == DT_BF16) {
    return __builtin_bit_cast(bf16x8, *(ptr)p0);
  } else {
    const i32x4 lo = *(ptr)p0, hi = *(ptr)p1;
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

template <int DT>
__device__ __forceinline__ f32x16 mfma(const typename FragT<DT>::type &b,
                                       const typename FragT<DT>::type &a, const f32x16 &c) {
  if constexpr (DT == DT_BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c, 0, 0, 0);
  } else {
    // operand formats 0 = e4m3 for both; zero scale operands select the unscaled instruction
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, 0, 0, 0, 0, 0, 0);
  }
}

// 16 x 16 blocks: lane l supplies row l % 16 of each operand, k-group l / 16 (8 bf16 or 32 e4m3),
// and holds C[m = l % 16][n = 4 (l / 16) + r], r = 0..3, of the block (B passed first).  Per
// MAC these move half the accumulator bytes of the 32 x 32 forms, which lowers the energy per
// FLOP and so raises the clock the chip holds under its power limit.
template <int DT>
__device__ __forceinline__ f32x4 mfma16(const typename FragT<DT>::type &b,
                                        const typename FragT<DT>::type &a, const f32x4 &c) {
  if constexpr (DT == DT_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, a, c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, c, 0, 0, 0, 0, 0, 0);
  }
}

// The same 16 x 16 MFMAs accumulating in place in an accumulation register.  With 64 blocks of
// accumulators per wave the compiler's register allocator, given the builtins above, keeps part
// of them in VGPRs and copies them in and out of AGPRs around every MFMA; written out, the
// instruction names its accumulator as both source and destination.  The compiler still sees
// the operands (and waits for the LDS reads that produce A and B), but not the MFMA's latency:
// callers leave wait states before reading an accumulator written here, and after writing one
// with a VALU instruction before its first MFMA.
__device__ __forceinline__ void mfma16_inplace(f32x4 &c, const bf16x8 &b, const bf16x8 &a) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(b), "v"(a));
}
__device__ __forceinline__ void mfma16_inplace(f32x4 &c, const i32x8 &b, const i32x8 &a) {
  asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0" : "+a"(c) : "v"(b), "v"(a));
}
// The same MFMAs starting from zero (C operand 0): the first k-step of a work item, which then
// needs no zeroed accumulators and leaves the previous item's values readable until each block's
// own first MFMA overwrites it.
__device__ __forceinline__ void mfma16_zero(f32x4 &c, const bf16x8 &b, const bf16x8 &a) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(c) : "v"(b), "v"(a));
}
__device__ __forceinline__ void mfma16_zero(f32x4 &c, const i32x8 &b, const i32x8 &a) {
  asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, 0" : "=a"(c) : "v"(b), "v"(a));
}

// Accumulator block of a configuration and the MFMA that updates it.
template <class CFG>
using acc_t = std::conditional_t<CFG::MI == 32, f32x16, f32x4>;

template <class CFG>
__device__ __forceinline__ void mfma_blk(acc_t<CFG> &c, const typename FragT<CFG::DT>::type &b,
                                         const typename FragT<CFG::DT>::type &a) {
  if constexpr (CFG::MI == 32)
    c = mfma<CFG::DT>(b, a, c);
  else
    mfma16_inplace(c, b, a);
}
template <class CFG>
__device__ __forceinline__ void mfma_blk_zero(acc_t<CFG> &c, const typename FragT<CFG::DT>::type &b,
                                              const typename FragT<CFG::DT>::type &a) {
  static_assert(CFG::MI == 16, "16 x 16 blocks");
  mfma16_zero(c, b, a);
}

// Wait states where the compiler cannot see an MFMA written as inline asm (mfma16_inplace), so
// its hazard recognizer inserts none.  Two places need them, both once per work item:
//  * after the accumulators are zeroed (VALU / accumulator-register writes) and before the first
//    MFMA reads them as its C operand: the ISA's dependency table asks for a few wait states
//    there (not in kernels whose first k-step starts from a zero C operand, mfma16_zero);
//  * after the last MFMA of the k-loop and before anything else reads its result (the epilogue's
//    accumulator reads, the Stream-K partial stores): an MFMA of P passes (four cycles each)
//    needs a little over P wait states before a non-MFMA instruction may read what it wrote.
//    The forms used here are 4-pass (16 x 16 x 32 bf16) and 8-pass (16 x 16 x 128 e4m3) -- 16
//    and 32 busy cycles per instruction in the SQ_VALU_MFMA_BUSY_CYCLES counter.
// Three s_nop 7 give 24 wait states, more than either place needs for these forms; a longer MFMA
// (more passes) or a new reader of the accumulators between the k-loop and this call would need
// this count revisited.
__device__ __forceinline__ void mfma_wait_states() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// ---- the kernel ------------------------------------------------------------------------------

// Producer side of the ring: the cursor of the next k-tile to load (uniform) and the lane's byte
// offsets inside a tile.  NW waves share the loads of a k-tile: load j of wave w fills tile rows
// (j * NW + w) * RPL + lane / CH with chunk (lane % CH) ^ swz(row) along K.  The swizzle does not
// change with j (NW * RPL rows is a whole number of swizzle periods), so load j is load 0 moved
// by the uniform stride j * NW * RPL rows: one lane offset per operand plus a scalar offset.
// Rows past M (N) of an edge tile and, for a ragged K, chunks past K get the offset kOOB in the
// lane's own (vector) offset, which the buffer range check turns into zeros.
template <class CFG, bool RAGGED_K, int NW = CFG::WAVES>
struct Producer {
  static constexpr int LA = CFG::A_BYTES / 1024 / NW, LB = CFG::B_BYTES / 1024 / NW;
  static_assert(CFG::A_BYTES % (1024 * NW) == 0 && CFG::B_BYTES % (1024 * NW) == 0, "load split");
  static_assert((NW * CFG::RPL) % (CFG::CH << CFG::SWZ) == 0, "swizzle must repeat per load");
  static_assert(LA + LB <= 63, "vmcnt range");
  Cursor cur;
  int32_t valid, k, ke, rows_a, rows_b, edge;
  __amdgpu_buffer_rsrc_t ra, rb;
  int32_t sta, stb;    // byte stride between loads j and j + 1 (uniform)
  uint32_t voa, vob;   // lane offsets of load 0
  uint32_t row0;       // tile row of the lane in load 0
  uint32_t chunk16;    // byte offset of the lane's chunk within a k-tile row

  __device__ __forceinline__ void init(const KernelArgs &args, int32_t b, int wave, int lane) {
    row0 = (uint32_t)(wave * CFG::RPL + lane / CFG::CH);
    chunk16 = (uint32_t)(((lane % CFG::CH) ^ ((row0 >> CFG::SWZ) & (CFG::CH - 1))) * 16);
    voa = row0 * (uint32_t)args.lda_bytes + chunk16;
    vob = row0 * (uint32_t)args.ldb_bytes + chunk16;
    sta = (int32_t)(NW * CFG::RPL * args.lda_bytes);
    stb = (int32_t)(NW * CFG::RPL * args.ldb_bytes);
    ra = rb = make_rsrc(args.A, 0);  // empty until an item sets them
    cursor_init(args.sp, b, cur);
    next_item(args);
  }

  __device__ __forceinline__ void next_item(const KernelArgs &args) {
    WorkItem w;
    // items without k-tiles (K == 0) load nothing
    while ((valid = cursor_next(args.sp, cur, w)) && w.kb == w.ke) {
    }
    if (valid) {
      k = w.kb;
      ke = w.ke;
      const int64_t m0 = (int64_t)w.m * CFG::BM, n0 = (int64_t)w.n * CFG::BN;
      rows_a = (int32_t)(args.M - m0 < CFG::BM ? args.M - m0 : CFG::BM);
      rows_b = (int32_t)(args.N - n0 < CFG::BN ? args.N - n0 : CFG::BN);
      edge = rows_a < CFG::BM || rows_b < CFG::BN;
      ra = make_rsrc(args.A + m0 * args.lda_bytes, (int64_t)rows_a * args.lda_bytes);
      rb = make_rsrc(args.B + n0 * args.ldb_bytes, (int64_t)rows_b * args.ldb_bytes);
    }
  }

  // Loads of one k-step are issued one instruction at a time: begin(stage) fixes the stage and
  // the k offset, load(j) issues 1 KiB load j (A loads first, then B), end() advances the cursor.
  uint32_t kbytes, koa, kob;
  lds_t *sa;

  __device__ __forceinline__ void begin(const KernelArgs &args, lds_t *smem, int stage) {
    kbytes = (uint32_t)k * CFG::ROWB;
    sa = smem + stage * CFG::STAGE_BYTES;
    koa = voa + kbytes;
    kob = vob + kbytes;
    if (RAGGED_K && (int64_t)(k + 1) * CFG::ROWB > args.K * CFG::EB) {  // chunks past K read 0
      if (chunk16 >= (uint32_t)(args.K * CFG::EB) - kbytes) koa = kob = kOOB;
    }
  }

  template <int J>
  __device__ __forceinline__ void load(int wave) {
    constexpr bool IS_A = J < LA;
    constexpr int j = IS_A ? J : J - LA;
    lds_t *dst = sa + (IS_A ? 0 : CFG::A_BYTES) + (j * NW + wave) * 1024;
    uint32_t off = IS_A ? koa : kob;
    if (edge && row0 + j * NW * CFG::RPL >= (uint32_t)(IS_A ? rows_a : rows_b)) off = kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(IS_A ? ra : rb, dst, 16, off, j * (IS_A ? sta : stb),
                                             0, 0);
  }

  __device__ __forceinline__ void end(const KernelArgs &args) {
    if (++k == ke) next_item(args);
  }
};

// MFMA operand fragments of one 16-deep (bf16) / 64-deep (fp8) sub-step of a k-tile.
template <class CFG>
struct Frags {
  typename FragT<CFG::DT>::type a[CFG::FM], b[CFG::FN];
};

// Fragment e of a sub-step: A fragments first (FM of them), then B (FN).
template <class CFG, int E>
__device__ __forceinline__ void load_frag(const lds_t *smem, int stage, int s,
                                          const uint32_t (&aoff)[CFG::KSUB][CFG::CPL],
                                          const uint32_t (&boff)[CFG::KSUB][CFG::CPL],
                                          Frags<CFG> &fr) {
  const lds_t *base = smem + stage * CFG::STAGE_BYTES;
  constexpr int H = CFG::CPL - 1;
  if constexpr (E < CFG::FM) {
    fr.a[E] = lds_frag<CFG::DT>(base + aoff[s][0] + E * CFG::MI * CFG::ROWB,
                                base + aoff[s][H] + E * CFG::MI * CFG::ROWB);
  } else {
    constexpr int G = E - CFG::FM;
    fr.b[G] = lds_frag<CFG::DT>(base + boff[s][0] + G * CFG::MI * CFG::ROWB,
                                base + boff[s][H] + G * CFG::MI * CFG::ROWB);
  }
}

// Load order of a sub-step's fragments: by first use in its MFMA sequence i = f * FN + g, so
// the first MFMA of a sub-step waits only for the two fragments it reads (a[0], b[0]) and each
// later fragment has until its own first MFMA to arrive.  Returns the fragment index of load e
// in load_frag's numbering (A fragments 0..FM-1, then B fragments).
template <class CFG>
__host__ __device__ constexpr int frag_order(int e) {
  int seen_a = 0, seen_b = 0, n = 0;
  for (int i = 0; i < CFG::FM * CFG::FN; ++i) {
    const int f = i / CFG::FN, g = i % CFG::FN;
    if (!((seen_a >> f) & 1)) {
      seen_a |= 1 << f;
      if (n++ == e) return f;
    }
    if (!((seen_b >> g) & 1)) {
      seen_b |= 1 << g;
      if (n++ == e) return CFG::FM + g;
    }
  }
  return -1;
}

// Slot plan: n memory operations spread over MFMA slots [a, b); operation j follows MFMA
// a + floor(j (b - a) / n).  ops_before(i, ...) counts the operations placed after MFMAs 0..i-1,
// so the operations that follow MFMA i are [ops_before(i), ops_before(i + 1)).
__host__ __device__ constexpr int ops_before(int i, int n, int a, int b) {
  int cnt = 0;
  for (int j = 0; j < n; ++j)
    if (a + (j * (b - a)) / n < i) ++cnt;
  return cnt;
}

// Spin (one lane) until *lock == want, at most max_spin polls; returns false on expiry.
__device__ __forceinline__ bool wait_lock(int *lock, int want, int max_spin) {
  for (int i = 0; i < max_spin; ++i) {
    if (__hip_atomic_load(lock, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == want) return true;
    __builtin_amdgcn_s_sleep(1);
  }
  return false;
}

// Output store of one accumulator quad: 4 consecutive n of row m, times alpha, cast.
template <class CFG>
__device__ __forceinline__ void store_quad(const KernelArgs &args, int64_t m, int64_t n, f32x4 v,
                                           float alpha) {
  if (m >= args.M || n >= args.N) return;
  v = v * alpha;
  if (args.out_bf16) {
    u32x2 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    *(u32x2 *)(args.C + (m * args.ldc + n) * 2) = pk;
  } else {
    *(f32x4 *)(args.C + (m * args.ldc + n) * 4) = v;
  }
}

// ---- fused epilogue ("H100 Kernel Design" lesson, section 12) ------------------------------
// Z = alpha * Acc (+ beta * S), + bias, Y = act(Z), amax over Y, then the cast -- for an e4m3
// output the code of Y / scale_d -- and the store, in the order of section 12.2 (steps 2 to 7).
// Kernels take this path in a fused instantiation, chosen at launch when EPI_* bits or an e4m3
// output are asked for; every other launch runs the plain epilogues above and below.  The
// wide-wave kernels have one fused instantiation per activation (no per-element branch on it),
// and one more per activation that also reads a source matrix S (FUSE_SRC); the cooperative
// kernel has one that reads the activation and the source from the EPI_* bits.
enum : uint32_t {
  EPI_BIAS_ROW = 0x1u,
  EPI_BIAS_COL = 0x2u,
  EPI_RELU = 0x4u,
  EPI_GELU = 0x8u,
  EPI_SILU = 0x10u,
  EPI_AMAX = 0x20u,
  EPI_SRC_F32 = 0x40u,
  EPI_SRC_BF16 = 0x80u
};

// FUSE template argument: FUSE_OFF = the plain epilogue; ACT_* = fused, with that activation;
// ACT_RT = fused, activation chosen by the EPI_* bits at run time.
enum { FUSE_OFF = -1, ACT_NONE = 0, ACT_RELU = 1, ACT_GELU = 2, ACT_SILU = 3, ACT_RT = 4 };
// FUSE_SRC added to a wide-wave kernel's ACT_*: that instantiation also reads a source matrix S,
// in its own copy of the kernel, so the others keep their registers.
enum { FUSE_SRC = 8 };
constexpr int fuse_act(int F) { return F < 0 ? F : (F & 7); }
constexpr bool fuse_src(int F) { return F >= 0 && (F & FUSE_SRC) != 0; }

// State of the fused epilogue in one lane: the output's inverse scale and the running max |Y|.
struct EpiCtx {
  float inv_d;  // 1 / scale_d for an e4m3 output, else 1
  float am;     // max |Y| over the elements this lane has written
};

__device__ __forceinline__ EpiCtx epi_init(const KernelArgs &args) {
  return EpiCtx{args.out_fp8 ? 1.0f / *args.scale_d : 1.0f, 0.0f};
}

// GELU in its exact form z Phi(z) = z (1 + erf(z / sqrt 2)) / 2, with erf from the rational
// approximation of Abramowitz and Stegun, formula 7.1.26 (after Hastings): for x >= 0,
//   erf(x) = 1 - P(t) exp(-x^2),  P(t) = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))),  t = 1/(1 + p x),
// absolute error below 1.5e-7, odd in x.  With x = |z| / sqrt 2 both signs of z collapse to
//   GELU(z) = max(z, 0) - |z| P(t) exp(-z^2 / 2) / 2
// (z >= 0: z (2 - P e) / 2;  z < 0: z P e / 2), the 1/2 folded into P's coefficients: ten
// VALU operations, a reciprocal and an exp2 per element, inline -- a library call would make
// the caller save the whole accumulator tile around it.
__device__ __forceinline__ float act_gelu(float z) {
  const float az = fabsf(z);
  const float t = __builtin_amdgcn_rcpf(fmaf(az, 0.3275911f * 0.70710678118654752f, 1.0f));
  float q = 0.5f * 1.061405429f;
  q = fmaf(q, t, 0.5f * -1.453152027f);
  q = fmaf(q, t, 0.5f * 1.421413741f);
  q = fmaf(q, t, 0.5f * -0.284496736f);
  q = fmaf(q, t, 0.5f * 0.254829592f);
  q = q * t;
  // exp(-z^2 / 2) = 2^(-z^2 log2(e) / 2): 0 once z^2 / 2 passes ~104, where the term vanishes
  const float e = __builtin_amdgcn_exp2f(z * z * -0.72134752044448170f);
  return fmaf(-az, q * e, fmaxf(z, 0.0f));
}
// SiLU z sigmoid(z) = z / (1 + exp(-z)); exp and reciprocal at hardware precision (a few ulp).
// exp(-z) = inf for very negative z gives -0, and 0 for very large z gives z.
__device__ __forceinline__ float act_silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
}

template <int ACT>
__device__ __forceinline__ float act_apply(float z) {
  if constexpr (ACT == ACT_RELU)
    return z < 0.0f ? 0.0f : z;  // NaN stays NaN
  else if constexpr (ACT == ACT_GELU)
    return act_gelu(z);
  else if constexpr (ACT == ACT_SILU)
    return act_silu(z);
  else
    return z;
}

// Y = act(Z) for one quad and, if the quad lies inside C (ok), |Y| into the amax.  ACT_RT: the
// uniform EPI_* bits choose.
template <int ACT>
__device__ __forceinline__ f32x4 epi_act(uint32_t epi, f32x4 z, float &am, bool ok = true) {
  if constexpr (ACT == ACT_RT) {
    if (epi & EPI_RELU) return epi_act<ACT_RELU>(epi, z, am, ok);
    if (epi & EPI_GELU) return epi_act<ACT_GELU>(epi, z, am, ok);
    if (epi & EPI_SILU) return epi_act<ACT_SILU>(epi, z, am, ok);
    return epi_act<ACT_NONE>(epi, z, am, ok);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) z[e] = act_apply<ACT>(z[e]);
  const float q = fmaxf(fmaxf(fabsf(z[0]), fabsf(z[1])), fmaxf(fabsf(z[2]), fabsf(z[3])));
  am = fmaxf(am, ok ? q : 0.0f);
  // fold each quad in as it goes: left free, the compiler regroups the max over the whole
  // tile and keeps the |Y| values live across the epilogue (spilling the kernel)
  asm volatile("" : "+v"(am));
  return z;
}

// e4m3 codes of four values already divided by the output scale, byte e = value e: clamped to
// +-448, the format's largest finite magnitude (NaN passes the comparisons unchanged), then
// rounded to nearest-even by the hardware conversion.
__device__ __forceinline__ uint32_t pack_e4m3x4(f32x4 v) {
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = v[e] > 448.0f ? 448.0f : (v[e] < -448.0f ? -448.0f : v[e]);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w, true);
  return (uint32_t)w;
}

// Fused store of one accumulator quad: 4 consecutive n of row m (n a multiple of 4, so a column
// bias quad is one aligned 16-byte load).
template <int F>
__device__ __forceinline__ void store_quad_fused(const KernelArgs &args, int64_t m, int64_t n,
                                                 f32x4 v, float alpha, EpiCtx &ec) {
  constexpr int ACT = fuse_act(F);
  if (m >= args.M || n >= args.N) return;
  v = v * alpha;
  if constexpr (F == ACT_RT || fuse_src(F)) {
    // Z = alpha * Acc + beta * S: the source quad is read before this thread writes the same
    // elements of C, so S may be C itself
    if (args.epi & EPI_SRC_F32) {
      const f32x4 s = *(const f32x4 *)(args.src + (m * args.ldc + n) * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = fmaf(args.beta, s[e], v[e]);
    } else if (args.epi & EPI_SRC_BF16) {
      const u32x2 s = *(const u32x2 *)(args.src + (m * args.ldc + n) * 2);
      const f32x4 sf = {__uint_as_float(s[0] << 16), __uint_as_float(s[0] & 0xFFFF0000u),
                        __uint_as_float(s[1] << 16), __uint_as_float(s[1] & 0xFFFF0000u)};
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = fmaf(args.beta, sf[e], v[e]);
    }
  }
  if (args.epi & EPI_BIAS_ROW) v = v + args.bias[m];
  if (args.epi & EPI_BIAS_COL) v = v + *(const f32x4 *)(args.bias + n);
  v = epi_act<ACT>(args.epi, v, ec.am);
  if (args.out_fp8) {
    *(uint32_t *)(args.C + m * args.ldc + n) = pack_e4m3x4(v * ec.inv_d);
  } else if (args.out_bf16) {
    u32x2 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    *(u32x2 *)(args.C + (m * args.ldc + n) * 2) = pk;
  } else {
    *(f32x4 *)(args.C + (m * args.ldc + n) * 4) = v;
  }
}

template <int FUSE, class CFG>
__device__ __forceinline__ void store_quad_sel(const KernelArgs &args, int64_t m, int64_t n,
                                               f32x4 v, float alpha, EpiCtx &ec) {
  if constexpr (FUSE != FUSE_OFF)
    store_quad_fused<FUSE>(args, m, n, v, alpha, ec);
  else
    store_quad<CFG>(args, m, n, v, alpha);
}

// The workgroup's largest amax, folded into *amax by one atomic max on its bit pattern (non-negative
// floats order like their bits).  red: WAVES floats of LDS that no wave uses any more once every
// wave has reached this point.
template <int WAVES>
__device__ __forceinline__ void publish_amax(float *amax, float am, lds_t *red, int wave,
                                             int lane) {
  typedef float __attribute__((address_space(3))) *pf;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
  __syncthreads();  // every wave is past its last use of `red`
  if (lane == 0) *(pf)(red + wave * 4) = am;
  __syncthreads();
  if (wave == 0 && lane == 0) {
    float m = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) m = fmaxf(m, *(pf)(red + w * 4));
    __hip_atomic_fetch_max((unsigned int *)amax, __float_as_uint(m), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <class CFG, int F, int G, int Q>
__device__ __forceinline__ f32x4 acc_quad(const f32x16 (&acc)[CFG::FM][CFG::FN]) {
  return f32x4{acc[F][G][4 * Q + 0], acc[F][G][4 * Q + 1], acc[F][G][4 * Q + 2],
               acc[F][G][4 * Q + 3]};
}

// Whole tile: C = cast(alpha * acc), one accumulator quad at a time.  The lane holds, for its
// MFMA block (f, g), rows m = f*32 + lane%32 and columns n = g*32 + 8q + 4*(lane/32) + 0..3.
template <class CFG, int FUSE = FUSE_OFF>
__device__ __forceinline__ void epilogue(const KernelArgs &args, const WorkItem &w,
                                         const f32x16 (&acc)[CFG::FM][CFG::FN], float alpha,
                                         int wm, int wn, int tid, EpiCtx &ec) {
  const int lane = tid & 63;
  const int64_t mbase = (int64_t)w.m * CFG::BM + wm * CFG::WM + (lane & 31);
  const int64_t nbase = (int64_t)w.n * CFG::BN + wn * CFG::WN + (lane >> 5) * 4;
#pragma unroll
  for (int f = 0; f < CFG::FM; ++f)
#pragma unroll
    for (int g = 0; g < CFG::FN; ++g)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = {acc[f][g][4 * q + 0], acc[f][g][4 * q + 1], acc[f][g][4 * q + 2],
                         acc[f][g][4 * q + 3]};
        store_quad_sel<FUSE, CFG>(args, mbase + f * 32, nbase + g * 32 + q * 8, v, alpha, ec);
      }
}

// Reads an accumulator that lives in an accumulation register (AGPR) into a VGPR.  The "a"
// constraint keeps the value in its AGPR until this point; without it the compiler moves a whole
// tile of accumulators out of the AGPRs at once when the k-loop ends.
__device__ __forceinline__ float agpr_read(float x) {
  float y;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(y) : "a"(x));
  return y;
}

template <bool AGPR, class BLK>
__device__ __forceinline__ f32x4 quad_of(const BLK &blk, int q) {
  if constexpr (AGPR)
    return f32x4{agpr_read(blk[4 * q + 0]), agpr_read(blk[4 * q + 1]), agpr_read(blk[4 * q + 2]),
                 agpr_read(blk[4 * q + 3])};
  else
    return f32x4{blk[4 * q + 0], blk[4 * q + 1], blk[4 * q + 2], blk[4 * q + 3]};
}

// Whole tile with bf16 output, staged through LDS so that every global store writes whole row
// segments: the wave converts its sub-tile to bf16 in rounds of 32 rows into its own 1/WAVES
// share of `stage` (a ring stage no wave reads any more), then reads the rows back 16 bytes per
// lane -- CPR lanes per row, CPR * 16 = WN * 2 contiguous bytes -- and stores them.  Only this
// wave touches its share, so the rounds need no workgroup barrier (LDS operations of one wave
// execute in order); the caller's barrier afterwards hands the stage back to the producer.
// Rows are padded by 16 bytes, which spreads the 32 rows one write touches over the banks while
// every address stays a per-lane base plus a constant.
template <class CFG, bool AGPR = false>
__device__ __forceinline__ void epilogue_staged(const KernelArgs &args, const WorkItem &w,
                                                const f32x16 (&acc)[CFG::FM][CFG::FN], float alpha,
                                                int wm, int wn, int wave, int lane, lds_t *smem,
                                                int stage) {
  typedef u32x2 __attribute__((address_space(3))) *p64;
  typedef u32x4 __attribute__((address_space(3))) *p128;
  constexpr int ROW_BYTES = CFG::WN * 2, CPR = ROW_BYTES / 16, PITCH = ROW_BYTES + 16;
  constexpr int SHARE = CFG::STAGE_BYTES / CFG::WAVES;
  static_assert(32 * PITCH <= SHARE, "one 32-row round must fit the wave's share");
  static_assert(64 % CPR == 0, "a wave-wide read covers whole rows");
  constexpr int RSTEP = 64 / CPR;        // rows per wave-wide read
  constexpr int READS = 32 / RSTEP;      // reads per lane per round
  lds_t *share = smem + stage * CFG::STAGE_BYTES + wave * SHARE;
  const int64_t m0 = (int64_t)w.m * CFG::BM + wm * CFG::WM;
  const int64_t n0 = (int64_t)w.n * CFG::BN + wn * CFG::WN;
  if (m0 >= args.M || n0 >= args.N) return;  // the wave's sub-tile lies past the edge of C
  // Stores go through a buffer resource based at the sub-tile origin and ending at the end of C:
  // rows at or past M fall outside it and are dropped by the hardware range check; a lane's
  // 8 columns are all inside or all outside N (N is a multiple of 8).
  const int64_t origin = m0 * args.ldc + n0;
  const __amdgpu_buffer_rsrc_t cr = make_rsrc(args.C + origin * 2, (args.M * args.ldc - origin) * 2);
  const int chunk_l = lane % CPR;
  const bool col_ok = n0 + chunk_l * 8 < args.N;
  const uint32_t ldc_b = (uint32_t)args.ldc * 2;
  lds_t *wr = share + (lane & 31) * PITCH + (lane >> 5) * 8;
  lds_t *rd_p = share + (lane / CPR) * PITCH + chunk_l * 16;
  const uint32_t st_off = (uint32_t)(lane / CPR) * ldc_b + chunk_l * 16;
#pragma unroll
  for (int f = 0; f < CFG::FM; ++f) {
#pragma unroll
    for (int g = 0; g < CFG::FN; ++g)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = quad_of<AGPR>(acc[f][g], q) * alpha;
        *(p64)(wr + (g * 4 + q) * 16) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        // one quad at a time: the accumulators leave their registers in small groups
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
    for (int j = 0; j < READS; ++j) {
      const u32x4 v = *(p128)(rd_p + j * RSTEP * PITCH);
      if (col_ok)
        __builtin_amdgcn_raw_buffer_store_b128(v, cr, st_off,
                                               (uint32_t)(f * 32 + j * RSTEP) * ldc_b, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Partial-tile slot layout: quad qi = (f * FN + g) * 4 + q of thread tid sits at
// quad index qi * THREADS + tid of the slot -- each access is a contiguous 1 KiB run per wave.
template <class CFG>
__device__ __forceinline__ uint32_t slot_byte(int64_t slot) {
  return (uint32_t)(slot * (CFG::BM * CFG::BN * 4));
}

// Chain fixup ("H100 Stream-K" lesson, section 6, deterministic mode): the first split stores its
// partial; every later split waits until the lock equals its K_idx, adds the slot to its own sum
// and either stores it back (middle) or finishes the tile (final).  The lock then becomes
// K_idx + k_tile_count.  Sums are formed left to right in K.
template <class CFG, int FUSE = FUSE_OFF>
__device__ __forceinline__ void fixup_chain(const KernelArgs &args, const WorkItem &w,
                                            const f32x16 (&acc)[CFG::FM][CFG::FN], float alpha,
                                            int wm, int wn, int tid, EpiCtx &ec) {
  const int lane = tid & 63;
  const bool add_slot = w.role == ROLE_MIDDLE || w.role == ROLE_LAST;
  const bool to_slot = w.role == ROLE_FIRST || w.role == ROLE_MIDDLE;
  int *lock = args.locks + w.sk_slot;
  const __amdgpu_buffer_rsrc_t pr = partial_rsrc(args.partials);
  const uint32_t slot = slot_byte<CFG>(w.sk_slot) + tid * 16;
  if (add_slot) {
    if (tid == 0 && !wait_lock(lock, w.kb, args.max_spin))
      __hip_atomic_store(args.error_word, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    lds_barrier();
  }
  const int64_t mbase = (int64_t)w.m * CFG::BM + wm * CFG::WM + (lane & 31);
  const int64_t nbase = (int64_t)w.n * CFG::BN + wn * CFG::WN + (lane >> 5) * 4;
  constexpr int NQ = CFG::FM * CFG::FN * 4;
  constexpr int BATCH = NQ < 4 ? NQ : 4;
  [&]<int... BI>(std::integer_sequence<int, BI...>) {
    (
        [&] {
          constexpr int q0 = BI * BATCH;
          f32x4 p[BATCH];
          if (add_slot) {
#pragma unroll
            for (int i = 0; i < BATCH; ++i)
              p[i] = load_coherent(pr, slot + (q0 + i) * CFG::THREADS * 16);
          }
#pragma unroll
          for (int i = 0; i < BATCH; ++i) {
            const int qi = q0 + i, fg = qi / 4, q = qi % 4, f = fg / CFG::FN, g = fg % CFG::FN;
            f32x4 v = {acc[f][g][4 * q + 0], acc[f][g][4 * q + 1], acc[f][g][4 * q + 2],
                       acc[f][g][4 * q + 3]};
            if (add_slot) v = p[i] + v;
            if (to_slot)
              store_coherent(pr, slot + qi * CFG::THREADS * 16, v);
            else
              store_quad_sel<FUSE, CFG>(args, mbase + f * 32, nbase + g * 32 + q * 8, v, alpha,
                                        ec);
          }
          // one batch of four loads in flight at a time: the accumulators fill most registers
          __builtin_amdgcn_sched_barrier(0);
        }(),
        ...);
  }(std::make_integer_sequence<int, NQ / BATCH>());
  if (to_slot) {
    wait_vmcnt<0>();  // this wave's slot stores are complete ...
    lds_barrier();    // ... and so are everyone's: publish
    const bool skip = (args.flags & KF_TEST_SKIP_PUBLISH) && w.sk_slot == 0 && w.role == ROLE_FIRST;
    if (tid == 0 && !skip)
      __hip_atomic_store(lock, w.ke, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Separate-reduction fixup, part 1: split (unit b on band tile t) stores its partial into its own
// partial slot (sk_partial_slot) and arrives on the tile's counter.
template <class CFG>
__device__ __forceinline__ void fixup_separate_store(const KernelArgs &args, const WorkItem &w,
                                                     const f32x16 (&acc)[CFG::FM][CFG::FN],
                                                     int32_t b, int tid) {
  const __amdgpu_buffer_rsrc_t pr = partial_rsrc(args.partials);
  const uint32_t slot = slot_byte<CFG>(sk_partial_slot(args.sp, b, w.sk_slot)) + tid * 16;
#pragma unroll
  for (int f = 0; f < CFG::FM; ++f)
#pragma unroll
    for (int g = 0; g < CFG::FN; ++g)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = {acc[f][g][4 * q + 0], acc[f][g][4 * q + 1], acc[f][g][4 * q + 2],
                         acc[f][g][4 * q + 3]};
        store_coherent(pr, slot + ((f * CFG::FN + g) * 4 + q) * CFG::THREADS * 16, v);
      }
  wait_vmcnt<0>();
  lds_barrier();
  const bool skip = (args.flags & KF_TEST_SKIP_PUBLISH) && w.sk_slot == 0 && w.role == ROLE_FIRST;
  if (tid == 0 && !skip)
    __hip_atomic_fetch_add(args.locks + w.sk_slot, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Separate-reduction fixup, part 2 (after every unit has stored its partials, so no unit ever
// waits on another unit's reduction): unit b, the j-th of the n units u0..u1 of tile t, waits for
// all n arrivals, then sums the n partials of its 1/n share of the tile in K order (u0 first --
// the same association as the chain) and writes that share of C.
template <class CFG, int FUSE = FUSE_OFF>
__device__ __forceinline__ void fixup_separate_reduce(const KernelArgs &args, const WorkItem &w,
                                                      float alpha, int32_t b, int tid,
                                                      EpiCtx &ec) {
  int32_t u0, u1;
  sk_tile_units(args.sp, w.sk_slot, u0, u1);
  const int n = u1 - u0 + 1, j = b - u0;
  if (tid == 0) {
    int *cnt = args.locks + w.sk_slot;
    bool ok = false;
    for (int i = 0; i < args.max_spin; ++i) {
      if (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n) {
        ok = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (!ok) __hip_atomic_store(args.error_word, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  lds_barrier();
  constexpr int NQ = CFG::BM * CFG::BN / 4;
  const int q_begin = (int)((int64_t)NQ * j / n), q_end = (int)((int64_t)NQ * (j + 1) / n);
  const __amdgpu_buffer_rsrc_t pr = partial_rsrc(args.partials);
  const uint32_t base = slot_byte<CFG>(sk_partial_slot(args.sp, u0, w.sk_slot));
  constexpr uint32_t SLOT = CFG::BM * CFG::BN * 4;
  for (int qq = q_begin + tid; qq < q_end; qq += CFG::THREADS) {
    // sum over u = 0..n-1 of the tile's consecutive slots, left to right; four loads in flight
    const uint32_t off = base + qq * 16;
    f32x4 sum = load_coherent(pr, off);
    int u = 1;
    for (; u + 4 <= n; u += 4) {
      const f32x4 p0 = load_coherent(pr, off + (u + 0) * SLOT);
      const f32x4 p1 = load_coherent(pr, off + (u + 1) * SLOT);
      const f32x4 p2 = load_coherent(pr, off + (u + 2) * SLOT);
      const f32x4 p3 = load_coherent(pr, off + (u + 3) * SLOT);
      sum = sum + p0;
      sum = sum + p1;
      sum = sum + p2;
      sum = sum + p3;
    }
    for (; u < n; ++u) sum = sum + load_coherent(pr, off + u * SLOT);
    // storage index qq = ((f * FN + g) * 4 + q) * THREADS + tid_src  ->  (m, n) of the quad
    const int tid_src = qq % CFG::THREADS, rest = qq / CFG::THREADS;
    const int q = rest % 4, fg = rest / 4, g = fg % CFG::FN, f = fg / CFG::FN;
    const int wave_src = tid_src >> 6, lane = tid_src & 63;
    const int wm = wave_src / CFG::WGN, wn = wave_src % CFG::WGN;
    const int64_t m = (int64_t)w.m * CFG::BM + wm * CFG::WM + f * 32 + (lane & 31);
    const int64_t nn = (int64_t)w.n * CFG::BN + wn * CFG::WN + g * 32 + q * 8 + (lane >> 5) * 4;
    store_quad_sel<FUSE, CFG>(args, m, nn, sum, alpha, ec);
  }
}

template <class CFG, bool RAGGED_K, bool FUSED = false>
__global__ void __attribute__((amdgpu_flat_work_group_size(CFG::THREADS, CFG::THREADS),
                               amdgpu_waves_per_eu(CFG::WAVES_PER_SIMD, CFG::WAVES_PER_SIMD)))
gemm_kernel(KernelArgs args) {
  // An even number of MFMA sub-steps per k-tile keeps the two fragment buffers in fixed roles,
  // so a fragment load never targets registers an in-flight MFMA is still reading.
  static_assert(CFG::KSUB % 2 == 0, "k-tile must hold an even number of MFMA sub-steps");
  static_assert(CFG::MI == 32, "32 x 32 MFMA blocks");
  __shared__ __attribute__((aligned(1024))) char smem_raw[CFG::LDS_BYTES];
  lds_t *smem = (lds_t *)(size_t)(uint32_t)(size_t)(lds_t *)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / CFG::WGN, wn = wave % CFG::WGN;
  const int32_t b = blockIdx.x;

  float alpha = 1.0f;
  if constexpr (CFG::DT == DT_FP8) alpha = (*args.scale_a) * (*args.scale_b);
  constexpr int FUSE = FUSED ? ACT_RT : FUSE_OFF;
  EpiCtx ec = {1.0f, 0.0f};
  if constexpr (FUSED) ec = epi_init(args);

  // Per-lane LDS read offsets of the MFMA operands (bytes within a stage).
  uint32_t aoff[CFG::KSUB][CFG::CPL], boff[CFG::KSUB][CFG::CPL];
  {
    const int r = lane & 31;
    const int swz = (r >> CFG::SWZ) & (CFG::CH - 1);
#pragma unroll
    for (int s = 0; s < CFG::KSUB; ++s)
#pragma unroll
      for (int h = 0; h < CFG::CPL; ++h) {
        const int chunk = (s * 2 + (lane >> 5)) * CFG::CPL + h;
        const uint32_t in_row = (uint32_t)((chunk ^ swz) * 16);
        aoff[s][h] = (uint32_t)((wm * CFG::WM + r) * CFG::ROWB) + in_row;
        boff[s][h] = (uint32_t)(CFG::A_BYTES + (wn * CFG::WN + r) * CFG::ROWB) + in_row;
      }
  }

  using Prod = Producer<CFG, RAGGED_K>;
  Prod prod;
  prod.init(args, b, wave, lane);

  Cursor ccur;
  cursor_init(args.sp, b, ccur);
  WorkItem cw;
  bool cvalid = cursor_next(args.sp, ccur, cw);

  // Ring bookkeeping: `issued` k-steps have been handed to the producer phase so far; the
  // consumer is at k-step c.  Handshake H(c), executed once per k-step, is FULL(c) -- every wave's
  // loads of step c have landed -- and EMPTY(c-1) -- every wave has finished its LDS reads of
  // step c-1 -- after which step c+S-1 may be loaded into stage (c-1) mod S.  Those loads are
  // issued during the first sub-step of step c (`pending`).
  constexpr int L = Prod::LA + Prod::LB;       // loads per wave per k-step
  constexpr int NM = CFG::FM * CFG::FN;       // MFMAs per sub-step
  constexpr int NF = CFG::FM + CFG::FN;       // fragments per sub-step
  int issued = 0;
#pragma unroll
  for (int s = 0; s < CFG::STAGES - 1; ++s)
    if (prod.valid) {
      prod.begin(args, smem, s);
      [&]<int... J>(std::integer_sequence<int, J...>) {
        (prod.template load<J>(wave), ...);
      }(std::make_integer_sequence<int, L>());
      prod.end(args);
      ++issued;
    }

  Frags<CFG> fr[2];
  int c = 0;
  bool pending = false;  // loads of step `issued` are begun but not yet issued
  auto handshake = [&](int step) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // own reads of step-1 are complete
    wait_loads_after<L>(issued - step - 1);
    lds_barrier();
    if (prod.valid) {
      prod.begin(args, smem, (step + CFG::STAGES - 1) % CFG::STAGES);
      pending = true;
    }
  };
  if (issued > 0) {
    handshake(0);
    [&]<int... E>(std::integer_sequence<int, E...>) {
      (load_frag<CFG, frag_order<CFG>(E)>(smem, 0, 0, aoff, boff, fr[0]), ...);
    }(std::make_integer_sequence<int, NF>());
  }

  // One sub-step: NM MFMAs on fr[CUR]; between them, per the slot plan, the fragments of the next
  // sub-step of this k-step, or -- in the last sub-step -- the handshake of the next k-step
  // followed by its first fragments and the producer's loads of the step after it, which may
  // fill the stage this k-step has just drained.  At the last k-step of a work item that stage
  // is kept for the epilogue, and the producer's loads move to the first sub-step of the next
  // k-step (as after the prologue).
  bool early = false;  // may the pending loads go out in this k-step's last sub-step?
  auto substep = [&](auto s_c, auto acc_ref) {
    constexpr int S = decltype(s_c)::value;
    constexpr int CUR = S & 1, NXT = (S + 1) & 1;
    constexpr bool LAST = S == CFG::KSUB - 1;
    constexpr int HS = LAST ? (CFG::KSUB == 1 ? NM / 2 : NM / 4) : NM;  // handshake slot
    auto &acc = *acc_ref;
    const int stage = c % CFG::STAGES;
    const bool have_next = c + 1 < issued;
    [&]<int... I>(std::integer_sequence<int, I...>) {
      (
          [&] {
            constexpr int i = I;
            constexpr int f = i / CFG::FN, g = i % CFG::FN;
            acc[f][g] = mfma<CFG::DT>(fr[CUR].b[g], fr[CUR].a[f], acc[f][g]);
            if constexpr (!LAST) {
              constexpr int lo = ops_before(i, NF, 0, NM);
              constexpr int hi = ops_before(i + 1, NF, 0, NM);
              [&]<int... E>(std::integer_sequence<int, E...>) {
                (load_frag<CFG, frag_order<CFG>(lo + E)>(smem, stage, S + 1, aoff, boff, fr[NXT]), ...);
              }(std::make_integer_sequence<int, hi - lo>());
            } else {
              if constexpr (i + 1 == HS) {
                if (have_next) handshake(c + 1);
              }
              constexpr int lo = ops_before(i, NF, HS, NM);
              constexpr int hi = ops_before(i + 1, NF, HS, NM);
              if (have_next) {
                [&]<int... E>(std::integer_sequence<int, E...>) {
                  (load_frag<CFG, frag_order<CFG>(lo + E)>(smem, (c + 1) % CFG::STAGES, 0, aoff, boff, fr[NXT]),
                   ...);
                }(std::make_integer_sequence<int, hi - lo>());
              }
              constexpr int plo = ops_before(i, L, HS, NM);
              constexpr int phi = ops_before(i + 1, L, HS, NM);
              if (pending && early) {
                [&]<int... J>(std::integer_sequence<int, J...>) {
                  (prod.template load<plo + J>(wave), ...);
                }(std::make_integer_sequence<int, phi - plo>());
                if constexpr (phi == L) {
                  prod.end(args);
                  ++issued;
                  pending = false;
                }
              }
            }
            __builtin_amdgcn_sched_barrier(0);
          }(),
          ...);
    }(std::make_integer_sequence<int, NM>());
  };

  int seq = 0;
  while (cvalid) {
    if ((args.flags & KF_TRACE) && tid == 0 && seq < args.trace_cap) {
      int *t = args.trace + ((int64_t)b * args.trace_cap + seq) * 8;
      t[0] = b; t[1] = seq; t[2] = cw.tile; t[3] = cw.m;
      t[4] = cw.n; t[5] = cw.kb; t[6] = cw.ke; t[7] = cw.role;
    }
    f32x16 acc[CFG::FM][CFG::FN];
#pragma unroll
    for (int f = 0; f < CFG::FM; ++f)
#pragma unroll
      for (int g = 0; g < CFG::FN; ++g)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[f][g][r] = 0.0f;

    for (int k = cw.kb; k < cw.ke; ++k, ++c) {
      // loads still pending from the prologue or an item boundary go out in the first sub-step
      if (pending) {
        [&]<int... J>(std::integer_sequence<int, J...>) {
          (prod.template load<J>(wave), ...);
        }(std::make_integer_sequence<int, L>());
        prod.end(args);
        ++issued;
        pending = false;
      }
      early = k + 1 < cw.ke;
      [&]<int... S>(std::integer_sequence<int, S...>) {
        (substep(std::integral_constant<int, S>(), &acc), ...);
      }(std::make_integer_sequence<int, CFG::KSUB>());
    }

    if (cw.role == ROLE_WHOLE) {
      if (FUSED) {
        epilogue<CFG, FUSE>(args, cw, acc, alpha, wm, wn, tid, ec);  // direct stores
      } else if (args.out_bf16) {
        // The stage read last (c - 1) becomes the staging area; its next fill is the pending
        // producer step, which is issued only after the barrier below.  Every wave has finished
        // reading it once the handshake of step c has run; without a next step (this worker's
        // last item) there was none, so wait for everyone's reads here.
        if (c >= issued) {
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          lds_barrier();
        }
        epilogue_staged<CFG>(args, cw, acc, alpha, wm, wn, wave, lane, smem,
                             (c + CFG::STAGES - 1) % CFG::STAGES);
        lds_barrier();
      } else {
        epilogue<CFG>(args, cw, acc, alpha, wm, wn, tid, ec);
      }
    } else if (args.sk_mode == SK_CHAIN)
      fixup_chain<CFG, FUSE>(args, cw, acc, alpha, wm, wn, tid, ec);
    else
      fixup_separate_store<CFG>(args, cw, acc, b, tid);

    ++seq;
    cvalid = cursor_next(args.sp, ccur, cw);
  }
  if (args.sk_mode == SK_SEPARATE && args.sp.sk_tiles > 0) {
    // second pass over this unit's splits: reduce its share of each tile it touched
    Cursor rc;
    cursor_init(args.sp, b, rc);
    WorkItem rw;
    while (cursor_next(args.sp, rc, rw))
      if (rw.role != ROLE_WHOLE) fixup_separate_reduce<CFG, FUSE>(args, rw, alpha, b, tid, ec);
  }
  wait_vmcnt<0>();
  if constexpr (FUSED)
    if (args.epi & EPI_AMAX) publish_amax<CFG::WAVES>(args.amax, ec.am, smem, wave, lane);
}

// ---- ping-pong kernel (data-parallel tiles) --------------------------------------------------
//
// The pages' ping-pong consumer schedule ("H100 Kernel Design" lesson, sections 7.3-7.5) mapped
// onto the two waves of each SIMD.  The 8 waves form two groups of four (one wave per SIMD each);
// group g owns rows [g*BM/2, (g+1)*BM/2) of the tile, each wave a WM x WN sub-tile.  A wave
// alternates a memory phase M(c) -- read every MFMA fragment of k-step c from LDS into registers
// -- and a compute phase C(c): the k-step's MFMAs back to back.  Group 1 runs one phase behind
// group 0, so in every phase one wave of each SIMD feeds the matrix core while the other reads LDS.
// The global->LDS loads of k-step c+1 go out in the memory phases M(c): group 0 issues the A
// loads after its fragment reads (phase 2c, the first phase the stage is free in), group 1 the B
// loads before its fragment reads (phase 2c+1), so each memory phase carries half of them.
// Loads placed between the MFMAs of a compute phase stretch that phase instead.
//
// Phases are separated by workgroup barriers (barrier n closes phase n for every wave).  With two
// stages the ring hand-offs are:
//  * EMPTY: stage c mod 2 is read in phase 2c (group 0) and 2c+1 (group 1); every wave retires its
//    reads (lgkmcnt(0)) before the barrier closing its memory phase, so from phase 2c+2 on the
//    stage may take k-step c+2.
//  * FULL: step c+1 is read from phase 2c+2 on.  Group 0 waits for its loads of it
//    (s_waitcnt vmcnt(0)) at the end of its C(c) and group 1 at the end of its M(c), both before
//    the barrier that closes phase 2c+1.
// The prologue loads steps 0 and 1.  Group 1 sits out phase 0 with one extra barrier and group 0
// balances it with one after its last phase.
// After an item's last C, the wave writes its sub-tile through its own 4 KiB slice of an LDS area
// outside the ring, during its next memory phase (under the other group's MFMAs).
template <class CFG>
__device__ __forceinline__ void epilogue_pp(const KernelArgs &args, const WorkItem &w,
                                            const f32x16 (&acc)[CFG::FM][CFG::FN], float alpha,
                                            int wm, int wn, int lane, lds_t *slice) {
  typedef u32x2 __attribute__((address_space(3))) *p64;
  typedef u32x4 __attribute__((address_space(3))) *p128;
  static_assert(CFG::WN * 2 == 128, "rows of the staged sub-tile are 128 bytes");
  // chunk c (16 bytes) of staged row r sits at chunk position c ^ (r mod 8): the 8 lanes reading a
  // row back touch 8 distinct bank groups
  const int64_t m0 = (int64_t)w.m * CFG::BM + wm * CFG::WM;
  const int64_t n0 = (int64_t)w.n * CFG::BN + wn * CFG::WN;
  if (m0 >= args.M || n0 >= args.N) return;  // the wave's sub-tile lies past the edge of C
  const int64_t origin = m0 * args.ldc + n0;
  const __amdgpu_buffer_rsrc_t cr = make_rsrc(args.C + origin * 2, (args.M * args.ldc - origin) * 2);
  const int chunk_l = lane & 7, rrow = lane >> 3;  // read-back: 8 rows per wave-wide read
  const bool col_ok = n0 + chunk_l * 8 < args.N;
  const uint32_t ldc_b = (uint32_t)args.ldc * 2;
  const uint32_t st_off = (uint32_t)rrow * ldc_b + chunk_l * 16;
  lds_t *rd_p = slice + rrow * 128 + ((chunk_l ^ rrow) * 16);
  lds_t *wr_row = slice + (lane & 31) * 128 + (lane >> 5) * 8;
  const int x = lane & 7;  // (row mod 8) of the lane's staged row
#pragma unroll
  for (int f = 0; f < CFG::FM; ++f) {
#pragma unroll
    for (int g = 0; g < CFG::FN; ++g)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = f32x4{acc[f][g][4 * q + 0], acc[f][g][4 * q + 1], acc[f][g][4 * q + 2],
                              acc[f][g][4 * q + 3]} * alpha;
        *(p64)(wr_row + (((g * 4 + q) ^ x) * 16)) =
            u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 v = *(p128)(rd_p + j * 1024);
      if (col_ok)
        __builtin_amdgcn_raw_buffer_store_b128(v, cr, st_off, (uint32_t)(f * 32 + j * 8) * ldc_b,
                                               0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

constexpr int kPPSlice = 4096;

  // per-wave epilogue staging area of the ping-pong kernel
template <class CFG>
constexpr int pp_lds_bytes() {
  return CFG::LDS_BYTES + CFG::WAVES * kPPSlice;
}

template <class CFG, bool RAGGED_K>
__global__ void __attribute__((amdgpu_flat_work_group_size(CFG::THREADS, CFG::THREADS),
                               amdgpu_waves_per_eu(2, 2)))
gemm_kernel_pp(KernelArgs args) {
  static_assert(CFG::WAVES == 8 && CFG::WGM == 2 && CFG::WGN == 4, "two groups of four waves");
  static_assert(CFG::STAGES == 2, "ping-pong ring of two stages");
  static_assert(CFG::MI == 32, "32 x 32 MFMA blocks");
  constexpr int EPI_SLICE = kPPSlice;
  static_assert(pp_lds_bytes<CFG>() <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) char smem_raw[pp_lds_bytes<CFG>()];
  lds_t *smem = (lds_t *)(size_t)(uint32_t)(size_t)(lds_t *)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / CFG::WGN, wn = wave % CFG::WGN;
  const int group = wm;
  const int32_t b = blockIdx.x;
  lds_t *slice = smem + CFG::LDS_BYTES + wave * EPI_SLICE;

  float alpha = 1.0f;
  if constexpr (CFG::DT == DT_FP8) alpha = (*args.scale_a) * (*args.scale_b);

  uint32_t aoff[CFG::KSUB][CFG::CPL], boff[CFG::KSUB][CFG::CPL];
  {
    const int r = lane & 31;
    const int swz = (r >> CFG::SWZ) & (CFG::CH - 1);
#pragma unroll
    for (int s = 0; s < CFG::KSUB; ++s)
#pragma unroll
      for (int h = 0; h < CFG::CPL; ++h) {
        const int chunk = (s * 2 + (lane >> 5)) * CFG::CPL + h;
        const uint32_t in_row = (uint32_t)((chunk ^ swz) * 16);
        aoff[s][h] = (uint32_t)((wm * CFG::WM + r) * CFG::ROWB) + in_row;
        boff[s][h] = (uint32_t)(CFG::A_BYTES + (wn * CFG::WN + r) * CFG::ROWB) + in_row;
      }
  }

  // the four waves of each group share a k-step's loads
  using Prod = Producer<CFG, RAGGED_K, 4>;
  constexpr int L = Prod::LA + Prod::LB;
  constexpr int NF = CFG::FM + CFG::FN;
  Prod prod;
  prod.init(args, b, wn, lane);
  Cursor ccur;
  cursor_init(args.sp, b, ccur);
  WorkItem cw;
  bool cvalid = cursor_next(args.sp, ccur, cw);

  constexpr int G0_HI = Prod::LA;  // group 0 issues the A loads [0, LA), group 1 the B loads
  int issued = 0;  // k-steps whose loads this wave has issued
  auto issue = [&](int stage) {
    prod.begin(args, smem, stage);
    if (group == 0) {
      [&]<int... J>(std::integer_sequence<int, J...>) {
        (prod.template load<J>(wn), ...);
      }(std::make_integer_sequence<int, G0_HI>());
    } else {
      [&]<int... J>(std::integer_sequence<int, J...>) {
        (prod.template load<G0_HI + J>(wn), ...);
      }(std::make_integer_sequence<int, L - G0_HI>());
    }
    prod.end(args);
  };
  {
#pragma unroll
    for (int s = 0; s < 2; ++s)
      if (prod.valid) {
        issue(s);
        ++issued;
      }
    wait_vmcnt<0>();
  }
  lds_barrier();                  // phase 0 opens: step 0 is in LDS
  if (group == 1) lds_barrier();  // group 1 sits out phase 0

  Frags<CFG> fr[CFG::KSUB];
  int c = 0;
  int seq = 0;
  while (cvalid) {
    if ((args.flags & KF_TRACE) && tid == 0 && seq < args.trace_cap) {
      int *t = args.trace + ((int64_t)b * args.trace_cap + seq) * 8;
      t[0] = b; t[1] = seq; t[2] = cw.tile; t[3] = cw.m;
      t[4] = cw.n; t[5] = cw.kb; t[6] = cw.ke; t[7] = cw.role;
    }
    ++seq;
    f32x16 acc[CFG::FM][CFG::FN];
#pragma unroll
    for (int f = 0; f < CFG::FM; ++f)
#pragma unroll
      for (int g = 0; g < CFG::FN; ++g)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[f][g][r] = 0.0f;

    for (int k = cw.kb; k < cw.ke; ++k, ++c) {
      // ---- M(c): every fragment of step c; group 0 also loads step c+1 when its stage is free
      const int stage = c & 1;
      // group 1: its loads of step c+1 first, to give them the whole phase
      if (group == 1 && prod.valid && issued == c + 1) {
        issue((c + 1) & 1);
        ++issued;
      }
#pragma unroll
      for (int t = 0; t < CFG::KSUB; ++t)
        [&]<int... E>(std::integer_sequence<int, E...>) {
          (load_frag<CFG, frag_order<CFG>(E)>(smem, stage, t, aoff, boff, fr[t]), ...);
        }(std::make_integer_sequence<int, NF>());
      // group 0: the loads of step c+1, whose stage became free with the phase that just began
      if (group == 0 && prod.valid && issued == c + 1) {
        issue((c + 1) & 1);
        ++issued;
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (group == 1) wait_vmcnt<0>();  // its loads of step c+1 have landed
      lds_barrier();
      // ---- C(c): the k-step's MFMAs, nothing else
#pragma unroll
      for (int t = 0; t < CFG::KSUB; ++t)
#pragma unroll
        for (int f = 0; f < CFG::FM; ++f)
#pragma unroll
          for (int g = 0; g < CFG::FN; ++g)
            acc[f][g] = mfma<CFG::DT>(fr[t].b[g], fr[t].a[f], acc[f][g]);
      if (group == 0) wait_vmcnt<0>();  // step c+1 is in LDS before M(c+1) reads it
      lds_barrier();
    }
    if (args.out_bf16) {
      epilogue_pp<CFG>(args, cw, acc, alpha, wm, wn, lane, slice);
    } else {
      EpiCtx ec_unused = {1.0f, 0.0f};
      epilogue<CFG>(args, cw, acc, alpha, wm, wn, tid, ec_unused);
    }
    cvalid = cursor_next(args.sp, ccur, cw);
  }
  if (group == 0) lds_barrier();  // balance the barrier group 1 skipped at the start
  wait_vmcnt<0>();
}

// ---- wide-wave kernel (data-parallel tiles) ---------------------------------------------------
//
// Four waves, one per SIMD, each owning a 128 x 128 sub-tile (4 x 4 MFMA blocks, accumulators in
// the accumulation registers), fed by the direct global->LDS loads of gemm_kernel.  Per MFMA a
// 128 x 128 sub-tile reads a third fewer fragment bytes from LDS than a 128 x 64 one, and with one
// wave per SIMD the wave interleaves its own memory instructions between its MFMAs: about one
// fragment read per two MFMAs and one load per four keep the matrix core fed.
//
// The k-tile keeps 128-byte rows in LDS (64 bf16 / 128 e4m3 deep), so each 1 KiB load covers 8
// whole 128-byte lines; half-depth tiles with 64-byte rows measured twice the L2 requests for
// the same bytes.  Two 64 KiB stages fill 128 KiB.  Per k-step c:
//  * handshake H(c+1) at slot HS of the last sub-step, as in gemm_kernel: FULL(c+1) by
//    vmcnt(n) -- n counts the loads issued after step c+1's -- and EMPTY(c) by lgkmcnt(0) (step
//    c's fragments are all in registers by then), then s_barrier;  after it stage c mod S may
//    take step c+S;
//  * right after the handshake, spread over the rest of that sub-step, the fragment reads of
//    step c+1 and the loads of step c+S: those loads get a whole k-step, until H(c+2), to land;
//  * in the other sub-steps, the fragment reads of the next sub-step between the MFMAs.
// The epilogue stages each wave's sub-tile through its own 8 KiB LDS slice outside the ring, so
// the ring keeps running across work items: the next tile's loads and first fragment reads are in
// flight while the wave stores the current tile.  With one sub-step per k-tile (e4m3) the two
// fragment buffers swap roles every k-step, so the k-loop is unrolled by two.
constexpr int kWideSlice = 8192;  // 32 rows x 256 bytes of bf16

template <class CFG>
constexpr int wide_lds_bytes() {
  return CFG::LDS_BYTES + CFG::WAVES * kWideSlice;
}

// Bias of a 16 x 16-block sub-tile as the lane meets it: rows m0 + 16f + lane%16 (one value per
// row block f, all loaded here) and columns n0 + 16g + 4(lane/16) + 0..3 (one quad per column
// block g, loaded by col() one block ahead of its use); zero where the bias is absent or past M
// or N (range-checked loads).  Without a bias no load is issued at all: a wait on one would also
// wait for the next item's operand loads, which are still in flight when the epilogue starts.
template <class CFG>
struct WideBias {
  __amdgpu_buffer_rsrc_t cols;
  int64_t nb;
  float row[CFG::FM];
  uint32_t ok;  // bit f: row block f inside C; bit 16 + g: column block g inside C
  bool by_col;

  __device__ __forceinline__ void init(const KernelArgs &args, int64_t m0, int64_t n0, int lane) {
    static_assert(CFG::FM <= 16 && CFG::FN <= 16, "one bit per block");
    const int64_t mb = m0 + (lane & 15);
    nb = n0 + (lane >> 4) * 4;
    by_col = (args.epi & EPI_BIAS_COL) != 0;
    cols = make_rsrc((const char *)args.bias, by_col ? args.N * 4 : 0);
    ok = 0;
#pragma unroll
    for (int f = 0; f < CFG::FM; ++f) {
      row[f] = 0.0f;
      ok |= (mb + f * 16 < args.M ? 1u : 0u) << f;
    }
    if (args.epi & EPI_BIAS_ROW) {
      const __amdgpu_buffer_rsrc_t rows = make_rsrc((const char *)args.bias, args.M * 4);
#pragma unroll
      for (int f = 0; f < CFG::FM; ++f)
        row[f] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rows, (uint32_t)((mb + f * 16) * 4), 0, 0));
    }
#pragma unroll
    for (int g = 0; g < CFG::FN; ++g) ok |= (nb + g * 16 < args.N ? 1u : 0u) << (16 + g);
  }
  __device__ __forceinline__ f32x4 col(int g) const {
    if (!by_col) return f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    return __builtin_bit_cast(
        f32x4, __builtin_amdgcn_raw_buffer_load_b128(cols, (uint32_t)((nb + g * 16) * 4), 0, 0));
  }
  __device__ __forceinline__ bool inside(int f, int g) const {
    return ((ok >> f) & (ok >> (16 + g)) & 1u) != 0;
  }
};

// Y of accumulator quad (f, g) of a 16 x 16-block sub-tile: alpha * Acc (+ beta * S) + bias, then
// the activation and, inside C, the amax (past the edge of C a row bias still reaches the columns
// past N, and a column bias the rows past M, so Y there need not be zero).  s: the source quad
// (FUSE_SRC instantiations).
template <class CFG, int ACT>
__device__ __forceinline__ f32x4 wide_fused_quad(const KernelArgs &args, const acc_t<CFG> &blk,
                                                 float alpha, f32x4 bcol, const WideBias<CFG> &bias,
                                                 EpiCtx &ec, int f, int g,
                                                 f32x4 s = f32x4{0.0f, 0.0f, 0.0f, 0.0f}) {
  const f32x4 a = quad_of<true>(blk, 0);
  f32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = fmaf(a[e], alpha, bcol[e] + bias.row[f]);
  if constexpr (fuse_src(ACT)) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = fmaf(args.beta, s[e], v[e]);
  }
  return epi_act<fuse_act(ACT)>(args.epi, v, ec.am, bias.inside(f, g));
}

// Source quads of a 16 x 16-block sub-tile for a FUSE_SRC epilogue (ES: element bytes, 4 for fp32,
// 2 for bf16; 0 = no source).  Quad (f, g) of the lane is S[m0 + 16f + lane%16][n0 + 16g +
// 4(lane/16) + 0..3], read through a buffer range that starts at the sub-tile's origin, like the
// direct stores: rows past M read zero, and a column block past N gets an offset past the range.
// The loads go out RING quads ahead of their use, in the order the epilogue consumes the quads,
// into a ring of registers: quad i is taken from slot i mod RING, which then takes quad i + RING.
template <class CFG, int ES>
struct WideSource {
  static constexpr int RING = CFG::WM == 128 && CFG::WN == 128 ? 4 : 8;
  using raw_t = std::conditional_t<ES == 4, u32x4, u32x2>;
  __amdgpu_buffer_rsrc_t r;
  uint32_t lane_off, row_b, cols_ok;
  raw_t ring[RING];

  __device__ __forceinline__ void init(const KernelArgs &args, int64_t m0, int64_t n0, int lane,
                                       uint32_t ok) {
    if constexpr (ES != 0) {
      const int64_t origin = m0 * args.ldc + n0;
      r = make_rsrc(args.src + origin * ES, (args.M * args.ldc - origin) * ES);
      row_b = (uint32_t)args.ldc * ES;
      asm volatile("" : "+s"(row_b));  // kept here, not hoisted ahead of the item loop
      lane_off = (uint32_t)(lane & 15) * row_b + (uint32_t)(lane >> 4) * 4 * ES;
      cols_ok = ok >> 16;  // bit g: column block g inside C
    }
  }
  __device__ __forceinline__ void issue(int i, int f, int g) {
    if constexpr (ES != 0) {
      const uint32_t off = ((cols_ok >> g) & 1u) ? lane_off + (uint32_t)(g * 16 * ES) : kOOB;
      const uint32_t soff = (uint32_t)(f * 16) * row_b;
      if constexpr (ES == 4)
        ring[i % RING] = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0);
      else
        ring[i % RING] = __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0);
    }
  }
  __device__ __forceinline__ f32x4 take(int i) const {
    if constexpr (ES == 4) {
      return __builtin_bit_cast(f32x4, ring[i % RING]);
    } else if constexpr (ES == 2) {
      const u32x2 x = ring[i % RING];
      return f32x4{__uint_as_float(x[0] << 16), __uint_as_float(x[0] & 0xFFFF0000u),
                   __uint_as_float(x[1] << 16), __uint_as_float(x[1] & 0xFFFF0000u)};
    } else {
      return f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }
};

// Runs body(std::integral_constant<int, ES>) with the source's element bytes of the launch
// (FUSE_SRC instantiations; ES = 0 for the others), so the epilogue loops hold no branch on it.
template <int FUSE, class Body>
__device__ __forceinline__ void with_source(const KernelArgs &args, Body &&body) {
  if constexpr (fuse_src(FUSE)) {
    if (args.epi & EPI_SRC_F32)
      body(std::integral_constant<int, 4>());
    else
      body(std::integral_constant<int, 2>());
  } else {
    body(std::integral_constant<int, 0>());
  }
}

// bf16 output of a 128-row sub-tile (128 or 112 columns) through the wave's LDS slice, 32 rows at
// a time, at a pitch of 256 bytes.  Chunk c (16 bytes) of staged row r sits at chunk position
// c ^ (r mod 16): the rows one write touches and the 4 rows one read-back touches each spread
// over every bank.  16 lanes store one row segment (the sub-tile's 14 or 16 chunks).  A fused
// FUSE adds the bias, the activation and the amax (16 x 16 blocks), and with SES (the source's
// element bytes) the source term.
template <class CFG, int FUSE = FUSE_OFF, int SES = 0>
__device__ __forceinline__ void epilogue_wide(const KernelArgs &args, const WorkItem &w,
                                              const acc_t<CFG> (&acc)[CFG::FM][CFG::FN],
                                              float alpha, int wm, int wn, int lane, lds_t *slice,
                                              EpiCtx &ec) {
  static_assert(FUSE == FUSE_OFF || CFG::MI == 16, "fused epilogue on 16 x 16 blocks");
  typedef u32x2 __attribute__((address_space(3))) *p64;
  typedef u32x4 __attribute__((address_space(3))) *p128;
  static_assert(CFG::WN * 2 <= 256 && CFG::WN % 16 == 0 && CFG::WM == 128,
                "staged sub-tile rows fit the slice's 256-byte pitch");
  const int64_t m0 = (int64_t)w.m * CFG::BM + wm * CFG::WM;
  const int64_t n0 = (int64_t)w.n * CFG::BN + wn * CFG::WN;
  if (m0 >= args.M || n0 >= args.N) return;  // the wave's sub-tile lies past the edge of C
  const int64_t origin = m0 * args.ldc + n0;
  const __amdgpu_buffer_rsrc_t cr = make_rsrc(args.C + origin * 2, (args.M * args.ldc - origin) * 2);
  const int chunk_l = lane & 15, rrow = lane >> 4;  // read-back: 4 rows per wave-wide read
  // 16 lanes cover a 256-byte pitch; a narrower sub-tile (112 columns: 14 chunks) leaves the
  // last chunks of each staged row unused
  const bool col_ok = chunk_l * 8 < CFG::WN && n0 + chunk_l * 8 < args.N;
  const uint32_t ldc_b = (uint32_t)args.ldc * 2;
  const uint32_t st_off = (uint32_t)rrow * ldc_b + chunk_l * 16;
  // read j covers rows rrow + 4j, whose swizzle is (rrow ^ 4 (j mod 4)): four lane bases
  lds_t *rd_p[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) rd_p[jj] = slice + rrow * 256 + ((chunk_l ^ rrow ^ (4 * jj)) * 16);
  // The reads go out four at a time ahead of their stores: the compiler keeps an LDS read behind
  // an earlier buffer store, so read, store, read, store would wait out one LDS round trip per
  // 16-byte chunk.
  auto read_back = [&](int round) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = *(p128)(rd_p[j] + (h * 4 + j) * 1024);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (col_ok)
          __builtin_amdgcn_raw_buffer_store_b128(v[j], cr, st_off,
                                                 (uint32_t)(round * 32 + (h * 4 + j) * 4) * ldc_b, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  if constexpr (CFG::MI == 32) {
    // block (f, g): the lane holds row f*32 + lane%32, columns g*32 + 8q + 4(lane/32) + 0..3
    const int wrow = lane & 31, x = wrow & 15;
    lds_t *wr_row = slice + wrow * 256 + (lane >> 5) * 8;
#pragma unroll
    for (int f = 0; f < CFG::FM; ++f) {
#pragma unroll
      for (int g = 0; g < CFG::FN; ++g)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v = quad_of<true>(acc[f][g], q) * alpha;
          *(p64)(wr_row + (((g * 4 + q) ^ x) * 16)) =
              u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          __builtin_amdgcn_sched_barrier(0);
        }
      read_back(f);
    }
  } else {
    // block (f, g): the lane holds row f*16 + lane%16, columns g*16 + 4(lane/16) + 0..3, i.e.
    // 16-byte chunk 2g + (lane/16)/2 of its row, half (lane/16) mod 2; two blocks per round
    const int wrow = lane & 15, kq = lane >> 4;
    lds_t *wr_row = slice + wrow * 256 + (kq & 1) * 8;
    // fused: column-block major inside each round of two row blocks, so one column bias quad
    // serves both (loaded one column block ahead)
    WideBias<CFG> bias;
    f32x4 bq = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (FUSE != FUSE_OFF) {
      bias.init(args, m0, n0, lane);
      bq = bias.col(0);
    }
    // source quads in consumption order: quad i is (row block 2p + fp, column block g) with
    // i = 2 FN p + 2 g + fp
    constexpr int NQ = CFG::FM * CFG::FN;
    using Src = WideSource<CFG, SES>;
    Src src;
    auto src_issue = [&](int j) {
      if (j < NQ) {
        const int p = j / (2 * CFG::FN), r = j % (2 * CFG::FN);
        src.issue(j, 2 * p + r % 2, r / 2);
      }
    };
    if constexpr (SES != 0) {
      src.init(args, m0, n0, lane, bias.ok);
#pragma unroll
      for (int j = 0; j < Src::RING; ++j) src_issue(j);
    }
#pragma unroll
    for (int p = 0; p < CFG::FM / 2; ++p) {
#pragma unroll
      for (int g = 0; g < CFG::FN; ++g) {
        // the next column block's bias (the first again for the next round); none after the
        // last quad: a load whose value nobody reads stays in flight past the epilogue, and the
        // next k-loop then waits on it before it reuses the registers it targets
        f32x4 bnext = bq;
        if constexpr (FUSE != FUSE_OFF)
          if (p + 1 < CFG::FM / 2 || g + 1 < CFG::FN) bnext = bias.col((g + 1) % CFG::FN);
#pragma unroll
        for (int fp = 0; fp < 2; ++fp) {
          f32x4 v;
          if constexpr (SES != 0) {
            const int i = 2 * CFG::FN * p + 2 * g + fp;
            const f32x4 s = src.take(i);
            src_issue(i + Src::RING);
            v = wide_fused_quad<CFG, FUSE>(args, acc[2 * p + fp][g], alpha, bq, bias, ec,
                                           2 * p + fp, g, s);
          } else if constexpr (FUSE != FUSE_OFF)
            v = wide_fused_quad<CFG, FUSE>(args, acc[2 * p + fp][g], alpha, bq, bias, ec,
                                           2 * p + fp, g);
          else
            v = quad_of<true>(acc[2 * p + fp][g], 0) * alpha;
          *(p64)(wr_row + fp * 16 * 256 + (((2 * g + (kq >> 1)) ^ wrow) * 16)) =
              u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (FUSE != FUSE_OFF) bq = bnext;
      }
      read_back(p);
    }
  }
}

// Output straight from the accumulation registers, one quad per lane and store (fp32; bf16 from
// kernels whose sub-tiles are too narrow to stage).
template <class CFG, int FUSE = FUSE_OFF>
__device__ __forceinline__ void epilogue_direct(const KernelArgs &args, const WorkItem &w,
                                                const acc_t<CFG> (&acc)[CFG::FM][CFG::FN],
                                                float alpha, int wm, int wn, int lane,
                                                EpiCtx &ec) {
  constexpr int MI = CFG::MI, NQ = MI == 32 ? 4 : 1;
  const int64_t mbase = (int64_t)w.m * CFG::BM + wm * CFG::WM + (lane % MI);
  const int64_t nbase = (int64_t)w.n * CFG::BN + wn * CFG::WN + (lane / MI) * 4;
#pragma unroll
  for (int f = 0; f < CFG::FM; ++f)
#pragma unroll
    for (int g = 0; g < CFG::FN; ++g)
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        store_quad_sel<FUSE, CFG>(args, mbase + f * MI, nbase + g * MI + q * 8,
                                   quad_of<true>(acc[f][g], q), alpha, ec);
        __builtin_amdgcn_sched_barrier(0);
      }
}

// Fused output of a 16 x 16-block sub-tile straight from the accumulation registers, one quad per
// store (16 bytes of fp32, 8 of bf16, 4 of e4m3 codes; for e4m3 this measured faster than
// staging the codes through LDS, which needs registers the e4m3 kernel does not have to spare;
// bf16 takes this path only on 64-wide sub-tiles, whose rows are too short to stage).
// Column-block major: the lane's row biases (one per row block) are loaded first, a column
// block's bias quad one block ahead of its use.  Without a bias of that orientation the loads go
// to an empty buffer range and read zero, so no branch sits in the loop.  One copy of the loop per
// output type (OUT: element bytes), and the stores go through a buffer range that starts at the
// sub-tile's origin: rows past M fall outside it, and a column block past N gets an offset past
// its end, so a store outside C is dropped without a branch around it.
template <class CFG, int ACT, int OUT, int SES = 0>
__device__ __forceinline__ void direct_fused_stores(const KernelArgs &args,
                                                    const acc_t<CFG> (&acc)[CFG::FM][CFG::FN],
                                                    float alpha, int64_t m0, int64_t n0, int lane,
                                                    const WideBias<CFG> &bias, EpiCtx &ec) {
  const int64_t origin = m0 * args.ldc + n0;
  const __amdgpu_buffer_rsrc_t cr =
      make_rsrc(args.C + origin * OUT, (args.M * args.ldc - origin) * OUT);
  uint32_t row_b = (uint32_t)args.ldc * OUT;
  // formed here, not ahead of the kernel's item loop: the row offsets below would otherwise be
  // hoisted there and held in scalar registers through the whole kernel
  asm volatile("" : "+s"(row_b));
  const uint32_t lane_off = (uint32_t)(lane & 15) * row_b + (uint32_t)(lane >> 4) * 4 * OUT;
  // source quads in consumption order: quad i is (f, g) with i = FM g + f
  constexpr int NQ = CFG::FM * CFG::FN;
  using Src = WideSource<CFG, SES>;
  Src src;
  auto src_issue = [&](int j) {
    if (j < NQ) src.issue(j, j % CFG::FM, j / CFG::FM);
  };
  if constexpr (SES != 0) {
    src.init(args, m0, n0, lane, bias.ok);
#pragma unroll
    for (int j = 0; j < Src::RING; ++j) src_issue(j);
  }
  f32x4 bq = bias.col(0);
#pragma unroll
  for (int g = 0; g < CFG::FN; ++g) {
    // no load after the last column block (see epilogue_wide)
    const f32x4 bnext = g + 1 < CFG::FN ? bias.col(g + 1) : bq;
    const uint32_t off = ((bias.ok >> (16 + g)) & 1u) ? lane_off + g * 16 * OUT : kOOB;
#pragma unroll
    for (int f = 0; f < CFG::FM; ++f) {
      f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (SES != 0) {
        s = src.take(CFG::FM * g + f);
        src_issue(CFG::FM * g + f + Src::RING);
      }
      const f32x4 v = wide_fused_quad<CFG, ACT>(args, acc[f][g], alpha, bq, bias, ec, f, g, s);
      const uint32_t soff = (uint32_t)(f * 16) * row_b;
      if constexpr (OUT == 1)
        __builtin_amdgcn_raw_buffer_store_b32(pack_e4m3x4(v * ec.inv_d), cr, off, soff, 0);
      else if constexpr (OUT == 2)
        __builtin_amdgcn_raw_buffer_store_b64(
            u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])}, cr, off, soff, 0);
      else
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), cr, off, soff, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    bq = bnext;
  }
}

template <class CFG, int ACT, int SES = 0>
__device__ __forceinline__ void epilogue_direct_fused(const KernelArgs &args, const WorkItem &w,
                                                      const acc_t<CFG> (&acc)[CFG::FM][CFG::FN],
                                                      float alpha, int wm, int wn, int lane,
                                                      EpiCtx &ec) {
  static_assert(CFG::MI == 16, "16 x 16 blocks");
  const int64_t m0 = (int64_t)w.m * CFG::BM + wm * CFG::WM;
  const int64_t n0 = (int64_t)w.n * CFG::BN + wn * CFG::WN;
  if (m0 >= args.M || n0 >= args.N) return;  // the wave's sub-tile lies past the edge of C
  WideBias<CFG> bias;
  bias.init(args, m0, n0, lane);
  if constexpr (CFG::DT == DT_FP8) {
    if (args.out_fp8)
      direct_fused_stores<CFG, ACT, 1, SES>(args, acc, alpha, m0, n0, lane, bias, ec);
    else if (args.out_bf16)
      direct_fused_stores<CFG, ACT, 2, SES>(args, acc, alpha, m0, n0, lane, bias, ec);
    else
      direct_fused_stores<CFG, ACT, 4, SES>(args, acc, alpha, m0, n0, lane, bias, ec);
  } else {
    // The bf16 kernels keep one loop that picks the store per quad (flat addresses, skipped
    // outside C): with the three copies above, the compiler put vmcnt waits inside the 256 x 224
    // fused kernel's k-loop (its bias + GELU workload measured 4 % slower), while none of the
    // benchmarked workloads sends a bf16 kernel down this path.
    const int64_t mb = m0 + (lane & 15), nb = n0 + (lane >> 4) * 4;
    constexpr int NQ = CFG::FM * CFG::FN;
    using Src = WideSource<CFG, SES>;
    Src src;
    auto src_issue = [&](int j) {
      if (j < NQ) src.issue(j, j % CFG::FM, j / CFG::FM);
    };
    if constexpr (SES != 0) {
      src.init(args, m0, n0, lane, bias.ok);
#pragma unroll
      for (int j = 0; j < Src::RING; ++j) src_issue(j);
    }
    f32x4 bq = bias.col(0);
#pragma unroll
    for (int g = 0; g < CFG::FN; ++g) {
      const f32x4 bnext = g + 1 < CFG::FN ? bias.col(g + 1) : bq;
      const int64_t n = nb + g * 16;
#pragma unroll
      for (int f = 0; f < CFG::FM; ++f) {
        const int64_t m = mb + f * 16;
        f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (SES != 0) {
          s = src.take(CFG::FM * g + f);
          src_issue(CFG::FM * g + f + Src::RING);
        }
        const f32x4 v = wide_fused_quad<CFG, ACT>(args, acc[f][g], alpha, bq, bias, ec, f, g, s);
        if (bias.inside(f, g)) {
          if (args.out_fp8)
            *(uint32_t *)(args.C + m * args.ldc + n) = pack_e4m3x4(v * ec.inv_d);
          else if (args.out_bf16)
            *(u32x2 *)(args.C + (m * args.ldc + n) * 2) =
                u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          else
            *(f32x4 *)(args.C + (m * args.ldc + n) * 4) = v;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      bq = bnext;
    }
  }
}

// Stream-K in the wide-wave kernels (separate reduction, "H100 Stream-K" lesson, section 6, with
// every split storing its own partial): the partial slot of (unit b, band tile t) is
// sk_partial_slot(b, t), like the cooperative kernel's, but laid out row-major -- element (r, c) of the BM x BN tile at
// (r BN + c) 4 bytes -- so the reduction reads whole rows whatever MFMA shape wrote them.
template <class CFG>
__device__ __forceinline__ void wide_partial_store(const KernelArgs &args, const WorkItem &w,
                                                   const acc_t<CFG> (&acc)[CFG::FM][CFG::FN],
                                                   int32_t b, int wm, int wn, int lane, int tid) {
  static_assert(CFG::MI == 16, "16 x 16 blocks");
  const __amdgpu_buffer_rsrc_t pr = partial_rsrc(args.partials);
  const uint32_t slot = slot_byte<CFG>(sk_partial_slot(args.sp, b, w.sk_slot));
  const uint32_t r0 = (uint32_t)(wm * CFG::WM + (lane & 15));
  const uint32_t c0 = (uint32_t)(wn * CFG::WN + (lane >> 4) * 4);
#pragma unroll
  for (int f = 0; f < CFG::FM; ++f)
#pragma unroll
    for (int g = 0; g < CFG::FN; ++g) {
      const uint32_t off = ((r0 + f * 16) * CFG::BN + c0 + g * 16) * 4;
      store_coherent(pr, slot + off, quad_of<true>(acc[f][g], 0));
      __builtin_amdgcn_sched_barrier(0);
    }
  wait_vmcnt<0>();  // this wave's partial is stored (the ring's loads in flight complete too) ...
  lds_barrier();    // ... and so is every wave's: arrive
  const bool skip = (args.flags & KF_TEST_SKIP_PUBLISH) && w.sk_slot == 0 && w.role == ROLE_FIRST;
  if (tid == 0 && !skip)
    __hip_atomic_fetch_add(args.locks + w.sk_slot, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The reduction of the row-major partials: unit b, the j-th of the n units u0..u1 of band tile t,
// waits for all n arrivals, then sums its 1/n share of the tile's quads over the n partials in K
// order (u0 first) and stores that share of C through the (fused) output path.
template <class CFG, int FUSE>
__device__ __forceinline__ void wide_reduce(const KernelArgs &args, const WorkItem &w, float alpha,
                                            int32_t b, int tid, EpiCtx &ec) {
  int32_t u0, u1;
  sk_tile_units(args.sp, w.sk_slot, u0, u1);
  const int n = u1 - u0 + 1, j = b - u0;
  if (tid == 0) {
    int *cnt = args.locks + w.sk_slot;
    bool ok = false;
    for (int i = 0; i < args.max_spin; ++i) {
      if (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n) {
        ok = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (!ok) __hip_atomic_store(args.error_word, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  lds_barrier();
  constexpr int QPR = CFG::BN / 4;  // quads per tile row
  constexpr int NQ = CFG::BM * QPR;
  constexpr uint32_t SLOT = CFG::BM * CFG::BN * 4;
  const int q_begin = (int)((int64_t)NQ * j / n), q_end = (int)((int64_t)NQ * (j + 1) / n);
  const __amdgpu_buffer_rsrc_t pr = partial_rsrc(args.partials);
  const uint32_t base = slot_byte<CFG>(sk_partial_slot(args.sp, u0, w.sk_slot));
  for (int qq = q_begin + tid; qq < q_end; qq += CFG::THREADS) {
    const uint32_t off = base + (uint32_t)qq * 16;
    f32x4 sum = load_coherent(pr, off);
    int u = 1;
    for (; u + 4 <= n; u += 4) {
      const f32x4 p0 = load_coherent(pr, off + (u + 0) * SLOT);
      const f32x4 p1 = load_coherent(pr, off + (u + 1) * SLOT);
      const f32x4 p2 = load_coherent(pr, off + (u + 2) * SLOT);
      const f32x4 p3 = load_coherent(pr, off + (u + 3) * SLOT);
      sum = sum + p0;
      sum = sum + p1;
      sum = sum + p2;
      sum = sum + p3;
    }
    for (; u < n; ++u) sum = sum + load_coherent(pr, off + u * SLOT);
    const int64_t m = (int64_t)w.m * CFG::BM + qq / QPR;
    const int64_t nn = (int64_t)w.n * CFG::BN + (qq % QPR) * 4;
    store_quad_sel<FUSE, CFG>(args, m, nn, sum, alpha, ec);
  }
}

// LEAN keeps only the first load's lane offset per operand and forms load j's as that plus j
// uniform row strides (one VALU add per load), instead of one register per load: 14 fewer
// VGPRs, which the e4m3 kernel (fragments of 128 VGPRs next to 256 accumulators) needs to keep
// its epilogue out of scratch.  Rows past the edge of an item's operand then get an offset past
// the end of the item's buffer range instead of kOOB: the range check zeroes them alike.  An
// exhausted producer switches to an empty range, so every offset reads zero.
template <class CFG, bool RAGGED_K, bool LEAN = false>
struct WideProducer {
  static constexpr int NW = CFG::WAVES;
  static constexpr int LA = CFG::A_BYTES / 1024 / NW, LB = CFG::B_BYTES / 1024 / NW;
  static constexpr int L = LA + LB;
  static constexpr int NV = LEAN ? 2 : L;  // lane offsets kept per item
  static_assert(CFG::A_BYTES % (1024 * NW) == 0 && CFG::B_BYTES % (1024 * NW) == 0, "load split");
  static_assert((NW * CFG::RPL) % (CFG::CH << CFG::SWZ) == 0, "swizzle must repeat per load");
  static_assert(L <= 63, "vmcnt range");
  Cursor cur;
  int32_t valid, k, ke;
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t vo[NV];     // lane offsets of the item's loads (LEAN: of the first A and B load)
  uint32_t step_a, step_b;  // LEAN: byte distance between consecutive loads' rows (uniform)
  uint32_t row0;       // tile row of the lane in load 0
  uint32_t chunk16;    // byte offset of the lane's swizzled chunk within a k-tile row
  uint32_t kbytes;     // byte offset of the k-step within a row (soffset of every load)
  uint32_t lds_wave;   // LDS address of the wave's first 1 KiB in the current stage
  bool k_oob;          // ragged K: the lane's chunk lies past K in this k-step

  __device__ __forceinline__ void init(const KernelArgs &args, int32_t b, int wave, int lane) {
    row0 = (uint32_t)(wave * CFG::RPL + lane / CFG::CH);
    chunk16 = (uint32_t)(((lane % CFG::CH) ^ ((row0 >> CFG::SWZ) & (CFG::CH - 1))) * 16);
    step_a = (uint32_t)(NW * CFG::RPL) * (uint32_t)args.lda_bytes;
    step_b = (uint32_t)(NW * CFG::RPL) * (uint32_t)args.ldb_bytes;
    ra = rb = make_rsrc(args.A, 0);  // empty until an item sets them
    cursor_init(args.sp, b, cur);
    next_item(args);
  }

  __device__ __forceinline__ void next_item(const KernelArgs &args) {
    WorkItem w;
    while ((valid = cursor_next(args.sp, cur, w)) && w.kb == w.ke) {
    }
    if (valid) {
      k = w.kb;
      ke = w.ke;
      const int64_t m0 = (int64_t)w.m * CFG::BM, n0 = (int64_t)w.n * CFG::BN;
      const int32_t rows_a = (int32_t)(args.M - m0 < CFG::BM ? args.M - m0 : CFG::BM);
      const int32_t rows_b = (int32_t)(args.N - n0 < CFG::BN ? args.N - n0 : CFG::BN);
      ra = make_rsrc(args.A + m0 * args.lda_bytes, (int64_t)rows_a * args.lda_bytes);
      rb = make_rsrc(args.B + n0 * args.ldb_bytes, (int64_t)rows_b * args.ldb_bytes);
      if constexpr (LEAN) {
        // rows past rows_a (rows_b) lie past the range's end: no per-row test needed
        vo[0] = row0 * (uint32_t)args.lda_bytes + chunk16;
        vo[1] = row0 * (uint32_t)args.ldb_bytes + chunk16;
      } else {
#pragma unroll
        for (int J = 0; J < L; ++J) {
          const bool is_a = J < LA;
          const uint32_t row = row0 + (uint32_t)((is_a ? J : J - LA) * NW * CFG::RPL);
          const uint32_t ld = (uint32_t)(is_a ? args.lda_bytes : args.ldb_bytes);
          vo[J] = row < (uint32_t)(is_a ? rows_a : rows_b) ? row * ld + chunk16 : kOOB;
        }
      }
    } else {
      if constexpr (LEAN) ra = rb = make_rsrc(args.A, 0);
#pragma unroll
      for (int J = 0; J < NV; ++J) vo[J] = kOOB;
    }
  }

  __device__ __forceinline__ void begin(const KernelArgs &args, uint32_t smem_base, int stage) {
    kbytes = (uint32_t)k * CFG::ROWB;
    lds_wave = smem_base + (uint32_t)stage * CFG::STAGE_BYTES;
    if constexpr (RAGGED_K) k_oob = (int64_t)chunk16 + kbytes >= args.K * CFG::EB;
  }

  // load J (A loads first): 1 KiB of the k-step into LDS; kOOB + kbytes stays below 2^32
  template <int J>
  __device__ __forceinline__ void load() {
    constexpr bool IS_A = J < LA;
    constexpr int j = IS_A ? J : J - LA;
    constexpr uint32_t dst_off = (IS_A ? 0 : CFG::A_BYTES) + j * NW * 1024;
    uint32_t off;
    if constexpr (LEAN)
      off = (IS_A ? vo[0] : vo[1]) + (uint32_t)j * (IS_A ? step_a : step_b);
    else
      off = vo[J];
    if constexpr (RAGGED_K) off = k_oob ? kOOB : off;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(IS_A ? ra : rb, (lds_t *)(size_t)(lds_wave + dst_off), 16,
                                             off, kbytes, 0, 0);
  }

  __device__ __forceinline__ void end(const KernelArgs &args) {
    if (valid && ++k == ke) next_item(args);
  }
};

template <class CFG, bool RAGGED_K, int FUSE = FUSE_OFF>
__global__ void __attribute__((amdgpu_flat_work_group_size(CFG::THREADS, CFG::THREADS),
                               amdgpu_waves_per_eu(1, 1)))
gemm_kernel_wide(KernelArgs args) {
  static_assert(CFG::WAVES == 4 && CFG::WGM == 2 && CFG::WGN == 2, "four waves, one per SIMD");
  static_assert(CFG::STAGES >= 2 && (CFG::STAGES & (CFG::STAGES - 1)) == 0,
                "stage = c mod S by mask");
  static_assert(wide_lds_bytes<CFG>() <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) char smem_raw[wide_lds_bytes<CFG>()];
  lds_t *smem = (lds_t *)(size_t)(uint32_t)(size_t)(lds_t *)smem_raw;
  const uint32_t smem_base = (uint32_t)(size_t)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / CFG::WGN, wn = wave % CFG::WGN;
  const int32_t b = blockIdx.x;
  lds_t *slice = smem + CFG::LDS_BYTES + wave * kWideSlice;

  float alpha = 1.0f;
  if constexpr (CFG::DT == DT_FP8) alpha = (*args.scale_a) * (*args.scale_b);
  EpiCtx ec = {1.0f, 0.0f};
  if constexpr (FUSE != FUSE_OFF) ec = epi_init(args);

  uint32_t aoff[CFG::KSUB][CFG::CPL], boff[CFG::KSUB][CFG::CPL];
  {
    const int r = lane % CFG::MI;  // fragment row; lane / MI is the lane's k-group
    const int swz = (r >> CFG::SWZ) & (CFG::CH - 1);
#pragma unroll
    for (int s = 0; s < CFG::KSUB; ++s)
#pragma unroll
      for (int h = 0; h < CFG::CPL; ++h) {
        const int chunk = (s * CFG::KG + lane / CFG::MI) * CFG::CPL + h;
        const uint32_t in_row = (uint32_t)((chunk ^ swz) * 16);
        aoff[s][h] = (uint32_t)((wm * CFG::WM + r) * CFG::ROWB) + in_row;
        boff[s][h] = (uint32_t)(CFG::A_BYTES + (wn * CFG::WN + r) * CFG::ROWB) + in_row;
      }
  }

  using Prod = WideProducer<CFG, RAGGED_K>;
  Prod prod;
  prod.init(args, b, wave, lane);
  const uint32_t lds_wave0 = smem_base + (uint32_t)wave * 1024;
  Cursor ccur;
  cursor_init(args.sp, b, ccur);
  WorkItem cw;
  bool cvalid = cursor_next(args.sp, ccur, cw);

  constexpr int L = Prod::L;              // loads per wave per k-step
  constexpr int NM = CFG::FM * CFG::FN;   // MFMAs per sub-step
  constexpr int NF = CFG::FM + CFG::FN;   // fragments per sub-step
  // handshake slot in the last sub-step: early, so the step's fragment reads and the loads of the
  // step it begins have most of the sub-step (measured: 3 % fewer cycles per k-step than NM / 4)
  constexpr int HS = CFG::KSUB == 1 ? NM / 2 : (NM / 8 > 0 ? NM / 8 : 1);

  if (!cvalid) return;  // no work (the whole workgroup alike)

  // Ring position: the loads of step c+S-1 go out in k-step c, those of steps 0..S-2 in the
  // prologue; handshake H(c) then waits for the loads of step c, followed by those of (S-2) later
  // steps, so vmcnt((S-2) L) -- loads of the exhausted producer included, they count alike.
  auto load_all = [&] {
    [&]<int... J>(std::integer_sequence<int, J...>) {
      (prod.template load<J>(), ...);
    }(std::make_integer_sequence<int, L>());
    prod.end(args);
  };
#pragma unroll
  for (int s = 0; s < CFG::STAGES - 1; ++s) {
    prod.begin(args, lds_wave0, s);
    load_all();
  }

  Frags<CFG> fr[2];
  int c = 0;
  auto handshake = [&](int step) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // own reads of step-1 are complete
    wait_vmcnt<((CFG::STAGES - 2) * L > 63 ? 63 : (CFG::STAGES - 2) * L)>();
    lds_barrier();
    prod.begin(args, lds_wave0, (step + CFG::STAGES - 1) & (CFG::STAGES - 1));
  };
  handshake(0);
  load_all();  // step S-1, begun by the handshake
  [&]<int... E>(std::integer_sequence<int, E...>) {
    (load_frag<CFG, frag_order<CFG>(E)>(smem, 0, 0, aoff, boff, fr[0]), ...);
  }(std::make_integer_sequence<int, NF>());

  // Sub-step S of k-step c on fragment buffer CUR: NM MFMAs; after MFMA i, in this order, the
  // fragment reads of the next sub-step, or in the last sub-step the handshake H(c+1) (slot HS)
  // followed by the fragment reads of step c+1 and the loads of step c+S, which H(c+1) began,
  // both spread over the slots after it: the loads have a whole k-step to land before H(c+2)
  // waits for them.  None of it is conditional: after the worker's last k-step the handshake,
  // reads and loads still run (every wave alike, so the barriers match), on a stage nobody uses
  // any more.
  auto substep = [&](auto s_c, auto cur_c, auto acc_ref) {
    constexpr int S = decltype(s_c)::value;
    constexpr int CUR = decltype(cur_c)::value, NXT = CUR ^ 1;
    constexpr bool LAST = S == CFG::KSUB - 1;
    auto &acc = *acc_ref;
    const int stage = c & (CFG::STAGES - 1);
    [&]<int... I>(std::integer_sequence<int, I...>) {
      (
          [&] {
            constexpr int i = I;
            constexpr int f = i / CFG::FN, g = i % CFG::FN;
            mfma_blk<CFG>(acc[f][g], fr[CUR].b[g], fr[CUR].a[f]);
            if constexpr (!LAST) {
              constexpr int lo = ops_before(i, NF, 0, NM);
              constexpr int hi = ops_before(i + 1, NF, 0, NM);
              [&]<int... E>(std::integer_sequence<int, E...>) {
                (load_frag<CFG, frag_order<CFG>(lo + E)>(smem, stage, S + 1, aoff, boff, fr[NXT]), ...);
              }(std::make_integer_sequence<int, hi - lo>());
            } else {
              if constexpr (i + 1 == HS) handshake(c + 1);
              constexpr int lo = ops_before(i, NF, HS, NM);
              constexpr int hi = ops_before(i + 1, NF, HS, NM);
              [&]<int... E>(std::integer_sequence<int, E...>) {
                (load_frag<CFG, frag_order<CFG>(lo + E)>(smem, (c + 1) & (CFG::STAGES - 1), 0, aoff,
                                                         boff, fr[NXT]),
                 ...);
              }(std::make_integer_sequence<int, hi - lo>());
              constexpr int plo = ops_before(i, L, HS, NM);
              constexpr int phi = ops_before(i + 1, L, HS, NM);
              [&]<int... J>(std::integer_sequence<int, J...>) {
                (prod.template load<plo + J>(), ...);
              }(std::make_integer_sequence<int, phi - plo>());
              if constexpr (phi == L && plo < L) prod.end(args);
            }
            __builtin_amdgcn_sched_barrier(0);
          }(),
          ...);
    }(std::make_integer_sequence<int, NM>());
  };
  // one k-step whose first sub-step reads fragment buffer P
  auto kstep = [&](auto p_c, auto acc_ref) {
    constexpr int P = decltype(p_c)::value;
    [&]<int... S>(std::integer_sequence<int, S...>) {
      (substep(std::integral_constant<int, S>(), std::integral_constant<int, (P + S) & 1>(),
               acc_ref),
       ...);
    }(std::make_integer_sequence<int, CFG::KSUB>());
    ++c;
  };

  int seq = 0;
  while (cvalid) {
    if ((args.flags & KF_TRACE) && tid == 0 && seq < args.trace_cap) {
      int *t = args.trace + ((int64_t)b * args.trace_cap + seq) * 8;
      t[0] = b; t[1] = seq; t[2] = cw.tile; t[3] = cw.m;
      t[4] = cw.n; t[5] = cw.kb; t[6] = cw.ke; t[7] = cw.role;
    }
    ++seq;
    acc_t<CFG> acc[CFG::FM][CFG::FN];
#pragma unroll
    for (int f = 0; f < CFG::FM; ++f)
#pragma unroll
      for (int g = 0; g < CFG::FN; ++g) acc[f][g] = acc_t<CFG>{};
    // 24 wait states: the zeroed accumulators reach the first (inline-asm) MFMA's C operand
    if constexpr (CFG::MI == 16) mfma_wait_states();

    if constexpr (CFG::KSUB % 2 == 0) {
      for (int k = cw.kb; k < cw.ke; ++k) kstep(std::integral_constant<int, 0>(), &acc);
    } else {
      // k-steps in pairs, so each item starts on buffer 0; after an odd last step the next
      // item's first fragments sit in buffer 1 and move over (once per item)
      int k = cw.kb;
      for (; k + 2 <= cw.ke; k += 2) {
        kstep(std::integral_constant<int, 0>(), &acc);
        kstep(std::integral_constant<int, 1>(), &acc);
      }
      if (k < cw.ke) {
        kstep(std::integral_constant<int, 0>(), &acc);
        fr[0] = fr[1];
      }
    }

    // 24 wait states (> 4 passes + the ISA's margin): the last MFMAs' results are written before
    // the epilogue or the partial store reads them
    if constexpr (CFG::MI == 16) mfma_wait_states();
    if (cw.role != ROLE_WHOLE) {  // a Stream-K split: its partial, reduced after all MAC work
      wide_partial_store<CFG>(args, cw, acc, b, wm, wn, lane, tid);
    } else if (CFG::WM == 128 && args.out_bf16) {  // staged through the wave's LDS slice
      if constexpr (CFG::WM == 128)
        with_source<FUSE>(args, [&](auto es) {
          epilogue_wide<CFG, FUSE, decltype(es)::value>(args, cw, acc, alpha, wm, wn, lane, slice,
                                                        ec);
        });
    } else if constexpr (FUSE != FUSE_OFF) {
      with_source<FUSE>(args, [&](auto es) {
        epilogue_direct_fused<CFG, FUSE, decltype(es)::value>(args, cw, acc, alpha, wm, wn, lane,
                                                              ec);
      });
    } else {
      epilogue_direct<CFG>(args, cw, acc, alpha, wm, wn, lane, ec);
    }
    cvalid = cursor_next(args.sp, ccur, cw);
  }
  if (args.sp.sk_tiles > 0) {
    // second pass over this unit's splits: reduce its share of each tile it touched
    Cursor rc;
    cursor_init(args.sp, b, rc);
    WorkItem rw;
    while (cursor_next(args.sp, rc, rw))
      if (rw.role != ROLE_WHOLE) wide_reduce<CFG, FUSE>(args, rw, alpha, b, tid, ec);
  }
  wait_vmcnt<0>();
  if constexpr (FUSE != FUSE_OFF)
    if (args.epi & EPI_AMAX)
      publish_amax<CFG::WAVES>(args.amax, ec.am, smem + CFG::LDS_BYTES, wave, lane);
}

// The staged bf16 output of a finished whole tile, written during the wave's next work item's
// first k-step instead of after its own last one (plain output; 16 x 16 blocks, 128-row
// sub-tiles).  That k-step's MFMAs start from a zero C operand, so block (f, g) of the finished
// tile stays in its accumulation registers until the new item's MFMA (f, g) replaces it: just
// before that MFMA the wave scales the block, converts it to bf16 and writes it into its LDS
// slice.  The slice holds two rows of blocks (16 sub-tile rows each, row f in half f mod 2,
// chunks swizzled as in epilogue_wide), so row f - 1 is read back and stored while row f is
// written into the other half: read j (4 staged rows) before MFMA (f, 2j), its store before MFMA
// (f, 2j + 2) -- one read (4 VGPRs) in flight at a time, which the e4m3 kernel's registers
// allow.  The last row goes out after the k-step (finish).  Rows and columns past the edge of C
// are dropped as in epilogue_wide; a sub-tile wholly past it stores nothing.
template <class CFG>
struct DeferredOut {
  static_assert(CFG::MI == 16 && CFG::WM == 128 && CFG::WN == 128 && CFG::FM == 8,
                "8 x 8 blocks of 16 x 16");
  typedef u32x2 __attribute__((address_space(3))) *p64;
  typedef u32x4 __attribute__((address_space(3))) *p128;
  __amdgpu_buffer_rsrc_t cr;
  uint32_t st_off, ldc_b;
  // LDS byte addresses: the lane's write of block column 0 and read 0 of a half.  Block column
  // G moves a write's 32-byte pair of chunks to chunk pair (G ^ wrow / 2): bits 5-7 of the
  // address, set to wrow / 2 here, XOR G; read J moves the read's chunk by 4 J: bits 6-7, XOR J.
  uint32_t wa, ra;
  u32x4 v[2];

  __device__ __forceinline__ void init(const KernelArgs &args, lds_t *slice, int lane) {
    clear(args);
    const uint32_t base = (uint32_t)(size_t)slice;  // 256-byte aligned
    const int wrow = lane & 15, kq = lane >> 4;
    // chunk (2 G + kq / 2) ^ wrow of row wrow, half kq mod 2 of it
    wa = base + wrow * 256 + ((kq >> 1) ^ (wrow & 1)) * 16 + (wrow >> 1) * 32 + (kq & 1) * 8;
    // row rrow (+ 4 J), chunk chunk_l ^ rrow (^ 4 J)
    const int chunk_l = lane & 15, rrow = lane >> 4;
    ra = base + rrow * 256 + ((chunk_l ^ rrow) * 16);
    ldc_b = (uint32_t)args.ldc * 2;
  }
  // the finished tile this carries: work item w, the wave's sub-tile (wm, wn); lanes whose
  // columns lie past N (or whose sub-tile lies past the edge of C) store to an offset outside
  // the buffer range, which drops the store; rows past M lie outside it too
  __device__ __forceinline__ void set(const KernelArgs &args, const WorkItem &w, int wm, int wn,
                                      int lane) {
    const int64_t m0 = (int64_t)w.m * CFG::BM + wm * CFG::WM;
    const int64_t n0 = (int64_t)w.n * CFG::BN + wn * CFG::WN;
    const bool inside = m0 < args.M && n0 < args.N;
    const int64_t origin = inside ? m0 * args.ldc + n0 : 0;
    cr = make_rsrc(args.C + origin * 2, (args.M * args.ldc - origin) * 2);
    const int chunk_l = lane & 15, rrow = lane >> 4;
    const bool ok = inside && n0 + chunk_l * 8 < args.N;
    st_off = ok ? (uint32_t)rrow * ldc_b + chunk_l * 16 : kOOB;
  }
  // nothing to carry: the stores go to an empty buffer range, which drops them
  __device__ __forceinline__ void clear(const KernelArgs &args) {
    cr = make_rsrc(args.C, 0);
    st_off = 0;
  }
  // Start of the k-step: the compiler may not form the addresses of all the step's writes and
  // row offsets ahead of time (it would hold them in registers the step does not have).
  __device__ __forceinline__ void begin() {
    asm volatile("" : "+v"(wa), "+v"(ra));
    asm volatile("" : "+s"(ldc_b));
  }
  template <int F, int G>
  __device__ __forceinline__ void write(const f32x4 &blk, float alpha) {
    const f32x4 x = quad_of<true>(blk, 0) * alpha;
    *(p64)(size_t)((wa ^ (G * 32)) + (F % 2) * 4096) =
        u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
  }
  template <int F, int J>
  __device__ __forceinline__ u32x4 read() {
    return *(p128)(size_t)((ra ^ (J * 64)) + ((F % 2) * 4 + J) * 1024);
  }
  template <int F, int J>
  __device__ __forceinline__ void store(const u32x4 &x) {
    __builtin_amdgcn_raw_buffer_store_b128(x, cr, st_off, (uint32_t)(F * 16 + J * 4) * ldc_b, 0);
  }
  // beside the new item's MFMA (f, g), before it: rows 0-6 go back out during rows 1-7
  template <int F, int G>
  __device__ __forceinline__ void slot(const f32x4 &blk, float alpha) {
    if constexpr (F >= 1 && G % 2 == 0) {
      if constexpr (G >= 2)
        store<F - 1, G / 2 - 1>(v[(G / 2 - 1) % 2]);
      else if constexpr (F >= 2)
        store<F - 2, 3>(v[1]);  // the last read of row F - 2, issued before MFMA (F - 1, 6)
      v[(G / 2) % 2] = read<F - 1, G / 2>();
    }
    write<F, G>(blk, alpha);
  }
  // the whole tile at once (the worker's last): the same steps without the MFMAs
  template <class ACC>
  __device__ __forceinline__ void flush(const ACC &acc, float alpha) {
    begin();
    [&]<int... I>(std::integer_sequence<int, I...>) {
      (
          [&] {
            constexpr int f = I / CFG::FN, g = I % CFG::FN;
            slot<f, g>(acc[f][g], alpha);
            __builtin_amdgcn_sched_barrier(0);
          }(),
          ...);
    }(std::make_integer_sequence<int, CFG::FM * CFG::FN>());
    finish();
  }
  // after the k-step: the last row
  __device__ __forceinline__ void finish() {
    constexpr int F = CFG::FM - 1;
    store<F - 1, 3>(v[1]);
    const u32x4 x0 = read<F, 0>(), x1 = read<F, 1>(), x2 = read<F, 2>(), x3 = read<F, 3>();
    store<F, 0>(x0);
    store<F, 1>(x1);
    store<F, 2>(x2);
    store<F, 3>(x3);
    __builtin_amdgcn_sched_barrier(0);
  }
};

// stands in for DeferredOut where a kernel never defers its output
struct NoDeferredOut {
  __device__ __forceinline__ void begin() {}
  template <int F, int G, class BLK>
  __device__ __forceinline__ void slot(const BLK &, float) {}
};

// ---- wide-wave kernel, one MFMA depth per k-tile (e4m3 16 x 16 x 128) ------------------------
//
// The wide-wave schedule for k-tiles exactly one MFMA deep.  A k-step's fragments then fill 128
// VGPRs, so they cannot all be double buffered next to 256 accumulators: B (read by every row of
// MFMAs) has two buffers, A one.  The MFMAs go row by row (f-major), and A[f] of step c+1 is read
// into A[f]'s registers right after the last MFMA of row f of step c, once handshake H(c+1) has
// passed -- so H(c+1) sits after row 0.  B of step c+1 goes into the other buffer, and the loads
// of step c+S (begun by H(c+1)) go out over the first half of the slots after the handshake,
// which leaves them more than half a k-step before H(c+2) waits for them.
template <class CFG, bool RAGGED_K, int FUSE = FUSE_OFF>
__global__ void __attribute__((amdgpu_flat_work_group_size(CFG::THREADS, CFG::THREADS),
                               amdgpu_waves_per_eu(1, 1)))
gemm_kernel_wide1(KernelArgs args) {
  static_assert(CFG::WAVES == 4 && CFG::WGM == 2 && CFG::WGN == 2, "four waves, one per SIMD");
  static_assert(CFG::KSUB == 1 && CFG::MI == 16, "one 16 x 16 MFMA depth per k-tile");
  static_assert(CFG::STAGES >= 2 && (CFG::STAGES & (CFG::STAGES - 1)) == 0, "stage = c mod S");
  static_assert(wide_lds_bytes<CFG>() <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) char smem_raw[wide_lds_bytes<CFG>()];
  lds_t *smem = (lds_t *)(size_t)(uint32_t)(size_t)(lds_t *)smem_raw;
  const uint32_t smem_base = (uint32_t)(size_t)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / CFG::WGN, wn = wave % CFG::WGN;
  const int32_t b = blockIdx.x;
  lds_t *slice = smem + CFG::LDS_BYTES + wave * kWideSlice;

  float alpha = 1.0f;
  if constexpr (CFG::DT == DT_FP8) alpha = (*args.scale_a) * (*args.scale_b);
  EpiCtx ec = {1.0f, 0.0f};
  if constexpr (FUSE != FUSE_OFF) ec = epi_init(args);

  uint32_t aoff[1][CFG::CPL], boff[1][CFG::CPL];
  {
    const int r = lane % CFG::MI;
    const int swz = (r >> CFG::SWZ) & (CFG::CH - 1);
#pragma unroll
    for (int h = 0; h < CFG::CPL; ++h) {
      // The lane's two 16-byte chunks of a 128-byte row are kq and kq + 4 (kq = lane / 16), not
      // 2 kq and 2 kq + 1: then each ds_read_b128 (one h) reads the same set of rows and chunks
      // as the bf16 kernel's read of one sub-step, which counts no LDS bank conflicts, where the
      // adjacent-pair order counted one extra 4-cycle pass per read (SQ_LDS_BANK_CONFLICT about
      // half of SQ_LDS_IDX_ACTIVE).  A and B use the same lane-to-k map, so the MFMA still sums
      // over all 128 k of the k-tile.
      const int chunk = h * CFG::KG + lane / CFG::MI;
      const uint32_t in_row = (uint32_t)((chunk ^ swz) * 16);
      aoff[0][h] = (uint32_t)((wm * CFG::WM + r) * CFG::ROWB) + in_row;
      boff[0][h] = (uint32_t)(CFG::A_BYTES + (wn * CFG::WN + r) * CFG::ROWB) + in_row;
    }
  }
  typedef typename FragT<CFG::DT>::type Frag;
  constexpr int H = CFG::CPL - 1;
  auto read_a = [&](Frag &dst, int stage, int f) {
    const lds_t *base = smem + stage * CFG::STAGE_BYTES + f * CFG::MI * CFG::ROWB;
    dst = lds_frag<CFG::DT>(base + aoff[0][0], base + aoff[0][H]);
  };
  auto read_b = [&](Frag &dst, int stage, int g) {
    const lds_t *base = smem + stage * CFG::STAGE_BYTES + g * CFG::MI * CFG::ROWB;
    dst = lds_frag<CFG::DT>(base + boff[0][0], base + boff[0][H]);
  };

  using Prod = WideProducer<CFG, RAGGED_K, true>;
  Prod prod;
  prod.init(args, b, wave, lane);
  const uint32_t lds_wave0 = smem_base + (uint32_t)wave * 1024;
  Cursor ccur;
  cursor_init(args.sp, b, ccur);
  WorkItem cw;
  bool cvalid = cursor_next(args.sp, ccur, cw);
  if (!cvalid) return;  // no work (the whole workgroup alike)

  constexpr int L = Prod::L;
  constexpr int FM = CFG::FM, FN = CFG::FN, NM = FM * FN;
  constexpr int HS = FN;  // the handshake follows row 0
  // the loads go out in the first half of the slots after it: the next handshake, in the next
  // k-step at slot HS, waits for them (vmcnt), and the ones issued last need the time to land
  constexpr int LW = HS + (NM - HS) / 2;
  auto load_all = [&] {
    [&]<int... J>(std::integer_sequence<int, J...>) {
      (prod.template load<J>(), ...);
    }(std::make_integer_sequence<int, L>());
    prod.end(args);
  };
#pragma unroll
  for (int s = 0; s < CFG::STAGES - 1; ++s) {
    prod.begin(args, lds_wave0, s);
    load_all();
  }

  Frag fa[FM], fb[2][FN];
  int c = 0;
  auto handshake = [&](int step) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    wait_vmcnt<((CFG::STAGES - 2) * L > 63 ? 63 : (CFG::STAGES - 2) * L)>();
    lds_barrier();
    prod.begin(args, lds_wave0, (step + CFG::STAGES - 1) & (CFG::STAGES - 1));
  };
  handshake(0);
  load_all();
#pragma unroll
  for (int g = 0; g < FN; ++g) read_b(fb[0][g], 0, g);
#pragma unroll
  for (int f = 0; f < FM; ++f) read_a(fa[f], 0, f);

  // the previous tile's staged output, carried into the next item's first k-step
  constexpr bool DEFER = FUSE == FUSE_OFF && CFG::WM == 128 && CFG::WN == 128;
  std::conditional_t<DEFER, DeferredOut<CFG>, NoDeferredOut> dout;
  if constexpr (DEFER) dout.init(args, slice, lane);

  // k-step c on B buffer P: MFMA i = (f, g) = (i / FN, i % FN); after MFMA i: the handshake
  // (i = HS - 1), A[f] of step c+1 (i = last of row f, from the handshake on), B reads of step
  // c+1 into buffer P^1 and the loads of step c+S, both spread over the slots after the handshake.
  // An item's first k-step (FIRST) starts its MFMAs from zero; with EPI, the previous tile's
  // block (f, g) goes to the LDS slice just before MFMA (f, g) replaces it.
  acc_t<CFG> acc[FM][FN];
  auto kstep = [&](auto p_c, auto first_c, auto epi_c) {
    constexpr int P = decltype(p_c)::value;
    constexpr bool FIRST = decltype(first_c)::value, EPI = decltype(epi_c)::value;
    const int nstage = (c + 1) & (CFG::STAGES - 1);
    if constexpr (EPI) dout.begin();
    [&]<int... I>(std::integer_sequence<int, I...>) {
      (
          [&] {
            constexpr int i = I;
            constexpr int f = i / FN, g = i % FN;
            if constexpr (EPI) dout.template slot<f, g>(acc[f][g], alpha);
            if constexpr (FIRST)
              mfma_blk_zero<CFG>(acc[f][g], fb[P][g], fa[f]);
            else
              mfma_blk<CFG>(acc[f][g], fb[P][g], fa[f]);
            if constexpr (i + 1 == HS) handshake(c + 1);
            if constexpr (i + 1 >= HS) {
              if constexpr (g == FN - 1) read_a(fa[f], nstage, f);
              constexpr int blo = ops_before(i, FN, HS, NM), bhi = ops_before(i + 1, FN, HS, NM);
              [&]<int... E>(std::integer_sequence<int, E...>) {
                (read_b(fb[P ^ 1][blo + E], nstage, blo + E), ...);
              }(std::make_integer_sequence<int, bhi - blo>());
              constexpr int plo = ops_before(i, L, HS, LW), phi = ops_before(i + 1, L, HS, LW);
              [&]<int... J>(std::integer_sequence<int, J...>) {
                (prod.template load<plo + J>(), ...);
              }(std::make_integer_sequence<int, phi - plo>());
              if constexpr (phi == L && plo < L) prod.end(args);
            }
            __builtin_amdgcn_sched_barrier(0);
          }(),
          ...);
    }(std::make_integer_sequence<int, NM>());
    ++c;
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using ON = std::true_type;
  using OFF = std::false_type;
  int seq = 0;
  if constexpr (DEFER) {
    // the first item's first k-step writes these (unset) values out to nowhere
#pragma unroll
    for (int f = 0; f < FM; ++f)
#pragma unroll
      for (int g = 0; g < FN; ++g) acc[f][g] = __builtin_nondeterministic_value(acc[f][g]);
  }
  while (cvalid) {
    if ((args.flags & KF_TRACE) && tid == 0 && seq < args.trace_cap) {
      int *t = args.trace + ((int64_t)b * args.trace_cap + seq) * 8;
      t[0] = b; t[1] = seq; t[2] = cw.tile; t[3] = cw.m;
      t[4] = cw.n; t[5] = cw.kb; t[6] = cw.ke; t[7] = cw.role;
    }
    ++seq;
    // Every item has at least one k-step (these kernels are not planned for K = 0).  The first
    // starts on B buffer 0, the rest go in pairs (1, 0); after an odd count the next item's B
    // sits in buffer 1 and moves over (once per item).
    // The first k-step always does the staged output's work: a copy of the step without it,
    // taken when nothing is carried, costs more registers than the step has; with nothing
    // carried (dout clear) the stores go nowhere.
    kstep(I0(), ON(), std::bool_constant<DEFER>());
    if constexpr (DEFER) dout.finish();
    int k = cw.kb + 1;
    for (; k + 2 <= cw.ke; k += 2) {
      kstep(I1(), OFF(), OFF());
      kstep(I0(), OFF(), OFF());
    }
    if (k < cw.ke) {
      kstep(I1(), OFF(), OFF());
    } else {
#pragma unroll
      for (int g = 0; g < FN; ++g) fb[0][g] = fb[1][g];
    }
    WorkItem nw;
    const bool nvalid = cursor_next(args.sp, ccur, nw);
    if (DEFER && args.out_bf16 && cw.role == ROLE_WHOLE) {
      // staged bf16 output: carried into the next item's first k-step, which writes it out from
      // the accumulators as they are; the worker's last tile goes out here, the same way
      if constexpr (DEFER) {
        dout.set(args, cw, wm, wn, lane);
        if (!nvalid) {
          mfma_wait_states();  // the last MFMAs' results are written before they are read
          dout.flush(acc, alpha);
        }
      }
    } else {
      if constexpr (DEFER) dout.clear(args);
      // 24 wait states (> 8 passes + the ISA's margin): the last MFMAs' results are written
      // before the epilogue or the partial store reads them
      mfma_wait_states();
      if (cw.role != ROLE_WHOLE) {  // a Stream-K split: its partial, reduced after all MAC work
        wide_partial_store<CFG>(args, cw, acc, b, wm, wn, lane, tid);
      } else if (!DEFER && CFG::WM == 128 && args.out_bf16) {  // staged through the LDS slice
        if constexpr (!DEFER && CFG::WM == 128)
          with_source<FUSE>(args, [&](auto es) {
            epilogue_wide<CFG, FUSE, decltype(es)::value>(args, cw, acc, alpha, wm, wn, lane,
                                                          slice, ec);
          });
      } else if constexpr (FUSE != FUSE_OFF) {
        with_source<FUSE>(args, [&](auto es) {
          epilogue_direct_fused<CFG, FUSE, decltype(es)::value>(args, cw, acc, alpha, wm, wn,
                                                                lane, ec);
        });
      } else {
        epilogue_direct<CFG>(args, cw, acc, alpha, wm, wn, lane, ec);
      }
    }
    cw = nw;
    cvalid = nvalid;
  }
  if (args.sp.sk_tiles > 0) {
    // second pass over this unit's splits: reduce its share of each tile it touched
    Cursor rc;
    cursor_init(args.sp, b, rc);
    WorkItem rw;
    while (cursor_next(args.sp, rc, rw))
      if (rw.role != ROLE_WHOLE) wide_reduce<CFG, FUSE>(args, rw, alpha, b, tid, ec);
  }
  wait_vmcnt<0>();
  if constexpr (FUSE != FUSE_OFF)
    if (args.epi & EPI_AMAX)
      publish_amax<CFG::WAVES>(args.amax, ec.am, smem + CFG::LDS_BYTES, wave, lane);
}

}  // namespace dg
