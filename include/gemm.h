/*
 * dense_gemm_design_amd -- C ABI of the tiled dense GEMM for MI355X (gfx950).
 *
 *   C = alpha * (A x B),  alpha = scale_a * scale_b for FP8 operands, 1 for BF16.
 *
 * The operation is the plain matrix product ("DeepGEMM on SM90" page, CTA <-> output tile
 * section: C[m, n] is the sum over k of A[m, k] B[k, n]) in BF16, or in FP8 e4m3 with one FP32
 * scale per tensor ("WGMMA part 2" lesson, section 11, tensor-wise scaling), accumulated in FP32
 * ("WGMMA part 2" lesson, section 14).  The fused epilogue applies alpha and casts to the output
 * type ("H100 Kernel Design" lesson, section 12: Z = alpha * Acc, then cast and store); on request
 * it also adds a bias, applies an activation, tracks amax and quantises to e4m3 (GEMM_EPI_*,
 * gemm_run_ex), all before the one store of C.  The work
 * is cut into BM x BN output tiles and BK-deep k-tiles, ordered by a tile mapping F(i) -> (m, n)
 * and handed to workgroups by a static, persistent or Stream-K scheduler ("DeepGEMM on SM90" page,
 * mapping table; "H100 Kernel Design" lesson, sections 9-10; "H100 Stream-K" lesson).
 *
 * Conventions
 *  - Every function returns a gemm_status (0 = success) and never prints or aborts.
 *  - Argument and plan errors are reported synchronously, before anything is enqueued.
 *  - Pointers passed to gemm_run are DEVICE pointers owned by the caller (A, B, C, the scales and
 *    the workspace); the library never allocates device memory.  The handle owns only host state.
 *  - gemm_run is asynchronous: it enqueues work on `stream` (a hipStream_t, NULL = the default
 *    stream) and returns; device faults surface at the caller's next synchronisation.
 *  - A handle is immutable after gemm_create; concurrent gemm_run calls on one handle are allowed
 *    if each uses its own workspace.
 */
#ifndef DENSE_GEMM_DESIGN_AMD_GEMM_H
#define DENSE_GEMM_DESIGN_AMD_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GEMM_OK = 0,
  GEMM_ERR_INVALID_ARG = -1,  /* bad enum, non-positive size, NULL handle/pointer ...        */
  GEMM_ERR_UNSUPPORTED = -2,  /* well-formed but outside what the kernels implement          */
  GEMM_ERR_ALIGNMENT = -3,    /* a device pointer is misaligned (16 bytes; 4 for one float)   */
  GEMM_ERR_WORKSPACE = -4,    /* workspace missing or smaller than gemm_workspace_bytes()     */
  GEMM_ERR_HIP = -5,          /* a HIP runtime call failed (no device, launch failure ...)    */
  GEMM_ERR_CAPACITY = -6,     /* a buffer passed to the library is too small for the result   */
  GEMM_ERR_SCRATCH_LIMIT = -7 /* gemm_run_noalloc: the plan's workspace exceeds the scratch   */
} gemm_status;

typedef enum { GEMM_BF16 = 0, GEMM_FP8_E4M3 = 1, GEMM_F32 = 2 } gemm_dtype;
typedef enum { GEMM_ROW_MAJOR = 0, GEMM_COL_MAJOR = 1 } gemm_layout;

/* Tile mapping F(i) -> (m, n) ("DeepGEMM on SM90" page, mapping-family table: linear, grouped
 * strips, 2D blocking / box, Morton / Z-order). */
typedef enum {
  GEMM_MAP_LINEAR_N = 0,   /* C00, C01, ..., C10, ...  (m = i / Nt, n = i % Nt)               */
  GEMM_MAP_LINEAR_M = 1,   /* C00, C10, ..., C01, ...  (m = i % Mt, n = i / Mt)               */
  GEMM_MAP_GROUPED_M = 2,  /* strips of G tile-rows, M-fast inside a strip                    */
  GEMM_MAP_GROUPED_N = 3,  /* strips of G tile-columns, N-fast inside a strip                 */
  GEMM_MAP_BLOCKED = 4,    /* 2D blocking: boxes of group x group_n tiles (rows x columns) hold
                              the tiles that run together; boxes walk along N, box rows along M;
                              M-fast inside a box.  group_n = Nt is GROUPED_M(group)          */
  GEMM_MAP_MORTON = 5      /* Z-order: tiles in the order of their bit-interleaved (m, n) code,
                              n in the even bits; codes outside the grid are skipped          */
} gemm_mapping;

/* Assignment of tasks to workgroups ("H100 Kernel Design" lesson, sections 9.2-10.3). */
typedef enum {
  GEMM_SCHED_STATIC = 0,      /* one workgroup per output tile, grid = tile count              */
  GEMM_SCHED_PERSISTENT = 1,  /* P resident workgroups, worker p takes tiles p, p + P, ...     */
  GEMM_SCHED_STREAMK = 2,     /* persistent data-parallel waves + Stream-K tail (<= half wave) */
  GEMM_SCHED_AUTO = 3         /* the planner picks one of the above                           */
} gemm_sched;

/* flags */
#define GEMM_FLAG_TRACE 0x1u         /* kernel records every work item it runs in the workspace  */
#define GEMM_FLAG_NO_XCD_REMAP 0x2u  /* keep worker id = workgroup id (no XCD-contiguous remap)  */
#define GEMM_FLAG_STREAMK_CHAIN 0x4u /* Stream-K fixup as the lock chain of "H100 Stream-K"
                                        section 6 (each split waits for its predecessor); default
                                        is the separate reduction, same sums in the same order   */
#define GEMM_FLAG_PINGPONG 0x8u      /* require the ping-pong kernel: two wave groups, one wave of
                                        each per SIMD, alternate a memory phase (fragments and
                                        loads) and an MFMA-only phase ("H100 Kernel Design"
                                        sections 7.3-7.5).  256 x 256 tiles, data-parallel
                                        schedules only (static or persistent, K > 0); other plans
                                        with this flag return GEMM_ERR_UNSUPPORTED              */
#define GEMM_FLAG_COOPERATIVE 0x10u  /* require the cooperative kernel (every wave loads and
                                        computes; also runs Stream-K and 128 x 128 tiles)        */
#define GEMM_FLAG_WIDE 0x40u         /* require the wide-wave kernel: four waves with 128 x 128
                                        (or 128 x 112, 64 x 64) sub-tiles fed by direct global ->
                                        LDS loads, 16 x 16 MFMAs.  Runs data-parallel plans and
                                        Stream-K with the separate reduction.  At most one
                                        kernel flag (else GEMM_ERR_INVALID_ARG); without one the
                                        planner picks, the wide-wave kernel for every plan with
                                        K > 0 that does not need the Stream-K lock chain        */
#define GEMM_FLAG_TEST_SKIP_PUBLISH 0x100u /* test only: the first Stream-K split of band tile 0
                                              does not publish its lock / arrival, so the bounded
                                              waits on it expire and report GEMM_DEVICE_ERR_SPIN */

/* Fused epilogue operations (gemm_desc.epilogue), "H100 Kernel Design" lesson, section 12: items
 * 1 (the linear combination with a source matrix), 2, 3 and 8 of its operation list, in the
 * order of its section 12.2 --
 *   Z = alpha * Acc + beta * S;  Z += bias;  Y = act(Z);  amax = max |Y|;
 *   D = cast(Y) (e4m3: of Y / scale_d)
 * -- all applied to the finished accumulators before C is stored once (a Stream-K tile: by the
 * split that writes it, after the full sum).  At most one source bit, one bias bit and one
 * activation bit.  A plan with epilogue bits or an e4m3 output runs on the wide-wave or the
 * cooperative kernel (GEMM_FLAG_PINGPONG with them: GEMM_ERR_UNSUPPORTED). */
#define GEMM_EPI_BIAS_ROW 0x1u  /* Z[m][n] += bias[m]; bias holds M floats                     */
#define GEMM_EPI_BIAS_COL 0x2u  /* Z[m][n] += bias[n]; bias holds N floats                     */
#define GEMM_EPI_RELU 0x4u      /* Y = max(Z, 0)                                                  */
#define GEMM_EPI_GELU 0x8u      /* Y = Z * Phi(Z) = Z * (1 + erf(Z / sqrt 2)) / 2 (exact form)    */
#define GEMM_EPI_SILU 0x10u     /* Y = Z / (1 + exp(-Z))                                          */
#define GEMM_EPI_AMAX 0x20u     /* *amax = max(*amax, max over C of |Y|): Y in fp32, before the
                                   output scale and cast.  The kernel folds its result into the
                                   float already there (an atomic max on the bit pattern), so the
                                   caller sets *amax (to 0, or a running value) before the run;
                                   NaN elements of Y are not propagated                          */
#define GEMM_EPI_SOURCE_F32 0x40u  /* Z = alpha * Acc + beta * S[m][n], S an M x N row-major
                                      fp32 matrix (gemm_epilogue_args.source, beta): C itself
                                      for C = alpha A B + beta C with an fp32 C, or any other */
#define GEMM_EPI_SOURCE_BF16 0x80u /* the same with S in bf16 (C itself for a bf16 C)          */

/* Problem description.  0 in an "auto" field lets the planner choose. */
typedef struct gemm_desc {
  int64_t M, N, K;           /* C is M x N, the reduction is over K (all >= 0; M or N == 0 is an
                                empty product and gemm_run does nothing; K == 0 writes C = 0)   */
  int32_t dtype_ab;          /* GEMM_BF16 or GEMM_FP8_E4M3                                      */
  int32_t dtype_c;           /* GEMM_F32, GEMM_BF16, or GEMM_FP8_E4M3 (e4m3 codes of Y / scale_d,
                                see gemm_epilogue_args; fused-epilogue plans only)            */
  int32_t layout_a;          /* must be GEMM_ROW_MAJOR: a(m,k) at A[m*K + k]                    */
  int32_t layout_b;          /* must be GEMM_COL_MAJOR: b(k,n) at B[n*K + k]                    */
  int32_t mapping;           /* gemm_mapping                                                     */
  int32_t group;             /* G for the grouped mappings, the box height in tile rows for
                                BLOCKED (>= 1, or 0 = chosen by the planner); ignored by the
                                linear ones and MORTON                                          */
  int32_t sched;             /* gemm_sched                                                       */
  int32_t num_workers;       /* P for persistent / Stream-K; 0 = CUs x resident workgroups/CU.
                                Stream-K workgroups wait on each other: a P above what the
                                device holds at once makes the bounded waits expire
                                (GEMM_DEVICE_ERR_SPIN in the error word)                        */
  int32_t bm, bn, bk;        /* tile shape; 0 = auto.  Supported: see gemm_create              */
  uint32_t flags;            /* GEMM_FLAG_*                                                      */
  uint32_t epilogue;         /* GEMM_EPI_* bits: fused bias / activation / amax (0 = none)      */
  int32_t group_n;           /* BLOCKED: box width in tile columns (>= 1, or 0 = chosen by the
                                planner, which then fills the box with the tiles one XCD runs
                                at a time); ignored by the other mappings                      */
  int32_t sk_groups;         /* Stream-K groups ("H100 Stream-K" lesson, section 7), 0..8; 1 =
                                one pool of units over the whole band, 0 = chosen by the
                                planner.  With G > 1 band tile j goes to group j mod G and
                                workgroups g P/G .. (g+1) P/G - 1 form group g, which splits its
                                own tiles' iterations equally; a requested G is lowered to the
                                largest count that divides P and is at most the band's tile
                                count.  The planner takes the largest such count up to 8 whose
                                P / G is a multiple of the XCD count and which keeps the fixup
                                mode of one pool (gemm_plan_info.sk_groups reports the count).
                                Ignored without a Stream-K band.                                */
} gemm_desc;

/* One unit of work as the scheduler hands it out (gemm_schedule_enumerate, device trace). */
typedef struct gemm_work_item {
  int32_t worker;            /* workgroup index in the launch                                   */
  int32_t seq;               /* position in that workgroup's processing order                   */
  int32_t tile;              /* linear task i                                                    */
  int32_t tile_m, tile_n;    /* F(i)                                                             */
  int32_t k_begin, k_end;    /* k-tiles [k_begin, k_end) of the tile (K_idx, K_idx + count)     */
  int32_t role;              /* 0 whole tile, 1 first split, 2 middle split, 3 final split      */
} gemm_work_item;

/* What the planner chose (read-only view of a handle). */
typedef struct gemm_plan_info {
  int32_t bm, bn, bk, stages;
  int32_t threads, grid;     /* workgroup size and launch grid                                  */
  int32_t mt, nt, kt;        /* tile counts                                                      */
  int32_t sched;             /* resolved scheduler (never AUTO)                                  */
  int32_t xcds;              /* XCD count used by the remap (1 = no remap)                      */
  int32_t lds_bytes;         /* LDS per workgroup                                                */
  int64_t dp_tiles, sk_tiles;
  int64_t workspace_bytes;
  int64_t trace_offset;      /* byte offset of the trace records in the workspace (-1: none)    */
  int32_t trace_capacity;    /* records per workgroup                                            */
  int32_t error_offset;      /* byte offset of the device error word in the workspace (-1: none)*/
  int32_t streamk_mode;      /* 0 lock chain, 1 separate reduction (meaningful when sk_tiles>0)  */
  int32_t kernel;            /* 0 cooperative, 1 ping-pong, 3 wide-wave (2 is not used)         */
  int32_t group;             /* G of a grouped mapping as planned (1 for the linear ones)       */
  int32_t group_n;           /* box width of BLOCKED as planned (1 for the other mappings)      */
  int32_t sk_groups;         /* Stream-K groups as planned (1 without a band)                   */
  int32_t xcd_box_r;         /* XCD box remap of a grouped mapping: each XCD runs an r x c box
                                of every data-parallel wave (r across the strip, c along it);
                                0 = contiguous runs of P / xcds workers per XCD               */
  int32_t xcd_box_c;
} gemm_plan_info;

/* device error word values (read back from the workspace after a run) */
#define GEMM_DEVICE_OK 0
#define GEMM_DEVICE_ERR_SPIN 1       /* a Stream-K lock wait hit its spin limit                 */

typedef struct gemm_plan *gemm_handle;

/* Validates the description and builds a plan.  The description carries the per-problem inputs
 * and knobs of the "DeepGEMM on SM90" page, section "Kernel Configuration Heuristic" (M, N, K,
 * the operand type, layout / GEMM type, and the chosen BM, BN, BK, G, stages and scheduler);
 * the plan records the tile grid of that section (Mt = ceil(M/BM), Nt = ceil(N/BN), one task per
 * output tile) and, for Stream-K, the workspace layout of the "H100 Stream-K" lesson, section 6
 * (The Lock).  The handle owns host memory only; it is freed by gemm_destroy.  On error *out is
 * left unchanged and nothing is allocated.  Supported in this version:
 *   dtype_ab BF16 with tiles (bm, bn, bk) in {(256,256,64), (256,224,64), (256,192,64),
 *   (128,128,64)},
 *   dtype_ab FP8_E4M3 with tiles in {(256,256,128), (256,224,128), (256,192,128),
 *   (128,128,128)}; 256 x 224 and 256 x 192 tiles run on the wide-wave kernel only (a plan that
 *   needs another kernel -- K = 0, the Stream-K lock chain, or a kernel flag other than
 *   GEMM_FLAG_WIDE -- returns GEMM_ERR_UNSUPPORTED);
 *   layout_a ROW and layout_b COL (both operands K-contiguous);
 *   K * sizeof(element) a multiple of 16 bytes and at most 2^30; N a multiple of 8 and at most
 *   2^22 (the kernels address the rows of an output tile with 32-bit byte offsets);
 *   M, N arbitrary otherwise (ragged tiles are masked), K ragged in the last k-tile.
 * Needs a visible GPU only when num_workers == 0 (it then queries the CU count). */
int gemm_create(const gemm_desc *desc, gemm_handle *out);

/* Device bytes the caller must pass to gemm_run as workspace (0 when none is needed).  The
 * workspace follows the "H100 Stream-K" lesson, section 6 (The Lock): the FP32 partial-tile
 * buffer first, the per-tile int lock (or arrival counter) array right after it in the same
 * allocation, then the device error word (and the trace, with GEMM_FLAG_TRACE); every lock is
 * zero when the kernel starts, because gemm_run clears them on the stream before the launch.
 * The caller owns and allocates it.  GEMM_ERR_INVALID_ARG for a NULL handle or pointer. */
int gemm_workspace_bytes(gemm_handle h, size_t *bytes);

/* Copies the plan as chosen (tile, grid, schedule counts, kernel, workspace layout) into *info,
 * a caller-owned struct.  GEMM_ERR_INVALID_ARG for a NULL handle or pointer. */
int gemm_plan_get(gemm_handle h, gemm_plan_info *info);

/* Enqueues C = alpha * A x B on `stream`.  The call follows the stream-ordered, asynchronous
 * model of the "DeepGEMM on SM90" page, CUDA programming-model section 1 (Host-Device
 * Execution): returning means the work is submitted, not complete; work on one stream runs in
 * order; the caller synchronises explicitly.  Its argument list has the shape of the library
 * call of the "Multi GPU Part 2" lesson (Lesson 10), section 6.1: buffers, sizes and datatype
 * (here fixed at gemm_create), the operation's operands, and the stream last.  A: M x K row-major, B: K x N column-major, C: M x N
 * row-major of dtype_c (A and B may be NULL when K == 0; nothing is needed when M or N is 0).  scale_a / scale_b: device pointers to one float each for FP8 (required),
 * ignored for BF16 (may be NULL).  workspace: device memory of at least gemm_workspace_bytes(),
 * 16-byte aligned; the library clears the parts it needs at the start of every run. */
int gemm_run(gemm_handle h, const void *A, const void *B, void *C, const float *scale_a,
             const float *scale_b, void *workspace, size_t workspace_bytes, void *stream);

/* Device operands of the fused epilogue; all DEVICE pointers owned by the caller. */
typedef struct gemm_epilogue_args {
  const float *bias;     /* with a GEMM_EPI_BIAS_* bit: M (row) or N (column) floats, 16-byte
                            aligned; else ignored                                                */
  const float *scale_d;  /* with dtype_c = GEMM_FP8_E4M3: one float, the output's dequantisation
                            scale (a code q stands for scale_d * q, so q = e4m3(Y / scale_d),
                            nearest-even, saturated to +-448); else ignored                    */
  float *amax;           /* with GEMM_EPI_AMAX: one float, 4-byte aligned, read and updated by
                            the kernel (see GEMM_EPI_AMAX); else ignored                        */
  const void *source;    /* with a GEMM_EPI_SOURCE_* bit and beta != 0: S, M x N row-major (N
                            elements per row) of the bit's type, 16-byte aligned (fp32) or
                            8-byte aligned (bf16); it may be C itself (each element of S is read
                            before the same element of C is written, by the same thread).  With
                            beta == 0 the kernels read no source (a NaN in S does not reach C)
                            and the pointer may be NULL.  Else ignored                         */
  float beta;            /* with a GEMM_EPI_SOURCE_* bit: the source's factor; else ignored     */
} gemm_epilogue_args;

/* gemm_run with the fused epilogue's operands.  `epi` may be NULL when the plan needs none of
 * them (gemm_run is this call with epi = NULL).  A missing required pointer is
 * GEMM_ERR_INVALID_ARG, a misaligned one GEMM_ERR_ALIGNMENT, both checked before anything is
 * enqueued.  Calls that overlap in time and share one amax combine their maxima. */
int gemm_run_ex(gemm_handle h, const void *A, const void *B, void *C, const float *scale_a,
                const float *scale_b, const gemm_epilogue_args *epi, void *workspace,
                size_t workspace_bytes, void *stream);

/* Frees the handle's host memory.  Work already enqueued with it is unaffected (a launch holds
 * its own copy of the arguments).  NULL is GEMM_ERR_INVALID_ARG. */
/* Size of the scratch array gemm_run_noalloc uses as workspace, in bytes (per GPU). */
#define GEMM_NOALLOC_SCRATCH_BYTES (32u << 20)

/* gemm_run_ex for callers that cannot allocate device memory -- code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation: the workspace is a file-scope device
 * array of GEMM_NOALLOC_SCRATCH_BYTES inside the library (one per GPU, allocated when the library's
 * code is loaded on that GPU and held until the process ends), so the call allocates nothing and
 * takes no workspace argument.  The caller still passes A, B, C, the scales and the epilogue
 * operands, as for gemm_run_ex, with the same checks and errors; the work is enqueued on `stream`,
 * which must belong to the current device (the scratch used is the current device's).  A plan
 * whose gemm_workspace_bytes() exceeds GEMM_NOALLOC_SCRATCH_BYTES returns GEMM_ERR_SCRATCH_LIMIT
 * before anything else happens (the largest Stream-K plans; 512 x 512 x 65536 on 256 workgroups
 * needs 17 MiB).  The parts of the scratch that must start at zero (the Stream-K locks and
 * counters, the error word) are cleared on the stream at the start of every call, with a fill
 * kernel.  Within a process, every call on one GPU shares that GPU's array and finds the previous
 * call's contents: calls that overlap in time on one GPU (from different streams or threads) race
 * on it, so the caller orders them. */
int gemm_run_noalloc(gemm_handle h, const void *A, const void *B, void *C, const float *scale_a,
                     const float *scale_b, const gemm_epilogue_args *epi, void *stream);

int gemm_destroy(gemm_handle h);

/* CPU replay of the plan's schedule: the tasks of the tile mapping F(i) -> (m, n) ("DeepGEMM on
 * SM90" page, mapping-family table), as the static / persistent assignment ("H100 Kernel Design"
 * lesson, sections 9.2-10.2: worker p takes tasks p, p + P, ...) or the Stream-K split ("H100
 * Stream-K" lesson, sections 2-5: equal iteration ranges per unit, cut at tile boundaries into
 * first / middle / final splits) hands them out.  Runs on the host with the same code the
 * kernels use; items is a caller-owned host array.  Writes up to `cap` items (grouped by worker,
 * each worker's items in processing order) and the total count to *n_out.  Returns GEMM_ERR_CAPACITY (with
 * *n_out set) when cap is too small. */
int gemm_schedule_enumerate(gemm_handle h, gemm_work_item *items, size_t cap, size_t *n_out);

/* One candidate configuration as the planner's cost model scores it (gemm_rank_configs). */
typedef struct gemm_config_score {
  int32_t bm, bn, bk;        /* tile                                                             */
  int32_t kernel;            /* as gemm_plan_info.kernel                                        */
  int32_t sched;             /* GEMM_SCHED_PERSISTENT or GEMM_SCHED_STREAMK                     */
  int32_t workers;           /* P the plan would launch                                         */
  int32_t group;             /* G for a grouped mapping, box height for BLOCKED (1 otherwise)  */
  int32_t group_n;           /* box width for BLOCKED (1 otherwise)                             */
  double cycles_mfma;        /* modelled clocks, whole GEMM, matrix-core side                   */
  double cycles_l2;          /* L2 -> CU side: A/B tile loads and C                             */
  double cycles_local;       /* LDS side: tile fills, fragment reads, C staging                 */
  double wave_efficiency;    /* tiles / (CUs x effective waves), a partial last wave with a
                                fraction f of the CUs busy counting f^0.39 of a full one (at
                                least 1/1.3: the busy CUs clock higher under the board's power
                                limit); Stream-K: busy unit slots over its units                 */
  double cycles_fixed;       /* not overlapped with the MAC loop: first loads, epilogues, and
                                Stream-K partial sums through device memory                    */
  double score;              /* max(mfma, l2, local) / wave_efficiency + fixed, times 1.03 for
                                Stream-K; lower is better                                       */
} gemm_config_score;

/* Kernel-configuration heuristic: the cost model of "DeepGEMM on SM90" (section "Kernel
 * Configuration Heuristic") -- candidates from a small discrete set, a resource filter, then
 * score = max(cycles_local, cycles_L2) / wave_efficiency with the minimum winning -- re-fitted to
 * gfx950: the candidates are this library's kernels and tiles (256 x 256, 256 x 224 and
 * 256 x 192 wide-wave data-parallel -- the narrower block widths from the page's aligned set fill
 * whole waves where 256 does not -- 128 x 128 wide-wave and cooperative data-parallel, Stream-K
 * tails on the 128 x 128 and 256 x 256 tiles, and for plans that read a source matrix the
 * cooperative kernel on 256 x 256 tiles),
 * the bandwidths and per-kernel MFMA efficiencies are measured on MI355X, a matrix-core term
 * joins the two data-movement terms, the costs that do not overlap the MAC loop are added, and a
 * Stream-K plan's score is scaled by 1.03 (measured).  Fills up to `cap` candidates, best first,
 * and the total to *n_out (GEMM_ERR_CAPACITY when cap is too small; items may be NULL with cap
 * 0).  gemm_create
 * takes the best one when bm = bn = bk = 0, sched = GEMM_SCHED_AUTO and no kernel flag is set;
 * with a grouped mapping and group = 0 it takes the G reported here.  Needs a visible GPU only
 * when num_workers == 0. */
int gemm_rank_configs(const gemm_desc *desc, gemm_config_score *items, size_t cap, size_t *n_out);

/* Static string for a gemm_status value (never NULL; unknown values give "unknown status").
 * The status codes are this library's own: the pages define no error interface; every call
 * reports through them instead of printing or aborting. */
const char *gemm_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif
