/*
 * Reference CPU implementation of the dense GEMM C = A x B -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may load this
 * library. The product path (the HIP library under dense_gemm_design_amd/) never links it,
 * includes it or calls it, and it shares no header, table or helper with that path.
 *
 * What it computes, and where the pages define it:
 *   - C[m][n] = sum over k of a(m,k) * b(k,n)  ("DeepGEMM on SM90" page, CTA <-> output tile
 *     section: C[0,0] is the sum over k of A[0,k] B[k,0]; "H100 Stream-K" lesson, section 1:
 *     an output tile is the sum of the products of its k-tiles).  The sum runs over k in
 *     increasing order in IEEE binary64, one product and one add per step (no contraction),
 *     so the result is a fixed, plainly defined number.
 *   - bf16 operands decode exactly: the 16 stored bits are the upper half of a binary32
 *     ("WGMMA part 1" lesson, section 12: two bf16 per 32-bit word, even element in the low half).
 *   - e4m3 operands decode from the format's definition: 1 sign bit, 4 exponent bits with bias 7,
 *     3 mantissa bits, subnormals at exponent 0, no infinities, S.1111.111 is NaN, so the largest
 *     finite magnitude is 448 ("WGMMA part 2" lesson, sections 9-10).
 *   - per-tensor FP32 scales multiply the exact integer-grid sum: C = s_a * s_b * sum q_a q_b
 *     ("WGMMA part 2" lesson, section 11, tensor-wise scaling).
 *   - oracle_encode_e4m3 (binary32 input) / _f64 / _array: round-to-nearest-even onto the e4m3
 *     grid with saturation to +-448 ("WGMMA part 2" lesson, sections 10 and 13: satfinite clamps
 *     out-of-range values to the signed maximum normal).  Checks the input generator's quantised
 *     bytes and gives the expected codes of an e4m3 output (fused-epilogue quantisation).
 *
 * Layout: A row-major means a(m,k) = A[m*K + k]; A column-major means a(m,k) = A[k*M + m].
 * B row-major (K x N) means b(k,n) = B[k*N + n]; B column-major means b(k,n) = B[n*K + k].
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_BF16 = 0, ORACLE_E4M3 = 1 };
enum { ORACLE_ROW = 0, ORACLE_COL = 1 };

double oracle_decode_bf16(uint16_t h) {
  uint32_t u = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

double oracle_decode_e4m3(uint8_t code) {
  int sign = code >> 7;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double mag;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    mag = ldexp((double)m, -9); /* m/8 * 2^(1-7) */
  else
    mag = ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* Nearest e4m3 code to x, ties to the code with an even mantissa, magnitudes above 448 saturate.
 * x is taken at full double precision, so a value just past a rounding midpoint rounds away from
 * it even when the nearest binary32 value would sit on the midpoint. */
uint8_t oracle_encode_e4m3_f64(double x) {
  uint8_t sign = 0;
  if (isnan(x)) return 0x7F;
  if (signbit(x)) {
    sign = 0x80;
    x = -x;
  }
  if (x >= 448.0) return sign | 0x7E;
  /* Walk the 127 non-negative finite codes (they are increasing in value) and keep the closest. */
  int best = 0;
  double best_err = x;
  for (int c = 1; c <= 0x7E; ++c) {
    double v = oracle_decode_e4m3((uint8_t)c);
    double err = fabs(v - x);
    if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      best_err = err;
    }
  }
  return sign | (uint8_t)best;
}

uint8_t oracle_encode_e4m3(float xf) { return oracle_encode_e4m3_f64((double)xf); }

/* out[i] = oracle_encode_e4m3_f64(x[i]) for i < n. */
void oracle_encode_e4m3_array(const double *x, uint8_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_encode_e4m3_f64(x[i]);
}

static double decode_one(int dtype, const void *p, int64_t idx) {
  if (dtype == ORACLE_BF16) return oracle_decode_bf16(((const uint16_t *)p)[idx]);
  return oracle_decode_e4m3(((const uint8_t *)p)[idx]);
}

typedef struct {
  int64_t M, N, K;
  int dtype, layout_a, layout_b;
  const void *A, *B;
  double scale;
  const double *Ad, *Bd; /* full mode: decoded a(m,k) at Ad[m*K+k], b(k,n) at Bd[n*K+k] */
  double *C;             /* full mode: row-major M x N output */
  const int64_t *sm, *sn;
  double *sout;          /* sampled mode: out[i] = C[sm[i]][sn[i]] */
  int64_t begin, end;    /* this thread's share of rows (full) or samples (sampled) */
} job_t;

static double a_at(const job_t *j, int64_t m, int64_t k) {
  int64_t idx = j->layout_a == ORACLE_ROW ? m * j->K + k : k * j->M + m;
  return decode_one(j->dtype, j->A, idx);
}
static double b_at(const job_t *j, int64_t k, int64_t n) {
  int64_t idx = j->layout_b == ORACLE_ROW ? k * j->N + n : n * j->K + k;
  return decode_one(j->dtype, j->B, idx);
}

/* sum over k = 0, 1, ..., K-1 of a[k] * b[k], one rounded product and one rounded add per step */
static double dot(const double *a, const double *b, int64_t K) {
  double s = 0.0;
  for (int64_t k = 0; k < K; ++k) {
    double p = a[k] * b[k];
    s = s + p;
  }
  return s;
}

static void *decode_a_rows(void *arg) {
  job_t *j = (job_t *)arg;
  double *Ad = (double *)j->Ad;
  for (int64_t m = j->begin; m < j->end; ++m)
    for (int64_t k = 0; k < j->K; ++k) Ad[m * j->K + k] = a_at(j, m, k);
  return NULL;
}

static void *decode_b_cols(void *arg) {
  job_t *j = (job_t *)arg;
  double *Bd = (double *)j->Bd;
  for (int64_t n = j->begin; n < j->end; ++n)
    for (int64_t k = 0; k < j->K; ++k) Bd[n * j->K + k] = b_at(j, k, n);
  return NULL;
}

static void *run_full(void *arg) {
  job_t *j = (job_t *)arg;
  for (int64_t m = j->begin; m < j->end; ++m)
    for (int64_t n = 0; n < j->N; ++n)
      j->C[m * j->N + n] = dot(j->Ad + m * j->K, j->Bd + n * j->K, j->K) * j->scale;
  return NULL;
}

static void *run_sampled(void *arg) {
  job_t *j = (job_t *)arg;
  double *arow = (double *)malloc(sizeof(double) * (size_t)(j->K + 1));
  double *bcol = (double *)malloc(sizeof(double) * (size_t)(j->K + 1));
  for (int64_t i = j->begin; i < j->end; ++i) {
    for (int64_t k = 0; k < j->K; ++k) arow[k] = a_at(j, j->sm[i], k);
    for (int64_t k = 0; k < j->K; ++k) bcol[k] = b_at(j, k, j->sn[i]);
    j->sout[i] = dot(arow, bcol, j->K) * j->scale;
  }
  free(arow);
  free(bcol);
  return NULL;
}

static int launch(const job_t *tmpl, int64_t count, int nthreads, void *(*fn)(void *)) {
  if (count <= 0) return 0;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > count) nthreads = (int)count;
  pthread_t th[256];
  job_t jobs[256];
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = *tmpl;
    jobs[t].begin = count * t / nthreads;
    jobs[t].end = count * (t + 1) / nthreads;
    if (pthread_create(&th[t], NULL, fn, &jobs[t]) != 0) return -1;
  }
  for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
  return 0;
}

static int check(int64_t M, int64_t N, int64_t K, int dtype, int la, int lb) {
  if (M < 0 || N < 0 || K < 0) return -1;
  if (dtype != ORACLE_BF16 && dtype != ORACLE_E4M3) return -1;
  if ((la != ORACLE_ROW && la != ORACLE_COL) || (lb != ORACLE_ROW && lb != ORACLE_COL)) return -1;
  return 0;
}

/* Full product: C (row-major M x N, fp64) = scale_a * scale_b * A x B.  For bf16 pass scales 1. */
int oracle_gemm(int64_t M, int64_t N, int64_t K, int dtype, const void *A, int layout_a,
                const void *B, int layout_b, double scale_a, double scale_b, double *C,
                int nthreads) {
  if (check(M, N, K, dtype, layout_a, layout_b)) return -1;
  job_t j;
  memset(&j, 0, sizeof j);
  j.M = M; j.N = N; j.K = K; j.dtype = dtype; j.layout_a = layout_a; j.layout_b = layout_b;
  j.A = A; j.B = B; j.scale = scale_a * scale_b; j.C = C;
  double *Ad = (double *)malloc(sizeof(double) * (size_t)(M * K + 1));
  double *Bd = (double *)malloc(sizeof(double) * (size_t)(N * K + 1));
  if (!Ad || !Bd) {
    free(Ad);
    free(Bd);
    return -2;
  }
  j.Ad = Ad;
  j.Bd = Bd;
  int rc = launch(&j, M, nthreads, decode_a_rows);
  if (!rc) rc = launch(&j, N, nthreads, decode_b_cols);
  if (!rc) rc = launch(&j, M, nthreads, run_full);
  free(Ad);
  free(Bd);
  return rc;
}

/* Sampled product: out[i] = C[sm[i]][sn[i]] for i < count, each computed exactly as above. */
int oracle_gemm_sampled(int64_t M, int64_t N, int64_t K, int dtype, const void *A, int layout_a,
                        const void *B, int layout_b, double scale_a, double scale_b,
                        const int64_t *sm, const int64_t *sn, int64_t count, double *out,
                        int nthreads) {
  if (check(M, N, K, dtype, layout_a, layout_b)) return -1;
  for (int64_t i = 0; i < count; ++i)
    if (sm[i] < 0 || sm[i] >= M || sn[i] < 0 || sn[i] >= N) return -1;
  job_t j;
  memset(&j, 0, sizeof j);
  j.M = M; j.N = N; j.K = K; j.dtype = dtype; j.layout_a = layout_a; j.layout_b = layout_b;
  j.A = A; j.B = B; j.scale = scale_a * scale_b; j.sm = sm; j.sn = sn; j.sout = out;
  return launch(&j, count, nthreads, run_sampled);
}
