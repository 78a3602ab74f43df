/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU reference for the output-stationary tiled
 * matrix multiply C = A @ B and for the analytic counts that the pages attach to
 * it. Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * load this library; the product path never does. It shares no code, header or
 * table with the GPU library.
 *
 * What it follows:
 *  - The operation is the plain matrix product C[i][j] = sum_k A[i][k] * B[k][j]
 *    (Mojo GPU puzzles, "Tiled Matrix Multiplication", section 3 "Optimized memory
 *    access layouts": the computation is standard A x B, not A x B^T). Tiling only
 *    reorders that sum ("Reading a matrix multiply through its tiles", section
 *    "Keep one output tile resident"), so the oracle computes the definition,
 *    without tiles.
 *  - Floating point: the stored 16-bit inputs are decoded exactly to binary64, each
 *    C[i][j] is summed in binary64 in ascending k, and the sum is rounded ONCE,
 *    round-to-nearest-even, to the output format. The fp32 accumulator of the pages
 *    (Helion listing: the C tile is an fp32 zero tile; "What fits in local
 *    storage?": FP16 inputs with FP32 accumulation) bounds the GPU's error; the
 *    oracle is deliberately more precise than the method.
 *  - int32: the same sum in unsigned 32-bit arithmetic, i.e. two's-complement
 *    wraparound modulo 2^32 (the pages leave overflow unstated; this reading makes
 *    the result independent of summation order, so any tiling must match bit-exactly).
 *  - Counts: 2*M*N*K operations ("Reading a matrix multiply through its tiles",
 *    opening paragraph); the no-reuse traffic of the output-stationary loop
 *    (section "Count the repeated reads"), summed tile by tile over the actual
 *    row/column/reduction ranges of every tile (section "Edge tiles still
 *    matter"); the per-step working set (section "What fits in local storage?",
 *    whose formulas did not survive extraction: A tile tm*tk*s_in, B tile
 *    tk*tn*s_in, accumulator tm*tn*4 bytes, the reading that reproduces the three
 *    1 KiB values printed for 16x16x32); and ragged tile ranges [i*t, min((i+1)*t, D))
 *    (Helion page: tiling 10 by 4 gives 0:4, 4:8, 8:10).
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off -fno-fast-math -pthread.
 * No FMA contraction, no fast-math: every product and sum is one IEEE binary64 op.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* element kinds */
enum { OR_I32 = 0, OR_F16 = 1, OR_BF16 = 2, OR_F32 = 3, OR_F64 = 4 };

/* ------------------------------------------------------------------------- */
/* Exact decoding of the 16-bit storage formats (IEEE 754 binary16, bfloat16). */

/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double oracle_decode_f16(uint16_t h) {
  int sign = h >> 15;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24); /* subnormal: f * 2^-10 * 2^-14 */
  } else if (e == 31) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(f + 1024), e - 15 - 10);
  }
  return sign ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits (upper half of binary32). */
double oracle_decode_bf16(uint16_t b) {
  int sign = b >> 15;
  int e = (b >> 7) & 0xff;
  int f = b & 0x7f;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -133); /* subnormal: f * 2^-7 * 2^-126 */
  } else if (e == 255) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(f + 128), e - 127 - 7);
  }
  return sign ? -v : v;
}

/* ------------------------------------------------------------------------- */
/* Correctly rounded (round-to-nearest, ties-to-even) binary64 -> narrow format.
 * A format is given by p (significand bits incl. the implicit one), emin (exponent
 * of the smallest normal) and emax (exponent of the largest finite). The result is
 * the bit pattern of the narrow format. One rounding, directly from binary64, so
 * no double rounding through binary32. */
static uint32_t encode_rne(double x, int p, int emin, int emax, int ebits) {
  uint32_t sign = signbit(x) ? 1u : 0u;
  uint32_t fbits = (uint32_t)(p - 1);
  uint32_t sign_bit = sign << (ebits + fbits);
  uint32_t exp_all = (1u << ebits) - 1u;
  if (isnan(x)) return sign_bit | (exp_all << fbits) | (1u << (fbits - 1)); /* quiet NaN */
  double ax = fabs(x);
  if (isinf(x)) return sign_bit | (exp_all << fbits);
  if (ax == 0.0) return sign_bit;
  int E; /* ax = m * 2^E with m in [0.5, 1): the leading bit has weight 2^(E-1) */
  frexp(ax, &E);
  int lead = E - 1;
  if (lead < emin) lead = emin; /* subnormal range: fixed quantum */
  int q = lead - (p - 1);       /* weight of the last kept bit */
  double r = nearbyint(ldexp(ax, -q)); /* default rounding mode: ties to even */
  double v = ldexp(r, q);
  if (v >= ldexp(1.0, emax + 1)) return sign_bit | (exp_all << fbits); /* overflow -> inf */
  /* encode v */
  if (v < ldexp(1.0, emin)) {
    /* subnormal (or zero after rounding): fraction = v / 2^(emin-(p-1)) */
    uint32_t frac = (uint32_t)ldexp(v, -(emin - (p - 1)));
    return sign_bit | frac;
  }
  int Ev;
  frexp(v, &Ev);
  int lv = Ev - 1;
  uint32_t frac = (uint32_t)(ldexp(v, -(lv - (p - 1))) - ldexp(1.0, p - 1));
  uint32_t bexp = (uint32_t)(lv - emin + 1);
  return sign_bit | (bexp << fbits) | frac;
}

uint16_t oracle_encode_f16(double x) { return (uint16_t)encode_rne(x, 11, -14, 15, 5); }
uint16_t oracle_encode_bf16(double x) { return (uint16_t)encode_rne(x, 8, -126, 127, 8); }
uint32_t oracle_encode_f32(double x) { return encode_rne(x, 24, -126, 127, 8); }

/* ------------------------------------------------------------------------- */
/* The product.                                                                */

typedef struct {
  int64_t M, N, K;
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb;
  int in_kind;
  void* C;
  int64_t ldc;
  int out_kind;
  /* rows to compute: either a contiguous range [r0, r1) or an explicit list */
  const int64_t* rows; /* if non-NULL, compute rows[idx] for idx in [r0, r1) and store C row idx */
  int64_t r0, r1;
  /* columns: NULL = all N columns (stored at column j), else cols[0..ncols) stored at column c */
  const int64_t* cols;
  int64_t ncols;
  const double* lut; /* 65536-entry exact decode table for 16-bit inputs */
} job_t;

static void store_out(void* C, int64_t ldc, int64_t i, int64_t j, int out_kind, double v) {
  switch (out_kind) {
    case OR_F64: ((double*)C)[i * ldc + j] = v; break;
    case OR_F32: ((uint32_t*)C)[i * ldc + j] = oracle_encode_f32(v); break;
    case OR_BF16: ((uint16_t*)C)[i * ldc + j] = oracle_encode_bf16(v); break;
    case OR_F16: ((uint16_t*)C)[i * ldc + j] = oracle_encode_f16(v); break;
    default: break;
  }
}

static void* run_job(void* arg) {
  job_t* jb = (job_t*)arg;
  const int64_t N = jb->N, K = jb->K;
  if (jb->in_kind == OR_I32) {
    const uint32_t* A = (const uint32_t*)jb->A;
    const uint32_t* B = (const uint32_t*)jb->B;
    uint32_t* C = (uint32_t*)jb->C;
    int64_t nc = jb->cols ? jb->ncols : N;
    uint32_t* acc = (uint32_t*)calloc((size_t)(nc > 0 ? nc : 1), sizeof(uint32_t));
    for (int64_t idx = jb->r0; idx < jb->r1; ++idx) {
      int64_t i = jb->rows ? jb->rows[idx] : idx;
      for (int64_t c = 0; c < nc; ++c) acc[c] = 0u;
      for (int64_t k = 0; k < K; ++k) {
        uint32_t a = A[i * jb->lda + k];
        const uint32_t* brow = B + k * jb->ldb;
        if (jb->cols) {
          for (int64_t c = 0; c < nc; ++c) acc[c] += a * brow[jb->cols[c]];
        } else {
          for (int64_t c = 0; c < nc; ++c) acc[c] += a * brow[c];
        }
      }
      for (int64_t c = 0; c < nc; ++c) C[idx * jb->ldc + c] = acc[c];
    }
    free(acc);
    return NULL;
  }
  /* 16-bit floating inputs, binary64 accumulation in ascending k */
  const uint16_t* A = (const uint16_t*)jb->A;
  const uint16_t* B = (const uint16_t*)jb->B;
  const double* lut = jb->lut;
  int64_t nc = jb->cols ? jb->ncols : N;
  double* acc = (double*)calloc((size_t)(nc > 0 ? nc : 1), sizeof(double));
  for (int64_t idx = jb->r0; idx < jb->r1; ++idx) {
    int64_t i = jb->rows ? jb->rows[idx] : idx;
    for (int64_t c = 0; c < nc; ++c) acc[c] = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      double a = lut[A[i * jb->lda + k]];
      const uint16_t* brow = B + k * jb->ldb;
      if (jb->cols) {
        for (int64_t c = 0; c < nc; ++c) acc[c] += a * lut[brow[jb->cols[c]]];
      } else {
        for (int64_t c = 0; c < nc; ++c) acc[c] += a * lut[brow[c]];
      }
    }
    for (int64_t c = 0; c < nc; ++c) store_out(jb->C, jb->ldc, idx, c, jb->out_kind, acc[c]);
  }
  free(acc);
  return NULL;
}

static int run_rows(job_t base, int64_t nrows, int threads) {
  double* lut = NULL;
  if (base.in_kind == OR_F16 || base.in_kind == OR_BF16) {
    lut = (double*)malloc(65536 * sizeof(double));
    if (!lut) return -1;
    for (uint32_t u = 0; u < 65536u; ++u)
      lut[u] = base.in_kind == OR_F16 ? oracle_decode_f16((uint16_t)u) : oracle_decode_bf16((uint16_t)u);
  }
  base.lut = lut;
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  if (nrows < threads) threads = nrows > 0 ? (int)nrows : 1;
  pthread_t tid[256];
  job_t jobs[256];
  int started[256];
  int64_t per = (nrows + threads - 1) / threads;
  for (int t = 0; t < threads; ++t) {
    jobs[t] = base;
    jobs[t].r0 = t * per < nrows ? t * per : nrows;
    jobs[t].r1 = (t + 1) * per < nrows ? (t + 1) * per : nrows;
    started[t] = pthread_create(&tid[t], NULL, run_job, &jobs[t]) == 0;
    if (!started[t]) run_job(&jobs[t]);
  }
  for (int t = 0; t < threads; ++t)
    if (started[t]) pthread_join(tid[t], NULL);
  free(lut);
  return 0;
}

static int kinds_ok(int in_kind, int out_kind) {
  if (in_kind == OR_I32) return out_kind == OR_I32;
  if (in_kind == OR_F16 || in_kind == OR_BF16)
    return out_kind == OR_F16 || out_kind == OR_BF16 || out_kind == OR_F32 || out_kind == OR_F64;
  return 0;
}

/* Full product: C (M x N, leading dimension ldc, elements of out_kind) = A @ B.
 * Returns 0 on success, -1 on a bad argument. */
int oracle_gemm(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                int in_kind, void* C, int64_t ldc, int out_kind, int threads) {
  if (M < 0 || N < 0 || K < 0 || !kinds_ok(in_kind, out_kind)) return -1;
  job_t jb;
  memset(&jb, 0, sizeof(jb));
  jb.M = M; jb.N = N; jb.K = K; jb.A = A; jb.lda = lda; jb.B = B; jb.ldb = ldb;
  jb.in_kind = in_kind; jb.C = C; jb.ldc = ldc; jb.out_kind = out_kind;
  return run_rows(jb, M, threads);
}

/* Selected full rows: out (nrows x N, dense) row r = row rows[r] of A @ B. */
int oracle_gemm_rows(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                     int in_kind, const int64_t* rows, int64_t nrows, void* out, int out_kind, int threads) {
  if (M < 0 || N < 0 || K < 0 || !kinds_ok(in_kind, out_kind)) return -1;
  for (int64_t r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= M) return -1;
  job_t jb;
  memset(&jb, 0, sizeof(jb));
  jb.M = M; jb.N = N; jb.K = K; jb.A = A; jb.lda = lda; jb.B = B; jb.ldb = ldb;
  jb.in_kind = in_kind; jb.C = out; jb.ldc = N; jb.out_kind = out_kind; jb.rows = rows;
  return run_rows(jb, nrows, threads);
}

/* Selected full columns: out (M x ncols, dense) column c = column cols[c] of A @ B. */
int oracle_gemm_cols(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                     int in_kind, const int64_t* cols, int64_t ncols, void* out, int out_kind, int threads) {
  if (M < 0 || N < 0 || K < 0 || !kinds_ok(in_kind, out_kind)) return -1;
  for (int64_t c = 0; c < ncols; ++c)
    if (cols[c] < 0 || cols[c] >= N) return -1;
  job_t jb;
  memset(&jb, 0, sizeof(jb));
  jb.M = M; jb.N = N; jb.K = K; jb.A = A; jb.lda = lda; jb.B = B; jb.ldb = ldb;
  jb.in_kind = in_kind; jb.C = out; jb.ldc = ncols; jb.out_kind = out_kind; jb.cols = cols; jb.ncols = ncols;
  return run_rows(jb, M, threads);
}

/* ------------------------------------------------------------------------- */
/* The pages' analytic counts.                                                 */

/* Operation count: one multiply plus one add per (i, j, k). */
int64_t oracle_ops(int64_t M, int64_t N, int64_t K) { return 2 * M * N * K; }

/* Number of tiles of size t covering D (the last may be partial). */
int64_t oracle_tile_count(int64_t D, int64_t t) { return D <= 0 ? 0 : (D + t - 1) / t; }

/* Tile i of size t over a dimension of length D covers [lo, hi). */
void oracle_tile_range(int64_t i, int64_t t, int64_t D, int64_t* lo, int64_t* hi) {
  int64_t a = i * t, b = (i + 1) * t;
  *lo = a < D ? a : D;
  *hi = b < D ? b : D;
}

/* No-reuse traffic of the output-stationary loop, in ELEMENTS, walked tile by
 * tile: for every output tile (mo, no) and every reduction chunk ko, the A tile
 * and the B tile of that step are read over their actual ranges; every output
 * tile is written once over its actual ranges. out[0] = A, out[1] = B, out[2] = C.
 * With padded != 0 every tile is counted at its full nominal size instead (the
 * overestimate the edge-tile section warns about). */
void oracle_traffic_elems(int64_t M, int64_t N, int64_t K, int64_t tm, int64_t tn, int64_t tk, int padded,
                          int64_t out[3]) {
  int64_t a = 0, b = 0, c = 0;
  int64_t nm = oracle_tile_count(M, tm), nn = oracle_tile_count(N, tn), nk = oracle_tile_count(K, tk);
  for (int64_t mi = 0; mi < nm; ++mi) {
    int64_t m0, m1;
    oracle_tile_range(mi, tm, M, &m0, &m1);
    int64_t rows = padded ? tm : m1 - m0;
    for (int64_t ni = 0; ni < nn; ++ni) {
      int64_t n0, n1;
      oracle_tile_range(ni, tn, N, &n0, &n1);
      int64_t colsn = padded ? tn : n1 - n0;
      for (int64_t ki = 0; ki < nk; ++ki) {
        int64_t k0, k1;
        oracle_tile_range(ki, tk, K, &k0, &k1);
        int64_t depth = padded ? tk : k1 - k0;
        a += rows * depth;  /* A_tile(mo, ko) */
        b += depth * colsn; /* B_tile(ko, no) */
      }
      c += rows * colsn; /* write_C_tile(mo, no) */
    }
  }
  out[0] = a;
  out[1] = b;
  out[2] = c;
}

/* The same counts in BYTES, for input element size s_in and output size s_out. */
void oracle_traffic_bytes(int64_t M, int64_t N, int64_t K, int64_t tm, int64_t tn, int64_t tk, int64_t s_in,
                          int64_t s_out, int padded, int64_t out[3]) {
  int64_t e[3];
  oracle_traffic_elems(M, N, K, tm, tn, tk, padded, e);
  out[0] = e[0] * s_in;
  out[1] = e[1] * s_in;
  out[2] = e[2] * s_out;
}

/* Resident working set of one tile step in bytes: A tile, B tile, accumulator.
 * out[0] = A, out[1] = B, out[2] = accumulator (s_acc bytes per element). */
void oracle_footprint_bytes(int64_t tm, int64_t tn, int64_t tk, int64_t s_in, int64_t s_acc, int64_t out[3]) {
  out[0] = tm * tk * s_in;
  out[1] = tk * tn * s_in;
  out[2] = tm * tn * s_acc;
}
