/* A C driver of the CPU oracle (oracle/oracle.c) for sanitizer builds: it calls every
 * exported entry point on small cases, including empty and ragged shapes, padded
 * leading dimensions, every input/output kind and several thread counts, and checks
 * what does not depend on rounding: the worked 9x9 int32 example against its closed
 * form, sampled rows and columns against the full product bit for bit, the results
 * for 1, 3 and 8 threads bit for bit, the pages' 576 KiB traffic example, and the
 * rejection of bad arguments. Exit status 0 and "oracle_client: ok" on success. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_gemm(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                int in_kind, void* C, int64_t ldc, int out_kind, int threads);
int oracle_gemm_rows(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                     int in_kind, const int64_t* rows, int64_t nrows, void* out, int out_kind, int threads);
int oracle_gemm_cols(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                     int in_kind, const int64_t* cols, int64_t ncols, void* out, int out_kind, int threads);
int64_t oracle_ops(int64_t M, int64_t N, int64_t K);
int64_t oracle_tile_count(int64_t D, int64_t t);
void oracle_tile_range(int64_t i, int64_t t, int64_t D, int64_t* lo, int64_t* hi);
void oracle_traffic_bytes(int64_t M, int64_t N, int64_t K, int64_t tm, int64_t tn, int64_t tk, int64_t s_in,
                          int64_t s_out, int padded, int64_t out[3]);
void oracle_footprint_bytes(int64_t tm, int64_t tn, int64_t tk, int64_t s_in, int64_t s_acc, int64_t out[3]);
double oracle_decode_f16(uint16_t h);
double oracle_decode_bf16(uint16_t b);
uint16_t oracle_encode_f16(double x);
uint16_t oracle_encode_bf16(double x);
uint32_t oracle_encode_f32(double x);

enum { I32 = 0, F16 = 1, BF16 = 2, F32 = 3, F64 = 4 };

#define EXPECT(c)                                                        \
  do {                                                                   \
    if (!(c)) {                                                          \
      fprintf(stderr, "oracle_client: %s:%d: %s\n", __FILE__, __LINE__, #c); \
      return 1;                                                          \
    }                                                                    \
  } while (0)

static size_t out_size(int kind) { return kind == F64 ? 8 : (kind == F32 || kind == I32) ? 4 : 2; }

static uint32_t lcg(uint32_t* s) {
  *s = *s * 1664525u + 1013904223u;
  return *s >> 8;
}

static int worked_example(void) {
  int32_t a[81], b[81], c[81];
  for (int i = 0; i < 9; ++i)
    for (int j = 0; j < 9; ++j) {
      a[9 * i + j] = 9 * i + j;
      b[9 * i + j] = 2 * (9 * i + j);
    }
  EXPECT(oracle_gemm(9, 9, 9, a, 9, b, 9, I32, c, 9, I32, 2) == 0);
  for (int i = 0; i < 9; ++i)
    for (int j = 0; j < 9; ++j) EXPECT(c[9 * i + j] == 3672 + 5832 * i + 72 * j + 162 * i * j);
  return 0;
}

/* One ragged case: full product with padded leading dimensions, for 1/3/8 threads,
 * against sampled rows and columns. */
static int ragged_case(int64_t M, int64_t N, int64_t K, int in_kind, int out_kind, uint32_t seed) {
  const int64_t lda = K + 3, ldb = N + 5, ldc = N + 2;
  const size_t ib = in_kind == I32 ? 4 : 2, ob = out_size(out_kind);
  unsigned char* A = calloc((size_t)(M > 0 ? M : 1) * (size_t)lda + 1, ib);
  unsigned char* B = calloc((size_t)(K > 0 ? K : 1) * (size_t)ldb + 1, ib);
  unsigned char* C1 = calloc((size_t)(M > 0 ? M : 1) * (size_t)ldc + 1, ob);
  unsigned char* C3 = calloc((size_t)(M > 0 ? M : 1) * (size_t)ldc + 1, ob);
  unsigned char* R = calloc((size_t)(N > 0 ? N : 1) * 2 + 1, ob);
  unsigned char* Q = calloc((size_t)(M > 0 ? M : 1) * 2 + 1, ob);
  if (!A || !B || !C1 || !C3 || !R || !Q) return 1;
  for (int64_t i = 0; i < M * lda; ++i) {
    const int v = (int)(lcg(&seed) % 17) - 8; /* small integers: exact in every input kind */
    if (in_kind == I32)
      ((int32_t*)A)[i] = v;
    else
      ((uint16_t*)A)[i] = in_kind == F16 ? oracle_encode_f16(v) : oracle_encode_bf16(v);
  }
  for (int64_t i = 0; i < K * ldb; ++i) {
    const int v = (int)(lcg(&seed) % 17) - 8;
    if (in_kind == I32)
      ((int32_t*)B)[i] = v;
    else
      ((uint16_t*)B)[i] = in_kind == F16 ? oracle_encode_f16(v) : oracle_encode_bf16(v);
  }
  EXPECT(oracle_gemm(M, N, K, A, lda, B, ldb, in_kind, C1, ldc, out_kind, 1) == 0);
  for (int t = 3; t <= 8; t += 5) {
    EXPECT(oracle_gemm(M, N, K, A, lda, B, ldb, in_kind, C3, ldc, out_kind, t) == 0);
    EXPECT(memcmp(C1, C3, (size_t)(M > 0 ? M : 1) * (size_t)ldc * ob) == 0);
  }
  if (M > 0 && N > 0) {
    const int64_t rows[2] = {0, M - 1}, cols[2] = {N - 1, 0};
    EXPECT(oracle_gemm_rows(M, N, K, A, lda, B, ldb, in_kind, rows, 2, R, out_kind, 2) == 0);
    EXPECT(oracle_gemm_cols(M, N, K, A, lda, B, ldb, in_kind, cols, 2, Q, out_kind, 3) == 0);
    for (int r = 0; r < 2; ++r)
      EXPECT(memcmp(R + (size_t)r * (size_t)N * ob, C1 + (size_t)rows[r] * (size_t)ldc * ob, (size_t)N * ob) == 0);
    for (int64_t i = 0; i < M; ++i)
      for (int c = 0; c < 2; ++c)
        EXPECT(memcmp(Q + ((size_t)i * 2 + (size_t)c) * ob, C1 + ((size_t)i * (size_t)ldc + (size_t)cols[c]) * ob,
                      ob) == 0);
    const int64_t bad[1] = {M};
    EXPECT(oracle_gemm_rows(M, N, K, A, lda, B, ldb, in_kind, bad, 1, R, out_kind, 1) == -1);
  }
  free(A);
  free(B);
  free(C1);
  free(C3);
  free(R);
  free(Q);
  return 0;
}

int main(void) {
  if (worked_example()) return 1;
  static const int64_t shapes[][3] = {{0, 5, 3}, {4, 0, 3}, {3, 4, 0}, {1, 1, 1}, {7, 5, 3}, {17, 19, 1}, {33, 20, 70}};
  static const int kinds[][2] = {{I32, I32}, {F16, F32}, {F16, F16}, {BF16, F32}, {BF16, BF16}, {BF16, F64},
                                 {F16, F64}};
  uint32_t seed = 12345;
  for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s)
    for (size_t k = 0; k < sizeof(kinds) / sizeof(kinds[0]); ++k)
      if (ragged_case(shapes[s][0], shapes[s][1], shapes[s][2], kinds[k][0], kinds[k][1], seed++)) {
        fprintf(stderr, "oracle_client: case %zu kind %zu\n", s, k);
        return 1;
      }
  /* bad arguments */
  int32_t x = 0;
  EXPECT(oracle_gemm(-1, 1, 1, &x, 1, &x, 1, I32, &x, 1, I32, 1) == -1);
  EXPECT(oracle_gemm(1, 1, 1, &x, 1, &x, 1, I32, &x, 1, F32, 1) == -1);
  EXPECT(oracle_gemm(1, 1, 1, &x, 1, &x, 1, F32, &x, 1, F32, 1) == -1);
  /* counts */
  EXPECT(oracle_ops(128, 128, 128) == 4194304);
  int64_t t[3], lo, hi;
  oracle_traffic_bytes(128, 128, 128, 16, 16, 32, 2, 4, 0, t);
  EXPECT(t[0] + t[1] + t[2] == 589824);
  oracle_footprint_bytes(16, 16, 32, 2, 4, t);
  EXPECT(t[0] == 1024 && t[1] == 1024 && t[2] == 1024);
  EXPECT(oracle_tile_count(10, 4) == 3 && oracle_tile_count(0, 4) == 0);
  oracle_tile_range(2, 4, 10, &lo, &hi);
  EXPECT(lo == 8 && hi == 10);
  /* encoders and decoders at the format limits */
  EXPECT(oracle_decode_f16(oracle_encode_f16(65504.0)) == 65504.0);
  EXPECT(oracle_encode_f16(65520.0) == 0x7C00);
  EXPECT(oracle_decode_bf16(oracle_encode_bf16(-3.0)) == -3.0);
  EXPECT(oracle_encode_f32(1e-46) == 0u && oracle_encode_f32(2e-45) == 1u);
  printf("oracle_client: ok\n");
  return 0;
}
