/* A plain C client of include/tgemm.h (no C++, no Python): what a C caller of the
 * library sees. Mode "host": only the host-side entry points (argument checks,
 * plans, counts, status strings) -- runs without a GPU. Mode "gpu": creates a
 * handle, multiplies two small bf16 matrices of small integers on the device and
 * compares with an exact host product. Exit status 0 on success. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h> /* device memory for the test (the HIP runtime's C API) */

#include "tgemm.h"

#define EXPECT(c)                                                     \
  do {                                                                \
    if (!(c)) {                                                       \
      fprintf(stderr, "abi_client: %s:%d: %s\n", __FILE__, __LINE__, #c); \
      return 1;                                                       \
    }                                                                 \
  } while (0)

static uint16_t bf16_of_int(int v) { /* small integers are exact in bfloat16 */
  float f = (float)v;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static int host_mode(void) {
  const void* p = (const void*)(uintptr_t)0x100000;
  gemm_plan_t plan;
  gemm_model_t model;
  EXPECT(gemm_check_args(64, 48, 32, p, 32, p, 48, p, 48, GEMM_BF16_BF16) == GEMM_OK);
  EXPECT(gemm_check_args(64, 48, 32, p, 31, p, 48, p, 48, GEMM_BF16_BF16) == GEMM_ERR_INVALID_ARG);
  EXPECT(gemm_check_args(64, 48, 32, p, 32, p, 48, p, 48, (gemm_dtype_t)9) == GEMM_ERR_UNSUPPORTED_DTYPE);
  EXPECT(gemm_check_args_op(GEMM_OP_T, GEMM_OP_T, 64, 48, 32, p, 64, p, 32, p, 48, GEMM_F16_F32) == GEMM_OK);
  EXPECT(gemm_plan(NULL, 8192, 8192, 8192, p, 8192, p, 8192, p, 8192, GEMM_BF16_BF16, &plan) == GEMM_OK);
  EXPECT(plan.kernel == 4 && plan.tile_m == 256 && plan.tile_n == 256 && plan.grid == 1024 && plan.split_k == 1);
  EXPECT(gemm_model(&plan, 8192, 8192, 8192, GEMM_BF16_BF16, &model) == GEMM_OK);
  EXPECT(model.flops == 2.0 * 8192.0 * 8192.0 * 8192.0 && model.tiles == 1024 && model.k_steps == 128);
  /* the pages' traffic example: 128^3, 16x16x32 tiles, fp16 in, fp32 C -> 576 KiB */
  memset(&plan, 0, sizeof(plan));
  plan.tile_m = plan.tile_n = 16;
  plan.tile_k = 32;
  plan.kernel = 3;
  plan.split_k = 1;
  EXPECT(gemm_model(&plan, 128, 128, 128, GEMM_F16_F32, &model) == GEMM_OK);
  EXPECT(model.bytes_a + model.bytes_b + model.bytes_c == 589824.0);
  EXPECT(strcmp(gemm_status_string(GEMM_OK), "GEMM_OK") == 0);
  EXPECT(gemm_destroy(NULL) == GEMM_ERR_INVALID_ARG);
  printf("abi_client host: ok\n");
  return 0;
}

static int gpu_mode(void) {
  enum { M = 200, N = 136, K = 520 };
  gemm_handle_t h = NULL;
  gemm_status_t st = gemm_create(&h);
  if (st != GEMM_OK) {
    fprintf(stderr, "abi_client: gemm_create: %s\n", gemm_status_string(st));
    return 1;
  }
  uint16_t* a = malloc(sizeof(uint16_t) * M * K);
  uint16_t* b = malloc(sizeof(uint16_t) * K * N);
  float* c = malloc(sizeof(float) * M * N);
  int* ai = malloc(sizeof(int) * M * K);
  int* bi = malloc(sizeof(int) * K * N);
  EXPECT(a && b && c && ai && bi);
  for (int i = 0; i < M * K; ++i) ai[i] = (int)((i * 7u + 3u) % 9u) - 4;
  for (int i = 0; i < K * N; ++i) bi[i] = (int)((i * 5u + 1u) % 9u) - 4;
  for (int i = 0; i < M * K; ++i) a[i] = bf16_of_int(ai[i]);
  for (int i = 0; i < K * N; ++i) b[i] = bf16_of_int(bi[i]);
  void *da = NULL, *db = NULL, *dc = NULL;
  EXPECT(hipMalloc(&da, sizeof(uint16_t) * M * K) == hipSuccess);
  EXPECT(hipMalloc(&db, sizeof(uint16_t) * K * N) == hipSuccess);
  EXPECT(hipMalloc(&dc, sizeof(float) * M * N) == hipSuccess);
  EXPECT(hipMemcpy(da, a, sizeof(uint16_t) * M * K, hipMemcpyHostToDevice) == hipSuccess);
  EXPECT(hipMemcpy(db, b, sizeof(uint16_t) * K * N, hipMemcpyHostToDevice) == hipSuccess);
  EXPECT(gemm_run(h, M, N, K, da, K, db, N, dc, N, GEMM_BF16_F32, NULL) == GEMM_OK);
  EXPECT(hipDeviceSynchronize() == hipSuccess);
  EXPECT(hipMemcpy(c, dc, sizeof(float) * M * N, hipMemcpyDeviceToHost) == hipSuccess);
  long bad = 0;
  for (int i = 0; i < M; ++i)
    for (int j = 0; j < N; ++j) {
      long s = 0;
      for (int k = 0; k < K; ++k) s += (long)ai[i * K + k] * bi[k * N + j];
      if (c[i * N + j] != (float)s) ++bad; /* |s| < 2^24: exact in fp32 whatever the order */
    }
  EXPECT(bad == 0);
  EXPECT(gemm_destroy(h) == GEMM_OK);
  (void)hipFree(da);
  (void)hipFree(db);
  (void)hipFree(dc);
  free(a), free(b), free(c), free(ai), free(bi);
  printf("abi_client gpu: ok (%dx%dx%d bf16 -> fp32, exact)\n", M, N, K);
  return 0;
}

/* Every planning path on the host: shapes from empty to past one round of 256x256
 * tiles, padded and odd leading dimensions, odd and even addresses, all operand forms
 * and dtypes. Each plan must be accepted, and its counts must hold 2MNK flops. */
static int sweep_mode(void) {
  static const int64_t dims[] = {0, 1, 7, 16, 63, 64, 65, 255, 256, 257, 1000, 4095, 4352, 8191, 8193, 20000};
  static const int64_t pads[] = {0, 1, 8, 64};
  static const uintptr_t bases[] = {0x100000, 0x100002, 0x100001};
  const int nd = (int)(sizeof(dims) / sizeof(dims[0]));
  long plans = 0;
  for (int dt = 0; dt <= 4; ++dt)
    for (int op = 0; op < 4; ++op)
      for (int im = 0; im < nd; ++im)
        for (int in = 0; in < nd; in += 2)
          for (int ik = (im + in) % 3; ik < nd; ik += 3) {
            const int64_t M = dims[im], N = dims[in], K = dims[ik];
            const gemm_op_t oa = (op & 1) ? GEMM_OP_T : GEMM_OP_N, ob = (op & 2) ? GEMM_OP_T : GEMM_OP_N;
            const int64_t pad = pads[(im + ik) % 4];
            const int64_t lda = (oa == GEMM_OP_T ? M : K) + pad, ldb = (ob == GEMM_OP_T ? K : N) + pad, ldc = N + pad;
            const void* A = (const void*)bases[(im + in) % 3];
            const void* B = (const void*)bases[(in + ik) % 3];
            void* C = (void*)bases[(im + 2 * ik) % 3];
            const gemm_dtype_t dtype = (gemm_dtype_t)dt;
            const gemm_status_t chk = gemm_check_args_op(oa, ob, M, N, K, A, lda, B, ldb, C, ldc, dtype);
            gemm_plan_t plan;
            gemm_model_t model;
            const gemm_status_t st = gemm_plan_op(NULL, oa, ob, M, N, K, A, lda, B, ldb, C, ldc, dtype, &plan);
            EXPECT(st == chk);
            if (st != GEMM_OK) continue;
            EXPECT(gemm_model(&plan, M, N, K, dtype, &model) == GEMM_OK);
            EXPECT(model.flops == 2.0 * (double)M * (double)N * (double)K);
            ++plans;
          }
  EXPECT(plans > 5000);
  printf("abi_client sweep: ok (%ld plans)\n", plans);
  return 0;
}

int main(int argc, char** argv) {
  if (argc > 1 && strcmp(argv[1], "gpu") == 0) return gpu_mode();
  if (argc > 1 && strcmp(argv[1], "sweep") == 0) return sweep_mode();
  return host_mode();
}
