// int32_valu.hip -- exact int32 path and the K = 0 zero fill.
//
// MFMA has no int32 x int32 form, so the integer product runs on the vector ALU
// with the same output-stationary schedule: one workgroup per tm x tn C tile with
// runtime tile sizes (the Mojo puzzle's 9x9 example uses 3 x 3 tiles), the A and
// B K-tiles of each step staged in LDS, guarded loads that read zeros outside the
// matrices, uniform barriers and a guarded store (Mojo GPU puzzles, "Tiled Matrix
// Multiplication", sections 3-6). Each thread keeps its C element in a register
// for the whole reduction. Products and sums are unsigned 32-bit, i.e. they wrap
// modulo 2^32, so the result does not depend on the order of the sum. A and B are
// addressed through element strides, which covers operands supplied transposed.
#include "device_common.h"
#include "launch.h"

namespace tg {

__global__ __launch_bounds__(1024) void i32_tile_kernel(I32Args p) {
  extern __shared__ __attribute__((aligned(16))) uint32_t smem_i32[];
  const int tm = p.tm, tn = p.tn, tk = p.tk;
  uint32_t* as = smem_i32;            // tm x tk
  uint32_t* bs = smem_i32 + tm * tk;  // tk x tn
  const int t = threadIdx.x, nthreads = blockDim.x;
  const int ty = t / tn, tx = t % tn;
  const int tile_m = blockIdx.x / p.tiles_n, tile_n = blockIdx.x % p.tiles_n;
  const int row0 = tile_m * tm, col0 = tile_n * tn;
  const int row = row0 + ty, col = col0 + tx;
  const uint32_t* A = (const uint32_t*)p.A;
  const uint32_t* B = (const uint32_t*)p.B;
  uint32_t acc = 0u;
  for (int k0 = 0; k0 < p.K; k0 += tk) {
    for (int q = t; q < tm * tk; q += nthreads) {
      const int r = q / tk, c = q % tk;
      as[q] = (row0 + r < p.M && k0 + c < p.K) ? A[(int64_t)(row0 + r) * p.sa_m + (int64_t)(k0 + c) * p.sa_k] : 0u;
    }
    for (int q = t; q < tk * tn; q += nthreads) {
      const int r = q / tn, c = q % tn;
      bs[q] = (k0 + r < p.K && col0 + c < p.N) ? B[(int64_t)(k0 + r) * p.sb_k + (int64_t)(col0 + c) * p.sb_n] : 0u;
    }
    __syncthreads();
    const int kmax = (p.K - k0) < tk ? (p.K - k0) : tk;
    if (ty < tm) {
      // a row of as is broadcast, bs[k][tx] is read by consecutive threads
      for (int k = 0; k < kmax; ++k) acc += as[ty * tk + k] * bs[k * tn + tx];
    }
    __syncthreads();
  }
  if (ty < tm && row < p.M && col < p.N) ((uint32_t*)p.C)[(int64_t)row * p.ldc + col] = acc;
}

hipError_t launch_i32(const I32Args& a, hipStream_t s, int64_t grid, int threads, int lds_bytes) {
  hipLaunchKernelGGL(i32_tile_kernel, dim3((unsigned)grid), dim3(threads), lds_bytes, s, a);
  return hipGetLastError();
}

// The empty sum (K = 0): every element of C becomes zero.
template <typename T>
__global__ __launch_bounds__(256) void zero_fill_kernel(T* C, int64_t M, int64_t N, int64_t ldc) {
  const int64_t total = M * N;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total; q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = q / N, c = q % N;
    C[r * ldc + c] = T(0);
  }
}

hipError_t launch_zero_fill(void* C, int64_t M, int64_t N, int64_t ldc, int elem_bytes, hipStream_t s) {
  const int64_t total = M * N;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (elem_bytes == 4)
    hipLaunchKernelGGL(zero_fill_kernel<uint32_t>, dim3((unsigned)blocks), dim3(256), 0, s, (uint32_t*)C, M, N, ldc);
  else
    hipLaunchKernelGGL(zero_fill_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, s, (uint16_t*)C, M, N, ldc);
  return hipGetLastError();
}

}  // namespace tg
