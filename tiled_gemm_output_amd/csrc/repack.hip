// repack.hip -- copy of a 16-bit operand into rows that start on 128-byte boundaries.
//
// The macro-tile kernel loads each K-tile row segment as whole 16-byte chunks. When
// an operand's rows do not start on 128-byte boundaries (a leading dimension that is
// not a multiple of 64 elements, or an offset base), every 128-byte segment of a
// K-contiguous row spans two cache lines and the load stream grows accordingly. A copy into rows padded to a
// multiple of 64 elements costs one read and one write of the operand; the host takes
// it when the estimated time saved is larger.
#include "device_common.h"
#include "launch.h"

namespace tg {

// rows x cols elements from src (row stride ld_src, 2-byte aligned) to dst (16-byte
// aligned, row stride ld_dst a multiple of 8). One 16-byte chunk per thread and step;
// the chunk that crosses the end of a row is completed with zeros.
__global__ __launch_bounds__(256) void repack_rows_kernel(const uint16_t* src, int64_t ld_src, uint16_t* dst,
                                                          int64_t ld_dst, int64_t rows, int64_t cols) {
  const int64_t chunks = (cols + 7) / 8, total = rows * chunks;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total; q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = q / chunks, c0 = (q - r * chunks) * 8;
    const uint16_t* s = src + r * ld_src + c0;
    i32x4 v;
    if (c0 + 8 <= cols) {
      __builtin_memcpy(&v, s, 16);  // 2-byte aligned 16-byte load
    } else {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = (c0 + 2 * e < cols) ? s[2 * e] : 0u;
        const uint32_t hi = (c0 + 2 * e + 1 < cols) ? s[2 * e + 1] : 0u;
        w[e] = lo | (hi << 16);
      }
      v = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    }
    *(i32x4*)(dst + r * ld_dst + c0) = v;
  }
}

hipError_t launch_repack(const uint16_t* src, int64_t ld_src, uint16_t* dst, int64_t ld_dst, int64_t rows,
                         int64_t cols, hipStream_t s) {
  const int64_t total = rows * ((cols + 7) / 8);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) return hipSuccess;
  hipLaunchKernelGGL(repack_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, ld_src, dst, ld_dst, rows, cols);
  return hipGetLastError();
}

}  // namespace tg
