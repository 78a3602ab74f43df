// launch.h -- kernel argument blocks and launchers (host side of the kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {

// Arguments of the MFMA kernels. Dimensions fit in int32 (checked by the host).
struct MacroArgs {
  const uint16_t* A;
  const uint16_t* B;
  void* C;
  int M, N, K;
  int64_t lda, ldb, ldc;
  int tiles_m, tiles_n, group_m;
  // split-K: workgroup (tile, blockIdx.y) reduces K-tiles [y * kt_per_split, (y+1) * kt_per_split)
  // and writes its fp32 partial tile at C + y * split_stride (elements); without split-K,
  // kt_per_split covers all K-tiles and gridDim.y == 1
  int kt_per_split;
  int64_t split_stride;
  // C's base is aligned to its element size: interior tiles are stored as 16-byte
  // chunks of consecutive columns, at whatever alignment the row start gives them
  // (gfx950 compute queues run with unaligned vector memory access).
  int c_vec;
};

struct MacroShape {
  int bm, bn, bk, threads, lds, stages;
};
constexpr int kNumMacroShapes = 7;
extern const MacroShape kMacroShapes[kNumMacroShapes];

// in: 0 = f16, 1 = bf16. out: 0 = f32, 1 = bf16, 2 = f16. ta: A is stored transposed
// (K x M, row stride lda); tb: B is stored transposed (N x K, row stride ldb).
hipError_t launch_macro(int shape, const MacroArgs& a, int in, int out, bool vec, hipStream_t s, int64_t grid,
                        int splits, bool ta, bool tb);
// The C tiles of the split-K launch whose partials are summed: their size, count, and
// whether the workgroups kept the hardware's order (MacroArgs::group_m == 0).
struct SplitTiles {
  int bm, bn, tiles_m, tiles_n;
  bool hw_order;
};
// C[0:M, 0:N] = sum over s < splits of ws[s][M][N] (dense fp32 partials, summed in slice order),
// rounded to the output format (out: 0 = f32, 1 = bf16, 2 = f16).
hipError_t launch_splitk_reduce(const float* ws, int splits, void* C, int64_t ldc, int M, int N, int out,
                                const SplitTiles& g, hipStream_t s);
hipError_t launch_small(const MacroArgs& a, int in, int out, bool vec, hipStream_t s, int64_t grid, bool ta, bool tb);

struct I32Args {
  const int32_t* A;
  const int32_t* B;
  int32_t* C;
  int M, N, K;
  int64_t sa_m, sa_k;  // element (m, k) of op(A) is A[m * sa_m + k * sa_k]
  int64_t sb_k, sb_n;  // element (k, n) of op(B) is B[k * sb_k + n * sb_n]
  int64_t ldc;
  int tm, tn, tk, tiles_n;
};
hipError_t launch_i32(const I32Args& a, hipStream_t s, int64_t grid, int threads, int lds_bytes);

// Copy a rows x cols matrix of 16-bit elements (row stride ld_src) into dst (16-byte
// aligned, row stride ld_dst >= cols, a multiple of 8), zeros completing the last
// 16-byte chunk of each row.
hipError_t launch_repack(const uint16_t* src, int64_t ld_src, uint16_t* dst, int64_t ld_dst, int64_t rows,
                         int64_t cols, hipStream_t s);

// C[0:M, 0:N] = 0 for element size 2 or 4 bytes.
hipError_t launch_zero_fill(void* C, int64_t M, int64_t N, int64_t ldc, int elem_bytes, hipStream_t s);

}  // namespace tg
