// macro_tile.hip -- launches of the macro-tile GEMM (the kernel is in
// macro_tile_kernel.h): the table of tile shapes, the dispatch over operand layouts
// and tiles, and the split-K reduction. The kernels themselves are instantiated in
// macro_tile_inst_*.hip.
#include "macro_tile_kernel.h"

namespace tg {

// Split-K reduction: the partial tiles of the K-slices are summed in slice order
// (deterministic) and rounded once to the output format.
template <int OUT>
__device__ __forceinline__ void store_out(void* C, int64_t off, float x) {
  if constexpr (OUT == OUT_F32)
    ((float*)C)[off] = x;
  else if constexpr (OUT == OUT_BF16)
    ((uint16_t*)C)[off] = f32_to_bf16_rne(x);
  else
    ((uint16_t*)C)[off] = f32_to_f16_rne(x);
}

// Each thread sums G consecutive elements of one row (G = 4 when N % 4 == 0: the
// workspace is dense, so every group is a 16-byte aligned vector of one row). VS:
// C's rows start on a multiple of four elements and C is aligned to four elements, so
// the four results go out in one store. The workspace is read once: non-temporal loads.
template <int OUT, int G, bool VS>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* ws, int splits, void* C, int64_t ldc, int M,
                                                           int N) {
  const int64_t slice = (int64_t)M * N, groups = slice / G;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < groups; q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = q * G, r = e / N, c = e - r * N;
    if constexpr (G == 4) {
      f32x4 acc = __builtin_nontemporal_load((const f32x4*)(ws + e));
      for (int s = 1; s < splits; ++s) {
        const f32x4 x = __builtin_nontemporal_load((const f32x4*)(ws + s * slice + e));
        acc.x += x.x;
        acc.y += x.y;
        acc.z += x.z;
        acc.w += x.w;
      }
      if constexpr (VS) {
        const int64_t off = r * ldc + c;
        if constexpr (OUT == OUT_F32) {
          *(f32x4*)((float*)C + off) = acc;
        } else if constexpr (OUT == OUT_BF16) {
          *(u32x2*)((uint16_t*)C + off) = u32x2{pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w)};
        } else {
          *(u32x2*)((uint16_t*)C + off) =
              u32x2{(uint32_t)f32_to_f16_rne(acc.x) | ((uint32_t)f32_to_f16_rne(acc.y) << 16),
                    (uint32_t)f32_to_f16_rne(acc.z) | ((uint32_t)f32_to_f16_rne(acc.w) << 16)};
        }
      } else {
        store_out<OUT>(C, r * ldc + c, acc.x);
        store_out<OUT>(C, r * ldc + c + 1, acc.y);
        store_out<OUT>(C, r * ldc + c + 2, acc.z);
        store_out<OUT>(C, r * ldc + c + 3, acc.w);
      }
    } else {
      float acc = ws[e];
      for (int s = 1; s < splits; ++s) acc += ws[s * slice + e];
      store_out<OUT>(C, r * ldc + c, acc);
    }
  }
}

// The same sum, organised by the GEMM's C tiles for a launch whose workgroups kept the
// hardware's order (tile = workgroup id) and whose tile count is a multiple of the 8
// XCDs: every K-slice of tile t then ran on XCD t % 8, which still holds the slices'
// partial tiles in its L2, and workgroup b of this kernel runs on XCD b % 8. So
// workgroup b sums part b / 8 % P of tile 8 * (b / 8 / P) + b % 8 (P parts of 1024
// elements per tile; rows and columns outside C are skipped; N % 4 == 0).
template <int OUT, bool VS, int BN>
__global__ __launch_bounds__(256) void splitk_reduce_tiles_kernel(const float* ws, int splits, void* C, int64_t ldc,
                                                                 int M, int N, int bm, int tiles_m) {
  constexpr int CPR = BN / 4;           // threads per tile row
  constexpr int RPP = 1024 / BN;        // tile rows per part
  const int P = bm / RPP;               // parts per tile
  const int b = blockIdx.x, x = b % 8, j = b / 8;
  const int t = x + 8 * (j / P), part = j % P;
  const int tm = t % tiles_m, tn = t / tiles_m;
  const int row = tm * bm + part * RPP + (int)threadIdx.x / CPR;
  const int col = tn * BN + 4 * ((int)threadIdx.x % CPR);
  if (row >= M || col >= N) return;
  const int64_t slice = (int64_t)M * N, e = (int64_t)row * N + col;
  f32x4 acc = __builtin_nontemporal_load((const f32x4*)(ws + e));
  for (int s = 1; s < splits; ++s) {
    const f32x4 v = __builtin_nontemporal_load((const f32x4*)(ws + s * slice + e));
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  const int64_t off = (int64_t)row * ldc + col;
  if constexpr (VS) {
    if constexpr (OUT == OUT_F32) {
      *(f32x4*)((float*)C + off) = acc;
    } else if constexpr (OUT == OUT_BF16) {
      *(u32x2*)((uint16_t*)C + off) = u32x2{pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w)};
    } else {
      *(u32x2*)((uint16_t*)C + off) =
          u32x2{(uint32_t)f32_to_f16_rne(acc.x) | ((uint32_t)f32_to_f16_rne(acc.y) << 16),
                (uint32_t)f32_to_f16_rne(acc.z) | ((uint32_t)f32_to_f16_rne(acc.w) << 16)};
    }
  } else {
    store_out<OUT>(C, off, acc.x);
    store_out<OUT>(C, off + 1, acc.y);
    store_out<OUT>(C, off + 2, acc.z);
    store_out<OUT>(C, off + 3, acc.w);
  }
}

template <int OUT, bool VS, int BN>
static void launch_reduce_tiles(const float* ws, int splits, void* C, int64_t ldc, int M, int N, const SplitTiles& g,
                                hipStream_t s) {
  const int64_t blocks = (int64_t)g.tiles_m * g.tiles_n * (g.bm * BN / 1024);
  hipLaunchKernelGGL((splitk_reduce_tiles_kernel<OUT, VS, BN>), dim3((unsigned)blocks), dim3(256), 0, s, ws, splits, C,
                     ldc, M, N, g.bm, g.tiles_m);
}

template <int OUT, bool VS>
static bool try_reduce_tiles(const float* ws, int splits, void* C, int64_t ldc, int M, int N, const SplitTiles& g,
                             hipStream_t s) {
  if (!g.hw_order || (int64_t)g.tiles_m * g.tiles_n % 8 != 0 || N % 4 != 0 || g.bn < 64 || g.bm % (1024 / g.bn) != 0)
    return false;
  switch (g.bn) {
    case 64: launch_reduce_tiles<OUT, VS, 64>(ws, splits, C, ldc, M, N, g, s); return true;
    case 128: launch_reduce_tiles<OUT, VS, 128>(ws, splits, C, ldc, M, N, g, s); return true;
    case 256: launch_reduce_tiles<OUT, VS, 256>(ws, splits, C, ldc, M, N, g, s); return true;
    default: return false;
  }
}

template <int OUT>
static void launch_reduce(const float* ws, int splits, void* C, int64_t ldc, int M, int N, const SplitTiles& g,
                          hipStream_t s) {
  const bool v4 = N % 4 == 0;
  const int64_t groups = (int64_t)M * N / (v4 ? 4 : 1);
  int64_t blocks = (groups + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  const int64_t ob = OUT == OUT_F32 ? 4 : 2;
  const bool vs = v4 && ldc % 4 == 0 && (uintptr_t)C % (uintptr_t)(4 * ob) == 0;
  if (vs ? try_reduce_tiles<OUT, true>(ws, splits, C, ldc, M, N, g, s)
         : try_reduce_tiles<OUT, false>(ws, splits, C, ldc, M, N, g, s))
    return;
  if (vs)
    hipLaunchKernelGGL((splitk_reduce_kernel<OUT, 4, true>), dim3((unsigned)blocks), dim3(256), 0, s, ws, splits, C, ldc,
                       M, N);
  else if (v4)
    hipLaunchKernelGGL((splitk_reduce_kernel<OUT, 4, false>), dim3((unsigned)blocks), dim3(256), 0, s, ws, splits, C,
                       ldc, M, N);
  else
    hipLaunchKernelGGL((splitk_reduce_kernel<OUT, 1, false>), dim3((unsigned)blocks), dim3(256), 0, s, ws, splits, C,
                       ldc, M, N);
}

hipError_t launch_splitk_reduce(const float* ws, int splits, void* C, int64_t ldc, int M, int N, int out,
                                const SplitTiles& g, hipStream_t s) {
  if (out == OUT_F32)
    launch_reduce<OUT_F32>(ws, splits, C, ldc, M, N, g, s);
  else if (out == OUT_BF16)
    launch_reduce<OUT_BF16>(ws, splits, C, ldc, M, N, g, s);
  else
    launch_reduce<OUT_F16>(ws, splits, C, ldc, M, N, g, s);
  return hipGetLastError();
}

const MacroShape kMacroShapes[kNumMacroShapes] = {
    {256, 256, 64, Cfg256x256w8::kThreads, Cfg256x256w8::kLds, Cfg256x256w8::NS},
    {256, 128, 64, Cfg256x128::kThreads, Cfg256x128::kLds, Cfg256x128::NS},
    {128, 128, 64, Cfg128x128::kThreads, Cfg128x128::kLds, Cfg128x128::NS},
    {64, 64, 64, Cfg64x64::kThreads, Cfg64x64::kLds, Cfg64x64::NS},
    {128, 128, 64, Cfg128x128s4::kThreads, Cfg128x128s4::kLds, Cfg128x128s4::NS},
    {64, 64, 64, Cfg64x64s4::kThreads, Cfg64x64s4::kLds, Cfg64x64s4::NS},
    {256, 256, 64, Cfg256x256w8a::kThreads, Cfg256x256w8a::kLds, Cfg256x256w8a::NS},
};

// The launchers live in macro_tile_inst_*.hip.
#define TG_EXTERN(TA, TB, I, CFG)                                                                          \
  extern template hipError_t launch_dtype<CFG, TA, TB>(const MacroArgs&, int, int, bool, hipStream_t, int64_t, \
                                                       int);
#define TG_EXTERN_NN(I, CFG) TG_EXTERN(false, false, I, CFG)
#define TG_EXTERN_NT(I, CFG) TG_EXTERN(false, true, I, CFG)
#define TG_EXTERN_TN(I, CFG) TG_EXTERN(true, false, I, CFG)
#define TG_EXTERN_TT(I, CFG) TG_EXTERN(true, true, I, CFG)
TG_MACRO_CONFIGS(TG_EXTERN_NN)
TG_MACRO_CONFIGS(TG_EXTERN_NT)
TG_MACRO_CONFIGS(TG_EXTERN_TN)
TG_MACRO_CONFIGS(TG_EXTERN_TT)

template <bool TA, bool TB>
static hipError_t launch_layout(int shape, const MacroArgs& a, int in, int out, bool vec, hipStream_t s, int64_t grid,
                                int splits) {
#define TG_CASE(I, CFG) \
  case I: return launch_dtype<CFG, TA, TB>(a, in, out, vec, s, grid, splits);
  switch (shape) {
    TG_MACRO_CONFIGS(TG_CASE)
    default: return hipErrorInvalidValue;
  }
#undef TG_CASE
}

hipError_t launch_macro(int shape, const MacroArgs& a, int in, int out, bool vec, hipStream_t s, int64_t grid,
                        int splits, bool ta, bool tb) {
  if (!ta && !tb) return launch_layout<false, false>(shape, a, in, out, vec, s, grid, splits);
  if (!ta && tb) return launch_layout<false, true>(shape, a, in, out, vec, s, grid, splits);
  if (ta && !tb) return launch_layout<true, false>(shape, a, in, out, vec, s, grid, splits);
  return launch_layout<true, true>(shape, a, in, out, vec, s, grid, splits);
}

}  // namespace tg
