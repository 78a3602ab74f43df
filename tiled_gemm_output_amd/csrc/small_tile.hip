// small_tile.hip -- one wave per 16 x 16 C tile, K-step 32: exactly one
// v_mfma_f32_16x16x32_{f16,bf16} per step. This is the tile of the traffic
// example in "Reading a matrix multiply through its tiles" (section "Count the
// repeated reads": M = N = K = 128 with 16 x 16 x 32 tiles), so the bytes this
// kernel requests are exactly the pages' no-reuse count: every step loads the
// 16 x 32 A tile (1 KiB) and the 32 x 16 B tile (1 KiB) once, and the C tile is
// stored once.
//
// The step structure is the macro-tile kernel's, scaled down: two LDS stages, a
// direct global->LDS load of each 1 KiB tile (one 16-byte buffer load per lane) or
// an element-wise guarded load when 16-byte loads are not possible, and fragment
// reads with ds_read_b128 (K-contiguous operands) or two ds_read_b64_tr_b16
// (M/N-contiguous operands: B as given, A supplied transposed).
#include "device_common.h"
#include "launch.h"

namespace tg {

// One 1 KiB operand K-tile: 16 positions along M (A) or N (B) by 32 along K.
// KMAJ (stored K-contiguous: A as given, B transposed): 16 LDS rows of 32 values
// (64 bytes), lane l moves row l/4, chunk l%4, and a fragment is one ds_read_b128.
// Otherwise (M/N-contiguous: B as given, A transposed): 32 rows of 16 values
// (32 bytes), lane l moves row l/2, chunk l%2, and a fragment is two
// ds_read_b64_tr_b16. Either way lane l ends up with position l%16 and reduction
// indices 8*(l/16) .. +7, the operand layout of v_mfma_f32_16x16x32.
template <bool KMAJ>
struct SmallOpnd {
  static constexpr int kRow = KMAJ ? 64 : 32;
  static constexpr int kChunks = kRow / 16;
  __device__ static __forceinline__ int row(int l) { return l / kChunks; }
  __device__ static __forceinline__ int chunk(int l) { return l % kChunks; }
  __device__ static __forceinline__ uint32_t frag(int l) {
    if constexpr (KMAJ) {
      return (uint32_t)((l & 15) * 64 + (l >> 4) * 16);
    } else {
      const int g = l >> 4, jj = l & 15;
      return (uint32_t)((8 * g + (jj >> 2)) * 32 + 4 * (jj & 3) * 2);
    }
  }
  __device__ static __forceinline__ i32x4 read(TG_LDS char* base, uint32_t off) {
    if constexpr (KMAJ) {
      return *(TG_LDS i32x4*)(base + off);
    } else {
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TG_LDS s16x4*)(base + off));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TG_LDS s16x4*)(base + off + 4 * 32));
      const int2 l2 = __builtin_bit_cast(int2, lo), h2 = __builtin_bit_cast(int2, hi);
      return i32x4{l2.x, l2.y, h2.x, h2.y};
    }
  }
};

// TA: A is supplied transposed (K x M); TB: B is supplied transposed (N x K).
template <int IN, int OUT, bool VEC, bool TA, bool TB>
__global__ __launch_bounds__(64) void small_tile_kernel(MacroArgs p) {
  using OA = SmallOpnd<!TA>;
  using OB = SmallOpnd<TB>;
  __shared__ __attribute__((aligned(1024))) char sA0[1024];
  __shared__ __attribute__((aligned(1024))) char sA1[1024];
  __shared__ __attribute__((aligned(1024))) char sB0[1024];
  __shared__ __attribute__((aligned(1024))) char sB1[1024];
  const int lane = threadIdx.x;
  const int tile_m = blockIdx.x / p.tiles_n, tile_n = blockIdx.x % p.tiles_n;
  const int row0 = tile_m * 16, col0 = tile_n * 16;
  const int M = p.M, N = p.N, K = p.K;
  const int64_t lda = p.lda, ldb = p.ldb;
  const int nk = (K + 31) / 32;

  // Lane l moves 8 consecutive elements of one stored row of each operand: tile
  // row r, chunk c. Stored (row, column) of the K-tile's origin and the stored
  // matrix's extents: A is (m, k) as given, (k, m) transposed; B is (k, n) as
  // given, (n, k) transposed.
  const int ar = OA::row(lane), ac = OA::chunk(lane);
  const int br = OB::row(lane), bc = OB::chunk(lane);
  const int a_rows = TA ? K : M, a_cols = TA ? M : K;
  const int b_rows = TB ? N : K, b_cols = TB ? K : N;
  i32x4 a_reg, b_reg;

  // 16 bytes of a stored row into one lane: direct to LDS (vector path; zeros
  // outside the matrix via an out-of-range offset) or guarded element loads.
  auto load8 = [&](const uint16_t* base, int64_t ld, int r0, int c0, int rows, int cols, int r, int c,
                   TG_LDS char* dst, i32x4& reg) {
    const int sr = r0 + r, sc = c0 + 8 * c;
    if constexpr (VEC) {
      const __amdgpu_buffer_rsrc_t rs =
          make_rsrc(base + (int64_t)r0 * ld + c0, ((int64_t)(rows - 1 - r0) * ld + (cols - c0)) * 2);
      const uint32_t off = (sr < rows && sc < cols) ? (uint32_t)(((int64_t)r * ld + 8 * c) * 2) : kOutOfRange;
      load_lds_x4(rs, dst, off);
    } else {
      const uint16_t* src = base + (int64_t)sr * ld + sc;
      if (sr < rows && sc + 7 < cols) {  // whole chunk: one 16-byte load at 2-byte alignment
        __builtin_memcpy(&reg, src, 16);
      } else {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = (sr < rows && sc + 2 * e < cols) ? src[2 * e] : 0u;
          const uint32_t hi = (sr < rows && sc + 2 * e + 1 < cols) ? src[2 * e + 1] : 0u;
          w[e] = lo | (hi << 16);
        }
        reg = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
      }
    }
  };
  auto load_tile = [&](TG_LDS char* sa, TG_LDS char* sb, int kt) {
    const int k0 = kt * 32;
    load8(p.A, lda, TA ? k0 : row0, TA ? row0 : k0, a_rows, a_cols, ar, ac, sa, a_reg);
    load8(p.B, ldb, TB ? col0 : k0, TB ? k0 : col0, b_rows, b_cols, br, bc, sb, b_reg);
  };
  auto commit_tile = [&](TG_LDS char* sa, TG_LDS char* sb) {
    if constexpr (VEC) {
      __builtin_amdgcn_s_waitcnt(0x0F70);
    } else {
      *(TG_LDS i32x4*)(sa + lane * 16) = a_reg;
      *(TG_LDS i32x4*)(sb + lane * 16) = b_reg;
    }
  };

  const uint32_t a_frag = OA::frag(lane), b_frag = OB::frag(lane);
  f32x4 acc = f32x4{};
  auto compute_tile = [&](TG_LDS char* sa, TG_LDS char* sb) {
    acc = mfma16<IN>(OA::read(sa, a_frag), OB::read(sb, b_frag), acc);
  };

  TG_LDS char* pA0 = (TG_LDS char*)sA0;
  TG_LDS char* pA1 = (TG_LDS char*)sA1;
  TG_LDS char* pB0 = (TG_LDS char*)sB0;
  TG_LDS char* pB1 = (TG_LDS char*)sB1;
  if (nk > 0) {
    load_tile(pA0, pB0, 0);
    commit_tile(pA0, pB0);
    __syncthreads();
  }
  for (int kt = 0; kt < nk; kt += 2) {
    if (kt + 1 < nk) load_tile(pA1, pB1, kt + 1);
    compute_tile(pA0, pB0);
    if (kt + 1 < nk) commit_tile(pA1, pB1);
    __syncthreads();
    if (kt + 1 >= nk) break;
    if (kt + 2 < nk) load_tile(pA0, pB0, kt + 2);
    compute_tile(pA1, pB1);
    if (kt + 2 < nk) commit_tile(pA0, pB0);
    __syncthreads();
  }

  // acc[i]: row 4*(lane/16) + i, column lane%16
  const int col = col0 + (lane & 15);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = row0 + 4 * (lane >> 4) + i;
    if (row < M && col < N) {
      if constexpr (OUT == OUT_F32)
        ((float*)p.C)[(int64_t)row * p.ldc + col] = acc[i];
      else if constexpr (OUT == OUT_BF16)
        ((uint16_t*)p.C)[(int64_t)row * p.ldc + col] = f32_to_bf16_rne(acc[i]);
      else
        ((uint16_t*)p.C)[(int64_t)row * p.ldc + col] = f32_to_f16_rne(acc[i]);
    }
  }
}

template <int IN, int OUT, bool TA, bool TB>
static hipError_t launch_small_t(const MacroArgs& a, bool vec, hipStream_t s, int64_t grid) {
  if (vec)
    hipLaunchKernelGGL((small_tile_kernel<IN, OUT, true, TA, TB>), dim3((unsigned)grid), dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((small_tile_kernel<IN, OUT, false, TA, TB>), dim3((unsigned)grid), dim3(64), 0, s, a);
  return hipGetLastError();
}

template <bool TA, bool TB>
static hipError_t launch_small_layout(const MacroArgs& a, int in, int out, bool vec, hipStream_t s, int64_t grid) {
  if (in == IN_BF16 && out == OUT_F32) return launch_small_t<IN_BF16, OUT_F32, TA, TB>(a, vec, s, grid);
  if (in == IN_BF16 && out == OUT_BF16) return launch_small_t<IN_BF16, OUT_BF16, TA, TB>(a, vec, s, grid);
  if (in == IN_F16 && out == OUT_F32) return launch_small_t<IN_F16, OUT_F32, TA, TB>(a, vec, s, grid);
  if (in == IN_F16 && out == OUT_F16) return launch_small_t<IN_F16, OUT_F16, TA, TB>(a, vec, s, grid);
  return hipErrorInvalidValue;
}

hipError_t launch_small(const MacroArgs& a, int in, int out, bool vec, hipStream_t s, int64_t grid, bool ta, bool tb) {
  if (!ta && !tb) return launch_small_layout<false, false>(a, in, out, vec, s, grid);
  if (!ta && tb) return launch_small_layout<false, true>(a, in, out, vec, s, grid);
  if (ta && !tb) return launch_small_layout<true, false>(a, in, out, vec, s, grid);
  return launch_small_layout<true, true>(a, in, out, vec, s, grid);
}

}  // namespace tg
