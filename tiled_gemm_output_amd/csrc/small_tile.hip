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
// an element-wise guarded load when 16-byte loads are not possible, an A fragment
// read with ds_read_b128 and a B fragment read with two ds_read_b64_tr_b16.
#include "device_common.h"
#include "launch.h"

namespace tg {

template <int IN, int OUT, bool VEC>
__global__ __launch_bounds__(64) void small_tile_kernel(MacroArgs p) {
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

  // loader: lane l moves A row l/4, chunk l%4 (64-byte rows) and B row l/2, chunk l%2 (32-byte rows)
  const int ar = lane >> 2, ac = lane & 3;
  const int bk = lane >> 1, bc = lane & 1;
  const uint32_t a_off = (row0 + ar < M) ? (uint32_t)(((int64_t)ar * lda + 8 * ac) * 2) : kOutOfRange;
  const uint32_t b_off = (col0 + 8 * bc < N) ? (uint32_t)(((int64_t)bk * ldb + 8 * bc) * 2) : kOutOfRange;
  i32x4 a_reg, b_reg;

  auto load_tile = [&](TG_LDS char* sa, TG_LDS char* sb, int kt) {
    const int k0 = kt * 32;
    if constexpr (VEC) {
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A + (int64_t)row0 * lda + k0, ((int64_t)(M - 1 - row0) * lda + (K - k0)) * 2);
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B + (int64_t)k0 * ldb + col0, ((int64_t)(K - 1 - k0) * ldb + (N - col0)) * 2);
      load_lds_x4(ra, sa, (k0 + 8 * ac < K) ? a_off : kOutOfRange);
      load_lds_x4(rb, sb, (k0 + bk < K) ? b_off : kOutOfRange);
    } else {
      uint32_t w[4];
      const int gr = row0 + ar, gk = k0 + 8 * ac;
      const uint16_t* sa_src = p.A + (int64_t)gr * lda + gk;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = (gr < M && gk + 2 * e < K) ? sa_src[2 * e] : 0u;
        const uint32_t hi = (gr < M && gk + 2 * e + 1 < K) ? sa_src[2 * e + 1] : 0u;
        w[e] = lo | (hi << 16);
      }
      a_reg = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
      const int gkb = k0 + bk, gc = col0 + 8 * bc;
      const uint16_t* sb_src = p.B + (int64_t)gkb * ldb + gc;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = (gkb < K && gc + 2 * e < N) ? sb_src[2 * e] : 0u;
        const uint32_t hi = (gkb < K && gc + 2 * e + 1 < N) ? sb_src[2 * e + 1] : 0u;
        w[e] = lo | (hi << 16);
      }
      b_reg = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    }
  };
  auto commit_tile = [&](TG_LDS char* sa, TG_LDS char* sb) {
    if constexpr (VEC) {
      __builtin_amdgcn_s_waitcnt(0x0F70);
    } else {
      *(TG_LDS i32x4*)(sa + lane * 16) = a_reg;
      *(TG_LDS i32x4*)(sb + lane * 16) = b_reg;
    }
  };

  // fragments: A row lane%16, chunk lane/16; B transpose read of rows 8g + jj/4 (+4), column 4*(jj%4)
  const uint32_t a_frag = (uint32_t)((lane & 15) * 64 + (lane >> 4) * 16);
  const int g = lane >> 4, jj = lane & 15;
  const uint32_t b_frag = (uint32_t)((8 * g + (jj >> 2)) * 32 + 4 * (jj & 3) * 2);
  f32x4 acc = f32x4{};
  auto compute_tile = [&](TG_LDS char* sa, TG_LDS char* sb) {
    const i32x4 a = *(TG_LDS i32x4*)(sa + a_frag);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TG_LDS s16x4*)(sb + b_frag));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TG_LDS s16x4*)(sb + b_frag + 4 * 32));
    const int2 l2 = __builtin_bit_cast(int2, lo), h2 = __builtin_bit_cast(int2, hi);
    acc = mfma16<IN>(a, i32x4{l2.x, l2.y, h2.x, h2.y}, acc);
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

template <int IN, int OUT>
static hipError_t launch_small_t(const MacroArgs& a, bool vec, hipStream_t s, int64_t grid) {
  if (vec)
    hipLaunchKernelGGL((small_tile_kernel<IN, OUT, true>), dim3((unsigned)grid), dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((small_tile_kernel<IN, OUT, false>), dim3((unsigned)grid), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_small(const MacroArgs& a, int in, int out, bool vec, hipStream_t s, int64_t grid) {
  if (in == IN_BF16 && out == OUT_F32) return launch_small_t<IN_BF16, OUT_F32>(a, vec, s, grid);
  if (in == IN_BF16 && out == OUT_BF16) return launch_small_t<IN_BF16, OUT_BF16>(a, vec, s, grid);
  if (in == IN_F16 && out == OUT_F32) return launch_small_t<IN_F16, OUT_F32>(a, vec, s, grid);
  if (in == IN_F16 && out == OUT_F16) return launch_small_t<IN_F16, OUT_F16>(a, vec, s, grid);
  return hipErrorInvalidValue;
}

}  // namespace tg
