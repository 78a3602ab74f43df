// macro_tile.hip -- the output-stationary macro-tile GEMM on gfx950 MFMA.
//
// One workgroup owns one BM x BN tile of C ("Reading a matrix multiply through its
// tiles", section "Keep one output tile resident"): its fp32 accumulator lives in
// the waves' registers for the whole reduction, the A (BM x BK) and B (BK x BN)
// K-tiles of each step are staged through LDS, and the tile is written to C once.
// Partial edge tiles use their actual ranges ("Edge tiles still matter"): loads
// outside A or B read zeros, stores outside C are dropped, and every thread reaches
// every barrier (the Mojo puzzle's manual kernel, sections 3-6, guards loads,
// compute and store but never the barriers).
//
// gfx950 design (differs from the pages' one-thread-per-element kernels):
//  * waves of 64 lanes, each owning a (BM/WM) x (BN/WN) sub-tile computed with
//    v_mfma_f32_32x32x16_{bf16,f16};
//  * two LDS stages (double buffering: the loads of step k+1 are in flight while
//    step k is multiplied), one barrier per step;
//  * vector path: 16-byte buffer loads straight from global memory into LDS
//    (buffer_load_dwordx4 ... lds), no register staging; out-of-range lanes use an
//    offset beyond the buffer and receive zeros;
//  * element path (unaligned pointers/leading dimensions, K or N not a multiple of
//    8): guarded 16-bit loads into registers, then 16-byte LDS writes;
//  * LDS layouts XOR-swizzled per 16-byte chunk so that A fragment reads
//    (ds_read_b128) and B fragment reads (ds_read_b64_tr_b16, which also performs
//    the k-major -> n-major transpose MFMA needs for row-major B) hit distinct banks;
//  * XCD-aware, grouped workgroup -> tile order (schedule_tile).
#include "device_common.h"
#include "launch.h"

namespace tg {

template <int BM_, int BN_, int BK_, int WM_, int WN_>
struct MacroCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kWTM = BM / WM, kWTN = BN / WN;  // wave sub-tile
  static constexpr int kFM = kWTM / 32, kFN = kWTN / 32;  // 32x32 MFMA blocks per wave
  static constexpr int kABytes = BM * BK * 2, kBBytes = BK * BN * 2;
  static constexpr int kARow = BK * 2, kBRow = BN * 2;    // LDS row pitch in bytes
  static constexpr int kAChunks = BK / 8, kBChunks = BN / 8;  // 16-byte chunks per row
  static constexpr int kABlocks = kABytes / 1024, kBBlocks = kBBytes / 1024;  // 1 KiB DMA blocks
  static constexpr int kBRowsPerBlock = 1024 / kBRow;
  static constexpr int kSubsteps = BK / 16;
  static constexpr int kLds = 2 * (kABytes + kBBytes);
  static_assert(BK == 64, "A swizzle assumes 8 chunks per A row");
  static_assert(kFM >= 1 && kFN >= 1 && kWTM % 32 == 0 && kWTN % 32 == 0, "wave tile must be a multiple of 32x32");
  static_assert(kABlocks % kWaves == 0 && kBBlocks % kWaves == 0, "DMA blocks must divide among waves");
  static_assert(kBRow <= 1024 && 1024 % kBRow == 0, "B rows must tile a 1 KiB block");
  static_assert(kBChunks >= 8, "B swizzle needs at least 8 chunks per row");
  static_assert(kLds <= 160 * 1024, "LDS budget");
};

// Physical 16-byte chunk of logical chunk c in A row r (8 chunks per row). For
// any 16 consecutive rows starting at a multiple of 16 and a fixed c, the 8-row
// halves see 8 distinct chunks, and rows of equal parity see 8 distinct chunks.
__device__ __forceinline__ int swz_a(int r) { return (r ^ (r >> 3)) & 7; }

// Physical chunk XOR for B row k (k-major rows of BN values). A transpose read
// touches 4 consecutive rows x 2 (or 4) consecutive chunks; these masks keep them
// on distinct banks.
template <int CH>
__device__ __forceinline__ int swz_b(int k) {
  const int m = k & 3;
  const int h = m == 0 ? 0 : (m == 1 ? 6 : (m == 2 ? 10 : 12));
  return h & (CH - 1);
}

// Direct-load geometry: DMA block t of a wave writes 1 KiB of LDS. For A (8 rows
// of 128 bytes per block) lane l fills row blk*8 + l/8, physical chunk l%8, i.e.
// logical chunk (l%8) ^ swz_a(row); for B (1024 / (2*BN) rows per block) lane l
// fills row blk*rows + l / chunks, physical chunk l % chunks.
#define A_DMA_HELPERS(Cfg)                                                                     \
  auto a_dma_row = [&](int w, int t, int l) { return (w * kAPer + t) * 8 + (l >> 3); };       \
  auto a_dma_chunk = [&](int r, int l) { return (l & 7) ^ swz_a(r); };                        \
  auto b_dma_row = [&](int w, int t, int l) {                                                  \
    return (w * kBPer + t) * Cfg::kBRowsPerBlock + l / Cfg::kBChunks;                          \
  };                                                                                           \
  auto b_dma_chunk = [&](int k, int l) { return (l % Cfg::kBChunks) ^ swz_b<Cfg::kBChunks>(k); };

// LOAD: kLoadElem = guarded element loads; kLoadVec = 16-byte direct loads, the last
// K-tile may be partial; kLoadVecFull = 16-byte direct loads, K is a multiple of BK.
enum { kLoadElem = 0, kLoadVec = 1, kLoadVecFull = 2 };

template <class Cfg, int IN, int OUT, int LOAD>
__global__ __launch_bounds__(Cfg::kThreads, 1) void macro_tile_kernel(MacroArgs p) {
  constexpr bool VEC = LOAD != kLoadElem;
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
  constexpr int FM = Cfg::kFM, FN = Cfg::kFN;
  __shared__ __attribute__((aligned(1024))) char sA0[Cfg::kABytes];
  __shared__ __attribute__((aligned(1024))) char sA1[Cfg::kABytes];
  __shared__ __attribute__((aligned(1024))) char sB0[Cfg::kBBytes];
  __shared__ __attribute__((aligned(1024))) char sB1[Cfg::kBBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;

  int tile_m, tile_n;
  schedule_tile(blockIdx.x, gridDim.x, p.tiles_m, p.group_m, tile_m, tile_n);
  const int row0 = tile_m * BM, col0 = tile_n * BN;
  const int M = p.M, N = p.N, K = p.K;
  const int64_t lda = p.lda, ldb = p.ldb;
  const int nk = (K + BK - 1) / BK;

  // ---------------- loader state ----------------
  constexpr int kAPer = Cfg::kABlocks / Cfg::kWaves;  // DMA blocks (or register chunks) per wave / thread
  constexpr int kBPer = Cfg::kBBlocks / Cfg::kWaves;
  A_DMA_HELPERS(Cfg)
  // vector path: per-lane byte offsets relative to the step's base
  uint32_t a_off[kAPer];
  uint32_t b_off[kBPer];
  // element path: each thread stages kAPer + kBPer chunks of 8 values in registers
  i32x4 a_reg[kAPer], b_reg[kBPer];
  uint32_t a_lds[kAPer], b_lds[kBPer];
  int a_r[kAPer], a_c[kAPer], b_k[kBPer], b_c[kBPer];

  if constexpr (VEC) {
#pragma unroll
    for (int t = 0; t < kAPer; ++t) {
      const int r = a_dma_row(wave, t, lane);
      const int c = a_dma_chunk(r, lane);
      a_off[t] = (row0 + r < M) ? (uint32_t)(((int64_t)r * lda + 8 * c) * 2) : kOutOfRange;
    }
#pragma unroll
    for (int t = 0; t < kBPer; ++t) {
      const int k = b_dma_row(wave, t, lane);
      const int c = b_dma_chunk(k, lane);
      b_off[t] = (col0 + 8 * c < N) ? (uint32_t)(((int64_t)k * ldb + 8 * c) * 2) : kOutOfRange;
    }
  } else {
#pragma unroll
    for (int t = 0; t < kAPer; ++t) {
      const int q = t * Cfg::kThreads + tid;  // chunk id within the A tile
      const int r = q / Cfg::kAChunks, c = q % Cfg::kAChunks;
      a_r[t] = r;
      a_c[t] = c;
      a_lds[t] = (uint32_t)(r * Cfg::kARow + ((c ^ swz_a(r)) << 4));
    }
#pragma unroll
    for (int t = 0; t < kBPer; ++t) {
      const int q = t * Cfg::kThreads + tid;
      const int k = q / Cfg::kBChunks, c = q % Cfg::kBChunks;
      b_k[t] = k;
      b_c[t] = c;
      b_lds[t] = (uint32_t)(k * Cfg::kBRow + ((c ^ swz_b<Cfg::kBChunks>(k)) << 4));
    }
  }

  const uint16_t* gA = p.A + (int64_t)row0 * lda;
  const uint16_t* gB = p.B + col0;

  // Issue the loads of K-tile kt into stage (sa, sb).
  auto load_tile = [&](TG_LDS char* sa, TG_LDS char* sb, int kt) {
    const int k0 = kt * BK;
    if (kt < 0) {  // the prepended zero tile
      if constexpr (VEC) {
        const __amdgpu_buffer_rsrc_t rz = make_rsrc(p.A, 0);
#pragma unroll
        for (int t = 0; t < kAPer; ++t) load_lds_x4(rz, sa + (wave * kAPer + t) * 1024, kOutOfRange);
#pragma unroll
        for (int t = 0; t < kBPer; ++t) load_lds_x4(rz, sb + (wave * kBPer + t) * 1024, kOutOfRange);
      } else {
#pragma unroll
        for (int t = 0; t < kAPer; ++t) a_reg[t] = i32x4{0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < kBPer; ++t) b_reg[t] = i32x4{0, 0, 0, 0};
      }
      return;
    }
    if constexpr (VEC) {
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(gA + k0, ((int64_t)(M - 1 - row0) * lda + (K - k0)) * 2);
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(gB + (int64_t)k0 * ldb, ((int64_t)(K - 1 - k0) * ldb + (N - col0)) * 2);
      if (LOAD == kLoadVecFull || k0 + BK <= K) {
#pragma unroll
        for (int t = 0; t < kAPer; ++t) load_lds_x4(ra, sa + (wave * kAPer + t) * 1024, a_off[t]);
#pragma unroll
        for (int t = 0; t < kBPer; ++t) load_lds_x4(rb, sb + (wave * kBPer + t) * 1024, b_off[t]);
      } else {
        // partial last K-tile: chunks at or beyond K read zeros
        int ln = lane;
        asm volatile("" : "+v"(ln));  // keep this tail-only arithmetic out of the main loop
#pragma unroll
        for (int t = 0; t < kAPer; ++t) {
          const int kc = 8 * a_dma_chunk(a_dma_row(wave, t, ln), ln);
          load_lds_x4(ra, sa + (wave * kAPer + t) * 1024, (k0 + kc < K) ? a_off[t] : kOutOfRange);
        }
#pragma unroll
        for (int t = 0; t < kBPer; ++t) {
          const int kr = b_dma_row(wave, t, ln);
          load_lds_x4(rb, sb + (wave * kBPer + t) * 1024, (k0 + kr < K) ? b_off[t] : kOutOfRange);
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < kAPer; ++t) {
        const int gr = row0 + a_r[t];
        const int gk = k0 + 8 * a_c[t];
        const uint16_t* src = p.A + (int64_t)gr * lda + gk;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = (gr < M && gk + 2 * e < K) ? src[2 * e] : 0u;
          const uint32_t hi = (gr < M && gk + 2 * e + 1 < K) ? src[2 * e + 1] : 0u;
          w[e] = lo | (hi << 16);
        }
        a_reg[t] = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
      }
#pragma unroll
      for (int t = 0; t < kBPer; ++t) {
        const int gk = k0 + b_k[t];
        const int gc = col0 + 8 * b_c[t];
        const uint16_t* src = p.B + (int64_t)gk * ldb + gc;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = (gk < K && gc + 2 * e < N) ? src[2 * e] : 0u;
          const uint32_t hi = (gk < K && gc + 2 * e + 1 < N) ? src[2 * e + 1] : 0u;
          w[e] = lo | (hi << 16);
        }
        b_reg[t] = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
      }
    }
  };

  // Make the stage's data visible: wait for the direct loads, or write the staged registers.
  auto commit_tile = [&](TG_LDS char* sa, TG_LDS char* sb) {
    if constexpr (VEC) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's LDS-DMA writes have landed
    } else {
#pragma unroll
      for (int t = 0; t < kAPer; ++t) *(TG_LDS i32x4*)(sa + a_lds[t]) = a_reg[t];
#pragma unroll
      for (int t = 0; t < kBPer; ++t) *(TG_LDS i32x4*)(sb + b_lds[t]) = b_reg[t];
    }
  };

  // ---------------- fragment addressing ----------------
  // A fragment of block i, substep s: row wm*WTM + 32i + lane%32, chunk 2s + lane/32.
  uint32_t a_frag[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int r = wm * Cfg::kWTM + 32 * i + (lane & 31);
    a_frag[i] = (uint32_t)(r * Cfg::kARow + (((lane >> 5) ^ swz_a(r)) << 4));
  }
  // B fragment of block j (lo half, substep 0): lane l in group g = l/16, jj = l%16
  // addresses row 8*(g/2) + jj/4, column wn*WTN + 32j + 16*(g%2) + 4*(jj%4).
  uint32_t b_frag[FN];
  {
    const int g = lane >> 4, jj = lane & 15;
    const int k = 8 * (g >> 1) + (jj >> 2);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = wn * Cfg::kWTN + 32 * j + 16 * (g & 1) + 4 * (jj & 3);
      b_frag[j] = (uint32_t)(k * Cfg::kBRow + (((n >> 3) ^ swz_b<Cfg::kBChunks>(k)) << 4) + (n & 7) * 2);
    }
  }

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

  // Fragments of substep s (16 reduction indices) of one stage.
  auto read_frags = [&](TG_LDS char* sa, TG_LDS char* sb, int s, i32x4(&a)[FM], i32x4(&b)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      // the substep selects chunk pair (2s, 2s+1); under the XOR swizzle that is an
      // XOR of the byte address with s << 5 (computed here, not hoisted out of the loop)
      uint32_t off = a_frag[i];
      asm volatile("" : "+v"(off));
      a[i] = *(TG_LDS i32x4*)(sa + (off ^ (uint32_t)(s << 5)));
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TG_LDS s16x4*)(sb + b_frag[j] + (16 * s) * Cfg::kBRow));
      const s16x4 hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((TG_LDS s16x4*)(sb + b_frag[j] + (16 * s + 4) * Cfg::kBRow));
      const int2 l2 = __builtin_bit_cast(int2, lo), h2 = __builtin_bit_cast(int2, hi);
      b[j] = i32x4{l2.x, l2.y, h2.x, h2.y};
    }
  };
  auto mfma_all = [&](const i32x4(&a)[FM], const i32x4(&b)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<IN>(a[i], b[j], acc[i][j]);
  };
  // Software pipeline over the substeps: the reads of substep s+1 are issued in the
  // same scheduling region as the MFMAs of substep s; sched_barrier keeps regions
  // apart so that at most two substeps' fragments are live.
  auto compute_tile = [&](TG_LDS char* sa, TG_LDS char* sb) {
    i32x4 a0[FM], b0[FN], a1[FM], b1[FN];
    read_frags(sa, sb, 0, a0, b0);
#pragma unroll
    for (int s = 0; s < Cfg::kSubsteps; s += 2) {
      read_frags(sa, sb, s + 1, a1, b1);
      mfma_all(a0, b0);
      __builtin_amdgcn_sched_barrier(0);
      if (s + 2 < Cfg::kSubsteps) read_frags(sa, sb, s + 2, a0, b0);
      mfma_all(a1, b1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  TG_LDS char* pA0 = (TG_LDS char*)sA0;
  TG_LDS char* pA1 = (TG_LDS char*)sA1;
  TG_LDS char* pB0 = (TG_LDS char*)sB0;
  TG_LDS char* pB1 = (TG_LDS char*)sB1;

  // ---------------- main loop: two stages, one barrier per K-step ----------------
  // K-tiles are processed in pairs (stage 0, stage 1) so that every compute call
  // is unconditional. When the number of K-tiles is odd, a zero tile (index -1,
  // every load out of range, so no memory is read) is prepended: it adds exact
  // zeros to the accumulator.
  const int kt0 = (nk & 1) ? -1 : 0;
  const int npairs = (nk - kt0) >> 1;
  load_tile(pA0, pB0, kt0);
  commit_tile(pA0, pB0);
  __syncthreads();
  for (int pr = 0, kt = kt0; pr < npairs; ++pr, kt += 2) {
    load_tile(pA1, pB1, kt + 1);
    compute_tile(pA0, pB0);
    commit_tile(pA1, pB1);
    __syncthreads();
    const bool more = pr + 1 < npairs;
    if (more) load_tile(pA0, pB0, kt + 2);
    compute_tile(pA1, pB1);
    if (more) commit_tile(pA0, pB0);
    __syncthreads();
  }

  // ---------------- epilogue: write the C tile once ----------------
  // acc[i][j][v] holds row 32i + 8*(v/4) + 4*(lane/32) + v%4, column 32j + lane%32
  // of the wave tile. Interior tiles store without bounds checks; edge tiles drop
  // the elements outside C.
  const int64_t ldc = p.ldc;
  const bool interior = row0 + BM <= M && col0 + BN <= N;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int rb = row0 + wm * Cfg::kWTM + 32 * i + 4 * (lane >> 5);
      const int col = col0 + wn * Cfg::kWTN + 32 * j + (lane & 31);
      const int64_t base = (int64_t)rb * ldc + col;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int dr = 8 * (v >> 2) + (v & 3);
        if (interior || (rb + dr < M && col < N)) {
          const int64_t off = base + (int64_t)dr * ldc;
          const float x = acc[i][j][v];
          if constexpr (OUT == OUT_F32)
            ((float*)p.C)[off] = x;
          else if constexpr (OUT == OUT_BF16)
            ((uint16_t*)p.C)[off] = f32_to_bf16_rne(x);
          else
            ((uint16_t*)p.C)[off] = f32_to_f16_rne(x);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host-side instantiation and launch

template <class Cfg, int IN, int OUT>
static hipError_t launch_cfg(const MacroArgs& a, bool vec, hipStream_t stream, int64_t grid) {
  const dim3 g((unsigned)grid), b(Cfg::kThreads);
  if (!vec)
    hipLaunchKernelGGL((macro_tile_kernel<Cfg, IN, OUT, kLoadElem>), g, b, 0, stream, a);
  else if (a.K % Cfg::BK == 0)
    hipLaunchKernelGGL((macro_tile_kernel<Cfg, IN, OUT, kLoadVecFull>), g, b, 0, stream, a);
  else
    hipLaunchKernelGGL((macro_tile_kernel<Cfg, IN, OUT, kLoadVec>), g, b, 0, stream, a);
  return hipGetLastError();
}

template <class Cfg>
static hipError_t launch_dtype(const MacroArgs& a, int in, int out, bool vec, hipStream_t s, int64_t grid) {
  if (in == IN_BF16 && out == OUT_F32) return launch_cfg<Cfg, IN_BF16, OUT_F32>(a, vec, s, grid);
  if (in == IN_BF16 && out == OUT_BF16) return launch_cfg<Cfg, IN_BF16, OUT_BF16>(a, vec, s, grid);
  if (in == IN_F16 && out == OUT_F32) return launch_cfg<Cfg, IN_F16, OUT_F32>(a, vec, s, grid);
  if (in == IN_F16 && out == OUT_F16) return launch_cfg<Cfg, IN_F16, OUT_F16>(a, vec, s, grid);
  return hipErrorInvalidValue;
}

using Cfg256x256w8 = MacroCfg<256, 256, 64, 2, 4>;  // 8 waves, 128 x 64 per wave
using Cfg256x256w4 = MacroCfg<256, 256, 64, 2, 2>;  // 4 waves, 128 x 128 per wave
using Cfg256x128 = MacroCfg<256, 128, 64, 4, 2>;
using Cfg128x128 = MacroCfg<128, 128, 64, 2, 2>;
using Cfg64x64 = MacroCfg<64, 64, 64, 2, 2>;

const MacroShape kMacroShapes[kNumMacroShapes] = {
    {256, 256, 64, Cfg256x256w8::kThreads, Cfg256x256w8::kLds},
    {256, 128, 64, Cfg256x128::kThreads, Cfg256x128::kLds},
    {128, 128, 64, Cfg128x128::kThreads, Cfg128x128::kLds},
    {64, 64, 64, Cfg64x64::kThreads, Cfg64x64::kLds},
    {256, 256, 64, Cfg256x256w4::kThreads, Cfg256x256w4::kLds},
};

hipError_t launch_macro(int shape, const MacroArgs& a, int in, int out, bool vec, hipStream_t s, int64_t grid) {
  switch (shape) {
    case 0: return launch_dtype<Cfg256x256w8>(a, in, out, vec, s, grid);
    case 1: return launch_dtype<Cfg256x128>(a, in, out, vec, s, grid);
    case 2: return launch_dtype<Cfg128x128>(a, in, out, vec, s, grid);
    case 3: return launch_dtype<Cfg64x64>(a, in, out, vec, s, grid);
    case 4: return launch_dtype<Cfg256x256w4>(a, in, out, vec, s, grid);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tg
