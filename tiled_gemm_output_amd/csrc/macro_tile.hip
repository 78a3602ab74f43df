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

// Loads: kLoadElem = guarded element loads staged in registers; kLoadVec = 16-byte
// direct loads, the last K-tile may be partial; kLoadVecFull = 16-byte direct loads,
// K is a multiple of BK.
enum { kLoadElem = 0, kLoadVec = 1, kLoadVecFull = 2 };

template <int N>
struct IC {
  static constexpr int value = N;
};
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(IC<I>{});
    static_for<I + 1, N>(f);
  }
}

// Workgroup barrier without a memory fence. The waits the pipeline needs are
// explicit s_waitcnt instructions placed before it (a fenced barrier would also
// wait for every load in flight); the empty asm statements keep the compiler from
// moving memory operations across it.
__device__ __forceinline__ void barrier_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Instruction order inside one scheduling region: each MFMA is followed by the
// next share of the region's LDS reads and global loads, so that reads for the
// next substep and refill loads are issued early and spread over the MFMAs.
template <int NM, int NR, int NV>
__device__ __forceinline__ void interleave() {
  constexpr int rper = NM > 0 ? (NR + NM - 1) / NM : 0;
  constexpr int vper = NM > 0 ? (NV + NM - 1) / NM : 0;
  static_for<0, NM>([&](auto q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    constexpr int r = NR - q.value * rper;
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r < rper ? r : rper, 0);  // DS read
    constexpr int v = NV - q.value * vper;
    if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x020, v < vper ? v : vper, 0);  // VMEM read
  });
}

template <class Cfg, int IN, int OUT, int LOAD>
__global__ __launch_bounds__(Cfg::kThreads, 1) void macro_tile_kernel(MacroArgs p) {
  constexpr bool VEC = LOAD != kLoadElem;
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
  constexpr int FM = Cfg::kFM, FN = Cfg::kFN;
  constexpr int kAPer = Cfg::kABlocks / Cfg::kWaves;  // 1 KiB blocks per wave and stage
  constexpr int kBPer = Cfg::kBBlocks / Cfg::kWaves;
  constexpr int NR = FM + 2 * FN;  // LDS reads per substep
  constexpr int NM = FM * FN;      // MFMAs per substep
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
  // K-tiles of this workgroup: [kt_base, kt_base + nk) (all of them without split-K)
  const int kt_base = blockIdx.y * p.kt_per_split;
  const int nk_all = (K + BK - 1) / BK;
  const int nk = (nk_all - kt_base) < p.kt_per_split ? (nk_all - kt_base) : p.kt_per_split;

  // ---------------- loader geometry ----------------
  // Block t of a wave fills 1 KiB of a stage. A: 8 rows of 128 bytes per block;
  // lane l fills row blk*8 + l/8 at physical chunk l%8, i.e. logical chunk
  // (l%8) ^ swz_a(row). B: 1024 / (2*BN) rows per block; lane l fills row
  // blk*rows + l/chunks at physical chunk l%chunks. The direct loads write lane
  // l's 16 bytes to block base + 16*l; the element path writes the same slot.
  auto a_row = [&](int t, int l) { return (wave * kAPer + t) * 8 + (l >> 3); };
  auto a_chunk = [&](int r, int l) { return (l & 7) ^ swz_a(r); };
  auto b_row = [&](int t, int l) { return (wave * kBPer + t) * Cfg::kBRowsPerBlock + l / Cfg::kBChunks; };
  auto b_chunk = [&](int k, int l) { return (l % Cfg::kBChunks) ^ swz_b<Cfg::kBChunks>(k); };

  uint32_t a_off[kAPer], b_off[kBPer];  // byte offsets from the K-tile's origin, vector path
  if constexpr (VEC) {
#pragma unroll
    for (int t = 0; t < kAPer; ++t) {
      const int r = a_row(t, lane);
      a_off[t] = (row0 + r < M) ? (uint32_t)(((int64_t)r * lda + 8 * a_chunk(r, lane)) * 2) : kOutOfRange;
    }
#pragma unroll
    for (int t = 0; t < kBPer; ++t) {
      const int k = b_row(t, lane);
      const int c = b_chunk(k, lane);
      b_off[t] = (col0 + 8 * c < N) ? (uint32_t)(((int64_t)k * ldb + 8 * c) * 2) : kOutOfRange;
    }
  }
  const uint16_t* gA = p.A + (int64_t)row0 * lda;
  const uint16_t* gB = p.B + col0;

  // Vector path: issue the direct loads of K-tile kt into a stage. Branch-free: a
  // K-tile outside [0, nk) gets a zero-length buffer, so every lane reads zeros and
  // no memory is touched (this keeps the compiler's tracking of which stage each
  // load writes exact, so it adds no waits before reads of the other stage).
  auto issue_loads = [&](TG_LDS char* sa, TG_LDS char* sb, int kt) {
    const bool ok = (unsigned)kt < (unsigned)nk;
    const int k0 = ok ? (kt_base + kt) * BK : 0;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(gA + k0, ok ? ((int64_t)(M - 1 - row0) * lda + (K - k0)) * 2 : 0);
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(gB + (int64_t)k0 * ldb, ok ? ((int64_t)(K - 1 - k0) * ldb + (N - col0)) * 2 : 0);
#pragma unroll
    for (int t = 0; t < kAPer; ++t) {
      uint32_t off = a_off[t];
      if constexpr (LOAD == kLoadVec) off = (k0 + 8 * a_chunk(a_row(t, lane), lane) < K) ? off : kOutOfRange;
      load_lds_x4(ra, sa + (wave * kAPer + t) * 1024, off);
    }
#pragma unroll
    for (int t = 0; t < kBPer; ++t) {
      uint32_t off = b_off[t];
      if constexpr (LOAD == kLoadVec) off = (k0 + b_row(t, lane) < K) ? off : kOutOfRange;
      load_lds_x4(rb, sb + (wave * kBPer + t) * 1024, off);
    }
  };

  // Element path: guarded 16-bit loads of K-tile kt into registers (zeros outside
  // the matrices and for kt outside [0, nk)), and their 16-byte LDS writes.
  i32x4 a_reg[kAPer], b_reg[kBPer];
  auto fetch_regs = [&](int kt) {
    const bool ok = (unsigned)kt < (unsigned)nk;
    const int k0 = (kt_base + kt) * BK;
#pragma unroll
    for (int t = 0; t < kAPer; ++t) {
      const int r = a_row(t, lane);
      const int gr = row0 + r, gk = k0 + 8 * a_chunk(r, lane);
      const bool rv = ok && gr < M;
      const uint16_t* src = p.A + (int64_t)gr * lda + gk;
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = (rv && gk + 2 * e < K) ? src[2 * e] : 0u;
        const uint32_t hi = (rv && gk + 2 * e + 1 < K) ? src[2 * e + 1] : 0u;
        w[e] = lo | (hi << 16);
      }
      a_reg[t] = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    }
#pragma unroll
    for (int t = 0; t < kBPer; ++t) {
      const int k = b_row(t, lane);
      const int gk = k0 + k, gc = col0 + 8 * b_chunk(k, lane);
      const bool kv = ok && gk < K;
      const uint16_t* src = p.B + (int64_t)gk * ldb + gc;
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = (kv && gc + 2 * e < N) ? src[2 * e] : 0u;
        const uint32_t hi = (kv && gc + 2 * e + 1 < N) ? src[2 * e + 1] : 0u;
        w[e] = lo | (hi << 16);
      }
      b_reg[t] = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    }
  };
  auto store_regs = [&](TG_LDS char* sa, TG_LDS char* sb) {
#pragma unroll
    for (int t = 0; t < kAPer; ++t) *(TG_LDS i32x4*)(sa + (wave * kAPer + t) * 1024 + lane * 16) = a_reg[t];
#pragma unroll
    for (int t = 0; t < kBPer; ++t) *(TG_LDS i32x4*)(sb + (wave * kBPer + t) * 1024 + lane * 16) = b_reg[t];
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

  // Fragments of substep s (16 reduction indices), read in the order the MFMAs
  // (row-major over the i x j blocks) consume them: a[0], every b[j], a[1..].
  auto read_a = [&](TG_LDS char* sa, int s, int i) {
    // the substep selects chunk pair (2s, 2s+1); under the XOR swizzle that is an
    // XOR of the byte address with s << 5 (kept in the loop, not hoisted)
    uint32_t off = a_frag[i];
    asm volatile("" : "+v"(off));
    return *(TG_LDS i32x4*)(sa + (off ^ (uint32_t)(s << 5)));
  };
  auto read_b = [&](TG_LDS char* sb, int s, int j) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TG_LDS s16x4*)(sb + b_frag[j] + (16 * s) * Cfg::kBRow));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TG_LDS s16x4*)(sb + b_frag[j] + (16 * s + 4) * Cfg::kBRow));
    const int2 l2 = __builtin_bit_cast(int2, lo), h2 = __builtin_bit_cast(int2, hi);
    return i32x4{l2.x, l2.y, h2.x, h2.y};
  };
  auto read_frags = [&](TG_LDS char* sa, TG_LDS char* sb, int s, i32x4(&a)[FM], i32x4(&b)[FN]) {
    a[0] = read_a(sa, s, 0);
#pragma unroll
    for (int j = 0; j < FN; ++j) b[j] = read_b(sb, s, j);
#pragma unroll
    for (int i = 1; i < FM; ++i) a[i] = read_a(sa, s, i);
  };
  // MFMAs of one substep; half 0 = block rows [0, FM/2), half 1 = the rest.
  auto mfma_rows = [&](const i32x4(&a)[FM], const i32x4(&b)[FN], int i0, int i1) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
      if (i >= i0 && i < i1)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<IN>(a[i], b[j], acc[i][j]);
  };

  TG_LDS char* pA0 = (TG_LDS char*)sA0;
  TG_LDS char* pA1 = (TG_LDS char*)sA1;
  TG_LDS char* pB0 = (TG_LDS char*)sB0;
  TG_LDS char* pB1 = (TG_LDS char*)sB1;

  // ---------------- main loop ----------------
  // Two stages; K-tile kt0 + st lives in stage st % 2. Each step multiplies its
  // stage in four substeps; the reads of substep s+1 are issued among the MFMAs
  // of substep s. The barrier that ends the step sits after the first half of the
  // last substep's MFMAs: once every wave is past it, the stage just consumed is
  // refilled with K-tile st + 2 and the next stage's first fragments are read,
  // both covered by the second half of those MFMAs. When the number of K-tiles is
  // odd, a zero K-tile (index -1) is prepended so that every step is unconditional.
  const int kt0 = (nk & 1) ? -1 : 0;
  const int nsteps = nk - kt0;  // even, >= 2
  i32x4 fa[FM], fb[FN], ga[FM], gb[FN];
  if constexpr (VEC) {
    issue_loads(pA0, pB0, kt0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  } else {
    fetch_regs(kt0);
    store_regs(pA0, pB0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  }
  barrier_nofence();
  if constexpr (VEC)
    issue_loads(pA1, pB1, kt0 + 1);
  else
    fetch_regs(kt0 + 1);
  read_frags(pA0, pB0, 0, fa, fb);

  auto step = [&](TG_LDS char* sa, TG_LDS char* sb, TG_LDS char* na, TG_LDS char* nb, int st) {
    read_frags(sa, sb, 1, ga, gb);
    mfma_rows(fa, fb, 0, FM);
    interleave<NM, NR, 0>();
    __builtin_amdgcn_sched_barrier(0);
    read_frags(sa, sb, 2, fa, fb);
    mfma_rows(ga, gb, 0, FM);
    interleave<NM, NR, 0>();
    __builtin_amdgcn_sched_barrier(0);
    read_frags(sa, sb, 3, ga, gb);
    mfma_rows(fa, fb, 0, FM);
    interleave<NM, NR, 0>();
    __builtin_amdgcn_sched_barrier(0);
    mfma_rows(ga, gb, 0, FM / 2);
    __builtin_amdgcn_sched_barrier(0);
    // the next stage must be complete in every wave before anyone reads it
    if constexpr (VEC) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of K-tile st + 1 landed
    } else {
      store_regs(na, nb);                  // K-tile st + 1, fetched one step ago
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    }
    barrier_nofence();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (VEC)
      issue_loads(sa, sb, kt0 + st + 2);  // out of range on the last two steps: zero-length, no traffic
    else
      fetch_regs(kt0 + st + 2);
    read_frags(na, nb, 0, fa, fb);
    mfma_rows(ga, gb, FM / 2, FM);
    interleave<(FM - FM / 2) * FN, NR, VEC ? kAPer + kBPer : 0>();
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int st = 0; st < nsteps; st += 2) {
    step(pA0, pB0, pA1, pB1, st);
    step(pA1, pB1, pA0, pB0, st + 1);
  }
  if constexpr (VEC) __builtin_amdgcn_s_waitcnt(0x0F70);  // trailing loads land before LDS is released

  // ---------------- epilogue: write the C tile once ----------------
  // acc[i][j][v] holds row 32i + 8*(v/4) + 4*(lane/32) + v%4, column 32j + lane%32
  // of the wave tile. Interior tiles store without bounds checks; edge tiles drop
  // the elements outside C.
  const int64_t ldc = p.ldc;
  char* const Cout = (char*)p.C + (int64_t)blockIdx.y * p.split_stride * (OUT == OUT_F32 ? 4 : 2);
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
            ((float*)Cout)[off] = x;
          else if constexpr (OUT == OUT_BF16)
            ((uint16_t*)Cout)[off] = f32_to_bf16_rne(x);
          else
            ((uint16_t*)Cout)[off] = f32_to_f16_rne(x);
        }
      }
    }
  }
}

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
// workspace is dense, so every group is a 16-byte aligned vector of one row).
template <int OUT, int G>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* ws, int splits, void* C, int64_t ldc, int M,
                                                           int N) {
  const int64_t slice = (int64_t)M * N, groups = slice / G;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < groups; q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = q * G, r = e / N, c = e - r * N;
    if constexpr (G == 4) {
      f32x4 acc = *(const f32x4*)(ws + e);
      for (int s = 1; s < splits; ++s) {
        const f32x4 x = *(const f32x4*)(ws + s * slice + e);
        acc.x += x.x;
        acc.y += x.y;
        acc.z += x.z;
        acc.w += x.w;
      }
      store_out<OUT>(C, r * ldc + c, acc.x);
      store_out<OUT>(C, r * ldc + c + 1, acc.y);
      store_out<OUT>(C, r * ldc + c + 2, acc.z);
      store_out<OUT>(C, r * ldc + c + 3, acc.w);
    } else {
      float acc = ws[e];
      for (int s = 1; s < splits; ++s) acc += ws[s * slice + e];
      store_out<OUT>(C, r * ldc + c, acc);
    }
  }
}

template <int OUT>
static void launch_reduce(const float* ws, int splits, void* C, int64_t ldc, int M, int N, hipStream_t s) {
  const bool v4 = N % 4 == 0;
  const int64_t groups = (int64_t)M * N / (v4 ? 4 : 1);
  int64_t blocks = (groups + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (v4)
    hipLaunchKernelGGL((splitk_reduce_kernel<OUT, 4>), dim3((unsigned)blocks), dim3(256), 0, s, ws, splits, C, ldc, M, N);
  else
    hipLaunchKernelGGL((splitk_reduce_kernel<OUT, 1>), dim3((unsigned)blocks), dim3(256), 0, s, ws, splits, C, ldc, M, N);
}

hipError_t launch_splitk_reduce(const float* ws, int splits, void* C, int64_t ldc, int M, int N, int out,
                                hipStream_t s) {
  if (out == OUT_F32)
    launch_reduce<OUT_F32>(ws, splits, C, ldc, M, N, s);
  else if (out == OUT_BF16)
    launch_reduce<OUT_BF16>(ws, splits, C, ldc, M, N, s);
  else
    launch_reduce<OUT_F16>(ws, splits, C, ldc, M, N, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// host-side instantiation and launch

template <class Cfg, int IN, int OUT>
static hipError_t launch_cfg(const MacroArgs& a, bool vec, hipStream_t stream, int64_t grid, int splits) {
  const dim3 g((unsigned)grid, (unsigned)splits), b(Cfg::kThreads);
  if (!vec)
    hipLaunchKernelGGL((macro_tile_kernel<Cfg, IN, OUT, kLoadElem>), g, b, 0, stream, a);
  else if (a.K % Cfg::BK == 0)
    hipLaunchKernelGGL((macro_tile_kernel<Cfg, IN, OUT, kLoadVecFull>), g, b, 0, stream, a);
  else
    hipLaunchKernelGGL((macro_tile_kernel<Cfg, IN, OUT, kLoadVec>), g, b, 0, stream, a);
  return hipGetLastError();
}

template <class Cfg>
static hipError_t launch_dtype(const MacroArgs& a, int in, int out, bool vec, hipStream_t s, int64_t grid,
                               int splits) {
  if (in == IN_BF16 && out == OUT_F32) return launch_cfg<Cfg, IN_BF16, OUT_F32>(a, vec, s, grid, splits);
  if (in == IN_BF16 && out == OUT_BF16) return launch_cfg<Cfg, IN_BF16, OUT_BF16>(a, vec, s, grid, splits);
  if (in == IN_F16 && out == OUT_F32) return launch_cfg<Cfg, IN_F16, OUT_F32>(a, vec, s, grid, splits);
  if (in == IN_F16 && out == OUT_F16) return launch_cfg<Cfg, IN_F16, OUT_F16>(a, vec, s, grid, splits);
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

hipError_t launch_macro(int shape, const MacroArgs& a, int in, int out, bool vec, hipStream_t s, int64_t grid,
                        int splits) {
  switch (shape) {
    case 0: return launch_dtype<Cfg256x256w8>(a, in, out, vec, s, grid, splits);
    case 1: return launch_dtype<Cfg256x128>(a, in, out, vec, s, grid, splits);
    case 2: return launch_dtype<Cfg128x128>(a, in, out, vec, s, grid, splits);
    case 3: return launch_dtype<Cfg64x64>(a, in, out, vec, s, grid, splits);
    case 4: return launch_dtype<Cfg256x256w4>(a, in, out, vec, s, grid, splits);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tg
