// macro_tile_kernel.h -- the output-stationary macro-tile GEMM on gfx950 MFMA.
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
// Operand layouts. Each operand is either K-contiguous in memory (A as given, or
// B supplied transposed, N x K) or M/N-contiguous (B as given, or A supplied
// transposed, K x M); the Mojo puzzle page's section on transposed loading
// describes reading a transposed operand through the shared tile. The two layouts
// are staged differently (see Opnd) and deliver identical MFMA fragments.
//
// gfx950 design (differs from the pages' one-thread-per-element kernels):
//  * waves of 64 lanes, each owning a (BM/WM) x (BN/WN) sub-tile computed with
//    v_mfma_f32_32x32x16_{bf16,f16};
//  * a pipeline of LDS stages with one barrier per K-step: K-tile kt lives in A
//    stage kt % NA and B stage kt % NB; A is loaded DA and B DB steps before the
//    step that multiplies it (two A stages and three B stages, DA = 2 and DB = 3;
//    three A stages and two B stages, DA = 3 and DB = 2; or four of each and
//    DA = DB = 3 for launches with at most one workgroup per compute unit). A stage is
//    only ever refilled once every wave's reads of it have completed (see the main
//    loop);
//  * vector path (A and B at even addresses: any shape and leading dimension):
//    16-byte buffer loads straight from global memory into LDS (buffer_load_dwordx4
//    ... lds), no register staging; out-of-range lanes use an offset beyond the
//    buffer and receive zeros; chunks that run past the end of a stored row are
//    cleaned up in LDS once the last K-tile has landed (fix_last);
//  * element path (an operand at an odd address, or a tile spanning more bytes of
//    an operand than a buffer range holds): whole 16-byte chunks, guarded 16-bit
//    loads where a chunk crosses the edge, into registers, then 16-byte LDS writes;
//  * LDS layouts XOR-swizzled per 16-byte chunk so that the fragment reads
//    (ds_read_b128 for K-contiguous tiles; ds_read_b64_tr_b16, which also performs
//    the transpose MFMA needs, for M/N-contiguous tiles) hit distinct banks;
//  * XCD-aware, grouped workgroup -> tile order (schedule_tile);
//  * the C tile is staged through LDS and stored as 16-byte chunks along its rows
//    (edge tiles drop the chunks outside C and store a chunk that crosses N
//    element by element).
#pragma once

#include "device_common.h"
#include "launch.h"

namespace tg {

constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }

// NS names the pipeline: 2 = two A stages, A loaded two steps ahead, and three B
// stages, B loaded three steps ahead; 3 = three A stages, A loaded three steps ahead,
// and two B stages, B loaded two steps ahead; 4 = four stages of each, loaded three
// steps ahead.
template <int BM_, int BN_, int BK_, int WM_, int WN_, int NS_ = 2>
struct MacroCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, NS = NS_;
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kWTM = BM / WM, kWTN = BN / WN;  // wave sub-tile
  static constexpr int kFM = kWTM / 32, kFN = kWTN / 32;  // 32x32 MFMA blocks per wave
  static constexpr int kABytes = BM * BK * 2, kBBytes = BK * BN * 2;
  static constexpr int kSubsteps = BK / 16;
  static constexpr int NA = NS == 2 ? 2 : NS;  // A stages
  static constexpr int NB = NS == 2 ? 3 : (NS == 3 ? 2 : NS);  // B stages
  // K-steps between a K-tile's load (issued right after one step's barrier) and the
  // step that multiplies it: every stage not holding a K-tile still to be multiplied.
  static constexpr int DA = NS == 4 ? NS - 1 : NA, DB = NS == 4 ? NS - 1 : NB;
  static constexpr int L = NA / gcd_c(NA, NB) * NB;  // steps after which the stage pattern repeats
  static constexpr int kLds = NA * kABytes + NB * kBBytes;
  static_assert(BK == 64, "four 16-deep substeps per K-step");
  static_assert(NS == 2 || NS == 3 || NS == 4, "three pipelines");
  // Every wave has completed its LDS reads of K-tile st when it reaches step st's
  // barrier, so the refill of K-tile st + DA (st + DB), issued right after it, may
  // take the stage of st but none of st + 1 .. st + DA - 1 (DB - 1): NA >= DA, NB >= DB.
  // In a batch of refills the operand loaded fewer steps ahead goes first, at most
  // one K-tile behind the other (the waits count loads in issue order).
  static_assert(DA >= 2 && DB >= 2 && NA >= DA && NB >= DB && DA - DB <= 1 && DB - DA <= 1,
                "refill targets a stage no wave still reads");
  static_assert(kFM >= 1 && kFN >= 1 && kWTM % 32 == 0 && kWTN % 32 == 0, "wave tile must be a multiple of 32x32");
  static_assert(kLds <= 160 * 1024, "LDS budget");
};

using Cfg256x256w8 = MacroCfg<256, 256, 64, 2, 4>;  // 8 waves, 128 x 64 per wave
using Cfg256x256w8a = MacroCfg<256, 256, 64, 2, 4, 3>;  // the same, A loaded three K-steps ahead
using Cfg256x128 = MacroCfg<256, 128, 64, 4, 2>;
using Cfg128x128 = MacroCfg<128, 128, 64, 2, 4>;      // 8 waves, 64 x 32 per wave
using Cfg64x64 = MacroCfg<64, 64, 64, 2, 2>;
using Cfg128x128s4 = MacroCfg<128, 128, 64, 2, 4, 4>;  // 4 stages, 8 waves: launches of at most one workgroup per CU
using Cfg64x64s4 = MacroCfg<64, 64, 64, 2, 2, 4>;

// Physical 16-byte chunk of logical chunk c in a K-contiguous row r (8 chunks per
// row): c ^ swz_a(r). For any 16 consecutive rows starting at a multiple of 16 and
// a fixed c, the 8-row halves see 8 distinct chunks, and rows of equal parity see
// 8 distinct chunks.
__device__ __forceinline__ int swz_a(int r) { return (r ^ (r >> 3)) & 7; }

// Physical chunk XOR for an M/N-contiguous row k (CH chunks per row). A transpose
// read touches 4 consecutive rows x 2 (or 4) consecutive chunks; these masks keep
// them on distinct banks.
template <int CH>
__device__ __forceinline__ int swz_b(int k) {
  const int m = k & 3;
  const int h = m == 0 ? 0 : (m == 1 ? 6 : (m == 2 ? 10 : 12));
  return h & (CH - 1);
}

// One operand's K-tile in LDS and the lanes that move it. X is the operand's
// extent along M (A) or N (B). KMAJ: K-contiguous in memory; the tile is stored
// as X rows of BK values (128 bytes) and a fragment is one ds_read_b128 per lane.
// Otherwise M/N-contiguous: BK rows of X values, and a fragment is two
// ds_read_b64_tr_b16 per lane. Either way lane l of fragment f, substep s holds
// position 32f + l%32 along X and reduction indices 16s + 8(l/32) .. +7, the
// operand layout of v_mfma_f32_32x32x16.
//
// "Stored" rows and columns below are those of the matrix as it lies in memory:
// for KMAJ a stored row is an X index and a stored column a K index, otherwise
// the reverse.
template <int X, int BK, bool KMAJ, int WAVES>
struct Opnd {
  static constexpr int kBytes = X * BK * 2;
  static constexpr int kRow = KMAJ ? BK * 2 : X * 2;  // LDS row pitch in bytes
  static constexpr int kChunks = kRow / 16;           // 16-byte chunks per row
  static constexpr int kRowsPerBlock = 1024 / kRow;   // rows per 1 KiB DMA block
  static constexpr int kPer = kBytes / 1024 / WAVES;  // DMA blocks per wave and stage
  static constexpr int kReads = KMAJ ? 1 : 2;         // LDS reads per fragment
  static_assert(!KMAJ || kChunks == 8, "K-contiguous swizzle assumes 8 chunks per row");
  static_assert(KMAJ || (kRow <= 1024 && kChunks >= 8), "M/N-contiguous rows must tile 1 KiB, >= 8 chunks");
  static_assert(kPer >= 1 && (kBytes / 1024) % WAVES == 0, "DMA blocks must divide among waves");

  __device__ static __forceinline__ int swz(int r) {
    if constexpr (KMAJ)
      return swz_a(r);
    else
      return swz_b<kChunks>(r);
  }
  // Tile row filled by lane l of DMA block t of wave w, and the logical chunk it
  // carries (its 16 bytes land at physical chunk l % kChunks of that row).
  __device__ static __forceinline__ int row(int w, int t, int l) { return (w * kPer + t) * kRowsPerBlock + l / kChunks; }
  __device__ static __forceinline__ int chunk(int r, int l) { return (l % kChunks) ^ swz(r); }
  // Reduction offset inside the K-tile of the data lane l of block t moves.
  __device__ static __forceinline__ int kpos(int w, int t, int l) {
    const int r = row(w, t, l);
    return KMAJ ? 8 * chunk(r, l) : r;
  }

  // Byte offset of a fragment's first read for lane l (xoff: the wave's offset
  // along X). For KMAJ, substep s is an XOR of s << 5 (the chunk pair 2s, 2s+1);
  // otherwise rows 16s (+4) are added.
  __device__ static __forceinline__ uint32_t frag(int xoff, int f, int l) {
    if constexpr (KMAJ) {
      const int r = xoff + 32 * f + (l & 31);
      return (uint32_t)(r * kRow + (((l >> 5) ^ swz(r)) << 4));
    } else {
      const int g = l >> 4, jj = l & 15;
      const int k = 8 * (g >> 1) + (jj >> 2);
      const int n = xoff + 32 * f + 16 * (g & 1) + 4 * (jj & 3);
      return (uint32_t)(k * kRow + (((n >> 3) ^ swz(k)) << 4) + (n & 7) * 2);
    }
  }
  __device__ static __forceinline__ i32x4 read(TG_LDS char* base, uint32_t off, int s) {
    if constexpr (KMAJ) {
      asm volatile("" : "+v"(off));  // keep the XOR in the loop (hoisting it costs registers)
      return *(TG_LDS i32x4*)(base + (off ^ (uint32_t)(s << 5)));
    } else {
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TG_LDS s16x4*)(base + off + (16 * s) * kRow));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TG_LDS s16x4*)(base + off + (16 * s + 4) * kRow));
      const int2 l2 = __builtin_bit_cast(int2, lo), h2 = __builtin_bit_cast(int2, hi);
      return i32x4{l2.x, l2.y, h2.x, h2.y};
    }
  }
};

// LDS buffer I of operand TAG (0 = A, 1 = B): one variable per (TAG, I, size), so
// that every stage is a distinct object. The compiler then knows which stage each
// direct load writes and waits only for those before a stage is read.
template <int TAG, int I, int BYTES>
__device__ __forceinline__ TG_LDS char* lds_stage() {
  __shared__ __attribute__((aligned(1024))) char buf[BYTES];
  return (TG_LDS char*)buf;
}

// s_waitcnt immediate for "at most n vector-memory operations outstanding" (gfx9
// encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }

// Loads: kLoadElem = guarded element loads staged in registers; kLoadVec = 16-byte
// direct loads, the last K-tile may be partial; kLoadVecFull = 16-byte direct loads,
// K is a multiple of BK.
enum { kLoadElem = 0, kLoadVec = 1, kLoadVecFull = 2 };

template <int N>
struct IC {
  static constexpr int value = N;
};
template <class T>
struct TypeIs {
  using type = T;
};
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(IC<I>{});
    static_for<I + 1, N>(f);
  }
}
// f(IC<I>), then f(IC<I + 1>) only if it returned true, and so on.
template <int I, int N, class F>
__device__ __forceinline__ void nested_for(F&& f) {
  if constexpr (I < N) {
    if (f(IC<I>{})) nested_for<I + 1, N>(f);
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

// TA: A is supplied transposed (stored K x M, lda >= M); TB: B is supplied
// transposed (stored N x K, ldb >= K). C is always M x N row-major.
template <class Cfg, int IN, int OUT, int LOAD, bool TA, bool TB>
__global__ __launch_bounds__(Cfg::kThreads, 1) void macro_tile_kernel(MacroArgs p) {
  constexpr bool VEC = LOAD != kLoadElem;
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
  constexpr int FM = Cfg::kFM, FN = Cfg::kFN;
  // Direct loads of an 8-wave workgroup are issued by half of its waves, one per
  // SIMD: a wave waiting to issue a load then leaves the SIMD's matrix core to the
  // other wave, which only multiplies (all waves do their share of the MFMAs).
  // Otherwise every wave loads its share of the K-tile.
  constexpr int LW = (VEC && Cfg::kWaves >= 8) ? Cfg::kWaves / 2 : Cfg::kWaves;  // loading waves
  using OA = Opnd<BM, BK, !TA, LW>;
  using OB = Opnd<BN, BK, TB, LW>;
  constexpr int kAPer = OA::kPer, kBPer = OB::kPer;
  constexpr int NR = FM * OA::kReads + FN * OB::kReads;  // LDS reads per substep
  constexpr int NM = FM * FN;                            // MFMAs per substep
  constexpr int NA = Cfg::NA, NB = Cfg::NB, DA = Cfg::DA, DB = Cfg::DB, L = Cfg::L;
  static_assert(VEC || Cfg::NS == 2, "the element loader stages one K-tile ahead in registers");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
  const int lwave = wave % LW;  // block index base of a loading wave (unused by the others)

  int tile_m, tile_n;
  schedule_tile(blockIdx.x, gridDim.x, p.tiles_m, p.group_m, tile_m, tile_n);
  const int row0 = tile_m * BM, col0 = tile_n * BN;
  const int M = p.M, N = p.N, K = p.K;
  const int64_t lda = p.lda, ldb = p.ldb;
  // K-tiles of this workgroup: [kt_base, kt_base + nk) (all of them without split-K);
  // below, K-tile indices kt count from kt_base
  const int kt_base = blockIdx.y * p.kt_per_split;
  const int nk_all = (K + BK - 1) / BK;
  const int nk = (nk_all - kt_base) < p.kt_per_split ? (nk_all - kt_base) : p.kt_per_split;

  // ---------------- loader geometry ----------------
  // Lane l of DMA block t fills tile row OX::row(wave, t, l) at physical chunk
  // l % kChunks; the direct loads write lane l's 16 bytes to block base + 16*l
  // and the element path writes the same slot. Per-lane byte offsets from the
  // K-tile's origin; the bound that does not depend on the K-tile (the M or N
  // extent) is folded in here as an out-of-range offset.
  uint32_t a_off[kAPer], b_off[kBPer];
  if constexpr (VEC) {
#pragma unroll
    for (int t = 0; t < kAPer; ++t) {
      const int r = OA::row(lwave, t, lane), c = OA::chunk(r, lane);
      const bool in = TA ? (row0 + 8 * c < M) : (row0 + r < M);
      a_off[t] = in ? (uint32_t)(((int64_t)r * lda + 8 * c) * 2) : kOutOfRange;
    }
#pragma unroll
    for (int t = 0; t < kBPer; ++t) {
      const int r = OB::row(lwave, t, lane), c = OB::chunk(r, lane);
      const bool in = TB ? (col0 + r < N) : (col0 + 8 * c < N);
      b_off[t] = in ? (uint32_t)(((int64_t)r * ldb + 8 * c) * 2) : kOutOfRange;
    }
  }
  // Origin of K-tile k0 (element offset) in each stored matrix, and the extent of
  // the stored matrix from there on (bytes), for the buffer descriptors.
  auto a_origin = [&](int k0) __attribute__((always_inline)) { return TA ? (int64_t)k0 * lda + row0 : (int64_t)row0 * lda + k0; };
  auto b_origin = [&](int k0) __attribute__((always_inline)) { return TB ? (int64_t)col0 * ldb + k0 : (int64_t)k0 * ldb + col0; };
  auto a_extent = [&](int k0) __attribute__((always_inline)) {
    return (TA ? (int64_t)(K - 1 - k0) * lda + (M - row0) : (int64_t)(M - 1 - row0) * lda + (K - k0)) * 2;
  };
  auto b_extent = [&](int k0) __attribute__((always_inline)) {
    return (TB ? (int64_t)(N - 1 - col0) * ldb + (K - k0) : (int64_t)(K - 1 - k0) * ldb + (N - col0)) * 2;
  };

  // Vector path: issue the direct loads of K-tile kt into a stage. Branch-free: a
  // K-tile outside [0, nk) gets a zero-length buffer, so every lane reads zeros and
  // no memory is touched (this keeps the compiler's tracking of which stage each
  // load writes exact, so it adds no waits before reads of the other stages).
  // Loads are whole 16-byte chunks at 2-byte alignment: a chunk that runs past the
  // end of a stored row reads the start of the next row (or its padding), which lands
  // at positions past M or N (outputs that are never stored) or past K (cleared once
  // the last K-tile has landed, see fix_last). Past the end of the matrix the range
  // check, which loads a dword only when all four of its bytes are in range, reads
  // zeros. With an odd stored row length (K for a K-contiguous operand, M or N
  // otherwise) the dword holding the matrix's last element also covers two bytes past
  // the end, so that element reads as zero too; it is written into LDS afterwards.
  auto issue_a = [&](TG_LDS char* sa, int kt) __attribute__((always_inline)) {
    const bool ok = (unsigned)kt < (unsigned)nk;
    const int k0 = ok ? (kt_base + kt) * BK : 0;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A + a_origin(k0), ok ? a_extent(k0) : 0);
#pragma unroll
    for (int t = 0; t < kAPer; ++t) {
      uint32_t off = a_off[t];
      if constexpr (LOAD == kLoadVec) off = (k0 + OA::kpos(lwave, t, lane) < K) ? off : kOutOfRange;
      load_lds_x4(ra, sa + (lwave * kAPer + t) * 1024, off);
    }
  };
  auto issue_b = [&](TG_LDS char* sb, int kt) __attribute__((always_inline)) {
    const bool ok = (unsigned)kt < (unsigned)nk;
    const int k0 = ok ? (kt_base + kt) * BK : 0;
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B + b_origin(k0), ok ? b_extent(k0) : 0);
#pragma unroll
    for (int t = 0; t < kBPer; ++t) {
      uint32_t off = b_off[t];
      if constexpr (LOAD == kLoadVec) off = (k0 + OB::kpos(lwave, t, lane) < K) ? off : kOutOfRange;
      load_lds_x4(rb, sb + (lwave * kBPer + t) * 1024, off);
    }
  };

  // Element path: guarded 16-bit loads of K-tile kt into registers (zeros outside
  // the matrices and for kt outside [0, nk)), and their 16-byte LDS writes. Lane l
  // of block t reads 8 consecutive elements of one stored row.
  i32x4 a_reg[kAPer], b_reg[kBPer];
  // A chunk wholly inside the row is one 16-byte load (2-byte aligned: gfx950
  // compute queues run with unaligned vector memory access); a chunk that crosses
  // the end of the row, or of the matrix, is loaded element by element.
  auto fetch8 = [](const uint16_t* src, bool row_ok, int col, int cols) __attribute__((always_inline)) {
    i32x4 v = i32x4{0, 0, 0, 0};
    if (row_ok && col + 7 < cols) {
      __builtin_memcpy(&v, src, 16);
    } else {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = (row_ok && col + 2 * e < cols) ? src[2 * e] : 0u;
        const uint32_t hi = (row_ok && col + 2 * e + 1 < cols) ? src[2 * e + 1] : 0u;
        w[e] = lo | (hi << 16);
      }
      v = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    }
    return v;
  };
  auto fetch_regs = [&](int kt) __attribute__((always_inline)) {
    const bool ok = (unsigned)kt < (unsigned)nk;
    const int k0 = (kt_base + kt) * BK;
#pragma unroll
    for (int t = 0; t < kAPer; ++t) {
      const int r = OA::row(wave, t, lane), c = OA::chunk(r, lane);
      // stored row / column of A: (m, k) as given, (k, m) transposed
      const int sr = TA ? k0 + r : row0 + r, sc = TA ? row0 + 8 * c : k0 + 8 * c;
      const int rows = TA ? K : M, cols = TA ? M : K;
      a_reg[t] = fetch8(p.A + (int64_t)sr * lda + sc, ok && sr < rows, sc, cols);
    }
#pragma unroll
    for (int t = 0; t < kBPer; ++t) {
      const int r = OB::row(wave, t, lane), c = OB::chunk(r, lane);
      // stored row / column of B: (k, n) as given, (n, k) transposed
      const int sr = TB ? col0 + r : k0 + r, sc = TB ? k0 + 8 * c : col0 + 8 * c;
      const int rows = TB ? N : K, cols = TB ? K : N;
      b_reg[t] = fetch8(p.B + (int64_t)sr * ldb + sc, ok && sr < rows, sc, cols);
    }
  };
  auto store_regs = [&](TG_LDS char* sa, TG_LDS char* sb) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < kAPer; ++t) *(TG_LDS i32x4*)(sa + (wave * kAPer + t) * 1024 + lane * 16) = a_reg[t];
#pragma unroll
    for (int t = 0; t < kBPer; ++t) *(TG_LDS i32x4*)(sb + (wave * kBPer + t) * 1024 + lane * 16) = b_reg[t];
  };

  // Vector path, the last K-tile of the matrix, once a loading wave's own loads of it
  // have landed in a stage: in a K-contiguous operand, clear the positions past K of
  // the chunk that straddles K in each tile row this wave loaded (they hold the next
  // row's data, possibly not even finite); and where the range check zeroed the
  // matrix's last element, write it. Then wait until these LDS writes are done.
  auto fix_operand = [&](auto OT, auto KM, TG_LDS char* st, const uint16_t* base, int64_t ld, int x0, int X, int XT,
                         int k0) __attribute__((always_inline)) {
    using O = typename decltype(OT)::type;
    constexpr bool KMAJ = decltype(KM)::value;
    if constexpr (KMAJ) {
      const int kv = K - k0;  // valid reduction indices in this K-tile
      if (kv & 7) {
        const int cs = kv >> 3, keep = kv & 7;
        constexpr int RPW = O::kPer * O::kRowsPerBlock;  // tile rows this wave loaded
#pragma unroll
        for (int i0 = 0; i0 < RPW; i0 += 64) {
          const int i = i0 + lane;
          if (RPW % 64 == 0 || i < RPW) {
            const int r = lwave * RPW + i;
            TG_LDS uint16_t* c = (TG_LDS uint16_t*)(st + r * O::kRow + ((cs ^ O::swz(r)) << 4));
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (e >= keep) c[e] = 0;
            if ((K & 1) && x0 + r == X - 1) c[keep - 1] = base[(int64_t)(X - 1) * ld + (K - 1)];
          }
        }
      }
    } else {
      const int kk = K - 1 - k0, xx = X - 1 - x0;  // the matrix's last element in this tile
      if ((X & 1) && xx >= 0 && xx < XT && lwave == (kk / O::kRowsPerBlock) / O::kPer && lane == 0)
        *(TG_LDS uint16_t*)(st + kk * O::kRow + (((xx >> 3) ^ O::swz(kk)) << 4) + (xx & 7) * 2) =
            base[(int64_t)(K - 1) * ld + (X - 1)];
    }
  };
  auto fix_last = [&](TG_LDS char* sa, TG_LDS char* sb, int kt) __attribute__((always_inline)) {
    // something to do: a K-contiguous operand with K not a multiple of 8, or an
    // M/N-contiguous operand with an odd row length
    const bool need = ((!TA || TB) && (K & 7)) || (TA && (M & 1)) || (!TB && (N & 1));
    if (kt_base + kt == nk_all - 1 && need) {
      const int k0 = (kt_base + kt) * BK;
      fix_operand(TypeIs<OA>{}, IC<!TA>{}, sa, p.A, lda, row0, M, BM, k0);
      fix_operand(TypeIs<OB>{}, IC<TB>{}, sb, p.B, ldb, col0, N, BN, k0);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    }
  };

  // ---------------- fragment addressing ----------------
  uint32_t a_frag[FM], b_frag[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) a_frag[i] = OA::frag(wm * Cfg::kWTM, i, lane);
#pragma unroll
  for (int j = 0; j < FN; ++j) b_frag[j] = OB::frag(wn * Cfg::kWTN, j, lane);

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

  // Fragments of substep s (16 reduction indices), read in the order the MFMAs
  // (row-major over the i x j blocks) consume them: a[0], every b[j], a[1..].
  auto read_frags = [&](TG_LDS char* sa, TG_LDS char* sb, int s, i32x4(&a)[FM], i32x4(&b)[FN]) {
    a[0] = OA::read(sa, a_frag[0], s);
#pragma unroll
    for (int j = 0; j < FN; ++j) b[j] = OB::read(sb, b_frag[j], s);
#pragma unroll
    for (int i = 1; i < FM; ++i) a[i] = OA::read(sa, a_frag[i], s);
  };
  // MFMAs of one substep; half 0 = block rows [0, FM/2), half 1 = the rest. The B
  // fragment goes in the instruction's first operand and the A fragment in its
  // second: both operands share one lane layout, so this computes the transposed
  // block, (A B)^T = B^T A^T, which leaves each lane holding runs of four
  // consecutive columns of one C row (see the epilogue).
  auto mfma_rows = [&](const i32x4(&a)[FM], const i32x4(&b)[FN], int i0, int i1) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
      if (i >= i0 && i < i1)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<IN>(b[j], a[i], acc[i][j]);
  };

  TG_LDS char* pA[NA];
  TG_LDS char* pB[NB];
  static_for<0, NA>([&](auto i) { pA[i.value] = lds_stage<0, i.value, Cfg::kABytes>(); });
  static_for<0, NB>([&](auto i) { pB[i.value] = lds_stage<1, i.value, Cfg::kBBytes>(); });

  // ---------------- main loop ----------------
  // K-tile kt lives in A stage kt % NA and B stage kt % NB. Step st multiplies
  // K-tile st in four substeps; the reads of substep s+1 are issued among the MFMAs
  // of substep s. The step's barrier sits after the first half of the last
  // substep's MFMAs: before it each wave waits until its own LDS reads have
  // completed, and each loading wave until its loads of K-tile st + 1 have landed
  // (later K-tiles may still be in flight); right after it the loading waves issue
  // B's K-tile st + DB and A's K-tile st + DA, and every wave reads the first
  // fragments of K-tile st + 1, all covered by the second half of those MFMAs.
  //
  // Why no stage is written while a wave may still read it ("Tiled Matrix
  // Multiplication", section 5: a barrier after the tile is consumed, before it
  // is overwritten). A wave's LDS read is complete once the wave has waited for
  // it (s_waitcnt lgkmcnt). Every read of K-tile st is issued before step st's
  // barrier (the last substep's fragments are read during the third substep's
  // MFMAs), and every wave waits for all its reads (lgkmcnt(0)) before that
  // barrier, so once a wave has passed it no wave reads K-tile st or an earlier one
  // any more. The refills issued right after step st's barrier go to the stages that
  // held K-tile st + DA - NA (A) and st + DB - NB (B): st or earlier, since
  // NA >= DA and NB >= DB. The writes before step st's barrier (the element loader's
  // K-tile st + 1, the clean-up of a last K-tile) go to the stages of K-tile st + 1,
  // which held K-tile st + 1 - NA and st + 1 - NB, at most st - 1, whose reads every
  // wave completed before step st - 1's barrier. (The fragments read after the last
  // step, from the stage of a K-tile past the slice, are never multiplied.)
  //
  // Loads complete in the order they are issued (a wave's s_waitcnt vmcnt counts
  // the loads still in flight), so each batch of refills issues first the operand
  // loaded fewer steps ahead (A when DB = DA + 1, B when DA = DB + 1). With DA == DB a
  // batch holds one K-tile, and K-tile st + 1 is complete once at most DA - 2 batches
  // are in flight. With DB = DA + 1, A's part of K-tile st + 1 comes first in batch
  // st + 1 - DA, the later of the two batches that hold K-tile st + 1 (B's part is in
  // batch st - DA); only the B part of that batch and the DA - 2 batches after it may
  // still be in flight (and the same with A and B swapped when DA = DB + 1).
  //
  // The stage pattern repeats every L steps: the loop body is one cycle of L
  // unrolled steps (stage indices are compile-time, so the compiler tracks the
  // direct loads of each stage apart), and the last nk % L steps follow it.
  constexpr int PER = kAPer + kBPer;  // direct loads per wave and K-tile
  // loads a loading wave may leave in flight once K-tile 0 (k0) or K-tile st + 1 (k1) is complete
  constexpr int kDS = DA < DB ? DA : DB;                           // the shorter distance
  constexpr int kLate = DA > DB ? kAPer : (DB > DA ? kBPer : 0);    // loads of the longer one per batch
  constexpr int kInFlight0 = DA == DB ? PER * (DA - 1) : kLate + PER * (kDS - 1);
  constexpr int kInFlight1 = DA == DB ? PER * (DA - 2) : kLate + PER * (kDS - 2);
  // The batch of refills issued right after step j's barrier (j < 0: the prologue's
  // batches; st = j there): A's K-tile st + DA and B's st + DB, the operand loaded
  // fewer steps ahead first; in the prologue K-tiles before 0 are skipped.
  auto refill = [&](auto J, int st) __attribute__((always_inline)) {
    constexpr int j = decltype(J)::value;
    constexpr int ia = ((j + DA) % NA + NA) % NA, ib = ((j + DB) % NB + NB) % NB;
    if constexpr (DB > DA) {
      if constexpr (j + DA >= 0) issue_a(pA[ia], st + DA);
      issue_b(pB[ib], st + DB);
    } else {
      if constexpr (j + DB >= 0) issue_b(pB[ib], st + DB);
      issue_a(pA[ia], st + DA);
    }
  };
  i32x4 fa[FM], fb[FN], ga[FM], gb[FN];
  // The pipeline, for a wave that loads (LOADER) or one that only multiplies; the
  // two are separate branch-free copies, so the compiler tracks each one's loads
  // exactly. A multiplying wave waits for nothing but its reads and the barriers:
  // each loading wave has waited for its own loads of a K-tile before it arrives there.
  auto run = [&](auto ROLE) __attribute__((always_inline)) {
    constexpr bool LOADER = decltype(ROLE)::value != 0;
    if constexpr (VEC) {
      if constexpr (LOADER) {
        // the batches of steps -max(DA, DB) .. -1 in the steady order
        constexpr int kDL = DA > DB ? DA : DB;
        static_for<0, kDL>([&](auto i) {
          constexpr int b = i.value - kDL;
          refill(IC<b>{}, b);
        });
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kInFlight0));  // K-tile 0 landed
        fix_last(pA[0], pB[0], 0);
      }
    } else {
      fetch_regs(0);
      store_regs(pA[0], pB[0]);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    }
    barrier_nofence();
    if constexpr (!VEC) fetch_regs(1);
    read_frags(pA[0], pB[0], 0, fa, fb);

    auto step = [&](auto J, int st) __attribute__((always_inline)) {
      constexpr int j = decltype(J)::value;
      TG_LDS char* const sa = pA[j % NA];  // K-tile st
      TG_LDS char* const sb = pB[j % NB];
      TG_LDS char* const na = pA[(j + 1) % NA];  // K-tile st + 1
      TG_LDS char* const nb = pB[(j + 1) % NB];
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
      // K-tile st + 1 must be complete in every wave before anyone reads it, and no
      // read of K-tile st may be in flight in any wave once the barrier is passed.
      if constexpr (VEC) {
        if constexpr (LOADER) {
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(kInFlight1));  // its loads of K-tile st + 1 landed
          fix_last(na, nb, st + 1);
        }
      } else {
        store_regs(na, nb);  // K-tile st + 1, fetched one step ago
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads and writes are done
      barrier_nofence();
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (VEC && LOADER) {
        refill(J, st);  // past the last K-tile: zero-length, no traffic
      } else if constexpr (!VEC) {
        fetch_regs(st + 2);
      }
      read_frags(na, nb, 0, fa, fb);
      mfma_rows(ga, gb, FM / 2, FM);
      interleave<(FM - FM / 2) * FN, NR, (VEC && LOADER) ? PER : 0>();
      __builtin_amdgcn_sched_barrier(0);
    };
    int st = 0;
    for (; st + L <= nk; st += L) static_for<0, L>([&](auto J) { step(J, st + J.value); });
    // The remaining nk % L steps, nested so that a skipped step leads only to the
    // end: a path that skipped a step never reaches a later one, so the compiler
    // keeps an exact account of which stage each load in flight writes (a join
    // that let it would make it wait for every load before the next fragment reads).
    nested_for<0, L - 1>([&](auto J) __attribute__((always_inline)) {
      if (st + J.value >= nk) return false;
      step(J, st + J.value);
      return true;
    });
  };
  if constexpr (LW == Cfg::kWaves)
    run(IC<1>{});
  else if (wave < LW)
    run(IC<1>{});
  else
    run(IC<0>{});
  if constexpr (VEC) __builtin_amdgcn_s_waitcnt(0x0F70);  // trailing loads land before LDS is released

  // ---------------- epilogue: write the C tile once ----------------
  // acc[i][j][v] holds row 32i + lane%32 and columns 32j + 8*(v/4) + 4*(lane/32) +
  // v%4 of the wave tile: for each g = v/4, four consecutive columns of one row. With
  // split-K, slice y writes its partial tile at C + y * split_stride.
  const int64_t ldc = p.ldc;
  char* const Cout = (char*)p.C + (int64_t)blockIdx.y * p.split_stride * (OUT == OUT_F32 ? 4 : 2);
  constexpr int SO = OUT == OUT_F32 ? 4 : 2;  // bytes per output element
  if (p.c_vec) {
    // Each block row (32 rows of the wave tile) goes through
    // a private LDS slice of the stage memory, written as runs of four elements and
    // read back as 16-byte chunks along the rows, so that every global store writes
    // whole 16-byte chunks of consecutive columns (CH lanes per row of the wave
    // tile). 16-byte chunks are XOR-swizzled by row within the slice; with 16-bit
    // outputs a lane writes half a chunk, and the halves are also swapped on rows
    // with bit 3 set, so that 16 consecutive rows write 16 distinct 8-byte slots of
    // a 128-byte bank window (the read-back swaps them again).
    constexpr int RB = Cfg::kWTN * SO;  // bytes per row of a wave tile
    constexpr int CH = RB / 16;         // 16-byte chunks per row
    constexpr int SLICE = 32 * RB;      // one block row
    constexpr int PER_OBJ = Cfg::kABytes / SLICE;
    static_assert(CH >= 2 && 64 % CH == 0 && PER_OBJ >= 1 && Cfg::kWaves <= NA * PER_OBJ,
                  "the wave slices fit in the A stages");
    // every wave is done with the stages, and no direct load is still landing
    __builtin_amdgcn_s_waitcnt(0);
    barrier_nofence();
    // wave w's slice: number w % PER_OBJ of A stage w / PER_OBJ (two-way choice at
    // most: an indexed choice among the stages would go through scratch memory)
    constexpr int NOBJ = (Cfg::kWaves + PER_OBJ - 1) / PER_OBJ;
    static_assert(NOBJ <= 2, "wave slices span at most two A stages");
    TG_LDS char* const slice =
        (NOBJ == 1 || wave < PER_OBJ ? pA[0] : pA[NOBJ - 1]) + (wave % PER_OBJ) * SLICE;
    const int r = lane & 31, h = lane >> 5;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float x0 = acc[i][j][4 * g], x1 = acc[i][j][4 * g + 1], x2 = acc[i][j][4 * g + 2],
                      x3 = acc[i][j][4 * g + 3];
          const int col = 32 * j + 8 * g + 4 * h;  // first of the four columns in the wave tile
          const int byte = col * SO;
          const int c = byte >> 4;
          const int half = SO == 2 ? ((byte >> 3) & 1) ^ ((r >> 3) & 1) : 0;
          const uint32_t at = (uint32_t)(r * RB + ((c ^ (r % CH)) << 4) + 8 * half);
          if constexpr (OUT == OUT_F32) {
            *(TG_LDS f32x4*)(slice + at) = f32x4{x0, x1, x2, x3};
          } else {
            uint32_t lo, hi;
            if constexpr (OUT == OUT_BF16) {
              lo = pack_bf16x2(x0, x1);
              hi = pack_bf16x2(x2, x3);
            } else {
              lo = (uint32_t)f32_to_f16_rne(x0) | ((uint32_t)f32_to_f16_rne(x1) << 16);
              hi = (uint32_t)f32_to_f16_rne(x2) | ((uint32_t)f32_to_f16_rne(x3) << 16);
            }
            *(TG_LDS u32x2*)(slice + at) = u32x2{lo, hi};
          }
        }
      }
      asm volatile("" ::: "memory");  // the reads below see this wave's writes (LDS is in order per wave)
      constexpr int ROWS = 64 / CH;  // rows per 64-lane read
      const int64_t gr0 = (int64_t)(row0 + wm * Cfg::kWTM + 32 * i);
      const int gc0 = col0 + wn * Cfg::kWTN;
      auto store_chunks = [&](auto EDGE) __attribute__((always_inline)) {
        constexpr int PER_CHUNK = 16 / SO;  // elements per 16-byte chunk
#pragma unroll
        for (int q = 0; q < 32 / ROWS; ++q) {
          const int rr = q * ROWS + lane / CH, c = lane % CH;
          i32x4 v = *(TG_LDS i32x4*)(slice + rr * RB + ((c ^ (rr % CH)) << 4));
          if (SO == 2 && ((rr >> 3) & 1)) v = i32x4{v.z, v.w, v.x, v.y};
          char* dst = Cout + ((gr0 + rr) * ldc + gc0) * SO + 16 * c;
          // C is written once and not read back here: non-temporal stores (1-2% on
          // products of one round of tiles, where all tiles store at once). The type
          // carries C's element alignment only: the chunk may straddle 16-byte words.
          typedef i32x4 i32x4_u __attribute__((aligned(2)));
          if constexpr (!decltype(EDGE)::value) {
            __builtin_nontemporal_store(v, (i32x4_u*)dst);
          } else {
            // rows past M and columns past N are dropped; a chunk that crosses N is
            // stored element by element
            const int64_t row = gr0 + rr;
            const int col = gc0 + PER_CHUNK * c;
            if (row < M && col < N) {
              if (col + PER_CHUNK <= N) {
                __builtin_nontemporal_store(v, (i32x4_u*)dst);
              } else {
#pragma unroll
                for (int k = 0; k < PER_CHUNK; ++k) {
                  if (col + k < N) {
                    if constexpr (SO == 2)
                      *(uint16_t*)(dst + 2 * k) = (uint16_t)((uint32_t)v[k / 2] >> (16 * (k % 2)));
                    else
                      *(uint32_t*)(dst + 4 * k) = (uint32_t)v[k];
                  }
                }
              }
            }
          }
        }
      };
      if (row0 + BM <= M && col0 + BN <= N)
        store_chunks(IC<0>{});
      else
        store_chunks(IC<1>{});
      asm volatile("" ::: "memory");  // the next block row's writes come after these reads
    }
  } else {
    // C not aligned to its element size: element by element, dropping what lies
    // outside C.
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = row0 + wm * Cfg::kWTM + 32 * i + (lane & 31);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int cb = col0 + wn * Cfg::kWTN + 32 * j + 4 * (lane >> 5);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int col = cb + 8 * (v >> 2) + (v & 3);
          if (row < M && col < N) {
            const int64_t off = (int64_t)row * ldc + col;
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
}

// ---------------------------------------------------------------------------
// host-side instantiation and launch of one operand layout

template <class Cfg, int IN, int OUT, bool TA, bool TB>
static hipError_t launch_cfg(const MacroArgs& a, bool vec, hipStream_t stream, int64_t grid, int splits) {
  using Cfg2 = MacroCfg<Cfg::BM, Cfg::BN, Cfg::BK, Cfg::WM, Cfg::WN, 2>;  // for the element loader
  const dim3 g((unsigned)grid, (unsigned)splits), b(Cfg::kThreads);
  if (!vec)
    hipLaunchKernelGGL((macro_tile_kernel<Cfg2, IN, OUT, kLoadElem, TA, TB>), g, b, 0, stream, a);
  else if (a.K % Cfg::BK == 0)
    hipLaunchKernelGGL((macro_tile_kernel<Cfg, IN, OUT, kLoadVecFull, TA, TB>), g, b, 0, stream, a);
  else
    hipLaunchKernelGGL((macro_tile_kernel<Cfg, IN, OUT, kLoadVec, TA, TB>), g, b, 0, stream, a);
  return hipGetLastError();
}

// Instantiated explicitly, one compilation unit per operand layout and group of tiles
// (macro_tile_inst_*.hip), so that they compile in parallel.
template <class Cfg, bool TA, bool TB>
hipError_t launch_dtype(const MacroArgs& a, int in, int out, bool vec, hipStream_t s, int64_t grid, int splits) {
  if (in == IN_BF16 && out == OUT_F32) return launch_cfg<Cfg, IN_BF16, OUT_F32, TA, TB>(a, vec, s, grid, splits);
  if (in == IN_BF16 && out == OUT_BF16) return launch_cfg<Cfg, IN_BF16, OUT_BF16, TA, TB>(a, vec, s, grid, splits);
  if (in == IN_F16 && out == OUT_F32) return launch_cfg<Cfg, IN_F16, OUT_F32, TA, TB>(a, vec, s, grid, splits);
  if (in == IN_F16 && out == OUT_F16) return launch_cfg<Cfg, IN_F16, OUT_F16, TA, TB>(a, vec, s, grid, splits);
  return hipErrorInvalidValue;
}

// The tile configurations, in the order of kMacroShapes (the shape index of launch_macro):
// X(index, configuration).
#define TG_MACRO_CONFIGS(X)                                                                           \
  X(0, Cfg256x256w8) X(1, Cfg256x128) X(2, Cfg128x128) X(3, Cfg64x64) X(4, Cfg128x128s4) X(5, Cfg64x64s4) \
  X(6, Cfg256x256w8a)

}  // namespace tg
