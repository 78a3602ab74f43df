// api.hip -- the C ABI of include/tgemm.h: handles, argument checks, kernel
// choice and launch. Argument errors are found here, on the host, before any HIP
// call; launches are asynchronous on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <unordered_set>

#include "launch.h"
#include "tgemm.h"

struct tgemm_handle {
  int device;
  int cus;
  int tm, tn, tk;   // forced tile, 0 = automatic
  int splits;       // forced K-slice count, 0 = automatic
  void* ws;         // split-K workspace (device memory owned by the handle), or null
  size_t ws_bytes;  // its size
};

namespace {

std::mutex g_mu;
std::unordered_set<const tgemm_handle*>& live() {
  static std::unordered_set<const tgemm_handle*> s;
  return s;
}
bool is_live(const tgemm_handle* h) {
  std::lock_guard<std::mutex> g(g_mu);
  return h != nullptr && live().count(h) != 0;
}

constexpr int64_t kI32Max = 0x7fffffffLL;
// Largest M, N, K: the kernels index rows, columns and K in 32-bit integers and add
// up to a tile (and a K-tile) to them, which stays below 2^31 from here.
constexpr int64_t kMaxDim = (int64_t)1 << 30;
constexpr int kMaxSplits = 64;  // largest K-slice count gemm_set_split_k accepts
constexpr int64_t kDeepMaxWorkgroups = 256;  // one per compute unit of MI355X
constexpr int64_t kDeepMinKTiles = 16;       // per K-slice, so the zero K-tiles padding a slice stay few
constexpr int64_t kMaxRecords = 0x7FFFFFF0LL;  // must match device_common.h

int out_bytes(int dtype) { return (dtype == GEMM_I32_I32 || dtype == GEMM_F16_F32 || dtype == GEMM_BF16_F32) ? 4 : 2; }
int in_kind(int dtype) { return (dtype == GEMM_BF16_F32 || dtype == GEMM_BF16_BF16) ? 1 : 0; }  // 1 = bf16
int out_kind(int dtype) {
  if (dtype == GEMM_BF16_BF16) return 1;
  if (dtype == GEMM_F16_F16) return 2;
  return 0;
}
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t max1(int64_t x) { return x > 1 ? x : 1; }

// Can the tile's 16-byte buffer loads be used? Needs 16-byte aligned A and B, row
// strides and the contiguous extent of each stored operand (K, or M / N for the
// M/N-contiguous layouts) in whole 8-element chunks, and every in-tile offset below
// the buffer range limit. ta / tb: A / B supplied transposed.
bool vector_ok(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb, int bm, int bn,
               int bk, bool ta, bool tb) {
  if (((uintptr_t)A & 15) || ((uintptr_t)B & 15)) return false;
  if ((lda & 7) || (ldb & 7)) return false;
  if (((ta ? M : K) & 7) || ((tb ? K : N) & 7)) return false;
  // largest in-tile byte offset: (tile rows - 1) * ld + row length of the stored tile
  const int64_t a_rows = ta ? bk : bm, a_len = ta ? bm : bk;
  const int64_t b_rows = tb ? bn : bk, b_len = tb ? bk : bn;
  if (((a_rows - 1) * lda + a_len) * 2 >= kMaxRecords) return false;
  if (((b_rows - 1) * ldb + b_len) * 2 >= kMaxRecords) return false;
  return true;
}

// Macro-tile configuration of a tile with the given number of LDS stages (the
// first one listed), or -1.
int find_macro(int tm, int tn, int tk, int stages = 2) {
  for (int i = 0; i < tg::kNumMacroShapes; ++i) {
    const tg::MacroShape& m = tg::kMacroShapes[i];
    if (m.bm == tm && m.bn == tn && m.bk == tk && m.stages == stages) return i;
  }
  return -1;
}

// Automatic tile: the largest macro tile that still gives the chip (256 CUs) a
// full wave of workgroups; smaller tiles for smaller problems.
int auto_macro(int64_t M, int64_t N) {
  const int64_t t256 = cdiv(M, 256) * cdiv(N, 256);
  if (t256 >= 256) return 0;
  const int64_t t256x128 = cdiv(M, 256) * cdiv(N, 128);
  if (t256x128 >= 256) return 1;
  const int64_t t128 = cdiv(M, 128) * cdiv(N, 128);
  if (t128 >= 64) return 2;
  return 3;
}

gemm_status_t plan_impl(const tgemm_handle* h, int op_a, int op_b, int64_t M, int64_t N, int64_t K, const void* A,
                        int64_t lda, const void* B, int64_t ldb, const void* C, int64_t ldc, int dtype,
                        gemm_plan_t* out) {
  gemm_status_t st = gemm_check_args_op((gemm_op_t)op_a, (gemm_op_t)op_b, M, N, K, A, lda, B, ldb, C, ldc,
                                        (gemm_dtype_t)dtype);
  if (st != GEMM_OK) return st;
  gemm_plan_t p;
  std::memset(&p, 0, sizeof(p));
  const int ftm = h ? h->tm : 0, ftn = h ? h->tn : 0, ftk = h ? h->tk : 0;
  const bool forced = ftm != 0;
  if (dtype == GEMM_I32_I32) {
    const int tm = forced ? ftm : 16, tn = forced ? ftn : 16, tk = forced ? ftk : 64;
    if ((int64_t)tm * tn > 1024 || ((int64_t)tm * tk + (int64_t)tk * tn) * 4 > 65536) return GEMM_ERR_UNSUPPORTED_TILE;
    p.tile_m = tm;
    p.tile_n = tn;
    p.tile_k = tk;
    p.threads = tm * tn;
    p.lds_bytes = (tm * tk + tk * tn) * 4;
    p.vector_loads = 0;
    p.kernel = 2;
  } else {
    int shape = -1;
    bool small = false;
    if (forced) {
      if (ftm == 16 && ftn == 16 && ftk == 32)
        small = true;
      else if ((shape = find_macro(ftm, ftn, ftk)) < 0)
        return GEMM_ERR_UNSUPPORTED_TILE;
    } else {
      shape = auto_macro(M, N);
    }
    if (small) {
      p.tile_m = 16;
      p.tile_n = 16;
      p.tile_k = 32;
      p.threads = 64;
      p.lds_bytes = 4096;
      p.kernel = 3;
    } else {
      const tg::MacroShape& s = tg::kMacroShapes[shape];
      p.tile_m = s.bm;
      p.tile_n = s.bn;
      p.tile_k = s.bk;
      p.threads = s.threads;
      p.lds_bytes = s.lds;
      p.kernel = 4;
    }
    p.vector_loads =
        vector_ok(M, N, K, A, lda, B, ldb, p.tile_m, p.tile_n, p.tile_k, op_a == GEMM_OP_T, op_b == GEMM_OP_T) ? 1 : 0;
  }
  p.split_k = 1;
  p.stages = p.kernel == 2 ? 1 : 2;
  if (M == 0 || N == 0) {
    p.kernel = 0;
    p.grid = 0;
    p.stages = 0;
  } else if (K == 0) {
    p.kernel = 1;
    p.stages = 0;
    p.grid = cdiv(M * N, 256) < 65536 ? cdiv(M * N, 256) : 65536;
  } else {
    p.grid = cdiv(M, p.tile_m) * cdiv(N, p.tile_n);
    if (p.grid > kI32Max) return GEMM_ERR_INVALID_ARG;
    // Split-K (automatic tiles only): when the C tiles cannot fill half of the chip
    // and the reduction is long, each tile's K range is cut into slices computed by
    // separate workgroups; their fp32 partial tiles are summed by a second kernel.
    // A forced slice count (gemm_set_split_k) replaces the heuristic. Slices hold
    // cdiv(nk, S) K-tiles each, and S is lowered so that none is empty.
    const int64_t nk = cdiv(K, p.tile_k);
    const int fs = h ? h->splits : 0;
    int64_t sk = 1;
    if (p.kernel == 4) {
      if (fs > 0) {
        sk = fs;
      } else if (!forced && p.grid < 128 && nk >= 8) {
        sk = 256 / p.grid;
        if (sk > 16) sk = 16;
        if (sk > nk / 4) sk = nk / 4;
      }
    }
    if (sk > nk) sk = nk;
    if (sk >= 2) p.split_k = (int32_t)cdiv(nk, cdiv(nk, sk));
    // Deeper pipeline: when the launch leaves at most one workgroup per compute unit
    // (so no other workgroup hides a workgroup's memory latency) and each K-slice is
    // long, the 4-stage twin of the tile keeps three K-tiles of loads in flight.
    if (p.kernel == 4 && p.vector_loads && p.grid * p.split_k <= kDeepMaxWorkgroups &&
        cdiv(nk, p.split_k) >= kDeepMinKTiles) {
      const int deep = find_macro(p.tile_m, p.tile_n, p.tile_k, 4);
      if (deep >= 0) {
        p.stages = 4;
        p.lds_bytes = tg::kMacroShapes[deep].lds;
      }
    }
  }
  *out = p;
  return GEMM_OK;
}

}  // namespace

extern "C" {

const char* gemm_status_string(gemm_status_t s) {
  switch (s) {
    case GEMM_OK: return "GEMM_OK";
    case GEMM_ERR_INVALID_ARG: return "GEMM_ERR_INVALID_ARG: invalid argument or handle";
    case GEMM_ERR_UNSUPPORTED_DTYPE: return "GEMM_ERR_UNSUPPORTED_DTYPE: unknown dtype";
    case GEMM_ERR_NO_DEVICE: return "GEMM_ERR_NO_DEVICE: no HIP device";
    case GEMM_ERR_ARCH: return "GEMM_ERR_ARCH: device is not gfx950";
    case GEMM_ERR_HIP: return "GEMM_ERR_HIP: HIP runtime or launch failure";
    case GEMM_ERR_OUT_OF_MEMORY: return "GEMM_ERR_OUT_OF_MEMORY: allocation of the handle or workspace failed";
    case GEMM_ERR_UNSUPPORTED_TILE: return "GEMM_ERR_UNSUPPORTED_TILE: no kernel has this tile for this dtype";
  }
  return "unknown status";
}

gemm_status_t gemm_check_args_op(gemm_op_t op_a, gemm_op_t op_b, int64_t M, int64_t N, int64_t K, const void* A,
                                 int64_t lda, const void* B, int64_t ldb, const void* C, int64_t ldc,
                                 gemm_dtype_t dtype) {
  const int d = (int)dtype;
  if (d < GEMM_I32_I32 || d > GEMM_F16_F16) return GEMM_ERR_UNSUPPORTED_DTYPE;
  if ((op_a != GEMM_OP_N && op_a != GEMM_OP_T) || (op_b != GEMM_OP_N && op_b != GEMM_OP_T))
    return GEMM_ERR_INVALID_ARG;
  if (M < 0 || N < 0 || K < 0) return GEMM_ERR_INVALID_ARG;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return GEMM_ERR_INVALID_ARG;
  // row length of each stored matrix: A is M x K (K x M transposed), B is K x N (N x K transposed)
  const int64_t a_len = op_a == GEMM_OP_N ? K : M, b_len = op_b == GEMM_OP_N ? N : K;
  if (lda < max1(a_len) || ldb < max1(b_len) || ldc < max1(N)) return GEMM_ERR_INVALID_ARG;
  if (lda > (int64_t)1 << 40 || ldb > (int64_t)1 << 40 || ldc > (int64_t)1 << 40) return GEMM_ERR_INVALID_ARG;
  if (M * K > 0 && A == nullptr) return GEMM_ERR_INVALID_ARG;
  if (K * N > 0 && B == nullptr) return GEMM_ERR_INVALID_ARG;
  if (M * N > 0 && C == nullptr) return GEMM_ERR_INVALID_ARG;
  return GEMM_OK;
}

gemm_status_t gemm_check_args(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                              int64_t ldb, const void* C, int64_t ldc, gemm_dtype_t dtype) {
  return gemm_check_args_op(GEMM_OP_N, GEMM_OP_N, M, N, K, A, lda, B, ldb, C, ldc, dtype);
}

gemm_status_t gemm_create(gemm_handle_t* out) {
  if (out == nullptr) return GEMM_ERR_INVALID_ARG;
  *out = nullptr;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return GEMM_ERR_NO_DEVICE;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GEMM_ERR_HIP;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GEMM_ERR_HIP;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return GEMM_ERR_ARCH;
  tgemm_handle* h = new (std::nothrow) tgemm_handle;
  if (h == nullptr) return GEMM_ERR_OUT_OF_MEMORY;
  h->device = dev;
  h->cus = prop.multiProcessorCount;
  h->tm = h->tn = h->tk = 0;
  h->splits = 0;
  h->ws = nullptr;
  h->ws_bytes = 0;
  {
    std::lock_guard<std::mutex> g(g_mu);
    live().insert(h);
  }
  *out = h;
  return GEMM_OK;
}

gemm_status_t gemm_destroy(gemm_handle_t h) {
  {
    std::lock_guard<std::mutex> g(g_mu);
    if (h == nullptr || live().erase(h) == 0) return GEMM_ERR_INVALID_ARG;
  }
  gemm_status_t st = GEMM_OK;
  if (h->ws != nullptr && hipFree(h->ws) != hipSuccess) st = GEMM_ERR_HIP;  // waits for work using it
  delete h;
  return st;
}

gemm_status_t gemm_set_tile(gemm_handle_t h, int32_t tm, int32_t tn, int32_t tk) {
  if (!is_live(h)) return GEMM_ERR_INVALID_ARG;
  const bool all_zero = tm == 0 && tn == 0 && tk == 0;
  if (!all_zero && (tm <= 0 || tn <= 0 || tk <= 0)) return GEMM_ERR_INVALID_ARG;
  h->tm = tm;
  h->tn = tn;
  h->tk = tk;
  return GEMM_OK;
}

gemm_status_t gemm_set_split_k(gemm_handle_t h, int32_t splits) {
  if (!is_live(h)) return GEMM_ERR_INVALID_ARG;
  if (splits < 0 || splits > kMaxSplits) return GEMM_ERR_INVALID_ARG;
  h->splits = splits;
  return GEMM_OK;
}

gemm_status_t gemm_plan_op(gemm_handle_t h, gemm_op_t op_a, gemm_op_t op_b, int64_t M, int64_t N, int64_t K,
                           const void* A, int64_t lda, const void* B, int64_t ldb, const void* C, int64_t ldc,
                           gemm_dtype_t dtype, gemm_plan_t* out) {
  if (out == nullptr) return GEMM_ERR_INVALID_ARG;
  if (h != nullptr && !is_live(h)) return GEMM_ERR_INVALID_ARG;
  return plan_impl(h, (int)op_a, (int)op_b, M, N, K, A, lda, B, ldb, C, ldc, (int)dtype, out);
}

gemm_status_t gemm_plan(gemm_handle_t h, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                        const void* B, int64_t ldb, const void* C, int64_t ldc, gemm_dtype_t dtype,
                        gemm_plan_t* out) {
  return gemm_plan_op(h, GEMM_OP_N, GEMM_OP_N, M, N, K, A, lda, B, ldb, C, ldc, dtype, out);
}

gemm_status_t gemm_run_op(gemm_handle_t h, gemm_op_t op_a, gemm_op_t op_b, int64_t M, int64_t N, int64_t K,
                          const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                          gemm_dtype_t dtype, void* stream) {
  if (!is_live(h)) return GEMM_ERR_INVALID_ARG;
  gemm_plan_t p;
  gemm_status_t st = plan_impl(h, (int)op_a, (int)op_b, M, N, K, A, lda, B, ldb, C, ldc, (int)dtype, &p);
  if (st != GEMM_OK) return st;
  const bool ta = op_a == GEMM_OP_T, tb = op_b == GEMM_OP_T;
  static const bool log = std::getenv("TGEMM_LOG") != nullptr;
  if (log)
    std::fprintf(stderr,
                 "tgemm: op=%c%c M=%lld N=%lld K=%lld dtype=%d kernel=%d tile=%dx%dx%d threads=%d vec=%d grid=%lld "
                 "split_k=%d\n",
                 ta ? 'T' : 'N', tb ? 'T' : 'N', (long long)M, (long long)N, (long long)K, (int)dtype, p.kernel,
                 p.tile_m, p.tile_n, p.tile_k, p.threads, p.vector_loads, (long long)p.grid, p.split_k);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  switch (p.kernel) {
    case 0: return GEMM_OK;
    case 1: e = tg::launch_zero_fill(C, M, N, ldc, out_bytes(dtype), s); break;
    case 2: {
      tg::I32Args a;
      a.A = (const int32_t*)A;
      a.B = (const int32_t*)B;
      a.C = (int32_t*)C;
      a.M = (int)M;
      a.N = (int)N;
      a.K = (int)K;
      a.sa_m = ta ? 1 : lda;
      a.sa_k = ta ? lda : 1;
      a.sb_k = tb ? 1 : ldb;
      a.sb_n = tb ? ldb : 1;
      a.ldc = ldc;
      a.tm = p.tile_m;
      a.tn = p.tile_n;
      a.tk = p.tile_k;
      a.tiles_n = (int)cdiv(N, p.tile_n);
      e = tg::launch_i32(a, s, p.grid, p.threads, p.lds_bytes);
      break;
    }
    default: {
      const int splits = p.split_k > 1 ? p.split_k : 1;
      if (splits > 1) {
        const size_t need = (size_t)splits * (size_t)M * (size_t)N * sizeof(float);
        if (h->ws_bytes < need) {
          if (h->ws != nullptr) {
            if (hipFree(h->ws) != hipSuccess) return GEMM_ERR_HIP;
            h->ws = nullptr;
            h->ws_bytes = 0;
          }
          if (hipMalloc(&h->ws, need) != hipSuccess) {
            (void)hipGetLastError();
            h->ws = nullptr;
            return GEMM_ERR_OUT_OF_MEMORY;
          }
          h->ws_bytes = need;
        }
      }
      tg::MacroArgs a;
      a.A = (const uint16_t*)A;
      a.B = (const uint16_t*)B;
      a.C = C;
      a.M = (int)M;
      a.N = (int)N;
      a.K = (int)K;
      a.lda = lda;
      a.ldb = ldb;
      a.ldc = ldc;
      a.tiles_m = (int)cdiv(M, p.tile_m);
      a.tiles_n = (int)cdiv(N, p.tile_n);
      a.group_m = a.tiles_m < 4 ? a.tiles_m : 4;
      const int64_t nk = cdiv(K, p.tile_k);
      a.kt_per_split = (int)cdiv(nk, splits);
      a.split_stride = (int64_t)M * N;
      if (p.kernel == 3) {
        e = tg::launch_small(a, in_kind(dtype), out_kind(dtype), p.vector_loads != 0, s, p.grid, ta, tb);
      } else if (splits == 1) {
        e = tg::launch_macro(find_macro(p.tile_m, p.tile_n, p.tile_k, p.stages), a, in_kind(dtype), out_kind(dtype),
                             p.vector_loads != 0, s, p.grid, 1, ta, tb);
      } else {
        // partial tiles (fp32, dense, ldc = N) into the workspace, then the ordered reduction
        tg::MacroArgs w = a;
        w.C = h->ws;
        w.ldc = N;
        e = tg::launch_macro(find_macro(p.tile_m, p.tile_n, p.tile_k, p.stages), w, in_kind(dtype), 0, p.vector_loads != 0, s,
                             p.grid, splits, ta, tb);
        if (e == hipSuccess)
          e = tg::launch_splitk_reduce((const float*)h->ws, splits, C, ldc, (int)M, (int)N, out_kind(dtype), s);
      }
      break;
    }
  }
  return e == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

gemm_status_t gemm_model(const gemm_plan_t* plan, int64_t M, int64_t N, int64_t K, gemm_dtype_t dtype,
                         gemm_model_t* out) {
  if (plan == nullptr || out == nullptr) return GEMM_ERR_INVALID_ARG;
  const int d = (int)dtype;
  if (d < GEMM_I32_I32 || d > GEMM_F16_F16) return GEMM_ERR_UNSUPPORTED_DTYPE;
  if (M < 0 || N < 0 || K < 0) return GEMM_ERR_INVALID_ARG;
  const gemm_plan_t& p = *plan;
  if (p.kernel < 0 || p.kernel > 4) return GEMM_ERR_INVALID_ARG;
  gemm_model_t m;
  std::memset(&m, 0, sizeof(m));
  const double s_in = d == GEMM_I32_I32 ? 4.0 : 2.0, s_out = (double)out_bytes(d);
  const double dM = (double)M, dN = (double)N, dK = (double)K;
  m.flops = 2.0 * dM * dN * dK;
  m.compulsory_bytes = s_in * (dM * dK + dK * dN) + s_out * dM * dN;
  if (M > 0 && N > 0) m.bytes_c = s_out * dM * dN;  // the zero fill (K = 0) writes C too
  if (p.kernel >= 2) {
    if (p.tile_m <= 0 || p.tile_n <= 0 || p.tile_k <= 0 || p.split_k < 1) return GEMM_ERR_INVALID_ARG;
    const int64_t tm = cdiv(M, p.tile_m), tn = cdiv(N, p.tile_n), nk = cdiv(K, p.tile_k);
    m.tiles = tm * tn;
    m.k_steps = nk;
    m.bytes_a = s_in * dM * dK * (double)tn;
    m.bytes_b = s_in * dK * dN * (double)tm;
    m.footprint_bytes = (int64_t)(s_in * (p.tile_m * p.tile_k + p.tile_k * p.tile_n)) + 4LL * p.tile_m * p.tile_n;
    m.lds_bytes = p.lds_bytes;
    const double tile_mn = (double)p.tile_m * p.tile_n * (double)m.tiles;
    if (p.kernel == 2) {
      m.executed_flops = 2.0 * tile_mn * dK;  // every thread of a tile runs the actual K range
    } else if (p.kernel == 3) {
      m.executed_flops = 2.0 * tile_mn * (double)(nk * p.tile_k);
    } else {
      // per K-slice: its K-tiles, plus the zero K-tiles prepended to make their number
      // a multiple of the stage count
      const int64_t per = cdiv(nk, p.split_k);
      const int64_t ns = p.stages > 0 ? p.stages : 2;
      double steps = 0;
      for (int64_t lo = 0; lo < nk; lo += per) {
        const int64_t n = (nk - lo) < per ? (nk - lo) : per;
        steps += (double)(n + (ns - n % ns) % ns);
      }
      m.executed_flops = 2.0 * tile_mn * steps * p.tile_k;
    }
    if (p.split_k > 1) m.bytes_workspace = 2.0 * 4.0 * (double)p.split_k * dM * dN;
  }
  *out = m;
  return GEMM_OK;
}

gemm_status_t gemm_run(gemm_handle_t h, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                       const void* B, int64_t ldb, void* C, int64_t ldc, gemm_dtype_t dtype, void* stream) {
  return gemm_run_op(h, GEMM_OP_N, GEMM_OP_N, M, N, K, A, lda, B, ldb, C, ldc, dtype, stream);
}

}  // extern "C"
