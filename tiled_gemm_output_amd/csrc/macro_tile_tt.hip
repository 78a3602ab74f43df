// macro_tile_tt.hip -- macro-tile GEMM instantiations for C = A^T @ B^T (A supplied as K x M, B as N x K).
#include "macro_tile_kernel.h"

namespace tg {

hipError_t launch_macro_tt(int shape, const MacroArgs& a, int in, int out, bool vec, hipStream_t s, int64_t grid,
                           int splits) {
  return launch_layout<true, true>(shape, a, in, out, vec, s, grid, splits);
}

}  // namespace tg
