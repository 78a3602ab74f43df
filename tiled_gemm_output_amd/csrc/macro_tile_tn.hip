// macro_tile_tn.hip -- macro-tile GEMM instantiations for C = A^T @ B (A supplied as K x M).
#include "macro_tile_kernel.h"

namespace tg {

hipError_t launch_macro_tn(int shape, const MacroArgs& a, int in, int out, bool vec, hipStream_t s, int64_t grid,
                           int splits) {
  return launch_layout<true, false>(shape, a, in, out, vec, s, grid, splits);
}

}  // namespace tg
