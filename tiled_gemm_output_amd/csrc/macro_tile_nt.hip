// macro_tile_nt.hip -- macro-tile GEMM instantiations for C = A @ B^T (B supplied as N x K).
#include "macro_tile_kernel.h"

namespace tg {

hipError_t launch_macro_nt(int shape, const MacroArgs& a, int in, int out, bool vec, hipStream_t s, int64_t grid,
                           int splits) {
  return launch_layout<false, true>(shape, a, in, out, vec, s, grid, splits);
}

}  // namespace tg
