// macro_tile_inst_tn_big3.hip -- macro-tile GEMM kernels for C = A^T @ B (A supplied as K x M), the 256x256 tile
// with A loaded three K-steps ahead.
#include "macro_tile_kernel.h"

namespace tg {

template hipError_t launch_dtype<Cfg256x256w8a, true, false>(const MacroArgs&, int, int, bool, hipStream_t, int64_t, int);

}  // namespace tg
