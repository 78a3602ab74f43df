// macro_tile_inst_tn_big.hip -- macro-tile GEMM kernels for C = A^T @ B (A supplied as K x M), the 256x256 tile.
#include "macro_tile_kernel.h"

namespace tg {

template hipError_t launch_dtype<Cfg256x256w8, true, false>(const MacroArgs&, int, int, bool, hipStream_t, int64_t, int);

}  // namespace tg
