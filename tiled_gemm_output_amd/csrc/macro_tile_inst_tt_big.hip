// macro_tile_inst_tt_big.hip -- macro-tile GEMM kernels for C = A^T @ B^T, the 256x256 tile.
#include "macro_tile_kernel.h"

namespace tg {

template hipError_t launch_dtype<Cfg256x256w8, true, true>(const MacroArgs&, int, int, bool, hipStream_t, int64_t, int);

}  // namespace tg
