// macro_tile_inst_nt_rest.hip -- macro-tile GEMM kernels for C = A @ B^T (B supplied as N x K), the other tiles.
#include "macro_tile_kernel.h"

namespace tg {

template hipError_t launch_dtype<Cfg256x128, false, true>(const MacroArgs&, int, int, bool, hipStream_t, int64_t, int);
template hipError_t launch_dtype<Cfg128x128, false, true>(const MacroArgs&, int, int, bool, hipStream_t, int64_t, int);
template hipError_t launch_dtype<Cfg64x64, false, true>(const MacroArgs&, int, int, bool, hipStream_t, int64_t, int);
template hipError_t launch_dtype<Cfg128x128s4, false, true>(const MacroArgs&, int, int, bool, hipStream_t, int64_t, int);
template hipError_t launch_dtype<Cfg64x64s4, false, true>(const MacroArgs&, int, int, bool, hipStream_t, int64_t, int);

}  // namespace tg
