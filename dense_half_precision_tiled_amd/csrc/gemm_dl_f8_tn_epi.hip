// gemm_dl_f8_tn_epi.hip -- instantiations of the direct-to-LDS kernel
// template for 8-bit float inputs (E4M3, E5M2): column-major B, general epilogue.
// One translation unit per family so the build compiles them in parallel.
#include "gemm_dl_kernel.h"

namespace dhpt {

hipError_t launch_dl_f8_tn_epi(int tile, int edge, const Problem& p, int group_m, hipStream_t s) {
    return dl::launch_family8<true, true>(tile, edge, p, group_m, s);
}

}  // namespace dhpt
