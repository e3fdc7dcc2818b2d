// gemm_dl_tn_epi.hip -- instantiations of the direct-to-LDS kernel template:
// column-major B (the TN layout), general epilogue.
// One translation unit per family so the build compiles them in parallel.
#include "gemm_dl_kernel.h"

namespace dhpt {

hipError_t launch_dl_tn_epi(int tile, int fd, int edge, const Problem& p, int group_m, hipStream_t s) {
    if (fd != 2) return hipErrorInvalidValue;
    return dl::launch_family<2, true, true>(tile, edge, p, group_m, s);
}

}  // namespace dhpt
