// gemm_dl_nn.hip -- instantiations of the direct-to-LDS kernel template:
// row-major B, plain epilogue (C = A.B): prefetch distance 1 and 2.
// One translation unit per family so the build compiles them in parallel.
#include "gemm_dl_kernel.h"

namespace dhpt {

hipError_t launch_dl_nn(int tile, int fd, int edge, const Problem& p, int group_m, hipStream_t s) {
    if (fd == 1) return dl::launch_family<1, false, false>(tile, edge, p, group_m, s);
    return dl::launch_family<2, false, false>(tile, edge, p, group_m, s);
}

}  // namespace dhpt
