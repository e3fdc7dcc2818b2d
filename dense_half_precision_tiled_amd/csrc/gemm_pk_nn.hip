// gemm_pk_nn.hip -- instantiations of the persistent 256x256 kernel of
// gemm_dl_kernel.h: row-major B, plain epilogue (C = A.B).
// One translation unit per family so the build compiles them in parallel.
#include "gemm_dl_kernel.h"

namespace dhpt {

hipError_t launch_pk_nn(int edge, const Problem& p, int group_m, hipStream_t s) {
    return dl::launch_persist_family<false, false>(edge, p, group_m, s);
}

}  // namespace dhpt
