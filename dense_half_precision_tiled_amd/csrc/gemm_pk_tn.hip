// gemm_pk_tn.hip -- instantiations of the persistent 256x256 kernel of
// gemm_dl_kernel.h: column-major B, plain epilogue.
// One translation unit per family so the build compiles them in parallel.
#include "gemm_dl_kernel.h"

namespace dhpt {

hipError_t launch_pk_tn(int edge, const Problem& p, int group_m, hipStream_t s) {
    return dl::launch_persist_family<true, false>(edge, p, group_m, s);
}

}  // namespace dhpt
