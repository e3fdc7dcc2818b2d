// gemm_ks.hip -- instantiations of the k-split-across-waves kernel template
// with the plain epilogue (C = A.B): row-major and column-major B.
#include "gemm_ks_kernel.h"

namespace dhpt {

hipError_t launch_ks(int edge, const Problem& p, int group_m, hipStream_t s) {
    return p.transB ? ks::launch_family<true, false>(edge, p, group_m, s)
                    : ks::launch_family<false, false>(edge, p, group_m, s);
}

}  // namespace dhpt
