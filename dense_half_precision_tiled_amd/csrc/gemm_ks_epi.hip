// gemm_ks_epi.hip -- instantiations of the k-split-across-waves kernel
// template with the general epilogue act(alpha*A.B + beta*C + bias).
#include "gemm_ks_kernel.h"

namespace dhpt {

hipError_t launch_ks_epi(int edge, const Problem& p, int group_m, hipStream_t s) {
    return p.transB ? ks::launch_family<true, true>(edge, p, group_m, s)
                    : ks::launch_family<false, true>(edge, p, group_m, s);
}

}  // namespace dhpt
