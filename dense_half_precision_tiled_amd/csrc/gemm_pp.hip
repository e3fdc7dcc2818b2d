// gemm_pp.hip -- instantiations of the ping-pong kernel template
// (gemm_pp_kernel.h): row-major and column-major B, plain and general
// epilogue.
#include "gemm_pp_kernel.h"

namespace dhpt {

hipError_t launch_pp(int ph, const Problem& p, int group_m, hipStream_t s) {
    if (ph == 2) {
        if (p.transB)
            return p.epi ? pp::launch_family<true, true, 2>(p, group_m, s) : pp::launch_family<true, false, 2>(p, group_m, s);
        return p.epi ? pp::launch_family<false, true, 2>(p, group_m, s) : pp::launch_family<false, false, 2>(p, group_m, s);
    }
    if (p.transB)
        return p.epi ? pp::launch_family<true, true, 4>(p, group_m, s) : pp::launch_family<true, false, 4>(p, group_m, s);
    return p.epi ? pp::launch_family<false, true, 4>(p, group_m, s) : pp::launch_family<false, false, 4>(p, group_m, s);
}

}  // namespace dhpt
