// Register-tiled and tall-block GEMM instances for the MLP (fc1 with GELU, fc2 with the residual).
#include "gemm_rk.h"
#include "gemm_tl.h"

namespace wf {

hipError_t launch_gemm_rk_b(int role, const GemmArgs &a, int mb, int nb, hipStream_t st) {
    switch (role) {
        case ROLE_FC1: return launch_rk_role<ROLE_FC1>(a, mb, nb, st);
        case ROLE_FC2: return launch_rk_role<ROLE_FC2>(a, mb, nb, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_tl_b(int role, const GemmArgs &a, int mb, hipStream_t st) {
    switch (role) {
        case ROLE_FC1: return launch_tl<ROLE_FC1>(a, mb, st);
        case ROLE_FC2: return launch_tl<ROLE_FC2>(a, mb, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace wf
