// Register-tiled and tall-block GEMM instances for the attention projections (QKV with the KV append, O, cross Q).
#include "gemm_rk.h"
#include "gemm_tl.h"

namespace wf {

hipError_t launch_gemm_rk_a(int role, const GemmArgs &a, int mb, int nb, hipStream_t st) {
    switch (role) {
        case ROLE_QKV: return launch_rk_role<ROLE_QKV>(a, mb, nb, st);
        case ROLE_OPROJ: return launch_rk_role<ROLE_OPROJ>(a, mb, nb, st);
        case ROLE_CROSS_Q: return launch_rk_role<ROLE_CROSS_Q>(a, mb, nb, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_tl_a(int role, const GemmArgs &a, int mb, hipStream_t st) {
    switch (role) {
        case ROLE_QKV: return launch_tl<ROLE_QKV>(a, mb, st);
        case ROLE_OPROJ: return launch_tl<ROLE_OPROJ>(a, mb, st);
        case ROLE_CROSS_Q: return launch_tl<ROLE_CROSS_Q>(a, mb, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace wf
