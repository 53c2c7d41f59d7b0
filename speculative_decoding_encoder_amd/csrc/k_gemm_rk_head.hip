// Register-tiled GEMM instances for the tied LM head and the drafter's
// projections; tall-block instances for the LM head, the drafter's QKV and
// the history K/V projection.
#include "gemm_rk.h"
#include "gemm_tl.h"

namespace wf {

hipError_t launch_gemm_rk_c(int role, const GemmArgs &a, int mb, int nb, hipStream_t st) {
    switch (role) {
        case ROLE_LM_HEAD: return launch_rk_role<ROLE_LM_HEAD>(a, mb, nb, st);
        case ROLE_DRAFT_QKV: return launch_rk_role<ROLE_DRAFT_QKV>(a, mb, nb, st);
        case ROLE_HIST: return launch_rk_role<ROLE_HIST>(a, mb, nb, st);
        case ROLE_HIST_KV: return launch_rk_role<ROLE_HIST_KV>(a, mb, nb, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_tl_c(int role, const GemmArgs &a, int mb, hipStream_t st) {
    switch (role) {
        case ROLE_LM_HEAD: return launch_tl<ROLE_LM_HEAD>(a, mb, st);
        case ROLE_DRAFT_QKV: return launch_tl<ROLE_DRAFT_QKV>(a, mb, st);
        case ROLE_HIST_KV: return launch_tl<ROLE_HIST_KV>(a, mb, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace wf
