// Key scoring on the bf16 matrix cores (kernel in score_mx.h) for bfloat16 caches that hold keys
// already rotated by RoPE, dense caches; paged ones in score_mx_post_paged.hip.  The dispatch rule
// is in score_mx.hip.
#include "score_mx.h"

namespace tri {

hipError_t launch_score_mx_post(const ScoreParams& p, int G_eff, bool interleaved, int grid, hipStream_t stream) {
#define TRI_MX_CASE(GG)                                                                   \
  case GG:                                                                                \
    return interleaved ? launch_mx_case<GG, true, false, true>(p, grid, stream)           \
                       : launch_mx_case<GG, false, false, true>(p, grid, stream);
  switch (G_eff) {
    TRI_MX_CASE(4)
    TRI_MX_CASE(5)
    TRI_MX_CASE(6)
    TRI_MX_CASE(7)
    TRI_MX_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef TRI_MX_CASE
}

}  // namespace tri
