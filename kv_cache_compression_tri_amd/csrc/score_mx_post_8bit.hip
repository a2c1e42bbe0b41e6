// Key scoring on the bf16 matrix cores (kernel in score_mx.h) for fp8 (OCP E4M3) and int8 caches
// that hold keys already rotated by RoPE, dense and paged.  The dispatch rule is in score_mx.hip.
#include "score_mx.h"

namespace tri {

template <bool PAGED>
static hipError_t launch_8bit(const ScoreParams& p, int G_eff, int dtype, bool interleaved, int grid,
                              hipStream_t stream) {
#define TRI_MX_CASE(GG)                                                                              \
  case GG:                                                                                           \
    if (dtype == 2)                                                                                  \
      return interleaved ? launch_mx_case<GG, true, PAGED, true, 2>(p, grid, stream)                 \
                         : launch_mx_case<GG, false, PAGED, true, 2>(p, grid, stream);               \
    return interleaved ? launch_mx_case<GG, true, PAGED, true, 3>(p, grid, stream)                   \
                       : launch_mx_case<GG, false, PAGED, true, 3>(p, grid, stream);
  switch (G_eff) {
    TRI_MX_CASE(2)
    TRI_MX_CASE(3)
    TRI_MX_CASE(4)
    TRI_MX_CASE(5)
    TRI_MX_CASE(6)
    TRI_MX_CASE(7)
    TRI_MX_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef TRI_MX_CASE
}

hipError_t launch_score_mx_post_8bit(const ScoreParams& p, int G_eff, int dtype, bool interleaved, bool paged,
                                     int grid, hipStream_t stream) {
  if (dtype != 2 && dtype != 3) return hipErrorInvalidValue;
  return paged ? launch_8bit<true>(p, G_eff, dtype, interleaved, grid, stream)
               : launch_8bit<false>(p, G_eff, dtype, interleaved, grid, stream);
}

}  // namespace tri
