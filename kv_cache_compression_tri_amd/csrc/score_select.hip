// Fused scoring and selection: dense bfloat16 caches, and the dispatch over the translation
// units of the other key types and layouts (score_select_*.hip).
#include "score_select.h"

namespace tri {

hipError_t launch_score_select(const ScoreParams& p, const SelectParams& s, int G_eff, int dtype, bool interleaved,
                               bool paged, int64_t units, hipStream_t stream) {
  if (dtype == 1) {
    return paged ? launch_score_select_bf16_paged(p, s, G_eff, interleaved, units, stream)
                 : launch_score_select_case<1, false>(p, s, G_eff, interleaved, units, stream);
  }
  if (dtype == 0) {
    return paged ? launch_score_select_f32_paged(p, s, G_eff, interleaved, units, stream)
                 : launch_score_select_f32(p, s, G_eff, interleaved, units, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace tri
