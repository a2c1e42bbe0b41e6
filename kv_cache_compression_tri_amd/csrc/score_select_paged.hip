// Fused scoring and selection, paged bfloat16 caches (dispatch in score_select.hip).
#include "score_select.h"

namespace tri {

hipError_t launch_score_select_bf16_paged(const ScoreParams& p, const SelectParams& s, int G_eff, bool interleaved,
                                          int64_t units, hipStream_t stream) {
  return launch_score_select_case<1, true>(p, s, G_eff, interleaved, units, stream);
}

}  // namespace tri
