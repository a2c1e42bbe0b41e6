// Fused scoring and selection, dense float32 caches (dispatch in score_select.hip).
#include "score_select.h"

namespace tri {

hipError_t launch_score_select_f32(const ScoreParams& p, const SelectParams& s, int G_eff, bool interleaved,
                                   int64_t units, hipStream_t stream) {
  return launch_score_select_case<0, false>(p, s, G_eff, interleaved, units, stream);
}

}  // namespace tri
