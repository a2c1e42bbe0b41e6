// Key scoring for caches that hold keys already rotated by RoPE at their positions (the
// kernel is in score_kernel.h; a translation unit of its own keeps compile times short).
#include "score_kernel.h"

namespace tri {

hipError_t launch_score_post(const ScoreParams& p, int G_eff, bool bf16, bool interleaved, bool paged,
                             int grid, hipStream_t stream) {
  return launch_groups<true>(p, G_eff, bf16, interleaved, paged, grid, stream);
}

}  // namespace tri
