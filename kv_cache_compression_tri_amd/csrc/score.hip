// Key scoring for caches that hold pre-RoPE keys (the kernel is in score_kernel.h).
#include "score_kernel.h"

namespace tri {

hipError_t launch_score(const ScoreParams& p, int G_eff, bool bf16, bool interleaved, bool paged,
                        bool post, int grid, hipStream_t stream) {
  if (post) return launch_score_post(p, G_eff, bf16, interleaved, paged, grid, stream);
  return launch_groups<false>(p, G_eff, bf16, interleaved, paged, grid, stream);
}

}  // namespace tri
