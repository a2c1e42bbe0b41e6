// Key scoring for fp8 (OCP E4M3) caches of keys already rotated by RoPE (the kernel is in
// score_kernel.h).
#include "score_kernel.h"

namespace tri {

hipError_t launch_score_post_fp8(const ScoreParams& p, int G_eff, bool interleaved, bool paged, int grid,
                                 hipStream_t stream) {
  return launch_groups<2, true>(p, G_eff, interleaved, paged, grid, stream);
}

}  // namespace tri
