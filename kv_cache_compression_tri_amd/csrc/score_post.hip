// Key scoring for float32 / bfloat16 caches that hold keys already rotated by RoPE at their
// positions (the kernel is in score_kernel.h; separate translation units keep compiles short).
#include "score_kernel.h"

namespace tri {

hipError_t launch_score_post(const ScoreParams& p, int G_eff, int dtype, bool interleaved, bool paged,
                             int grid, hipStream_t stream) {
  return dtype == 1 ? launch_groups<1, true>(p, G_eff, interleaved, paged, grid, stream)
                    : launch_groups<0, true>(p, G_eff, interleaved, paged, grid, stream);
}

}  // namespace tri
