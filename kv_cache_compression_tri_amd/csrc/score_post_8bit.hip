// Key scoring for 8-bit caches (fp8 OCP E4M3 or int8 codes) of keys already rotated by RoPE
// (the kernel is in score_kernel.h).
#include "score_kernel.h"

namespace tri {

hipError_t launch_score_post_8bit(const ScoreParams& p, int G_eff, int dtype, bool interleaved, bool paged, int grid,
                  hipStream_t stream) {
  return dtype == 3 ? launch_groups<3, true>(p, G_eff, interleaved, paged, grid, stream)
                    : launch_groups<2, true>(p, G_eff, interleaved, paged, grid, stream);
}

}  // namespace tri
