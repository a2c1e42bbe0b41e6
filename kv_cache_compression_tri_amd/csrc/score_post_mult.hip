// Multiplicative score form (phase-only cosine series times the centre and key norms) for
// float32 / bfloat16 keys already rotated by RoPE (the kernel is in score_kernel.h).
#include "score_kernel.h"

namespace tri {

hipError_t launch_score_post_mult(const ScoreParams& p, int G_eff, int dtype, bool interleaved, bool paged, int grid,
                  hipStream_t stream) {
  return dtype == 1 ? launch_groups<1, true, true>(p, G_eff, interleaved, paged, grid, stream)
                    : launch_groups<0, true, true>(p, G_eff, interleaved, paged, grid, stream);
}

}  // namespace tri
