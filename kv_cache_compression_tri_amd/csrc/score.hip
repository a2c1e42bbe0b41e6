// Key scoring, pre-RoPE float32 / bfloat16 keys, and the dispatch over the instantiating
// translation units (the vector kernel is in score_kernel.h, the matrix-core one in
// score_mx.h).
#include "score_kernel.h"

namespace tri {

hipError_t launch_score(const ScoreParams& p, int G_eff, int dtype, bool interleaved, bool paged,
                        bool post, bool mult, int grid, hipStream_t stream) {
  if (score_mx_applies(G_eff, dtype, post, mult, p.pos != nullptr, p.reduce_mean != 0))
    return launch_score_mx(p, G_eff, dtype, interleaved, paged, post, grid, stream);
  if (p.pos && !post) return launch_score_pos(p, G_eff, dtype, interleaved, paged, grid, stream);
  if (mult) {
    if (dtype >= 2)
      return post ? launch_score_post_mult_8bit(p, G_eff, dtype, interleaved, paged, grid, stream)
                  : launch_score_mult_8bit(p, G_eff, dtype, interleaved, paged, grid, stream);
    return post ? launch_score_post_mult(p, G_eff, dtype, interleaved, paged, grid, stream)
                : launch_score_mult(p, G_eff, dtype, interleaved, paged, grid, stream);
  }
  if (dtype >= 2)
    return post ? launch_score_post_8bit(p, G_eff, dtype, interleaved, paged, grid, stream)
                : launch_score_8bit(p, G_eff, dtype, interleaved, paged, grid, stream);
  if (post) return launch_score_post(p, G_eff, dtype, interleaved, paged, grid, stream);
  return dtype == 1 ? launch_groups<1, false>(p, G_eff, interleaved, paged, grid, stream)
                    : launch_groups<0, false>(p, G_eff, interleaved, paged, grid, stream);
}

}  // namespace tri
