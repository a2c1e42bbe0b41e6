// Key scoring on the bf16 matrix cores (kernel in score_mx.h): bfloat16 keys before RoPE at
// consecutive positions or cached after RoPE, additive form, max over 4..8 query heads per KV
// head.  Dense caches
// here, paged ones in score_mx_paged.hip (two translation units so they compile in parallel).
#include "score_mx.h"

namespace tri {

// The vector kernel's time grows with the group, this kernel's does not: same-process medians of
// the 32K pass's scoring (36 x 8 units of 32768 bfloat16 keys; group statistics of that
// workload, G changed), vector / matrix cores: G = 3 0.456 / 0.474 ms, G = 4 0.482 / 0.478,
// G = 5 0.540 / 0.475, G = 6 0.600 / 0.478; the 128K pass (G = 7) 0.981 / 0.754 ms; the paged
// pass of 64 sequences (G = 4) 20.30 / 19.84 ms.  So it takes G >= 4.  Keys cached after RoPE
// (no rotation; the trig products take the raw keys), same measure on two boxes: G = 2
// 0.407 / 0.433 ms, G = 3 0.385 / 0.437, G = 4 0.423 / 0.429 and 0.448 / 0.438, G = 5
// 0.490 / 0.438, G = 6 0.513 / 0.440, 128K 0.823 / 0.629 and 0.847 / 0.677 ms, paged 16.79 /
// 15.17 and 17.70 / 16.82 ms: the same rule.
constexpr int kMxMinGroup = 4;

// 8-bit keys cached after RoPE (fp8 / int8 caches of the 32K pass's shape, same measure): the
// vector kernel takes G = 2 0.292, G = 3 0.312, G = 4 0.361 / 0.371 (fp8 / int8), G = 7 0.512 ms,
// this kernel 0.25-0.26 ms at every G (4: 0.252 / 0.256, 7: 0.254), so it takes G >= 2.
constexpr int kMxMinGroup8 = 2;

bool score_mx_applies(int G_eff, int dtype, bool post, bool mult, bool positions, bool reduce_mean) {
  // keys cached after RoPE carry their positions, so explicit positions are not read for them; 8-bit
  // keys take this kernel only after RoPE (before RoPE their rotation and split cost what the
  // products save)
  if (mult || reduce_mean || G_eff > kMaxGroup) return false;
  if (dtype == 2 || dtype == 3) return post && G_eff >= kMxMinGroup8;
  return dtype == 1 && (post || !positions) && G_eff >= kMxMinGroup;
}

hipError_t launch_score_mx(const ScoreParams& p, int G_eff, int dtype, bool interleaved, bool paged, bool post,
                           int grid, hipStream_t stream) {
  if (dtype != 1) return launch_score_mx_post_8bit(p, G_eff, dtype, interleaved, paged, grid, stream);
  if (post) return paged ? launch_score_mx_post_paged(p, G_eff, interleaved, grid, stream)
                         : launch_score_mx_post(p, G_eff, interleaved, grid, stream);
  if (paged) return launch_score_mx_paged(p, G_eff, interleaved, grid, stream);
#define TRI_MX_CASE(GG)                                                                   \
  case GG:                                                                                \
    return interleaved ? launch_mx_case<GG, true, false, false>(p, grid, stream)                 \
                       : launch_mx_case<GG, false, false, false>(p, grid, stream);
  switch (G_eff) {
    TRI_MX_CASE(4)
    TRI_MX_CASE(5)
    TRI_MX_CASE(6)
    TRI_MX_CASE(7)
    TRI_MX_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef TRI_MX_CASE
}

}  // namespace tri
