// Key scoring on the bf16 matrix cores (kernel in score_mfma.h): bfloat16 keys before RoPE at
// consecutive positions, additive form, max over 6..8 query heads per KV head.
#include "score_mfma.h"

namespace tri {

// Its time does not depend on the group size; the vector kernel's grows with it.  Same-process
// timings of the 32K pass's scoring (36 x 8 units of 32768 bf16 keys): vector kernel 0.52 /
// 0.58 / 0.62 / 0.71 ms at G = 4 / 5 / 6 / 8, this kernel 0.59 ms at every G; the 128K pass
// (G = 7) 1.04 -> 0.93 ms.  So it takes G >= 6.
constexpr int kMfmaMinGroup = 6;

bool score_mfma_applies(int G_eff, int dtype, bool post, bool mult, bool positions, bool reduce_mean) {
  return dtype == 1 && !post && !mult && !positions && !reduce_mean && G_eff >= kMfmaMinGroup &&
         G_eff <= kMaxGroup;
}

hipError_t launch_score_mfma(const ScoreParams& p, bool interleaved, bool paged, int grid, hipStream_t stream) {
  if (interleaved) return paged ? launch_mfma_case<true, true>(p, grid, stream) : launch_mfma_case<true, false>(p, grid, stream);
  return paged ? launch_mfma_case<false, true>(p, grid, stream) : launch_mfma_case<false, false>(p, grid, stream);
}

}  // namespace tri
