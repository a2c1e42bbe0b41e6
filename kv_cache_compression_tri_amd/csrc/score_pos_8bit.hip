// Key scoring at explicit positions for 8-bit (fp8 or int8) pre-RoPE keys (the kernel is in
// score_kernel.h).
#include "score_kernel.h"

namespace tri {

hipError_t launch_score_pos_8bit(const ScoreParams& p, int G_eff, int dtype, bool interleaved, bool paged,
                                 int grid, hipStream_t stream) {
  return dtype == 3 ? launch_groups<3, false, false, true>(p, G_eff, interleaved, paged, grid, stream)
                    : launch_groups<2, false, false, true>(p, G_eff, interleaved, paged, grid, stream);
}

}  // namespace tri
