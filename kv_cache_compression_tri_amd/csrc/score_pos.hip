// Key scoring for pre-RoPE caches whose keys sit at explicit positions (a cache compacted
// before: its slots no longer equal positions), float32 / bfloat16 keys, and the dispatch
// to the 8-bit unit; the kernel is in score_kernel.h.
#include "score_kernel.h"

namespace tri {

hipError_t launch_score_pos(const ScoreParams& p, int G_eff, int dtype, bool interleaved, bool paged, int grid,
                            hipStream_t stream) {
  switch (dtype) {
    case 0: return launch_groups<0, false, false, true>(p, G_eff, interleaved, paged, grid, stream);
    case 1: return launch_groups<1, false, false, true>(p, G_eff, interleaved, paged, grid, stream);
    default: return launch_score_pos_8bit(p, G_eff, dtype, interleaved, paged, grid, stream);
  }
}

}  // namespace tri
