// Launcher of the fused scoring and selection kernel (score_select_kernel in score_kernel.h) for
// one key type and layout; each score_select*.hip instantiates one, so they compile in parallel.
#pragma once
#include "score_kernel.h"

namespace tri {
namespace {

template <int DT, bool PAGED>
hipError_t launch_score_select_case(const ScoreParams& p, const SelectParams& s, int G_eff, bool interleaved,
                                    int64_t units, hipStream_t st) {
  const dim3 blk{kScoreWaves * 64, 1, 1}, grd{unsigned(units), 1, 1};
#define TRI_FUSED_CASE(GG)                                                                                   \
  case GG:                                                                                                   \
    if (interleaved) hipLaunchKernelGGL((score_select_kernel<GG, DT, true, PAGED>), grd, blk, 0, st, p, s);    \
    else hipLaunchKernelGGL((score_select_kernel<GG, DT, false, PAGED>), grd, blk, 0, st, p, s);              \
    return hipGetLastError();
  switch (G_eff) {
    TRI_FUSED_CASE(1)
    TRI_FUSED_CASE(2)
    TRI_FUSED_CASE(3)
    TRI_FUSED_CASE(4)
    TRI_FUSED_CASE(5)
    TRI_FUSED_CASE(6)
    TRI_FUSED_CASE(7)
    TRI_FUSED_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef TRI_FUSED_CASE
}

}  // namespace
}  // namespace tri
