// Fused scoring and selection (score_select_kernel in score_kernel.h): bfloat16 keys here,
// float32 keys in score_select_f32.hip (two translation units so they compile in parallel).
#include "score_kernel.h"

namespace tri {

template <int DT>
hipError_t launch_score_select_dt(const ScoreParams& p, const SelectParams& s, int G_eff, bool interleaved,
                                  int64_t units, hipStream_t st) {
  const dim3 blk{kScoreWaves * 64, 1, 1}, grd{unsigned(units), 1, 1};
#define TRI_FUSED_CASE(GG)                                                                          \
  case GG:                                                                                          \
    if (interleaved) hipLaunchKernelGGL((score_select_kernel<GG, DT, true>), grd, blk, 0, st, p, s);   \
    else hipLaunchKernelGGL((score_select_kernel<GG, DT, false>), grd, blk, 0, st, p, s);             \
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

#ifdef TRI_SCORE_SELECT_F32
hipError_t launch_score_select_f32(const ScoreParams& p, const SelectParams& s, int G_eff, bool interleaved,
                                   int64_t units, hipStream_t stream) {
  return launch_score_select_dt<0>(p, s, G_eff, interleaved, units, stream);
}
#else
hipError_t launch_score_select(const ScoreParams& p, const SelectParams& s, int G_eff, int dtype, bool interleaved,
                               int64_t units, hipStream_t stream) {
  if (dtype == 0) return launch_score_select_f32(p, s, G_eff, interleaved, units, stream);
  if (dtype == 1) return launch_score_select_dt<1>(p, s, G_eff, interleaved, units, stream);
  return hipErrorInvalidValue;
}
#endif

}  // namespace tri
