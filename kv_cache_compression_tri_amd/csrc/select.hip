// Top-B selection kernel of the TriAttention compression pass (gfx950): one workgroup per
// unit; the selection itself is in select_core.h.
#include "select_core.h"

namespace tri {
namespace {

template <bool kStream, int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) void select_kernel(const SelectParams P) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[kLevels][kBins];   // read as 16-byte pieces
  __shared__ uint32_t sub[kSubHist * kBins];
  __shared__ SelSmall<NT / 64> sm;
  const SelLds<NT / 64> S{hist, sub, &sm};
  select_unit<NT, kResident, kStream, false>(P, blockIdx.x, S, nullptr);
}

}  // namespace

hipError_t launch_select(const SelectParams& p, int64_t n_units, hipStream_t stream) {
  // units longer than the register-resident capacity re-read their scores on every sweep
  if (p.score_stride <= kResident)
    hipLaunchKernelGGL((select_kernel<false, kResThreads>), dim3(unsigned(n_units)), dim3(kResThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((select_kernel<true, kStreamThreads>), dim3(unsigned(n_units)), dim3(kStreamThreads), 0,
                       stream, p);
  return hipGetLastError();
}

}  // namespace tri
