// Calibration kernel: per-band query statistics from pre-RoPE query samples (gfx950).
//
// The centre of a head is the mean of its pre-RoPE queries over a calibration set
// ("TriAttention: Trigonometric KV Compression for Efficient Long Reasoning", section "Key
// Concepts"); the statistics are a property of the model's weights ("TriAttention:
// trigonometric KV cache compression for long reasoning", section "Calibration statistics
// are tied to a specific model").  Per (layer, query head, band f):
//   center[f]   = mean_n q_{n,f}      (complex band value, re/im)
//   mean_abs[f] = mean_n |q_{n,f}|
// One workgroup per (layer, head); lane f of each wave owns band f, the 4 waves stride over
// the samples, and the partial float64 sums are combined in LDS.
#include "tri_internal.h"

namespace tri {
namespace {

constexpr int kCalibThreads = 256;

template <bool BF16, bool IL>
__global__ __launch_bounds__(kCalibThreads) void calib_kernel(const CalibParams P) {
  __shared__ double part[3][kCalibThreads];
  const int tid = threadIdx.x;
  const int f = tid & 63, sub = tid >> 6;
  const int64_t lh = blockIdx.x;
  const int64_t stride = int64_t(P.n_layer) * P.n_qh * kHeadDim;
  const int ia = IL ? 2 * f : f, ib = IL ? 2 * f + 1 : f + kBands;
  double sr = 0.0, si = 0.0, sa = 0.0;
  for (int64_t i = sub; i < P.n; i += kCalibThreads / 64) {
    const int64_t base = i * stride + lh * kHeadDim;
    double a, b;
    if (BF16) {
      const uint16_t* q = static_cast<const uint16_t*>(P.q);
      a = __uint_as_float(uint32_t(q[base + ia]) << 16);
      b = __uint_as_float(uint32_t(q[base + ib]) << 16);
    } else {
      const float* q = static_cast<const float*>(P.q);
      a = q[base + ia];
      b = q[base + ib];
    }
    sr += a;
    si += b;
    sa += sqrt(a * a + b * b);
  }
  part[0][tid] = sr;
  part[1][tid] = si;
  part[2][tid] = sa;
  __syncthreads();
  if (sub == 0) {
    for (int w = 1; w < kCalibThreads / 64; ++w) {
      sr += part[0][w * 64 + f];
      si += part[1][w * 64 + f];
      sa += part[2][w * 64 + f];
    }
    const double inv = 1.0 / double(P.n);
    P.center[(lh * kBands + f) * 2 + 0] = float(sr * inv);
    P.center[(lh * kBands + f) * 2 + 1] = float(si * inv);
    P.mean_abs[lh * kBands + f] = float(sa * inv);
  }
}

}  // namespace

hipError_t launch_calib(const CalibParams& p, bool bf16, bool interleaved, hipStream_t stream) {
  const dim3 grid(unsigned(int64_t(p.n_layer) * p.n_qh)), blk(kCalibThreads);
  if (bf16) {
    if (interleaved) hipLaunchKernelGGL((calib_kernel<true, true>), grid, blk, 0, stream, p);
    else hipLaunchKernelGGL((calib_kernel<true, false>), grid, blk, 0, stream, p);
  } else {
    if (interleaved) hipLaunchKernelGGL((calib_kernel<false, true>), grid, blk, 0, stream, p);
    else hipLaunchKernelGGL((calib_kernel<false, false>), grid, blk, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace tri
