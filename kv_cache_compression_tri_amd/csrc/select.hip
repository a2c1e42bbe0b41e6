// Top-B selection kernels of the TriAttention compression pass (gfx950): one workgroup per
// unit, or, for units longer than the register capacity and a caller's workspace, two stages
// over many workgroups (below); the selection itself is in select_core.h.
#include <algorithm>

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

// Tournament for units longer than kResident slots, which the single-workgroup kernel would
// stream from memory on every sweep with one CU per unit.  The candidates (all but the last
// W' = min(window, B) slots) are cut into runs of kResident slots; stage 1 selects each run's
// best B' = B - W' (one workgroup per run, register-resident) and keeps their slots and order
// keys; stage 2 selects the unit's best B' among those (register-resident: n_runs * B' <=
// kResident) and appends the window.  It is exact: a candidate among the unit's best B' by
// (score descending, slot ascending) has fewer than B' candidates before it in that order, so
// fewer than B' in its own run, and the runs' kept lists, concatenated in run order, are in
// slot order, so stage 2 breaks ties by slot as well.
struct TourParams {
  int32_t* cand_pos;     // [units][n_runs][B'] candidate slots
  uint32_t* cand_key;    // [units][n_runs][B'] their order keys
  int32_t n_runs;        // runs per unit: ceil(score_stride / kResident)
};

template <int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) void select_runs_kernel(const SelectParams P,
                                                                                             const TourParams T) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[kLevels][kBins];
  __shared__ uint32_t sub[kSubHist * kBins];
  __shared__ SelSmall<NT / 64> sm;
  const int64_t unit = blockIdx.x / T.n_runs;
  const int run = int(blockIdx.x - unit * T.n_runs);
  const int s = int(unit / P.units_per_seq);
  const int L = min(max(P.seq_len[s], 0), int(P.score_stride));
  const int B = P.budget;
  const int bp = B - min(P.window, B);
  const int ncand = L - min(P.window, B);
  const int start = run * kResident;
  if (L <= B || start >= ncand) return;   // stage 2 keeps every slot / no candidates in this run
  SelJob J;
  J.in = P.scores + unit * P.score_stride + start;
  J.L = min(kResident, ncand - start);
  J.B = bp;
  J.window = 0;
  const int64_t at = (unit * T.n_runs + run) * int64_t(bp);
  J.out = T.cand_pos + at;
  J.out_key = T.cand_key + at;
  J.pos_map = nullptr;
  J.base = start;
  J.kept_n = nullptr;
  const SelLds<NT / 64> S{hist, sub, &sm};
  select_job<NT, kResident, false, false>(J, S, nullptr);
}

template <int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) void select_final_kernel(const SelectParams P,
                                                                                              const TourParams T) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[kLevels][kBins];
  __shared__ uint32_t sub[kSubHist * kBins];
  __shared__ SelSmall<NT / 64> sm;
  const int64_t unit = blockIdx.x;
  const int s = int(unit / P.units_per_seq);
  const int L = min(max(P.seq_len[s], 0), int(P.score_stride));
  const int B = P.budget;
  const int w = min(P.window, B);
  const int bp = B - w;
  int32_t* out = P.kept + unit * int64_t(B);
  if (threadIdx.x == 0 && unit % P.units_per_seq == 0) P.kept_n[s] = min(L, B);
  if (L <= B) {
    for (int i = threadIdx.x; i < B; i += NT) out[i] = i < L ? i : -1;
    return;
  }
  const int ncand = L - w;
  const int runs = (ncand + kResident - 1) / kResident;
  const int last = ncand - (runs - 1) * kResident;
  SelJob J;
  const int64_t at = unit * T.n_runs * int64_t(bp);
  J.in = T.cand_key + at;
  J.L = (runs - 1) * bp + min(bp, last);
  J.B = bp;
  J.window = 0;
  J.out = out;
  J.out_key = nullptr;
  J.pos_map = T.cand_pos + at;
  J.base = 0;
  J.kept_n = nullptr;
  const SelLds<NT / 64> S{hist, sub, &sm};
  select_job<NT, kResident, false, false, true>(J, S, nullptr);
  for (int t = threadIdx.x; t < w; t += NT) out[bp + t] = ncand + t;   // the window, after every candidate
}

// runs per unit and whether the tournament takes this launch
int tour_runs(const SelectParams& p) {
  if (p.score_stride <= kResident) return 0;
  const int64_t runs = (p.score_stride + kResident - 1) / kResident;
  const int64_t bp = p.budget - std::min(p.window, p.budget);
  return (bp >= 1 && runs * bp <= kResident) ? int(runs) : 0;
}

}  // namespace

size_t select_workspace_bytes(const SelectParams& p, int64_t n_units) {
  const int runs = tour_runs(p);
  if (!runs) return 0;
  const int64_t bp = p.budget - std::min(p.window, p.budget);
  return size_t(n_units) * size_t(runs) * size_t(bp) * (sizeof(int32_t) + sizeof(uint32_t));
}

hipError_t launch_select(const SelectParams& p, int64_t n_units, void* ws, hipStream_t stream) {
  const int runs = tour_runs(p);
  if (ws && runs) {
    const int64_t bp = p.budget - std::min(p.window, p.budget);
    TourParams t;
    t.cand_pos = static_cast<int32_t*>(ws);
    t.cand_key = reinterpret_cast<uint32_t*>(t.cand_pos + n_units * runs * bp);
    t.n_runs = runs;
    hipLaunchKernelGGL((select_runs_kernel<kResThreads>), dim3(unsigned(n_units * runs)), dim3(kResThreads), 0, stream,
                       p, t);
    hipLaunchKernelGGL((select_final_kernel<kResThreads>), dim3(unsigned(n_units)), dim3(kResThreads), 0, stream, p,
                       t);
    return hipGetLastError();
  }
  // units longer than the register-resident capacity re-read their scores on every sweep
  if (p.score_stride <= kResident)
    hipLaunchKernelGGL((select_kernel<false, kResThreads>), dim3(unsigned(n_units)), dim3(kResThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((select_kernel<true, kStreamThreads>), dim3(unsigned(n_units)), dim3(kStreamThreads), 0,
                       stream, p);
  return hipGetLastError();
}

}  // namespace tri
