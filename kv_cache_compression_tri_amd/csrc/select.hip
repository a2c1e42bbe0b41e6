// Top-B selection kernel of the TriAttention compression pass (gfx950).
//
// Per unit (one workgroup): keep the last W' = min(window, budget) slots, then the best
// budget - W' of the remaining candidates ranked by (score descending, slot ascending), and
// write the kept slots in ascending order ("TriAttention: Trigonometric KV Compression for
// Efficient Long Reasoning", section "Core Mechanism": only the top-scoring keys are kept;
// "TriAttention: trigonometric KV cache compression for long reasoning", section "The KV
// budget is a runtime knob ...": the budget bounds the whole kept cache).
//
// Method: scores map to order-preserving 32-bit keys (NaN and -inf to the lowest key, -0 to
// +0).  Four radix passes of 8 bits over the candidates find the exact key tau of the
// (budget - W')-th best candidate and how many keys equal to tau must be taken
// (lowest slots first).  The histograms live in LDS; lanes of a wave that hit the same bin
// are merged with a ballot before the atomic add (scores of one head cluster in a few
// bins).  The ordered write uses one ballot + mbcnt per wave per tile and a workgroup scan
// of the per-wave counts, so the output is ascending without a sort.
#include "tri_internal.h"

namespace tri {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kTilesPerSeg = 64;   // groups per segment = kTilesPerSeg * waves = threads

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t b = __float_as_uint(x);
  if (x != x) return 0x007FFFFFu;              // NaN ranks as -inf
  if (b == 0x80000000u) b = 0u;                // -0 == +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
}

// Add 1 to hist[bin] for every active lane, merging the two most common bins of the wave.
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t bin, bool active, int lane) {
#pragma unroll
  for (int round = 0; round < 2; ++round) {
    const uint64_t m = __ballot(active);
    if (m == 0) return;
    const int leader = __ffsll((unsigned long long)m) - 1;
    const uint32_t b0 = __shfl(bin, leader);
    const bool same = active && bin == b0;
    const uint64_t sm = __ballot(same);
    if (lane == leader) atomicAdd(&hist[b0], uint32_t(__popcll(sm)));
    active = active && !same;
  }
  if (active) atomicAdd(&hist[bin], 1u);
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  return v;
}

// Exclusive scan of (a, b) across the workgroup; totals returned in ta, tb.
__device__ __forceinline__ void block_scan2(uint32_t& a, uint32_t& b, uint32_t& ta, uint32_t& tb,
                                            uint32_t* wa, uint32_t* wb, int lane, int wave) {
  const uint32_t ia = wave_incl_scan(a, lane), ib = wave_incl_scan(b, lane);
  if (lane == 63) {
    wa[wave] = ia;
    wb[wave] = ib;
  }
  __syncthreads();
  uint32_t pa = 0, pb = 0;
  ta = 0;
  tb = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const uint32_t x = wa[w], y = wb[w];
    if (w < wave) {
      pa += x;
      pb += y;
    }
    ta += x;
    tb += y;
  }
  a = pa + ia - a;
  b = pb + ib - b;
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(const SelectParams P) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t grp_a[kSelThreads], grp_b[kSelThreads];
  __shared__ uint32_t wsum_a[kSelWaves], wsum_b[kSelWaves];
  __shared__ uint32_t pick[2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t unit = blockIdx.x;
  const int s = int(unit / P.units_per_seq);
  const int L = min(max(P.seq_len[s], 0), int(P.score_stride));
  const int B = P.budget;
  const float* sc = P.scores + unit * P.score_stride;
  int32_t* out = P.kept + unit * int64_t(B);

  if (tid == 0 && unit % P.units_per_seq == 0) P.kept_n[s] = min(L, B);
  if (L <= B) {
    for (int i = tid; i < B; i += kSelThreads) out[i] = i < L ? i : -1;
    return;
  }
  const int w = min(P.window, B);
  const int ncand = L - w;
  const int need = B - w;

  // ---- radix select of the need-th largest candidate key ----------------------------
  uint32_t prefix = 0u, pmask = 0u;
  uint32_t remaining = uint32_t(need);
  if (need > 0) {
    const int span = (ncand + kSelThreads - 1) / kSelThreads * kSelThreads;
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0u;
      __syncthreads();
      for (int j = tid; j < span; j += kSelThreads) {
        const bool in = j < ncand;
        const uint32_t u = in ? order_key(sc[j]) : 0u;
        hist_add(hist, (u >> shift) & 255u, in && (u & pmask) == prefix, lane);
      }
      __syncthreads();
      if (wave == 0) {
        // lane holds bins 4*lane .. 4*lane+3; count candidates in higher bins
        uint32_t hb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) hb[i] = hist[4 * lane + i];
        const uint32_t lsum = hb[0] + hb[1] + hb[2] + hb[3];
        // suffix sum over lanes: reverse the lane order and scan
        const uint32_t rev = wave_incl_scan(__shfl(lsum, 63 - lane), lane);
        const uint32_t incl = __shfl(rev, 63 - lane);   // sum of lanes >= lane
        uint32_t above = incl - lsum;                    // sum of lanes > lane
        if (above < remaining && remaining <= incl) {
#pragma unroll
          for (int i = 3; i >= 0; --i) {
            if (above + hb[i] >= remaining) {
              pick[0] = uint32_t(4 * lane + i);
              pick[1] = above;
              break;
            }
            above += hb[i];
          }
        }
      }
      __syncthreads();
      const uint32_t digit = pick[0];
      remaining -= pick[1];
      prefix |= digit << shift;
      pmask |= 255u << shift;
      __syncthreads();
    }
  }
  const uint32_t tau = prefix;
  const uint32_t need_eq = need > 0 ? remaining : 0u;

  // ---- ordered write: slot order = (tile, wave, lane) ----------------------------------
  uint32_t carry_a = 0u, carry_b = 0u;
  for (int seg = 0; seg < L; seg += kTilesPerSeg * kSelThreads) {
    for (int t = 0; t < kTilesPerSeg; ++t) {
      const int slot = seg + t * kSelThreads + tid;
      bool a = false, b = false;
      if (slot < L) {
        if (slot >= ncand) {
          a = true;
        } else if (need > 0) {
          const uint32_t u = order_key(sc[slot]);
          a = u > tau;
          b = u == tau;
        }
      }
      const uint64_t ma = __ballot(a), mb = __ballot(b);
      if (lane == 0) {
        grp_a[t * kSelWaves + wave] = uint32_t(__popcll(ma));
        grp_b[t * kSelWaves + wave] = uint32_t(__popcll(mb));
      }
    }
    __syncthreads();
    uint32_t ga = grp_a[tid], gb = grp_b[tid], ta, tb;
    block_scan2(ga, gb, ta, tb, wsum_a, wsum_b, lane, wave);
    __syncthreads();
    grp_a[tid] = ga + carry_a;
    grp_b[tid] = gb + carry_b;
    __syncthreads();
    for (int t = 0; t < kTilesPerSeg; ++t) {
      const int slot = seg + t * kSelThreads + tid;
      bool a = false, b = false;
      if (slot < L) {
        if (slot >= ncand) {
          a = true;
        } else if (need > 0) {
          const uint32_t u = order_key(sc[slot]);
          a = u > tau;
          b = u == tau;
        }
      }
      const uint64_t ma = __ballot(a), mb = __ballot(b);
      const uint32_t ra = grp_a[t * kSelWaves + wave] + lanes_below(ma);
      const uint32_t rb = grp_b[t * kSelWaves + wave] + lanes_below(mb);
      const uint32_t at = ra + min(rb, need_eq);
      if ((a || (b && rb < need_eq)) && at < uint32_t(B)) out[at] = slot;
    }
    carry_a += ta;
    carry_b += tb;
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_select(const SelectParams& p, int64_t n_units, hipStream_t stream) {
  hipLaunchKernelGGL(select_kernel, dim3(unsigned(n_units)), dim3(kSelThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace tri
