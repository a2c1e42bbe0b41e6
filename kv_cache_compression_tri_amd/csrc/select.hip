// Top-B selection kernel of the TriAttention compression pass (gfx950).
//
// Per unit (one workgroup): keep the last W' = min(window, budget) slots, then the best
// budget - W' of the remaining candidates ranked by (score descending, slot ascending), and
// write the kept slots in ascending order ("TriAttention: Trigonometric KV Compression for
// Efficient Long Reasoning", section "Core Mechanism": only the top-scoring keys are kept;
// "TriAttention: trigonometric KV cache compression for long reasoning", section "The KV
// budget is a runtime knob ...": the budget bounds the whole kept cache).
//
// Scores map to order-preserving 32-bit keys (NaN and -inf to the lowest key, -0 to +0).
// The exact threshold key tau of the need-th best candidate is found in three steps:
//   1. a strided sample of 4096 candidates is brought to LDS and two sample quantiles that
//      bracket the target rank with a wide safety margin are found (radix select in LDS);
//   2. one pass over the unit counts the candidates above the bracket and appends the
//      ones inside it (typically ~3% of the unit) to LDS with ballot compaction;
//   3. a radix select inside that band gives tau and how many keys equal to tau are taken.
// If the bracket misses the target or the band overflows LDS (e.g. massive ties), the
// kernel falls back to radix passes over the whole unit in global memory.  The ordered
// write uses one ballot + mbcnt per wave per tile and a workgroup scan of the per-wave
// counts, so the output is ascending without a sort; ties at tau go to the lowest slots.
#include "tri_internal.h"

namespace tri {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSample = 4096;
constexpr int kBandCap = 8192;
constexpr int kBatchTiles = 16;                        // tiles of keys held in registers
constexpr int kBatch = kBatchTiles * kSelThreads;      // 16384 slots per batch

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

__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t* wsum, int lane, int wave) {
  v = wave_incl_scan(v, lane);
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) t += wsum[w];
  __syncthreads();
  return t;
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

struct SelShared {
  uint32_t hist[256];
  uint32_t pick[2];
  uint32_t band_n;
  uint32_t wsum_a[kSelWaves], wsum_b[kSelWaves];
  uint32_t grp_a[kBatchTiles * kSelWaves], grp_b[kBatchTiles * kSelWaves];
  uint32_t band_u[kBandCap];      // sample keys, then band keys
  uint32_t band_slot[kBandCap];
};

// After all radix levels: the rank-th largest value (1-based) and the count above it.
// `fetch(i)` gives element i (i < n) and `in(i)` whether it takes part.
template <typename Fetch>
__device__ __forceinline__ void radix_select(Fetch fetch, int n, uint32_t rank, SelShared& sh,
                                             int tid, int lane, int wave, uint32_t& tau,
                                             uint32_t& above) {
  uint32_t prefix = 0u, pmask = 0u, remaining = rank, gt = 0u;
  const int span = (n + kSelThreads - 1) / kSelThreads * kSelThreads;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) sh.hist[tid] = 0u;
    __syncthreads();
    for (int i = tid; i < span; i += kSelThreads) {
      bool act = i < n;
      const uint32_t u = act ? fetch(i) : 0u;
      act = act && (u & pmask) == prefix;
      hist_add(sh.hist, (u >> shift) & 255u, act, lane);
    }
    __syncthreads();
    if (wave == 0) {
      // lane holds bins 4*lane .. 4*lane+3; count the values in higher bins
      uint32_t hb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) hb[i] = sh.hist[4 * lane + i];
      const uint32_t lsum = hb[0] + hb[1] + hb[2] + hb[3];
      const uint32_t rev = wave_incl_scan(__shfl(lsum, 63 - lane), lane);
      const uint32_t incl = __shfl(rev, 63 - lane);   // sum over lanes >= lane
      uint32_t abv = incl - lsum;                      // sum over lanes > lane
      if (abv < remaining && remaining <= incl) {
#pragma unroll
        for (int i = 3; i >= 0; --i) {
          if (abv + hb[i] >= remaining) {
            sh.pick[0] = uint32_t(4 * lane + i);
            sh.pick[1] = abv;
            break;
          }
          abv += hb[i];
        }
      }
    }
    __syncthreads();
    const uint32_t digit = sh.pick[0], a = sh.pick[1];
    remaining -= a;
    gt += a;
    prefix |= digit << shift;
    pmask |= 255u << shift;
    __syncthreads();
  }
  tau = prefix;
  above = gt;
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(const SelectParams P) {
  __shared__ SelShared sh;
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

  // keys of one batch of slots, one per tile, kept in registers (loaded in one burst)
  uint32_t u[kBatchTiles];
  auto load_batch = [&](int b0) {
#pragma unroll
    for (int t = 0; t < kBatchTiles; ++t) {
      const int slot = b0 + t * kSelThreads + tid;
      u[t] = slot < ncand ? order_key(sc[slot]) : 0u;
    }
  };

  uint32_t tau = 0xFFFFFFFFu, need_eq = 0u;
  if (need > 0) {
    // ---- 1. bracket the target rank with two sample quantiles -------------------------
    uint32_t v_lo = 0u, v_hi = 0xFFFFFFFFu;
    if (ncand > kBandCap) {
      for (int i = tid; i < kSample; i += kSelThreads) {
        const int j = int((int64_t(i) * ncand) / kSample);
        sh.band_u[i] = order_key(sc[j]);
      }
      __syncthreads();
      const double p = double(need) / double(ncand);
      const double r = p * kSample;
      const double sd = sqrt(r * (1.0 - p));
      const int margin = int(4.0 * sd) + 16;
      const int r_hi = int(r) - margin;        // ranks are 0-based, descending
      const int r_lo = int(r) + margin;
      auto fs = [&](int i) { return sh.band_u[i]; };
      uint32_t ab;
      if (r_hi >= 0) radix_select(fs, kSample, uint32_t(r_hi + 1), sh, tid, lane, wave, v_hi, ab);
      if (r_lo < kSample) radix_select(fs, kSample, uint32_t(r_lo + 1), sh, tid, lane, wave, v_lo, ab);
      __syncthreads();
    }
    // ---- 2. count above the bracket, collect the band ----------------------------------
    if (tid == 0) sh.band_n = 0u;
    __syncthreads();
    uint32_t my_above = 0u;
    for (int b0 = 0; b0 < ncand; b0 += kBatch) {
      load_batch(b0);
#pragma unroll
      for (int t = 0; t < kBatchTiles; ++t) {
        const int j = b0 + t * kSelThreads + tid;
        const bool in = j < ncand;
        my_above += (in && u[t] > v_hi) ? 1u : 0u;
        const bool band = in && u[t] >= v_lo && u[t] <= v_hi;
        const uint64_t m = __ballot(band);
        if (m) {
          uint32_t base = 0u;
          if (lane == 0) base = atomicAdd(&sh.band_n, uint32_t(__popcll(m)));
          base = __shfl(base, 0);
          const uint32_t at = base + lanes_below(m);
          if (band && at < uint32_t(kBandCap)) {
            sh.band_u[at] = u[t];
            sh.band_slot[at] = uint32_t(j);
          }
        }
      }
    }
    const uint32_t above = block_sum(my_above, sh.wsum_a, lane, wave);
    const uint32_t band_n = sh.band_n;
    if (above < uint32_t(need) && uint32_t(need) <= above + band_n && band_n <= uint32_t(kBandCap)) {
      // ---- 3. exact select inside the band -------------------------------------------
      uint32_t ab;
      auto fb = [&](int i) { return sh.band_u[i]; };
      radix_select(fb, int(band_n), uint32_t(need) - above, sh, tid, lane, wave, tau, ab);
      need_eq = uint32_t(need) - above - ab;
    } else {
      // ---- fallback: radix passes over the whole unit --------------------------------
      uint32_t ab;
      auto fg = [&](int i) { return order_key(sc[i]); };
      radix_select(fg, ncand, uint32_t(need), sh, tid, lane, wave, tau, ab);
      need_eq = uint32_t(need) - ab;
    }
  }

  // ---- ordered write: slot order = (tile, wave, lane) within each batch -----------------
  uint32_t carry_a = 0u, carry_b = 0u;
  for (int b0 = 0; b0 < L; b0 += kBatch) {
    load_batch(b0);
    auto classify = [&](int t, bool& a, bool& b) {
      const int slot = b0 + t * kSelThreads + tid;
      a = false;
      b = false;
      if (slot < L) {
        if (slot >= ncand) {
          a = true;                       // recent window
        } else if (need > 0) {
          a = u[t] > tau;
          b = u[t] == tau;
        }
      }
    };
#pragma unroll
    for (int t = 0; t < kBatchTiles; ++t) {
      bool a, b;
      classify(t, a, b);
      const uint64_t ma = __ballot(a), mb = __ballot(b);
      if (lane == 0) {
        sh.grp_a[t * kSelWaves + wave] = uint32_t(__popcll(ma));
        sh.grp_b[t * kSelWaves + wave] = uint32_t(__popcll(mb));
      }
    }
    __syncthreads();
    constexpr int kGroups = kBatchTiles * kSelWaves;
    uint32_t ga = tid < kGroups ? sh.grp_a[tid] : 0u, gb = tid < kGroups ? sh.grp_b[tid] : 0u, ta, tb;
    block_scan2(ga, gb, ta, tb, sh.wsum_a, sh.wsum_b, lane, wave);
    __syncthreads();
    if (tid < kGroups) {
      sh.grp_a[tid] = ga + carry_a;
      sh.grp_b[tid] = gb + carry_b;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < kBatchTiles; ++t) {
      bool a, b;
      classify(t, a, b);
      const uint64_t ma = __ballot(a), mb = __ballot(b);
      const uint32_t ra = sh.grp_a[t * kSelWaves + wave] + lanes_below(ma);
      const uint32_t rb = sh.grp_b[t * kSelWaves + wave] + lanes_below(mb);
      const uint32_t at = ra + min(rb, need_eq);
      if ((a || (b && rb < need_eq)) && at < uint32_t(B)) out[at] = b0 + t * kSelThreads + tid;
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
