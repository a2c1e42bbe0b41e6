// Top-B selection of one unit, shared by the selection kernel (select.hip) and the fused
// score-and-select kernel (fused.hip) of the TriAttention compression pass (gfx950).
//
// Per unit (one workgroup): keep the last W' = min(window, budget) slots, then the best
// budget - W' of the remaining candidates ranked by (score descending, slot ascending), and
// write the kept slots in ascending order ("TriAttention: Trigonometric KV Compression for
// Efficient Long Reasoning", section "Core Mechanism": only the top-scoring keys are kept;
// "TriAttention: trigonometric KV cache compression for long reasoning", section "The KV
// budget is a runtime knob ...": the budget bounds the whole kept cache).
//
// Scores map to order-preserving 32-bit keys (NaN and -inf to the lowest candidate key, -0
// to +0).  Each wave of a 1024-thread workgroup owns a contiguous range of slots, four
// consecutive slots per lane; up to 32768 values are read from memory (or LDS) once into
// registers (2048 per wave), longer inputs are re-read on every sweep (select.hip can instead
// split them into register-resident runs).  The threshold is found by refining linear
// histograms instead of sorting:
//   level 1: 2048 bins spanning [min, max] of the candidate keys, counted in four copies (lane
//            l adds into copy l % 4, so lanes of one instruction that hit the same bin mostly
//            hit different LDS words; a lane adds a run of its slots in one bin at once) and
//            then folded;
//   level k+1: 2048 sub-bins of the bin that holds the target rank;
// until either the whole target bin is kept (its lower edge becomes the threshold: keep
// key >= T) or the bins are single key values (at most three levels, because the key span
// has 32 bits and each level resolves 11).  In the second case only some of the keys equal
// to the threshold are kept: the lowest slots among them, found with one more sweep.
// The ordered write counts the kept slots per wave, turns the counts into offsets, and
// writes each wave's kept slots in order from ballots (mbcnt ranks), without a sort.
#pragma once
#include "tri_internal.h"

namespace tri {
namespace {

// Workgroup sizes: a unit that fits in registers (up to kResident slots) uses kResThreads
// threads holding kResident / kResThreads keys each; longer units stream their scores
// with kStreamThreads threads.
constexpr int kResThreads = 1024;
constexpr int kStreamThreads = 1024;
constexpr int kVec = 4;                       // consecutive slots per lane in a tile
constexpr int kTile = 64 * kVec;              // slots per wave tile
constexpr int kResident = 32768;              // slots a workgroup holds in registers
constexpr int kBinBits = 11;
constexpr int kBins = 1 << kBinBits;
constexpr int kLevels = 3;                    // ceil(32 / kBinBits)
constexpr int kSubHist = 4;                   // level 1: lane l adds into copy l % 4 (fewer same-bin conflicts)
constexpr uint32_t kKeyNone = 0u;             // slot outside the wave's range
constexpr uint32_t kKeyWindow = 0xFFFFFFFFu;  // recent-window slot, always kept

// Candidate keys lie in [0x007FFFFF, 0xFF800000], strictly between the two sentinels.
__device__ __forceinline__ uint32_t order_key(uint32_t b) {
  const float x = __uint_as_float(b);
  if (b == 0x80000000u) b = 0u;                              // -0 ranks as +0
  const uint32_t k = b ^ (uint32_t(int32_t(b) >> 31) | 0x80000000u);
  return x != x ? 0x007FFFFFu : k;                           // NaN ranks as -inf
}

// acc + number of set bits of m in lanes below this one
__device__ __forceinline__ uint32_t mbcnt(uint64_t m, uint32_t acc) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), acc));
}

// Inclusive prefix sum over the 64 lanes: row shifts inside 16-lane rows, then row
// broadcasts of lane 15 and lane 31 into the rows above.
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) {
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x111, 0xF, 0xF, true));   // row_shr:1
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x112, 0xF, 0xF, true));   // row_shr:2
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x114, 0xF, 0xF, true));   // row_shr:4
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x118, 0xF, 0xF, true));   // row_shr:8
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x142, 0xA, 0xF, false));  // row_bcast:15
  v += uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x143, 0xC, 0xF, false));  // row_bcast:31
  return v;
}

__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = min(v, uint32_t(__shfl_xor(int(v), d, 64)));
  return v;
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = max(v, uint32_t(__shfl_xor(int(v), d, 64)));
  return v;
}

// Per-wave partial results of one unit's selection.
template <int NW>
struct SelSmall {
  uint32_t wmin[NW], wmax[NW];
  uint32_t wties[NW], wkeep[NW];
  int32_t jstar;
};

// Where a unit's selection keeps its LDS state: the refinement histograms, the level-1
// copies (copy c = lane % kSubHist at c * kBins) and the per-wave partials.  The caller owns
// the memory, so a fused kernel can lay these over LDS that an earlier phase used.
template <int NW>
struct SelLds {
  uint32_t (*hist)[kBins];   // [kLevels][kBins]
  uint32_t* sub;             // [kSubHist * kBins]
  SelSmall<NW>* sm;
};

// The bin holding the rank-th largest (1-based) histogram entry, the number of entries in
// higher bins and in the bin itself.  Every lane of the calling wave gets the same result.
// Lane l first sums bins [kBins - 32(l+1), kBins - 32l), so lanes ascending walk the bins
// descending; the 16-byte reads are rotated per lane to spread them over the LDS banks.
__device__ __forceinline__ void find_bin(const uint32_t* hist, uint32_t rank, int lane, uint32_t& tbin,
                                         uint32_t& above, uint32_t& cnt) {
  const uint4* hv = reinterpret_cast<const uint4*>(hist + kBins - 32 * (lane + 1));
  uint32_t lsum = 0;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint4 q = hv[(c + lane) & 7];
    lsum += (q.x + q.y) + (q.z + q.w);
  }
  const uint32_t incl = wave_incl_sum(lsum);
  const uint64_t hit = __ballot(incl >= rank);
  const int fl = hit ? __ffsll((unsigned long long)hit) - 1 : 63;
  const uint32_t abv = uint32_t(__builtin_amdgcn_readlane(int(incl - lsum), fl));
  const int top = kBins - 1 - 32 * fl;
  const uint32_t v = lane < 32 ? hist[top - lane] : 0u;
  const uint32_t incl2 = abv + wave_incl_sum(v);
  const uint64_t hit2 = __ballot(lane < 32 && incl2 >= rank);
  const int k = hit2 ? __ffsll((unsigned long long)hit2) - 1 : 31;
  cnt = uint32_t(__builtin_amdgcn_readlane(int(v), k));
  above = uint32_t(__builtin_amdgcn_readlane(int(incl2), k)) - cnt;
  tbin = uint32_t(top - k);
}

// One selection: L values (scores, or with kKeysIn order keys already), keep the last
// min(window, B) positions and the best B - min(window, B) others; write the kept positions
// ascending.
struct SelJob {
  const void* in;            // the L values (global memory; with kLds the LDS argument instead)
  int L, B, window;
  int32_t* out;              // B entries: kept positions ascending, -1 past the kept count
  uint32_t* out_key;         // optional: the kept positions' order keys, in the same order
  const int32_t* pos_map;    // optional: write pos_map[j] instead of base + j
  int32_t base;              // added to the written positions (without pos_map)
  int32_t* kept_n;           // optional: receives min(L, B)
};

// Selection by a workgroup of NT threads, whose lanes hold up to kCap values in registers
// (kCap / NT per lane); longer inputs (kStream) are re-read on every sweep.  With kLds the
// values are lds_sc (already in LDS and complete: the caller synchronises first).
template <int NT, int kCap, bool kStream, bool kLds, bool kKeysIn = false>
__device__ __forceinline__ void select_job(const SelJob& J, const SelLds<NT / 64>& S, const float* lds_sc) {
  constexpr int kSelThreads = NT;
  constexpr int kSelWaves = NT / 64;
  constexpr int kBatchTiles = kCap / (NT * kVec);   // tiles of keys a wave holds in registers
  static_assert(kBatchTiles * NT * kVec == kCap, "register capacity");
  static_assert(!(kStream && kLds), "LDS-resident scores are never streamed");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int L = J.L;
  const int B = J.B;
  const float* sc = kLds ? nullptr : static_cast<const float*>(J.in);
  int32_t* out = J.out;
  auto position = [&](int j) __attribute__((always_inline)) -> int32_t {
    return J.pos_map ? J.pos_map[j] : J.base + j;
  };

  if (tid == 0 && J.kept_n) *J.kept_n = min(L, B);
  if (L <= B) {
    for (int i = tid; i < B; i += kSelThreads) {
      out[i] = i < L ? position(i) : -1;
      if (J.out_key && i < L) {
        const uint32_t raw = kLds ? __float_as_uint(lds_sc[i]) : __float_as_uint(sc[i]);
        J.out_key[i] = kKeysIn ? raw : order_key(raw);
      }
    }
    return;
  }
  const int w = min(J.window, B);
  const int ncand = L - w;                 // >= 1 because L > B >= w
  const uint32_t need = uint32_t(B - w);   // candidates to keep

  // this wave's slots [r0, r1), in tiles of 64 lanes x 4 consecutive slots
  const int per_wave = (L + kSelWaves * kTile - 1) / (kSelWaves * kTile) * kTile;
  const int r0 = min(L, wave * per_wave), r1 = min(L, r0 + per_wave);
  const int n_tiles = (r1 - r0 + kTile - 1) / kTile;
  const int cand_end = min(r1, ncand);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(sc), (short)0, L * 4, 0x00020000);

  uint32_t u[kBatchTiles][kVec];
  // raw scores of the tiles from t0 into r (no waiting here: the loads stay in flight)
  auto issue = [&](int t0, uint32_t (&r)[kBatchTiles][kVec]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < kBatchTiles; ++t) {
      if (t0 + t < n_tiles) {
        const int j = r0 + (t0 + t) * kTile + lane * kVec;
        uint4 q;
        if constexpr (kLds) {   // within the unit's slots: tiles end at a multiple of kTile <= score_stride
          q = *reinterpret_cast<const uint4*>(lds_sc + j);
        } else {
          q = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, j * 4, 0, 0));
        }
        r[t][0] = q.x;
        r[t][1] = q.y;
        r[t][2] = q.z;
        r[t][3] = q.w;
      }
    }
  };
  // scores in u -> order keys, with the window and padding sentinels
  auto to_keys = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < kBatchTiles; ++t) {
      const int jt = r0 + (t0 + t) * kTile;
      if (t0 + t < n_tiles) {
        if (jt + kTile <= cand_end) {
#pragma unroll
          for (int e = 0; e < kVec; ++e) u[t][e] = kKeysIn ? u[t][e] : order_key(u[t][e]);
        } else {
#pragma unroll
          for (int e = 0; e < kVec; ++e) {
            const int j = jt + lane * kVec + e;
            u[t][e] = j >= r1 ? kKeyNone : j >= ncand ? kKeyWindow : kKeysIn ? u[t][e] : order_key(u[t][e]);
          }
        }
      }
    }
  };
  // body(t, jt) runs for every tile of the wave with keys u[t][*] of slots jt + 4*lane + e;
  // the scheduling barrier keeps the tiles in order so that ballots do not pile up in SGPRs.
  // Streaming: the next batch's loads are issued into a second buffer before the current
  // batch is processed, so their latency overlaps the work instead of stalling each batch.
  auto sweep = [&](auto&& body) __attribute__((always_inline)) {
    if constexpr (kStream) {
      uint32_t nxt[kBatchTiles][kVec];
      issue(0, nxt);
      for (int t0 = 0; t0 < n_tiles; t0 += kBatchTiles) {
#pragma unroll
        for (int t = 0; t < kBatchTiles; ++t)
#pragma unroll
          for (int e = 0; e < kVec; ++e) u[t][e] = nxt[t][e];
        to_keys(t0);
        if (t0 + kBatchTiles < n_tiles) issue(t0 + kBatchTiles, nxt);
#pragma unroll
        for (int t = 0; t < kBatchTiles; ++t) {
          if (t0 + t < n_tiles) body(t, r0 + (t0 + t) * kTile);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < kBatchTiles; ++t) {
        if (t < n_tiles) body(t, r0 + t * kTile);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  if constexpr (!kStream) {
    issue(0, u);
    to_keys(0);
    // kLds: the caller may lay the histograms over the scores' LDS; every wave has its keys
    // in registers before any of it is written
    if constexpr (kLds) __syncthreads();
  }

  // kept: key > tau, or key == tau and slot <= jstar (jstar = -1 when all ties at tau are
  // kept, i.e. the threshold is key >= tau + 1)
  uint32_t tau = kKeyWindow - 1u;
  int jstar = -1;
  bool partial = false;
  if (need > 0) {
    // ---- range of the candidate keys (sentinels wrap out of the min and the max) --------
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
    sweep([&](int t, int) __attribute__((always_inline)) {
#pragma unroll
      for (int e = 0; e < kVec; ++e) {
        mn = min(mn, u[t][e] - 1u);
        mx = max(mx, u[t][e] + 1u);
      }
    });
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (lane == 0) {
      S.sm->wmin[wave] = mn;
      S.sm->wmax[wave] = mx;
    }
    for (int i = tid; i < kLevels * kBins; i += kSelThreads) (&S.hist[0][0])[i] = 0u;
    for (int i = tid; i < kSubHist * kBins; i += kSelThreads) S.sub[i] = 0u;
    __syncthreads();
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int i = 0; i < kSelWaves; ++i) {
      lo = min(lo, S.sm->wmin[i]);
      hi = max(hi, S.sm->wmax[i]);
    }
    lo += 1u;
    hi -= 1u;

    // ---- histogram refinement ------------------------------------------------------------
    uint32_t base = lo, span = hi - lo, rank = need;   // in range: key - base <= span
    const int bitlen = 32 - __clz(int(span));
    int shift = bitlen > kBinBits ? bitlen - kBinBits : 0;
    for (int lev = 0; lev < kLevels; ++lev) {
      uint32_t* hist = S.hist[lev];
      if (lev == 0) {
        const uint32_t copy = uint32_t(lane & (kSubHist - 1)) * kBins;
        sweep([&](int t, int) __attribute__((always_inline)) {
          // a lane's 4 consecutive slots often share a bin: runs of equal bins add once
          uint32_t pb = 0xFFFFFFFFu, pc = 0;
#pragma unroll
          for (int e = 0; e < kVec; ++e) {
            const uint32_t d = u[t][e] - base;
            if (d <= span) {
              const uint32_t b = d >> shift;
              if (b == pb) {
                ++pc;
              } else {
                if (pc) atomicAdd(&S.sub[copy + pb], pc);
                pb = b;
                pc = 1;
              }
            }
          }
          if (pc) atomicAdd(&S.sub[copy + pb], pc);
        });
        __syncthreads();
        for (int i = tid; i < kBins; i += kSelThreads) {   // fold the copies
          uint32_t v = 0;
#pragma unroll
          for (int c = 0; c < kSubHist; ++c) v += S.sub[c * kBins + i];
          hist[i] = v;
        }
      } else {
        sweep([&](int t, int) __attribute__((always_inline)) {
#pragma unroll
          for (int e = 0; e < kVec; ++e) {
            const uint32_t d = u[t][e] - base;
            if (d <= span) atomicAdd(&hist[d >> shift], 1u);
          }
        });
      }
      __syncthreads();
      uint32_t tbin, above, cnt;
      find_bin(hist, rank, lane, tbin, above, cnt);
      rank -= above;
      const uint32_t edge = base + (tbin << shift);
      if (rank == cnt) {             // the whole bin is kept
        tau = edge - 1u;
        break;
      }
      if (shift == 0) {              // keys equal to edge: only the first `rank` are kept
        tau = edge;
        partial = true;
        break;
      }
      base = edge;
      span = (1u << shift) - 1u;
      shift = shift > kBinBits ? shift - kBinBits : 0;
    }

    if (partial) {
      // ---- slot of the rank-th key equal to tau, in slot order -------------------------
      uint32_t ct = 0;
      sweep([&](int t, int) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < kVec; ++e) ct += uint32_t(__popcll(__ballot(u[t][e] == tau)));
      });
      if (lane == 0) S.sm->wties[wave] = ct;
      __syncthreads();
      uint32_t run = 0;
      for (int i = 0; i < wave; ++i) run += S.sm->wties[i];
      if (run < rank && rank <= run + ct) {
        sweep([&](int t, int jt) __attribute__((always_inline)) {
          uint64_t m[kVec];
#pragma unroll
          for (int e = 0; e < kVec; ++e) m[e] = __ballot(u[t][e] == tau);
          uint32_t r = run;
#pragma unroll
          for (int e = 0; e < kVec; ++e) r = mbcnt(m[e], r);
#pragma unroll
          for (int e = 0; e < kVec; ++e) {
            const bool f = u[t][e] == tau;
            if (f && r == rank - 1u) S.sm->jstar = jt + lane * kVec + e;
            r += f ? 1u : 0u;
          }
#pragma unroll
          for (int e = 0; e < kVec; ++e) run += uint32_t(__popcll(m[e]));
        });
      }
      __syncthreads();
      jstar = S.sm->jstar;
    }
  }

  // ---- ordered write --------------------------------------------------------------------
  auto keep = [&](uint32_t k, int j) __attribute__((always_inline)) {
    return k > tau || (k == tau && j <= jstar);
  };
  uint32_t ck = 0;
  sweep([&](int t, int jt) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < kVec; ++e) ck += uint32_t(__popcll(__ballot(keep(u[t][e], jt + lane * kVec + e))));
  });
  if (lane == 0) S.sm->wkeep[wave] = ck;
  __syncthreads();
  uint32_t run = 0;
  for (int i = 0; i < wave; ++i) run += S.sm->wkeep[i];
  sweep([&](int t, int jt) __attribute__((always_inline)) {
    bool f[kVec];
    uint64_t m[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      f[e] = keep(u[t][e], jt + lane * kVec + e);
      m[e] = __ballot(f[e]);
    }
    uint32_t r = run;
#pragma unroll
    for (int e = 0; e < kVec; ++e) r = mbcnt(m[e], r);
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      if (f[e] && r < uint32_t(B)) {
        out[r] = position(jt + lane * kVec + e);
        if (J.out_key) J.out_key[r] = u[t][e];
      }
      r += f[e] ? 1u : 0u;
    }
#pragma unroll
    for (int e = 0; e < kVec; ++e) run += uint32_t(__popcll(m[e]));
  });
}

// Selection of unit `unit` of a SelectParams launch (its scores, length, budget and window).
template <int NT, int kCap, bool kStream, bool kLds>
__device__ __forceinline__ void select_unit(const SelectParams& P, const int64_t unit, const SelLds<NT / 64>& S,
                                            const float* lds_sc) {
  const int s = int(unit / P.units_per_seq);
  SelJob J;
  J.in = kLds ? nullptr : P.scores + unit * P.score_stride;
  J.L = min(max(P.seq_len[s], 0), int(P.score_stride));
  J.B = P.budget;
  J.window = P.window;
  J.out = P.kept + unit * int64_t(P.budget);
  J.out_key = nullptr;
  J.pos_map = nullptr;
  J.base = 0;
  J.kept_n = unit % P.units_per_seq == 0 ? P.kept_n + s : nullptr;
  select_job<NT, kCap, kStream, kLds>(J, S, lds_sc);
}

}  // namespace
}  // namespace tri
