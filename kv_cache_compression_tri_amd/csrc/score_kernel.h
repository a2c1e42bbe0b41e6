// Key-scoring kernel of the TriAttention compression pass (gfx950), shared by the
// translation units that instantiate it (score.hip / score_post.hip: pre-RoPE keys / keys
// cached after RoPE, float32 or bfloat16; score_8bit.hip / score_post_8bit.hip: fp8 and
// int8 codes; score_*mult*.hip: the same for the multiplicative form; score_pos*.hip: keys
// at explicit positions; score_select*.hip: scoring fused with the selection, FUSE below).
//
// What it computes (per unit = sequence s, layer l, KV head h; key slot j at position p_j;
// query heads hq of the group with centre c_f = E[q_f] and m_f = E|q_f|):
//
//   s_hq(j) = mean_Delta sum_f |c_f||k_f| cos((Q - p_j + Delta) theta_f + arg c_f - arg k_f)
//           + sum_f (1 - R_f) m_f |k_f|,          R_f = |c_f| / m_f
//
// The first term is the cosine series in the query-key distance that fixed pre-RoPE
// centres produce after RoPE ("TriAttention: Trigonometric KV Compression for Efficient
// Long Reasoning", sections "Core Mechanism" and "Key Concepts"); the second blends in a
// norm-only signal weighted by the measured concentration ("TriAttention: How a Geometric
// Trick Cuts LLM Memory Use by 10x Without Losing Accuracy", section "The Core Idea: Q/K
// Concentration in Pre-RoPE Space").
//
// Evaluation (exact algebraic rewrite; the only per-key transcendental is |k_f|):
//   |c||k| cos(d theta + arg c - arg k) = Re(c conj(k) e^{i d theta}), so with an anchor
//   slot p_a and r = p_j - p_a,
//     s_hq(j) = sum_f Re( W_f x_f ) + N_f |k_f|,   x_f = e^{-i r theta_f} conj(k_f),
//     W_f = c_f C_f e^{i (Q - p_a) theta_f},  C_f = mean_Delta e^{i Delta theta_f},
//     N_f = m_f - |c_f|  (= (1 - R_f) m_f).
// The anchor phase is formed in float64 per segment; e^{-i r theta_f} (r < kChunk) comes from
// an LDS table built in float64 and rounded once to float32.  Large phases never go through
// a float32 sin/cos.  At each chunk boundary the weights rotate by e^{-i kChunk theta_f}.
// For the mean reduction W and N are averaged over the group first (both terms are linear
// in them).  bf16 keys are widened exactly to float32 (one shift or mask per element),
// fp8 (OCP E4M3) codes are converted exactly, two per instruction, and int8 codes one per
// instruction; all arithmetic is float32.  A per-(layer, KV head) key scale (stored key = true key / scale) multiplies W
// and N once per segment, since both terms are linear in the key.
//
// Mapping: 8 lanes per key; lane g of a key owns bands 8g..8g+7, so the 8 lanes of a key
// read its row as coalesced 16-byte pieces and a wave scores 8 keys per step.  Per-lane
// partial sums are combined with three DPP steps inside each 8-lane group.  Each wave owns
// an equal, contiguous share of all 8-key steps of all units and walks it unit by unit; the
// weights of the current unit live in registers.  Key rows are fetched with raw buffer
// loads from a wave-uniform base plus a per-lane constant offset, a few steps ahead, into a
// ring of registers.  Scores of 8 steps are gathered into one lane each and written as one
// coalesced 256-byte store.  The grid is persistent (one workgroup of kScoreWaves waves per
// CU), so the 128 KB phase table is built once per CU.
//
// Multiplicative form (MULT; "TriAttention: Trigonometric KV Compression for Efficient Long
// Reasoning", section "Core Mechanism": the series, then weighted by the query and key
// norms): s_hq(j) = mean_Delta sum_f cos(d theta_f + arg c_f - arg k_f) ||c|| ||k_j||.  The
// same rewrite applies to unit bands: W_f = (c_f / |c_f|) ||c|| C_f e^{i(Q - p_a) theta_f} and
// x_f = e^{-i r theta_f} conj(k_f) / |k_f| (one v_rsq_f32 per band; a band with |k_f|^2 = 0
// contributes 0), and the reduced score is multiplied by ||k_j|| = sqrt(sum_f |k_f|^2).  There
// is no norm term.
//
// Keys cached after RoPE (POST): key j was stored as k'_f = k_f e^{i p_j theta_f}, so
// c conj(k) e^{i(Q - p_j + Delta) theta} = c conj(k') e^{i(Q + Delta) theta}: the weights
// become W_f = c_f C_f e^{i Q theta_f} for every key of the unit and x_f = conj(k'_f); there is
// no per-key rotation, no phase table and no chunk re-anchoring, and |k'_f| = |k_f|.
#pragma once
#include "device_util.h"
#include "select_core.h"
#include "tri_internal.h"

namespace tri {
namespace {

// Block-table entries are read through the constant address space: the table is read-only
// during the kernel and its addresses are wave-uniform, so these become scalar loads (they
// do not pass through the vector memory counter that tracks the key stream).
typedef __attribute__((address_space(4))) const int32_t* const_i32_ptr;

// Cache policy of the key-stream buffer loads: non-temporal (NT).  Every key row is read
// exactly once, so the stream is marked as such instead of being kept in the caches; on
// gfx950 this raises the sustained read rate of the stream (a plain streaming-read probe of
// the same access pattern: about 6.1 TB/s without the bit, 6.9-7.0 TB/s with it).
constexpr int kStreamPolicy = 2;

// Element types of the key cache: DT 0 = float32, 1 = bfloat16, 2 = fp8 (OCP E4M3 codes),
// 3 = int8.  A step fragment holds a lane's 8 bands of one key: 64 B (f32), 32 B (bf16),
// 16 B (8-bit).
template <int DT>
struct Frag {
  uint4 d[DT == 0 ? 4 : (DT == 1 ? 2 : 1)];
};

// Signed byte i (0..3) of a word as float32 (exact; one SDWA conversion).
__device__ __forceinline__ float i8_at(uint32_t w, int i) { return float(int8_t(w >> (8 * i))); }

// (re, im) of band b (0..7) of the lane's fragment.
template <int DT, bool IL>
__device__ __forceinline__ void band_of(const Frag<DT>& fr, int b, float& re, float& im) {
  if constexpr (DT == 3) {
    if constexpr (IL) {       // bytes (re_b, im_b) sit next to each other
      const uint32_t w = word(fr.d[0], b >> 1);
      re = i8_at(w, 2 * (b & 1));
      im = i8_at(w, 2 * (b & 1) + 1);
    } else {                  // re codes in words x, y; im codes in words z, w
      re = i8_at(word(fr.d[0], b >> 2), b & 3);
      im = i8_at(word(fr.d[0], 2 + (b >> 2)), b & 3);
    }
  } else if constexpr (DT == 2) {
    // exact E4M3 -> float32 conversion of two codes at a time (bytes 0,1 or 2,3 of a word;
    // b is a constant once the band loop is unrolled, so each branch folds away)
    if constexpr (IL) {       // bytes (re_b, im_b) sit next to each other
      const int w = int(word(fr.d[0], b >> 1));
      const auto v = (b & 1) ? __builtin_amdgcn_cvt_pk_f32_fp8(w, true) : __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
      re = v[0];
      im = v[1];
    } else {                  // re codes in words x, y; im codes in words z, w
      const int wr = int(word(fr.d[0], b >> 2)), wi = int(word(fr.d[0], 2 + (b >> 2)));
      const auto vr = (b & 2) ? __builtin_amdgcn_cvt_pk_f32_fp8(wr, true) : __builtin_amdgcn_cvt_pk_f32_fp8(wr, false);
      const auto vi = (b & 2) ? __builtin_amdgcn_cvt_pk_f32_fp8(wi, true) : __builtin_amdgcn_cvt_pk_f32_fp8(wi, false);
      re = vr[b & 1];
      im = vi[b & 1];
    }
  } else if constexpr (DT == 1) {
    if constexpr (IL) {
      const uint32_t w = word(fr.d[b >> 2], b & 3);
      re = bf16_lo(w);
      im = bf16_hi(w);
    } else {
      const uint32_t wr = word(fr.d[0], b >> 1), wi = word(fr.d[1], b >> 1);
      re = (b & 1) ? bf16_hi(wr) : bf16_lo(wr);
      im = (b & 1) ? bf16_hi(wi) : bf16_lo(wi);
    }
  } else {
    if constexpr (IL) {
      re = __uint_as_float(word(fr.d[b >> 1], 2 * (b & 1)));
      im = __uint_as_float(word(fr.d[b >> 1], 2 * (b & 1) + 1));
    } else {
      re = __uint_as_float(word(fr.d[b >> 2], b & 3));
      im = __uint_as_float(word(fr.d[2 + (b >> 2)], b & 3));
    }
  }
}

// A wave-uniform 64-bit value held in scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(v)));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(v) >> 32));
  return int64_t((uint64_t(hi) << 32) | lo);
}

// LDS phase table: entry (r, f), r < kChunk, holds (c, s) = e^{-i r theta_f} as float32.
// Step it = r / 8, key kk = r % 8, band group g = f / 8 and band b = f % 8 are arranged so
// that the 64 lanes of a step read 64 consecutive 16-byte slots per instruction (one slot
// holds bands 2m and 2m+1 of the lane's key).
__device__ __forceinline__ int tab_slot(int r, int f) {
  const int it = r >> 3, kk = r & 7, g = f >> 3, b = f & 7;
  return ((it * 4 + (b >> 1)) * 64 + kk * 8 + g) * 2 + (b & 1);   // float2 index
}

// Work division of the scoring kernels: the units' keys, in (sequence, layer, head) order and
// in steps of KEYS keys (a unit of L keys has ceil(L / KEYS) steps), are split into one
// contiguous, equal share per wave, so ragged lengths do not unbalance the grid.  Consecutive
// steps of one unit form a segment: the weights carry over (rotated chunk by chunk) and the
// loads stream without a break.  seq_len lives on the device, so each wave sums it itself.
// body(s, u_in, st0, n_steps) runs for each segment of the wave's share: sequence s, unit u_in
// of the sequence (layer * n_kvh + head), first step st0 and n_steps steps.
template <int KEYS, typename Body>
__device__ __forceinline__ void for_each_segment(const ScoreParams& P, int lane, int64_t w_id, int64_t n_waves,
                                                 Body&& body) {
  const int ups = P.n_layer * P.n_kvh;
  auto unit_steps = [&](int sq) -> int64_t {
    return (int64_t(min(max(P.seq_len[sq], 0), int(P.score_stride))) + KEYS - 1) / KEYS;
  };
  int64_t total = 0;
  for (int s0 = 0; s0 < P.n_seq; s0 += 64) {
    int64_t c = s0 + lane < P.n_seq ? unit_steps(s0 + lane) : 0;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) c += __shfl_xor(c, d, 64);
    total += uniform64(c);
  }
  total *= ups;
  const int64_t share = total / n_waves, extra = total % n_waves;
  const int64_t g0 = w_id * share + min(w_id, extra);
  const int64_t g1 = g0 + share + (w_id < extra ? 1 : 0);
  // sequence holding step g0, and the global index of that sequence's first step
  int s = 0;
  int64_t seq_base = 0;
  if (g0 < g1) {
    for (int s0 = 0; s0 < P.n_seq; s0 += 64) {
      const int64_t c = s0 + lane < P.n_seq ? unit_steps(s0 + lane) * ups : 0;
      int64_t incl = c;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int64_t t = __shfl_up(incl, d, 64);
        if (lane >= d) incl += t;
      }
      const uint64_t hit = __ballot(seq_base + incl > g0);
      if (hit) {
        const int ln = __ffsll((unsigned long long)hit) - 1;
        s = s0 + ln;
        seq_base += uniform64(__shfl(incl - c, ln, 64));
        break;
      }
      seq_base += uniform64(__shfl(incl, 63, 64));
    }
  }
  int64_t gs = g0;
  while (gs < g1 && s < P.n_seq) {
    const int64_t spu = unit_steps(s);
    const int64_t rel = gs - seq_base;
    if (rel >= spu * ups) {            // past the end of sequence s (or s is empty)
      seq_base += spu * ups;
      ++s;
      continue;
    }
    const int u_in = int(rel / spu);
    const int st0 = int(rel - int64_t(u_in) * spu);
    const int64_t seg_end = min(g1, seq_base + (int64_t(u_in) + 1) * spu);
    const int seg_steps = int(seg_end - gs);
    gs = seg_end;
    body(s, u_in, st0, seg_steps);
  }
}

// Fused scoring and selection (FUSE; dense or paged caches): one workgroup per unit of at most
// kFuseMax slots scores
// the unit into LDS, each wave an equal run of whole 64-key groups, and then selects its top B
// from there (select_core.h), so the scores never go to memory.  The LDS is the phase table,
// on a kFuseChunk-offset chunk (32 KB), and the unit's scores (128 KB): the CU's whole 160 KB,
// so the anchors and the chunk step are kept in registers instead, and the selection lays its
// histograms over the table and its level-1 copies over the scores once they are in registers.
constexpr int kFuseMax = kFuseMaxSlots;
constexpr int kFuseChunk = 64;

// LDS of the scoring kernel besides the phase table.
template <bool FUSE, int NW>
struct ScoreSmem {
  float2 stepc[kBands];        // e^{-i kChunk theta_f}
  float2 anc[NW][kBands];      // per-wave anchors
};
template <int NW>
struct ScoreSmem<true, NW> {
  float sc[kFuseMax];          // the unit's scores
};

template <int GE, int DT, bool IL, bool PAGED, bool POST, bool MULT, bool XP, bool FUSE>
__device__ __forceinline__ void score_impl(const ScoreParams& P, const SelectParams& SP) {
  // XP: pre-RoPE keys at explicit positions (P.pos): each key is rotated by its own phase,
  // formed like the anchor (float64 turns) and evaluated by v_cos / v_sin; no table
  static_assert(!FUSE || (!POST && !MULT && !XP && DT <= 1), "fused: pre-RoPE additive f32/bf16");
  constexpr int NW = kScoreWaves;
  constexpr int NT = NW * 64;
  constexpr int CH = FUSE ? kFuseChunk : kChunk;   // phase-table offsets
  constexpr int STEPS = CH / 8;                // 8 keys per wave step
  constexpr int PF = GE <= 4 ? 4 : 2;          // steps of loads in flight
  constexpr int ESZ = DT == 0 ? 4 : (DT == 1 ? 2 : 1);
  constexpr bool B8 = DT >= 2;                 // one byte per element
  constexpr int ROW = kHeadDim * ESZ;
  static_assert(STEPS % PF == 0 && STEPS % 8 == 0, "chunk geometry");

  constexpr bool TABLE = !POST && !XP;          // consecutive positions: LDS phase table
  __shared__ float4 tab[TABLE ? CH * kBands / 2 : 1];
  __shared__ __attribute__((aligned(16))) ScoreSmem<FUSE, NW> sm;

  const int tid = threadIdx.x;
  // ---- phase table: float64 recurrence per (band, run of offsets), rounded once -------
  if constexpr (TABLE) {
    constexpr int RL = CH * kBands / NT;       // offsets per thread
    const int f = tid & 63, run = tid >> 6;
    const double th = P.theta[f];
    double s1, c1, zr, zi;
    sincos(-th, &s1, &c1);
    sincos(-double(run * RL) * th, &zi, &zr);
    float2* t2 = reinterpret_cast<float2*>(tab);
    for (int m = 0; m < RL; ++m) {
      t2[tab_slot(run * RL + m, f)] = make_float2(float(zr), float(zi));
      const double nr = zr * c1 - zi * s1;
      zi = zr * s1 + zi * c1;
      zr = nr;
    }
    if constexpr (!FUSE) {
      if (tid < kBands) {
        double ss, cc;
        sincos(-double(CH) * th, &ss, &cc);
        sm.stepc[tid] = make_float2(float(cc), float(ss));
      }
    }
  }
  __syncthreads();

  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kk = lane >> 3;   // key of the step
  const int g = lane & 7;     // band group
  // FUSE: e^{-i CH theta_f} of the lane's 8 bands, in registers: lane f forms band f's (one
  // float64 sincos per lane) and each lane reads its bands' across lanes
  float2 sreg[FUSE ? 8 : 1];
  if constexpr (FUSE) {
    double ss, cc;
    sincos(-double(CH) * P.theta[lane], &ss, &cc);
    const float sx = float(cc), sy = float(ss);
#pragma unroll
    for (int b = 0; b < 8; ++b) sreg[b] = make_float2(__shfl(sx, g * 8 + b, 64), __shfl(sy, g * 8 + b, 64));
  }
  double th_turns[XP ? 8 : 1];   // XP: theta_f / (2 pi) of the lane's bands
  if constexpr (XP) {
#pragma unroll
    for (int b = 0; b < 8; ++b) th_turns[b] = P.theta[g * 8 + b] * 0.15915494309189535;
  }
  const int ups = P.n_layer * P.n_kvh;
  const int n_qh = P.n_kvh * P.group;
  // per-lane constant byte offsets of the lane's pieces inside a step's 8 rows
  uint32_t off[DT == 0 ? 4 : 2];
  if constexpr (B8) {
    off[0] = kk * ROW + (IL ? g * 16 : g * 8);          // interleaved: one 16-byte piece
    off[1] = kk * ROW + 64 + g * 8;                      // half: re codes, then im codes
  } else if constexpr (DT == 1) {
    off[0] = kk * ROW + (IL ? g * 32 : g * 16);
    off[1] = kk * ROW + (IL ? g * 32 + 16 : 128 + g * 16);
  } else {
    off[0] = kk * ROW + (IL ? g * 64 : g * 32);
    off[1] = off[0] + 16;
    off[2] = kk * ROW + (IL ? g * 64 + 32 : 256 + g * 32);
    off[3] = off[2] + 16;
  }

  const int64_t n_waves = int64_t(gridDim.x) * NW;
  const int64_t w_id = int64_t(blockIdx.x) * NW + wave;
  auto body = [&](const int s, const int u_in, const int st0, const int seg_steps) __attribute__((always_inline)) {
    const int64_t unit = int64_t(s) * ups + u_in;
    const int l = u_in / P.n_kvh;
    const int h = u_in - l * P.n_kvh;
    const int L = min(max(P.seq_len[s], 0), int(P.score_stride));
    const int p0 = 8 * st0;
    const int nkeys = min(L - p0, 8 * seg_steps);
    const int n_steps = seg_steps;
    const int64_t Q = P.query_pos ? P.query_pos[s] : int64_t(L) - 1;

    // ---- key stream: raw buffer loads; reads past the segment return zero ------------
    const char* kbase = static_cast<const char*>(P.k);
    const_i32_ptr bt = PAGED ? (const_i32_ptr)(P.block_table + int64_t(s) * P.max_pages) : nullptr;
    // paged: page of step n, read one step before the step's load is issued
    auto page_of = [&](int n) -> int32_t { return bt[(p0 + 8 * min(n, n_steps - 1)) >> 4]; };
    int32_t pg_next = PAGED ? page_of(0) : 0;   // widened only where it is used
    // paged: bytes per page id (all layers and heads) and this unit's slice of a page
    const uint64_t pg_bytes = uint64_t(P.n_layer) * uint64_t(P.n_kvh) * uint64_t(kPage * ROW);
    const char* ubase = kbase + (int64_t(l) * P.n_kvh + h) * int64_t(kPage * ROW);
    Frag<DT> ring[PF];
    const int32_t* kpos = XP ? P.pos + unit * P.score_stride : nullptr;
    int32_t pring[XP ? PF : 1];   // XP: position of the lane's key, fetched with the key
    // Loads of step n into ring slot sl.  They are issued whatever n is (past the segment's last
    // step the range is empty: the loads return zeros and touch no memory), so that a ring
    // register never merges with an older value under a branch; such a merge makes the compiler
    // wait for every load in flight instead of the one step it needs.
    auto load_step = [&](int n, int sl) __attribute__((always_inline)) {
      Frag<DT>& fr = ring[sl];
      const int key0 = p0 + 8 * min(n, n_steps - 1);
      if constexpr (XP) pring[sl] = (n < n_steps && key0 + kk < p0 + nkeys) ? kpos[key0 + kk] : 0;
      const char* base;
      if constexpr (PAGED) {
        const int32_t page = pg_next;
        pg_next = page_of(n + 1);
        base = ubase + uint64_t(uint32_t(page)) * pg_bytes + (key0 & 15) * ROW;
      } else {
        base = kbase + (unit * P.max_len + key0) * ROW;
      }
      const int rem = nkeys - 8 * n;
      const int rows = __builtin_amdgcn_readfirstlane(n < n_steps ? (rem < 8 ? rem : 8) : 0);
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, rows * ROW, 0x00020000);
      if constexpr (B8 && !IL) {
        const uint2 re = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, off[0], 0, kStreamPolicy));
        const uint2 im = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, off[1], 0, kStreamPolicy));
        fr.d[0] = make_uint4(re.x, re.y, im.x, im.y);
      } else if constexpr (B8) {
        fr.d[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off[0], 0, kStreamPolicy));
      } else {
#pragma unroll
        for (int i = 0; i < (DT == 1 ? 2 : 4); ++i)
          fr.d[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off[i], 0, kStreamPolicy));
      }
    };
#pragma unroll
    for (int i = 0; i < PF; ++i) load_step(i, i);

    float wr[GE][8], wn[GE][8], nn[MULT ? 1 : GE][8];
    const int64_t hrow0 = int64_t(l) * n_qh + int64_t(h) * P.group;
    if constexpr (!MULT) {
      // per-head statistics of the lane's bands, loaded into the weight registers before the
      // float64 anchor work so that their latency overlaps it (turned into weights below)
      const float2* c2 = reinterpret_cast<const float2*>(P.center);
      if (!P.reduce_mean) {
#pragma unroll
        for (int hh = 0; hh < GE; ++hh)
#pragma unroll
          for (int b = 0; b < 8; ++b) {
            const int64_t idx = (hrow0 + hh) * kBands + g * 8 + b;
            const float2 c = c2[idx];
            wr[hh][b] = c.x;
            wn[hh][b] = c.y;
            nn[hh][b] = P.mean_abs[idx];
          }
      } else {
        // mean over the group: W and N are linear in the head statistics, so the centres
        // and norm weights are averaged first and the anchor is applied once below
#pragma unroll
        for (int b = 0; b < 8; ++b) wr[0][b] = wn[0][b] = nn[0][b] = 0.0f;
        for (int hh = 0; hh < P.group; ++hh) {
          float2 c[8];
          float m[8];
#pragma unroll
          for (int b = 0; b < 8; ++b) {
            const int64_t idx = (hrow0 + hh) * kBands + g * 8 + b;
            c[b] = c2[idx];
            m[b] = P.mean_abs[idx];
          }
#pragma unroll
          for (int b = 0; b < 8; ++b) {
            wr[0][b] += c[b].x;
            wn[0][b] += c[b].y;
            // (1 - R_f) m_f = m_f - |c_f|; a band with m_f = 0 carries no norm term
            nn[0][b] += (m[b] > 0.0f) ? m[b] - __builtin_sqrtf(c[b].x * c[b].x + c[b].y * c[b].y) : 0.0f;
          }
        }
        const float inv = 1.0f / float(P.group);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          wr[0][b] *= inv;
          wn[0][b] *= inv;
          nn[0][b] *= inv;
        }
      }
    }

    // anchor of this segment (float64), one band per lane; after RoPE the anchor is 0.  Each
    // lane reads its 8 bands' through LDS, or FUSE (no LDS to spare) across lanes
    float2 areg[FUSE ? 8 : 1];
    {
      const double ang = double((POST || XP) ? Q : Q - p0) * P.theta[lane];
      double sa, ca;
      sincos(ang, &sa, &ca);
      const double cr = P.c_re[lane], ci = P.c_im[lane];
      const float ax = float(cr * ca - ci * sa), ay = float(cr * sa + ci * ca);
      if constexpr (FUSE) {
#pragma unroll
        for (int b = 0; b < 8; ++b) areg[b] = make_float2(__shfl(ax, g * 8 + b, 64), __shfl(ay, g * 8 + b, 64));
      } else {
        sm.anc[wave][lane] = make_float2(ax, ay);
        __builtin_amdgcn_wave_barrier();
      }
    }
    // anchor of the lane's band b (0..7)
    auto anchor = [&](int b) __attribute__((always_inline)) -> float2 {
      if constexpr (FUSE) return areg[b];
      else return sm.anc[wave][g * 8 + b];
    };

    if constexpr (MULT) {
      // multiplicative form: the weight of band f is (c_f / |c_f|) ||c|| C_f A_f (a centre
      // band of 0 has no phase and weighs 0); ||c|| sums |c_f|^2 over the 8 lanes of a key
      // group, which hold the head's 64 bands
      const float2* cbase = reinterpret_cast<const float2*>(P.center) + hrow0 * kBands + g * 8;
      auto unit_weights = [&](int hh, float (&r)[8], float (&i)[8]) __attribute__((always_inline)) {
        const float2* cr = cbase + int64_t(hh) * kBands;
        float c2 = 0.0f;
#pragma unroll
        for (int b = 0; b < 8; ++b) c2 = fmaf(cr[b].x, cr[b].x, fmaf(cr[b].y, cr[b].y, c2));
        const float cn = __builtin_sqrtf(sum8(c2));
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const float2 c = cr[b], A = anchor(b);
          const float m = __builtin_sqrtf(c.x * c.x + c.y * c.y);
          const float sc = m > 0.0f ? cn / m : 0.0f;
          r[b] = sc * (c.x * A.x - c.y * A.y);
          i[b] = sc * (c.x * A.y + c.y * A.x);
        }
      };
      if (P.reduce_mean) {
        float sr[8], si[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) sr[b] = si[b] = 0.0f;
        for (int hh = 0; hh < P.group; ++hh) {
          float r[8], i[8];
          unit_weights(hh, r, i);
#pragma unroll
          for (int b = 0; b < 8; ++b) {
            sr[b] += r[b];
            si[b] += i[b];
          }
        }
        const float inv = 1.0f / float(P.group);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          wr[0][b] = sr[b] * inv;
          wn[0][b] = -si[b] * inv;
        }
      } else {
#pragma unroll
        for (int hh = 0; hh < GE; ++hh) {
          float r[8], i[8];
          unit_weights(hh, r, i);
#pragma unroll
          for (int b = 0; b < 8; ++b) {
            wr[hh][b] = r[b];
            wn[hh][b] = -i[b];
          }
        }
      }
    } else {
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const float2 A = anchor(b);
      if (P.reduce_mean) {   // group-mean centre (already averaged) times the anchor
        const float cx = wr[0][b], cy = wn[0][b];
        wr[0][b] = cx * A.x - cy * A.y;
        wn[0][b] = -(cx * A.y + cy * A.x);
      } else {
#pragma unroll
        for (int hh = 0; hh < GE; ++hh) {   // W = c A
          const float cx = wr[hh][b], cy = wn[hh][b], m = nn[hh][b];
          wr[hh][b] = cx * A.x - cy * A.y;
          wn[hh][b] = -(cx * A.y + cy * A.x);
          nn[hh][b] = (m > 0.0f) ? m - __builtin_sqrtf(cx * cx + cy * cy) : 0.0f;   // (1 - R_f) m_f
        }
      }
    }
    }

    if (P.k_scale) {   // stored key = true key / scale: the score is linear in the key
      const float ks = P.k_scale[int64_t(l) * P.n_kvh + h];
#pragma unroll
      for (int hh = 0; hh < GE; ++hh)
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          wr[hh][b] *= ks;
          wn[hh][b] *= ks;
          if constexpr (!MULT) nn[hh][b] *= ks;
        }
    }

    float* out = P.scores + unit * P.score_stride + p0;
    const int lane_key = 8 * g + kk;   // key this lane stores within a group of 8 steps
    float keep = 0.0f;
    // n0: first step of the current chunk; steps n0 + it >= n_steps of the last chunk compute
    // nothing, but still issue their (empty) loads
    for (int n0 = 0; n0 < n_steps; n0 += STEPS) {
      const int c = n0 / STEPS;
      // The table is read-only, so its per-step reads are invariant across chunks; an opaque
      // base keeps them inside their step instead of being hoisted (and held in registers)
      // for all steps of the chunk.
      int tz = lane;
      asm volatile("" : "+v"(tz));
      if (TABLE && c > 0) {  // next chunk: W <- W e^{-i kChunk theta_f}
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          float2 R;
          if constexpr (FUSE) R = sreg[b];
          else R = sm.stepc[(tz & 7) * 8 + b];
#pragma unroll
          for (int hh = 0; hh < GE; ++hh) {
            const float a = wr[hh][b], q = wn[hh][b];
            wr[hh][b] = fmaf(a, R.x, q * R.y);
            wn[hh][b] = fmaf(q, R.x, -(a * R.y));
          }
        }
      }
#pragma unroll
      for (int it = 0; it < STEPS; ++it) {
        const int n = n0 + it;
        const bool live = n < n_steps;     // wave-uniform
        float acc[GE];
        float k2sum = 0.0f;   // multiplicative form: sum_f |k_f|^2 of the lane's bands
        if (live) {
          Frag<DT>& cur = ring[it % PF];
#pragma unroll
          for (int hh = 0; hh < GE; ++hh) acc[hh] = 0.0f;
          if constexpr (POST) {
#pragma unroll
            for (int b = 0; b < 8; ++b) {
              float a, q;
              band_of<DT, IL>(cur, b, a, q);
              if constexpr (MULT) {   // unit band: the series keeps phases only
                const float k2 = fmaf(a, a, q * q);
                k2sum += k2;
                const float rinv = k2 > 0.0f ? __builtin_amdgcn_rsqf(k2) : 0.0f;
                a *= rinv;
                q *= rinv;
              }
              const float nk = MULT ? 0.0f : __builtin_amdgcn_sqrtf(fmaf(a, a, q * q));
#pragma unroll
              for (int hh = 0; hh < GE; ++hh) {        // x = conj(k'): Re(W x) = Wr a + Wi q
                acc[hh] = fmaf(wr[hh][b], a, acc[hh]);
                acc[hh] = fmaf(wn[hh][b], -q, acc[hh]);
                if constexpr (!MULT) acc[hh] = fmaf(nn[hh][b], nk, acc[hh]);
              }
            }
          } else {
          float4 t4[4];
          if constexpr (TABLE) {
            const float4* tp = tab + it * 4 * 64 + tz;
            t4[0] = tp[0];
            t4[1] = tp[64];
            t4[2] = tp[128];
            t4[3] = tp[192];
          } else {   // e^{-i p theta_f} of the key's own position p
            const double pk = double(pring[it % PF]);
#pragma unroll
            for (int b = 0; b < 8; ++b) {
              double turns = pk * th_turns[b];
              turns -= __builtin_floor(turns);
              const float cs = __builtin_amdgcn_cosf(float(turns)), sn = __builtin_amdgcn_sinf(float(turns));
              if (b & 1) { t4[b >> 1].z = cs; t4[b >> 1].w = -sn; } else { t4[b >> 1].x = cs; t4[b >> 1].y = -sn; }
            }
          }
#pragma unroll
          for (int b = 0; b < 8; ++b) {
            float a, q;
            band_of<DT, IL>(cur, b, a, q);
            if constexpr (MULT) {   // unit band: the series keeps phases only
              const float k2 = fmaf(a, a, q * q);
              k2sum += k2;
              const float rinv = k2 > 0.0f ? __builtin_amdgcn_rsqf(k2) : 0.0f;
              a *= rinv;
              q *= rinv;
            }
            const float tc = (b & 1) ? t4[b >> 1].z : t4[b >> 1].x;
            const float ts = (b & 1) ? t4[b >> 1].w : t4[b >> 1].y;
            const float xr = fmaf(tc, a, ts * q);      // Re(e^{-i r theta} conj(k))
            const float xi = fmaf(ts, a, -(tc * q));   // Im(...)
            const float nk = MULT ? 0.0f : __builtin_amdgcn_sqrtf(fmaf(a, a, q * q));
#pragma unroll
            for (int hh = 0; hh < GE; ++hh) {
              acc[hh] = fmaf(wr[hh][b], xr, acc[hh]);
              acc[hh] = fmaf(wn[hh][b], xi, acc[hh]);
              if constexpr (!MULT) acc[hh] = fmaf(nn[hh][b], nk, acc[hh]);
            }
          }
          }
        }
        // the slot is free again: fetch the step PF ahead into it
        load_step(n + PF, it % PF);
        if (live) {
          float sc = sum8(acc[0]);
#pragma unroll
          for (int hh = 1; hh < GE; ++hh) sc = fmaxf(sc, sum8(acc[hh]));
          if constexpr (MULT) sc *= __builtin_sqrtf(sum8(k2sum));   // times ||k|| (>= 0)
          if ((it & 7) == g) keep = sc;
          if ((it & 7) == 7 || n == n_steps - 1) {
            // lane (kk, g) holds the score of step (n & ~7) + g, key kk
            const int key = 8 * (n & ~7) + lane_key;
            // the scores are written once here and read once by the selection pass (FUSE: into
            // LDS, and to memory only if asked for)
            if (g <= (n & 7) && key < nkeys) {
              if constexpr (FUSE) {
                sm.sc[p0 + key] = keep;
                if (P.scores) __builtin_nontemporal_store(keep, out + key);
              } else {
                __builtin_nontemporal_store(keep, out + key);
              }
            }
          }
        }
        // keep each step's table reads and arithmetic inside its own step
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  if constexpr (FUSE) {
    // one unit per workgroup: wave w scores steps [w S, (w + 1) S) of it, S a multiple of 8
    // (whole 64-key store groups); then the workgroup selects from the scores in LDS
    const int64_t unit = blockIdx.x;
    const int s = int(unit / ups), u_in = int(unit - int64_t(s) * ups);
    const int L = min(max(P.seq_len[s], 0), int(P.score_stride));
    const int steps = (L + 7) / 8;
    const int share = (steps + 8 * NW - 1) / (8 * NW) * 8;
    const int st0 = wave * share;
    const int n = min(share, steps - st0);
    if (n > 0) body(s, u_in, st0, n);
    __syncthreads();
    // the selection's state over LDS the scoring has finished with: histograms and per-wave
    // partials over the phase table, level-1 copies over the scores (select_unit reads the
    // scores into registers and synchronises before it writes those)
    static_assert(sizeof(tab) >= kLevels * kBins * 4 + sizeof(SelSmall<NW>), "table region too small");
    static_assert(sizeof(sm) >= kSubHist * kBins * 4, "score region too small");
    const SelLds<NW> S{reinterpret_cast<uint32_t(*)[kBins]>(tab), reinterpret_cast<uint32_t*>(sm.sc),
                       reinterpret_cast<SelSmall<NW>*>(reinterpret_cast<char*>(tab) + kLevels * kBins * 4)};
    select_unit<NT, kFuseMax, false, true>(SP, unit, S, sm.sc);
  } else {
    for_each_segment<8>(P, lane, w_id, n_waves, body);
  }
}

template <int GE, int DT, bool IL, bool PAGED, bool POST, bool MULT, bool XP>
__global__ __launch_bounds__(kScoreWaves * 64) void score_kernel(const ScoreParams P) {
  score_impl<GE, DT, IL, PAGED, POST, MULT, XP, false>(P, SelectParams{});
}

// scoring and selection of one unit per workgroup (FUSE above)
template <int GE, int DT, bool IL, bool PAGED>
__global__ __launch_bounds__(kScoreWaves * 64) void score_select_kernel(const ScoreParams P, const SelectParams S) {
  score_impl<GE, DT, IL, PAGED, false, false, false, true>(P, S);
}

template <int GE, int DT, bool POST, bool MULT, bool XP>
hipError_t launch_ge(const ScoreParams& p, bool il, bool paged, int grid, hipStream_t st) {
  const dim3 blk(kScoreWaves * 64), grd(grid);
#define TRI_SCORE_CASE(I, PG)                                                              \
  if (il == I && paged == PG) {                                                            \
    hipLaunchKernelGGL((score_kernel<GE, DT, I, PG, POST, MULT, XP>), grd, blk, 0, st, p);\
    return hipGetLastError();                                                              \
  }
  TRI_SCORE_CASE(false, false)
  TRI_SCORE_CASE(false, true)
  TRI_SCORE_CASE(true, false)
  TRI_SCORE_CASE(true, true)
#undef TRI_SCORE_CASE
  return hipErrorInvalidValue;
}

template <int DT, bool POST, bool MULT = false, bool XP = false>
hipError_t launch_groups(const ScoreParams& p, int G_eff, bool interleaved, bool paged, int grid,
                         hipStream_t stream) {
  switch (G_eff) {
    case 1: return launch_ge<1, DT, POST, MULT, XP>(p, interleaved, paged, grid, stream);
    case 2: return launch_ge<2, DT, POST, MULT, XP>(p, interleaved, paged, grid, stream);
    case 3: return launch_ge<3, DT, POST, MULT, XP>(p, interleaved, paged, grid, stream);
    case 4: return launch_ge<4, DT, POST, MULT, XP>(p, interleaved, paged, grid, stream);
    case 5: return launch_ge<5, DT, POST, MULT, XP>(p, interleaved, paged, grid, stream);
    case 6: return launch_ge<6, DT, POST, MULT, XP>(p, interleaved, paged, grid, stream);
    case 7: return launch_ge<7, DT, POST, MULT, XP>(p, interleaved, paged, grid, stream);
    case 8: return launch_ge<8, DT, POST, MULT, XP>(p, interleaved, paged, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace tri
