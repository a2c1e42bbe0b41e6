// Attention of the newest token over a compressed cache (gfx950): the consumer of the
// compaction outputs.
//
// After compression the surviving keys are rotated by RoPE at their own positions and read
// by standard attention ("TriAttention: Trigonometric KV Compression for Efficient Long
// Reasoning", section "Core Mechanism"); compacted slots no longer equal positions, so the
// positions come from the compaction's position output.  For query head hq (pre-RoPE q at
// position Q) and kept key j (pre-RoPE k_j at position p_j, value v_j):
//
//   a_j = (R(Q) q) . (R(p_j) k_j) / sqrt(d) = sum_f Re(q_f conj(k_f) e^{i (Q - p_j) theta_f}) / sqrt(d)
//   out = sum_j softmax(a)_j v_j
//
// (keys cached after RoPE: a_j = (R(Q) q) . k'_j / sqrt(d)).  The distance phase is formed
// as (Q - p) theta_f / 2pi in float64, reduced to a fraction of a turn, and evaluated by
// v_sin_f32 / v_cos_f32 (which take turns), so large positions keep full accuracy.
//
// Mapping: one workgroup of 4 waves per (sequence, layer, KV head, slot split).  Wave w takes
// every 4th step of 4 keys of its split, with 16 lanes per key (lane g owns bands 4g..4g+3 of
// the key and dims 8g..8g+7 of its value), and scores each key for all query heads of the
// group: the key's phase and value row are formed once and serve every head.  The next
// steps' rows are in flight while a step is processed.  Each lane keeps an online softmax
// per head (reference maximum, sum and 8 accumulated value dims) for its key slot; slots are
// merged with a log-sum-exp reduction across lanes, then across waves through LDS.  A lane
// holds at most 128 VGPRs (bfloat16), so four workgroups share a CU and one's start-up and
// tail overlap the others' streaming.  With one split the workgroup writes the output; with
// several (so that few, long units still fill the GPU) each writes its partial state
// (maximum, sum, unnormalised value sums) to the caller's workspace and a second kernel
// merges the splits the same way.
#include <algorithm>

#include "device_util.h"
#include "tri_internal.h"

namespace tri {
namespace {

constexpr int kDecodeWaves = 4;
constexpr int kLanesPerKey = 16;
constexpr int kStepKeys = 64 / kLanesPerKey;       // keys a wave takes per step
constexpr int kLaneBands = kBands / kLanesPerKey;  // bands of the key a lane owns
constexpr int kLaneDims = kHeadDim / kLanesPerKey; // value dims a lane owns

// 2^x by v_exp_f32 (maxima and partial states are kept in base-2 units)
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
// A slot's reference maximum may trail its true maximum by this much (base 2) before the slot
// is rescaled.
constexpr float kLazyRescale = 8.0f;
// Reference maximum of a slot that has seen no key: finite, so that 2^(-inf - kNoMax) = 0 for
// a dead slot's weight and 2^(kNoMax - m) = 0 when slots are merged.
constexpr float kNoMax = -1e30f;

// DPP lane moves within a 16-lane row (lane i of the row takes the lane named): quad_perm
// [1,0,3,2] and [2,3,0,1] (i ^ 1, i ^ 2), row_half_mirror (i ^ 7 within 8 lanes) and row_ror
// by 4, 8 and 12 lanes (rotations of the row; by 8 that is i ^ 8).
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppXor7 = 0x141;
constexpr int kDppRor4 = 0x124, kDppRor8 = 0x128, kDppRor12 = 0x12C;
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

// bfloat16 half `hi` (0 or 1, a constant after unrolling) of a word, widened to float32
__device__ __forceinline__ float bf16_half(uint32_t w, int hi) { return hi ? bf16_hi(w) : bf16_lo(w); }

// One workgroup per (sequence, layer, KV head, pass, split): wave w takes every 4th step of 4
// keys of the split and scores each key for up to GE query heads hq0.. of the group (the
// key's phase and value row serve every head); groups of more than GE heads take a second
// pass.
// bfloat16 rows fit 128 VGPRs (4 waves per SIMD); float32 rows take more (3 per SIMD).
template <int GE, bool BF16, bool IL, bool PAGED, bool POST>
__global__ __launch_bounds__(kDecodeWaves * 64) __attribute__((amdgpu_waves_per_eu(BF16 ? 4 : 2)))
void decode_attention_kernel(const DecodeParams P) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int ROW = kHeadDim * ESZ;
  constexpr int NW = kDecodeWaves;
  constexpr int NB = kLaneBands, ND = kLaneDims;
  __shared__ float red_m[NW][GE], red_l[NW][GE];
  __shared__ float red_acc[NW][GE][kHeadDim];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kk = lane / kLanesPerKey, g = lane % kLanesPerKey;   // key slot of the step, band group
  int64_t wg = blockIdx.x;
  const int split = int(wg % P.n_split);
  wg /= P.n_split;
  const int64_t unit_pass = wg;                         // (sequence, layer, KV head, pass)
  const int pass = int(wg % P.n_pass);
  wg /= P.n_pass;
  const int hq0 = pass * GE;                            // first head of this pass
  const int nh = min(GE, P.group - hq0);
  const int h = int(wg % P.n_kvh);
  wg /= P.n_kvh;
  const int lr = int(wg % P.n_layers);
  const int s = int(wg / P.n_layers);
  const int l = P.layer0 + lr;
  const int L_all = min(max(P.seq_len[s], 0), int(P.slots));
  const int j_begin = int(min(int64_t(L_all), int64_t(split) * P.split_len));
  const int L = int(min(int64_t(L_all), int64_t(j_begin) + P.split_len));   // end of this split's slots
  const int n_qh = P.n_kvh * P.group;
  const int64_t qrow0 = (int64_t(s) * P.n_layers + lr) * n_qh + int64_t(h) * P.group + hq0;
  const int64_t Q = P.query_pos[s];
  // logits in base-2 units: log2(e) / sqrt(128), so that every weight is one v_exp_f32
  const float scale = 0.08838834764831845f * 1.4426950408889634f;

  // the lane's query bands of each head (pre-RoPE; POST: rotated to the query position)
  float qr[GE][NB], qi[GE][NB];
  double th[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) th[b] = P.theta_turns[g * NB + b];
#pragma unroll
  for (int hh = 0; hh < GE; ++hh) {
    const float* q = P.q + (qrow0 + min(hh, nh - 1)) * kHeadDim;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int f = g * NB + b;
      const float re = IL ? q[2 * f] : q[f];
      const float im = IL ? q[2 * f + 1] : q[f + kBands];
      if constexpr (POST) {
        double turns = double(Q) * th[b];
        turns -= __builtin_floor(turns);
        const float c = __builtin_amdgcn_cosf(float(turns)), sn = __builtin_amdgcn_sinf(float(turns));
        qr[hh][b] = re * c - im * sn;
        qi[hh][b] = re * sn + im * c;
      } else {
        qr[hh][b] = re;
        qi[hh][b] = im;
      }
    }
  }

  const int64_t unit = (int64_t(s) * P.n_layer + l) * P.n_kvh + h;
  const int32_t* kpos = P.pos ? P.pos + unit * P.pos_stride : nullptr;
  const int32_t* bt = PAGED ? P.block_table + int64_t(s) * P.max_pages : nullptr;
  const char* kb = static_cast<const char*>(P.k);
  const char* vb = static_cast<const char*>(P.v);
  // the step's keys j0..j0+3 (j0 a multiple of 4) share one page: its block-table entry is a
  // wave-uniform (scalar) load, so the row addresses wait on no vector load
  auto row_off = [&](int j0, int jj) -> int64_t {
    if constexpr (PAGED) {
      const int page = __builtin_amdgcn_readfirstlane(bt[min(j0, L - 1) >> 4]);
      return ((((int64_t(page) * P.n_layer + l) * P.n_kvh + h) * kPage) + (jj & 15)) * ROW;
    } else {
      return (unit * P.max_len + jj) * ROW;
    }
  };
  // lane pieces: key bands 4g..4g+3 (bfloat16 half layout: words 0-1 real, 2-3 imaginary;
  // interleaved: one (re, im) word per band) and value dims 8g..8g+7
  struct Step {
    uint4 k[BF16 ? 1 : 2];
    uint4 v[BF16 ? 1 : 2];
    int32_t p;
  };
  // Every fetch issues the same loads (slots past the split's end clamped to its last slot,
  // the position of a cache without positions read from a dummy word), so that the wait
  // before a step counts only the loads of that step and the ones issued before it, never
  // the prefetches behind it.  Called only when the split has slots (L > j_begin).
  const int32_t* pos_word = kpos ? kpos : P.seq_len + s;
  auto fetch = [&](int j0, Step& st) __attribute__((always_inline)) {
    const int jj = min(j0 + kk, L - 1);                // dead slots are not used
    const int64_t off = row_off(j0, jj);
    const char* kr = kb + off;
    const char* vr = vb + off;
    if constexpr (BF16) {
      if constexpr (IL) {
        st.k[0] = *reinterpret_cast<const uint4*>(kr + 16 * g);
      } else {
        const uint2 re = *reinterpret_cast<const uint2*>(kr + 8 * g);
        const uint2 im = *reinterpret_cast<const uint2*>(kr + kHeadDim + 8 * g);
        st.k[0] = make_uint4(re.x, re.y, im.x, im.y);
      }
      st.v[0] = *reinterpret_cast<const uint4*>(vr + 16 * g);
    } else {
      st.k[0] = *reinterpret_cast<const uint4*>(kr + (IL ? 32 * g : 16 * g));
      st.k[1] = *reinterpret_cast<const uint4*>(kr + (IL ? 32 * g + 16 : 2 * kHeadDim + 16 * g));
      st.v[0] = *reinterpret_cast<const uint4*>(vr + 32 * g);
      st.v[1] = *reinterpret_cast<const uint4*>(vr + 32 * g + 16);
    }
    st.p = pos_word[kpos ? jj : 0];                    // the slot's position, or the dummy word
  };
  auto key_band = [&](const Step& st, int b, float& a, float& c) __attribute__((always_inline)) {
    if constexpr (BF16) {
      if constexpr (IL) {
        const uint32_t w = word(st.k[0], b);
        a = bf16_half(w, 0);
        c = bf16_half(w, 1);
      } else {
        const uint32_t wr = word(st.k[0], b >> 1), wi = word(st.k[0], 2 + (b >> 1));
        a = bf16_half(wr, b & 1);
        c = bf16_half(wi, b & 1);
      }
    } else {
      if constexpr (IL) {
        a = __uint_as_float(word(st.k[b >> 1], 2 * (b & 1)));
        c = __uint_as_float(word(st.k[b >> 1], 2 * (b & 1) + 1));
      } else {
        a = __uint_as_float(word(st.k[0], b));
        c = __uint_as_float(word(st.k[1], b));
      }
    }
  };
  auto value_dim = [&](const Step& st, int d) __attribute__((always_inline)) -> float {
    if constexpr (BF16) return bf16_half(word(st.v[0], d >> 1), d & 1);
    else return __uint_as_float(word(st.v[d >> 2], d & 3));
  };

  // Each row of 16 lanes holds one key of the step.  Its lanes' partial dot products (4 bands
  // each) for the 4 heads are reduced by a reduce-scatter over the row: lanes swap half of
  // their heads with lane ^ 8, then half of the rest with lane ^ 7, then sum with lanes ^ 2 and
  // ^ 1, so the 4 lanes of quad h end with the full dot product of head h.  Quad h keeps that
  // head's online softmax for the slot (reference maximum, sum); the row's lanes take the
  // other quads' weights by rotations of the row by 4, 8 and 12 lanes, so a lane's value
  // sums acc[r] belong to the head of the quad it takes from by rotation r, head_of[r].
  static_assert(GE == 4 && kLanesPerKey == 16, "a row's quads of lanes take one head each");
  const bool swap8 = (g & 8) != 0, swap4 = (g & 4) != 0;
  const int quad = g >> 2;
  float m_l = kNoMax, lsum_l = 0.0f, acc[GE][ND];
#pragma unroll
  for (int r = 0; r < GE; ++r)
#pragma unroll
    for (int d = 0; d < ND; ++d) acc[r][d] = 0.0f;
  const double Qd = double(Q);
  auto process = [&](const Step& cur, int j0) __attribute__((always_inline)) {
    const bool live = j0 + kk < L;
    float part[GE];
#pragma unroll
    for (int hh = 0; hh < GE; ++hh) part[hh] = 0.0f;
    const double dq = Qd - double(kpos ? cur.p : j0 + kk);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float a, c;
      key_band(cur, b, a, c);
      if constexpr (!POST) {   // u = k e^{-i (Q - p) theta}: then Re(q conj(k) e^{i..}) = Re(q conj(u))
        const double turns = __builtin_amdgcn_fract(dq * th[b]);   // fraction of a turn, in [0, 1)
        const float cs = __builtin_amdgcn_cosf(float(turns)), sn = __builtin_amdgcn_sinf(float(turns));
        const float ur = fmaf(a, cs, c * sn);
        const float ui = fmaf(c, cs, -(a * sn));
        a = ur;
        c = ui;
      }
#pragma unroll
      for (int hh = 0; hh < GE; ++hh) part[hh] = fmaf(qr[hh][b], a, fmaf(qi[hh][b], c, part[hh]));
    }
    // reduce-scatter over the row: heads {0, 1} stay with g < 8 and {2, 3} with g >= 8, then
    // the head of quad g / 4
    const float k0 = swap8 ? part[2] : part[0], s0 = swap8 ? part[0] : part[2];
    const float k1 = swap8 ? part[3] : part[1], s1 = swap8 ? part[1] : part[3];
    const float x0 = k0 + dpp<kDppRor8>(s0), x1 = k1 + dpp<kDppRor8>(s1);
    float dot = (swap4 ? x1 : x0) + dpp<kDppXor7>(swap4 ? x0 : x1);
    dot += dpp<kDppXor2>(dot);
    dot += dpp<kDppXor1>(dot);
    const float logit = live ? dot * scale : -INFINITY;
    // the slot's reference maximum moves (and rescales the slot's state) only when a key
    // exceeds it by more than kLazyRescale, so weights stay below 2^kLazyRescale; the branch
    // is rare once a few keys have been seen and is taken by the whole wave or skipped; the
    // result is the same softmax, as sum and value sums share the reference
    const bool grow = logit > m_l + kLazyRescale;
    if (__any(grow)) {
      const float keep = grow ? exp2_fast(m_l - logit) : 1.0f;
      m_l = grow ? logit : m_l;
      lsum_l *= keep;
      const float kr[GE] = {keep, dpp<kDppRor4>(keep), dpp<kDppRor8>(keep), dpp<kDppRor12>(keep)};
#pragma unroll
      for (int r = 0; r < GE; ++r)
#pragma unroll
        for (int d = 0; d < ND; ++d) acc[r][d] *= kr[r];
    }
    const float w = exp2_fast(logit - m_l);   // 0 for a dead slot (logit -inf, m_l finite)
    lsum_l += w;
    const float wr[GE] = {w, dpp<kDppRor4>(w), dpp<kDppRor8>(w), dpp<kDppRor12>(w)};
#pragma unroll
    for (int r = 0; r < GE; ++r)
#pragma unroll
      for (int d = 0; d < ND; ++d) acc[r][d] = fmaf(wr[r], value_dim(cur, d), acc[r][d]);
  };
  // steps j0 = j_begin + 4 wave + 4 NW t; three register buffers, the loads of the next two
  // steps in flight while a step is processed
  constexpr int STRIDE = kStepKeys * NW;
  constexpr int DEPTH = 3;
  int j0 = j_begin + kStepKeys * wave;
  if (j_begin < L) {
    // the wave's steps in rounds of DEPTH; the loop has no exit but its end, and every round
    // issues the same loads, so each step waits only for its own rows
    const int n_steps = j0 < L ? (L - j0 + STRIDE - 1) / STRIDE : 0;
    Step st[DEPTH];
#pragma unroll
    for (int i = 0; i + 1 < DEPTH; ++i) fetch(j0 + i * STRIDE, st[i]);
    for (int t = 0; t < n_steps; t += DEPTH) {
#pragma unroll
      for (int i = 0; i < DEPTH; ++i) {
        fetch(j0 + (DEPTH - 1) * STRIDE, st[(i + DEPTH - 1) % DEPTH]);
        if (t + i < n_steps) process(st[i], j0);
        j0 += STRIDE;
      }
    }
  }
  // merge the 4 key slots of the wave (rows; head h's state in quad h of each row), then the
  // waves through LDS
  float m_all = m_l;
#pragma unroll
  for (int x = kLanesPerKey; x < 64; x <<= 1) m_all = fmaxf(m_all, __shfl_xor(m_all, x, 64));
  const float f = exp2_fast(m_l - m_all);   // 0 for a slot that saw no key (1 if none did: zero sums)
  float ls = lsum_l * f;
#pragma unroll
  for (int x = kLanesPerKey; x < 64; x <<= 1) ls += __shfl_xor(ls, x, 64);
  const float fr[GE] = {f, dpp<kDppRor4>(f), dpp<kDppRor8>(f), dpp<kDppRor12>(f)};
#pragma unroll
  for (int r = 0; r < GE; ++r)
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      float a = acc[r][d] * fr[r];
#pragma unroll
      for (int x = kLanesPerKey; x < 64; x <<= 1) a += __shfl_xor(a, x, 64);
      acc[r][d] = a;
    }
  if (kk == 0) {
    if ((g & 3) == 0) {
      red_m[wave][quad] = m_all;
      red_l[wave][quad] = ls;
    }
    const int head_of[GE] = {quad, dpp<kDppRor4>(quad), dpp<kDppRor8>(quad), dpp<kDppRor12>(quad)};
#pragma unroll
    for (int r = 0; r < GE; ++r)
#pragma unroll
      for (int d = 0; d < ND; ++d) red_acc[wave][head_of[r]][ND * g + d] = acc[r][d];
  }
  __syncthreads();
  // thread t: head t / 128 (when < G), dim t % 128
  const int64_t part = unit_pass * P.n_split + split;
  for (int t = threadIdx.x; t < nh * kHeadDim; t += NW * 64) {
    const int hh = t / kHeadDim, d = t % kHeadDim;
    float mt = kNoMax;
    for (int w = 0; w < NW; ++w) mt = fmaxf(mt, red_m[w][hh]);
    float lt = 0.0f, at = 0.0f;   // a wave that saw no key has zero sums
    for (int w = 0; w < NW; ++w) {
      const float f = exp2_fast(red_m[w][hh] - mt);
      lt = fmaf(red_l[w][hh], f, lt);
      at = fmaf(red_acc[w][hh][d], f, at);
    }
    if (P.n_split == 1) {
      P.out[(qrow0 + hh) * kHeadDim + d] = lt > 0.0f ? at / lt : 0.0f;   // no keys: zeros
    } else {
      P.part_acc[(part * GE + hh) * kHeadDim + d] = at;
      if (d == 0) {
        P.part_ml[(part * GE + hh) * 2] = mt;
        P.part_ml[(part * GE + hh) * 2 + 1] = lt;
      }
    }
  }
}

// Merge of the splits: one 128-thread workgroup per (sequence, layer, KV head, pass, head of
// the pass); thread d combines value dim d of every split by log-sum-exp.
template <int GE>
__global__ __launch_bounds__(kHeadDim) void decode_merge_kernel(const DecodeParams P) {
  const int d = threadIdx.x;
  int64_t wg = blockIdx.x;
  const int hh = int(wg % GE);
  wg /= GE;
  const int64_t unit_pass = wg;
  const int pass = int(wg % P.n_pass);
  wg /= P.n_pass;
  const int h = int(wg % P.n_kvh);
  wg /= P.n_kvh;
  const int lr = int(wg % P.n_layers);
  const int s = int(wg / P.n_layers);
  const int hq = pass * GE + hh;
  if (hq >= P.group) return;
  const int64_t qrow = (int64_t(s) * P.n_layers + lr) * (int64_t(P.n_kvh) * P.group) + int64_t(h) * P.group + hq;
  const int64_t part0 = unit_pass * P.n_split;
  float mt = kNoMax;
  for (int sp = 0; sp < P.n_split; ++sp) mt = fmaxf(mt, P.part_ml[((part0 + sp) * GE + hh) * 2]);
  float lt = 0.0f, at = 0.0f;   // a split with no keys has zero sums
  for (int sp = 0; sp < P.n_split; ++sp) {
    const float f = exp2_fast(P.part_ml[((part0 + sp) * GE + hh) * 2] - mt);
    lt = fmaf(P.part_ml[((part0 + sp) * GE + hh) * 2 + 1], f, lt);
    at = fmaf(P.part_acc[((part0 + sp) * GE + hh) * kHeadDim + d], f, at);
  }
  P.out[qrow * kHeadDim + d] = lt > 0.0f ? at / lt : 0.0f;
}

template <int GE>
hipError_t launch_decode_ge(const DecodeParams& p, bool bf16, bool interleaved, bool paged, bool post,
                            hipStream_t stream) {
  const int64_t unit_passes = int64_t(p.n_seq) * p.n_layers * p.n_kvh * p.n_pass;
  const dim3 grid(unsigned(unit_passes * p.n_split)), block(kDecodeWaves * 64);
#define TRI_DECODE_CASE(B, I, PG, PO)                                                                  \
  if (bf16 == B && interleaved == I && paged == PG && post == PO) {                                    \
    hipLaunchKernelGGL((decode_attention_kernel<GE, B, I, PG, PO>), grid, block, 0, stream, p);      \
    if (p.n_split > 1)                                                                                 \
      hipLaunchKernelGGL((decode_merge_kernel<GE>), dim3(unsigned(unit_passes * GE)), dim3(kHeadDim), 0, \
                         stream, p);                                                                   \
    return hipGetLastError();                                                                          \
  }
  TRI_DECODE_CASE(true, false, false, false)
  TRI_DECODE_CASE(true, false, true, false)
  TRI_DECODE_CASE(true, true, false, false)
  TRI_DECODE_CASE(true, true, true, false)
  TRI_DECODE_CASE(false, false, false, false)
  TRI_DECODE_CASE(false, false, true, false)
  TRI_DECODE_CASE(false, true, false, false)
  TRI_DECODE_CASE(false, true, true, false)
  TRI_DECODE_CASE(true, false, false, true)
  TRI_DECODE_CASE(true, false, true, true)
  TRI_DECODE_CASE(true, true, false, true)
  TRI_DECODE_CASE(true, true, true, true)
  TRI_DECODE_CASE(false, false, false, true)
  TRI_DECODE_CASE(false, false, true, true)
  TRI_DECODE_CASE(false, true, false, true)
  TRI_DECODE_CASE(false, true, true, true)
#undef TRI_DECODE_CASE
  return hipErrorInvalidValue;
}

}  // namespace

int64_t decode_workspace_bytes(int64_t unit_passes, int n_split) {
  if (n_split <= 1) return 0;
  const int64_t parts = unit_passes * n_split * kDecodeHeadsPerPass;
  return ((parts * 2 * 4 + 255) / 256) * 256 + parts * kHeadDim * 4;
}

int decode_splits(int64_t unit_passes, int64_t slots) {
  // the fewest (a power of two) that give every CU kDecodeMinGroupsPerCU workgroups, with at
  // least kDecodeMinSplitLen slots per split
  int n = 1;
  while (n < kDecodeMaxSplits && unit_passes * n < int64_t(kDecodeMinGroupsPerCU) * kDecodeCUs &&
         slots >= int64_t(2 * n) * kDecodeMinSplitLen)
    n *= 2;
  return n;
}

hipError_t launch_decode_attention(const DecodeParams& p, bool bf16, bool interleaved, bool paged, bool post,
                                   hipStream_t stream) {
  // a wave holds kDecodeHeadsPerPass query heads; larger groups take more passes over the keys
  DecodeParams q = p;
  q.n_pass = (p.group + kDecodeHeadsPerPass - 1) / kDecodeHeadsPerPass;
  if (q.n_split < 1) q.n_split = 1;
  if (q.n_split == 1) q.split_len = q.slots;
  return launch_decode_ge<kDecodeHeadsPerPass>(q, bf16, interleaved, paged, post, stream);
}

}  // namespace tri
