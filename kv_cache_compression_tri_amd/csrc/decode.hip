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
// Mapping: one workgroup of 8 waves per (sequence, layer, KV head, slot split).  Wave w takes
// every 8th step of 8 keys of its split, with 8 lanes per key (lane g owns bands 8g..8g+7 of
// the key and dims 16g..16g+15 of its value), and scores each key for all query heads of the
// group: the key's phase and value row are formed once and serve every head.  The next
// steps' rows are in flight while a step is processed.  Each lane keeps an online softmax
// per head (running max, sum and 16 accumulated value dims) for its key slot; slots are
// merged with a log-sum-exp reduction across lanes, then across waves through LDS.  With
// one split the workgroup writes the output; with several (so that few, long units still
// fill the GPU) each writes its partial state (max, sum, unnormalised value sums) to the
// caller's workspace and a second kernel merges the splits the same way.
#include <algorithm>

#include "device_util.h"
#include "tri_internal.h"

namespace tri {
namespace {

constexpr int kDecodeWaves = 8;

// bfloat16 half `hi` (0 or 1, a constant after unrolling) of a word, widened to float32
__device__ __forceinline__ float bf16_half(uint32_t w, int hi) { return hi ? bf16_hi(w) : bf16_lo(w); }

// One workgroup per (sequence, layer, KV head, pass, split): wave w takes every 8th step of 8
// keys of the split and scores each key for up to GE query heads hq0.. of the group (the
// key's phase and value row serve every head); groups of more than GE heads take a second
// pass.
template <int GE, bool BF16, bool IL, bool PAGED, bool POST>
__global__ __launch_bounds__(kDecodeWaves * 64) void decode_attention_kernel(const DecodeParams P) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int ROW = kHeadDim * ESZ;
  constexpr int NW = kDecodeWaves;
  __shared__ float red_m[NW][GE], red_l[NW][GE];
  __shared__ float red_acc[NW][GE][kHeadDim];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kk = lane >> 3, g = lane & 7;             // key slot of the step, band group
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
  const float scale = 0.08838834764831845f;            // 1 / sqrt(128)

  // the lane's 8 query bands of each head (pre-RoPE; POST: rotated to the query position)
  float qr[GE][8], qi[GE][8];
  double th[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) th[b] = P.theta_turns[g * 8 + b];
#pragma unroll
  for (int hh = 0; hh < GE; ++hh) {
    const float* q = P.q + (qrow0 + min(hh, nh - 1)) * kHeadDim;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int f = g * 8 + b;
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
  auto row_off = [&](int j) -> int64_t {
    if constexpr (PAGED) return ((((int64_t(bt[j >> 4]) * P.n_layer + l) * P.n_kvh + h) * kPage) + (j & 15)) * ROW;
    else return (unit * P.max_len + j) * ROW;
  };
  // lane pieces: key bands 8g..8g+7 (re, im) and value dims 16g..16g+15
  struct Step {
    uint4 k[BF16 ? 2 : 4];
    uint4 v[BF16 ? 2 : 4];
    int32_t p;
  };
  auto fetch = [&](int j0, Step& st) __attribute__((always_inline)) {
    const int j = j0 + kk;
    if (j0 >= L) return;
    const bool live = j < L;
    const int jj = live ? j : L - 1;                   // clamped: dead slots are not used
    const char* kr = kb + row_off(jj);
    const char* vr = vb + row_off(jj);
    if constexpr (BF16) {
      st.k[0] = *reinterpret_cast<const uint4*>(kr + (IL ? 32 * g : 16 * g));
      st.k[1] = *reinterpret_cast<const uint4*>(kr + (IL ? 32 * g + 16 : 128 + 16 * g));
      st.v[0] = *reinterpret_cast<const uint4*>(vr + 32 * g);
      st.v[1] = *reinterpret_cast<const uint4*>(vr + 32 * g + 16);
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        st.k[i] = *reinterpret_cast<const uint4*>(kr + (IL ? 64 * g : 32 * g) + 16 * i);
        st.k[2 + i] = *reinterpret_cast<const uint4*>(kr + (IL ? 64 * g + 32 : 256 + 32 * g) + 16 * i);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) st.v[i] = *reinterpret_cast<const uint4*>(vr + 64 * g + 16 * i);
    }
    st.p = kpos ? kpos[jj] : jj;
  };
  auto key_band = [&](const Step& st, int b, float& a, float& c) __attribute__((always_inline)) {
    if constexpr (BF16) {
      if constexpr (IL) {
        const uint32_t w = word(st.k[b >> 2], b & 3);
        a = bf16_half(w, 0);
        c = bf16_half(w, 1);
      } else {
        const uint32_t wr = word(st.k[0], b >> 1), wi = word(st.k[1], b >> 1);
        a = bf16_half(wr, b & 1);
        c = bf16_half(wi, b & 1);
      }
    } else {
      if constexpr (IL) {
        a = __uint_as_float(word(st.k[b >> 1], 2 * (b & 1)));
        c = __uint_as_float(word(st.k[b >> 1], 2 * (b & 1) + 1));
      } else {
        a = __uint_as_float(word(st.k[b >> 2], b & 3));
        c = __uint_as_float(word(st.k[2 + (b >> 2)], b & 3));
      }
    }
  };
  auto value_dim = [&](const Step& st, int d) __attribute__((always_inline)) -> float {
    if constexpr (BF16) return bf16_half(word(st.v[d >> 3], (d & 7) >> 1), d & 1);
    else return __uint_as_float(word(st.v[d >> 2], d & 3));
  };

  float m[GE], lsum[GE], acc[GE][16];
#pragma unroll
  for (int hh = 0; hh < GE; ++hh) {
    m[hh] = -INFINITY;
    lsum[hh] = 0.0f;
#pragma unroll
    for (int d = 0; d < 16; ++d) acc[hh][d] = 0.0f;
  }
  auto process = [&](const Step& cur, int j0) __attribute__((always_inline)) {
    const bool live = j0 + kk < L;
    float part[GE];
#pragma unroll
    for (int hh = 0; hh < GE; ++hh) part[hh] = 0.0f;
    const double dq = double(Q - int64_t(cur.p));
#pragma unroll
    for (int b = 0; b < 8; ++b) {
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
#pragma unroll
    for (int hh = 0; hh < GE; ++hh) {
      const float logit = live ? sum8(part[hh]) * scale : -INFINITY;
      // a new running maximum rescales the slot's state (rare once a few keys have been seen,
      // so the branch is usually skipped by the whole wave); e^{-inf} = 0 for an empty slot
      if (logit > m[hh]) {
        const float keep = __expf(m[hh] - logit);
        lsum[hh] *= keep;
#pragma unroll
        for (int d = 0; d < 16; ++d) acc[hh][d] *= keep;
        m[hh] = logit;
      }
      const float w = logit == -INFINITY ? 0.0f : __expf(logit - m[hh]);
      lsum[hh] += w;
#pragma unroll
      for (int d = 0; d < 16; ++d) acc[hh][d] = fmaf(w, value_dim(cur, d), acc[hh][d]);
    }
  };
  // steps j0 = j_begin + 8 wave + 8 NW t; register buffers with the next steps' loads in
  // flight (bfloat16: three buffers, two steps ahead; float32: two buffers, one step ahead)
  constexpr int STRIDE = 8 * NW;
  int j0 = j_begin + 8 * wave;
  if constexpr (BF16) {
    Step s0, s1, s2;
    fetch(j0, s0);
    fetch(j0 + STRIDE, s1);
    while (j0 < L) {
      fetch(j0 + 2 * STRIDE, s2);
      process(s0, j0);
      j0 += STRIDE;
      if (j0 >= L) break;
      fetch(j0 + 2 * STRIDE, s0);
      process(s1, j0);
      j0 += STRIDE;
      if (j0 >= L) break;
      fetch(j0 + 2 * STRIDE, s1);
      process(s2, j0);
      j0 += STRIDE;
    }
  } else {
    Step s0, s1;
    fetch(j0, s0);
    while (j0 < L) {
      fetch(j0 + STRIDE, s1);
      process(s0, j0);
      j0 += STRIDE;
      if (j0 >= L) break;
      fetch(j0 + STRIDE, s0);
      process(s1, j0);
      j0 += STRIDE;
    }
  }
  // merge the 8 key slots of the wave (lanes kk * 8 + g, same g), then the waves through LDS
#pragma unroll
  for (int hh = 0; hh < GE; ++hh) {
    float m_all = m[hh];
#pragma unroll
    for (int x = 8; x < 64; x <<= 1) m_all = fmaxf(m_all, __shfl_xor(m_all, x, 64));
    const float f = (m[hh] == -INFINITY) ? 0.0f : __expf(m[hh] - m_all);
    float ls = lsum[hh] * f;
#pragma unroll
    for (int d = 0; d < 16; ++d) acc[hh][d] *= f;
#pragma unroll
    for (int x = 8; x < 64; x <<= 1) {
      ls += __shfl_xor(ls, x, 64);
#pragma unroll
      for (int d = 0; d < 16; ++d) acc[hh][d] += __shfl_xor(acc[hh][d], x, 64);
    }
    if (lane == 0) {
      red_m[wave][hh] = m_all;
      red_l[wave][hh] = ls;
    }
    if (kk == 0) {
#pragma unroll
      for (int d = 0; d < 16; ++d) red_acc[wave][hh][16 * g + d] = acc[hh][d];
    }
  }
  __syncthreads();
  // thread t: head t / 128 (when < G), dim t % 128
  const int64_t part = unit_pass * P.n_split + split;
  for (int t = threadIdx.x; t < nh * kHeadDim; t += NW * 64) {
    const int hh = t / kHeadDim, d = t % kHeadDim;
    float mt = -INFINITY;
    for (int w = 0; w < NW; ++w) mt = fmaxf(mt, red_m[w][hh]);
    float lt = 0.0f, at = 0.0f;
    if (mt != -INFINITY)
      for (int w = 0; w < NW; ++w) {
        if (red_m[w][hh] == -INFINITY) continue;
        const float f = __expf(red_m[w][hh] - mt);
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
  float mt = -INFINITY;
  for (int sp = 0; sp < P.n_split; ++sp) mt = fmaxf(mt, P.part_ml[((part0 + sp) * GE + hh) * 2]);
  float lt = 0.0f, at = 0.0f;
  if (mt != -INFINITY)
    for (int sp = 0; sp < P.n_split; ++sp) {
      const float m = P.part_ml[((part0 + sp) * GE + hh) * 2];
      if (m == -INFINITY) continue;                     // a split with no keys
      const float f = __expf(m - mt);
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
  int best = 1;
  double best_cost = 0.0;
  for (int n = 1; n <= kDecodeMaxSplits; ++n) {
    if (n > 1 && slots < int64_t(n) * kDecodeMinSplitLen) break;
    const double rounds = double((unit_passes * n + kDecodeCUs - 1) / kDecodeCUs);
    const double cost = rounds * (kDecodeGroupCost + double(slots) / n) + (n > 1 ? kDecodeMergeCost : 0);
    if (n == 1 || cost < best_cost) {
      best = n;
      best_cost = cost;
    }
  }
  return best;
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
