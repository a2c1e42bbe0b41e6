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
// Mapping: one workgroup per (sequence, layer, KV head) with one wave per query head of the
// group.  A wave reads 8 keys per step with 8 lanes per key (lane g owns bands 8g..8g+7 of
// the key and dims 16g..16g+15 of its value), sums the key's logit with three DPP steps and
// keeps an online softmax (running max, sum and 16 accumulated value dims) per key slot.  The
// 8 key slots are merged with a log-sum-exp reduction at the end.
#include "tri_internal.h"

namespace tri {
namespace {

constexpr int kDecodeMaxGroup = 8;

__device__ __forceinline__ float sum8d(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  return v;
}

template <bool BF16>
__device__ __forceinline__ float elem(const char* row, int i) {
  if constexpr (BF16) return __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(row)[i]) << 16);
  else return reinterpret_cast<const float*>(row)[i];
}

template <bool BF16, bool IL, bool PAGED, bool POST>
__global__ __launch_bounds__(kDecodeMaxGroup * 64) void decode_attention_kernel(const DecodeParams P) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int ROW = kHeadDim * ESZ;
  const int lane = threadIdx.x & 63;
  const int hq_in = threadIdx.x >> 6;                 // query head within the group
  const int kk = lane >> 3, g = lane & 7;             // key slot of the step, band group
  int64_t wg = blockIdx.x;
  const int h = int(wg % P.n_kvh);
  wg /= P.n_kvh;
  const int lr = int(wg % P.n_layers);
  const int s = int(wg / P.n_layers);
  const int l = P.layer0 + lr;
  const int L = min(max(P.seq_len[s], 0), int(P.slots));
  const int n_qh = P.n_kvh * P.group;
  const int hq = h * P.group + hq_in;
  const int64_t qrow = (int64_t(s) * P.n_layers + lr) * n_qh + hq;
  const float* q = P.q + qrow * kHeadDim;
  const int64_t Q = P.query_pos[s];
  const float scale = 0.08838834764831845f;            // 1 / sqrt(128)

  // the lane's 8 query bands (pre-RoPE; POST: rotated to the query position here)
  float qr[8], qi[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int f = g * 8 + b;
    const float re = IL ? q[2 * f] : q[f];
    const float im = IL ? q[2 * f + 1] : q[f + kBands];
    if constexpr (POST) {
      double turns = double(Q) * P.theta_turns[f];
      turns -= __builtin_floor(turns);
      const float c = __builtin_amdgcn_cosf(float(turns)), sn = __builtin_amdgcn_sinf(float(turns));
      qr[b] = re * c - im * sn;
      qi[b] = re * sn + im * c;
    } else {
      qr[b] = re;
      qi[b] = im;
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

  float m = -INFINITY, lsum = 0.0f, acc[16];
#pragma unroll
  for (int d = 0; d < 16; ++d) acc[d] = 0.0f;
  for (int j0 = 0; j0 < L; j0 += 8) {
    const int j = j0 + kk;
    if (j < L) {   // lanes of a key slot past the end keep their state
      const char* krow = kb + row_off(j);
      const char* vrow = vb + row_off(j);
      const int64_t p = kpos ? int64_t(kpos[j]) : int64_t(j);
      float part = 0.0f;
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const int f = g * 8 + b;
        const float a = elem<BF16>(krow, IL ? 2 * f : f);
        const float c = elem<BF16>(krow, IL ? 2 * f + 1 : f + kBands);
        if constexpr (POST) {   // (R(Q) q) . k'
          part = fmaf(qr[b], a, fmaf(qi[b], c, part));
        } else {                // Re(q conj(k) e^{i (Q - p) theta})
          double turns = double(Q - p) * P.theta_turns[f];
          turns -= __builtin_floor(turns);
          const float cs = __builtin_amdgcn_cosf(float(turns)), sn = __builtin_amdgcn_sinf(float(turns));
          const float zr = fmaf(qr[b], a, qi[b] * c);
          const float zi = fmaf(qi[b], a, -(qr[b] * c));
          part = fmaf(zr, cs, fmaf(-zi, sn, part));
        }
      }
      const float logit = sum8d(part) * scale;
      const float m_new = fmaxf(m, logit);
      const float keep = __expf(m - m_new), w = __expf(logit - m_new);
      lsum = fmaf(lsum, keep, w);
#pragma unroll
      for (int d = 0; d < 16; ++d) acc[d] = fmaf(acc[d], keep, w * elem<BF16>(vrow, 16 * g + d));
      m = m_new;
    }
  }
  // merge the 8 key slots (lanes kk * 8 + g, same g): log-sum-exp
  float m_all = m;
#pragma unroll
  for (int x = 8; x < 64; x <<= 1) m_all = fmaxf(m_all, __shfl_xor(m_all, x, 64));
  const float f = (m == -INFINITY) ? 0.0f : __expf(m - m_all);
  lsum *= f;
#pragma unroll
  for (int d = 0; d < 16; ++d) acc[d] *= f;
#pragma unroll
  for (int x = 8; x < 64; x <<= 1) {
    lsum += __shfl_xor(lsum, x, 64);
#pragma unroll
    for (int d = 0; d < 16; ++d) acc[d] += __shfl_xor(acc[d], x, 64);
  }
  if (kk == 0) {
    float* o = P.out + qrow * kHeadDim + 16 * g;
    const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;   // no keys: zeros
#pragma unroll
    for (int d = 0; d < 16; ++d) o[d] = acc[d] * inv;
  }
}

}  // namespace

hipError_t launch_decode_attention(const DecodeParams& p, bool bf16, bool interleaved, bool paged, bool post,
                                   hipStream_t stream) {
  const dim3 grid(unsigned(int64_t(p.n_seq) * p.n_layers * p.n_kvh)), block(p.group * 64);
#define TRI_DECODE_CASE(B, I, PG, PO)                                                                  \
  if (bf16 == B && interleaved == I && paged == PG && post == PO) {                                    \
    hipLaunchKernelGGL((decode_attention_kernel<B, I, PG, PO>), grid, block, 0, stream, p);          \
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

}  // namespace tri
