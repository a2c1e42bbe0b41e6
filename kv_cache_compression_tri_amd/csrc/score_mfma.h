// Key scoring with the head contraction on the bf16 matrix cores (gfx950): bfloat16 keys
// before RoPE at consecutive positions, additive form, max over a group of query heads (used
// for 6..8 heads, where it is faster than the vector kernel).
//
// It computes what the vector kernel in score_kernel.h computes (same rewrite:
// s_h(j) = sum_f Re(W_hf x_f) + N_hf |k_f|, x_f = e^{-i r theta_f} conj(k_f), from "TriAttention:
// Trigonometric KV Compression for Efficient Long Reasoning", sections "Core Mechanism" and
// "Key Concepts", and the norm term of "TriAttention: How a Geometric Trick Cuts LLM Memory
// Use by 10x Without Losing Accuracy", section "The Core Idea: Q/K Concentration in Pre-RoPE
// Space").  Per key the three real features of each band (Re x_f, Im x_f, |k_f|) are formed
// in float32 on the vector ALUs as before; the contraction with the G heads' weights, 3G
// FMAs per band on the vector ALUs, becomes a 16-key x 16-column x 384 product on
// v_mfma_f32_16x16x32_bf16:
//   - every feature x splits exactly into a bfloat16 high part (x with its low 16 bits
//     cleared) and a bfloat16 remainder (x minus that, rounded to nearest): x_hi + x_lo
//     carries 16 significand bits (relative error below 2^-16);
//   - every weight w splits the same way; column h (< 8) of the weight matrix holds w_hi of
//     head h, column 8 + h holds w_lo;
//   - the products run over the features twice, with A = x_hi and A = x_lo, so
//     C[key][h] + C[key][8 + h] = sum (x_hi + x_lo)(w_hi + w_lo), accumulated in float32.
// The vector work per key no longer grows with G: about 165 VALU instructions per 8 keys at
// any G, against 187 (G = 4) to 285 (G = 7) in the vector kernel.  The 12 dependent products
// of a step stall the issuing wave, so the time only drops below the vector kernel's from
// G = 6 on.
//
// Mapping: a wave step is 16 keys.  Lane l holds key m = l % 16 and bands 8q..8q+7 and
// 32+8q..32+8q+7 (q = l / 16), i.e. 4 lanes per key, 16 bands per lane, read as four 16-byte
// pieces.  In v_mfma_f32_16x16x32_bf16, lane l supplies row l % 16 of A and column l % 16 of
// B, each as 8 values of the k-range of its lane group l / 16, and receives C[4(l/16) + i][l %
// 16], i = 0..3 (checked with a GPU probe).  So a lane's own features are its A operand, and the
// same lane, as column n = l % 16, holds the weights of those features for head n % 8 (high
// part for n < 8, remainder for n >= 8): no data crosses lanes before the product.  The sum of
// the two halves is one DPP row rotation by 8, the max over heads three DPP steps inside each
// 8-lane half-row.  The phase table, anchors, chunk re-anchoring, work division and key stream
// follow score_kernel.h.  A lane's features are ordered Re x_j, Im x_j (at 2j, 2j + 1) for its
// 16 local bands, then |k_j| (at 32 + j); products 0..5 take 8 consecutive features each.
#pragma once
#include "score_kernel.h"   // uniform64, kStreamPolicy

namespace tri {
namespace {

typedef __bf16 mf_bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 mf_bf16x2 __attribute__((ext_vector_type(2)));
typedef float mf_f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t mf_u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMfKeys = 16;                 // keys per wave step
constexpr int kMfFeat = 48;                 // features per lane: 16 bands x (Re x, Im x, |k|)
constexpr int kMfProducts = kMfFeat / 8;    // 16x16x32 products per half (x_hi or x_lo)

// band of local band j (0..15) of lane group q (0..3)
__device__ __forceinline__ int mf_band(int q, int j) { return j < 8 ? 8 * q + j : 24 + 8 * q + j; }

// float2 index of the phase table entry (r, f), r < kChunk: the 64 lanes of step r / 16 read
// 64 consecutive 16-byte slots per instruction (instruction jj: the lane's local bands 2jj
// and 2jj + 1)
__device__ __forceinline__ int mf_tab_index(int r, int f) {
  const int q = (f & 31) >> 3, j = (f & 7) + (f >= 32 ? 8 : 0);
  const int it = r >> 4, m = r & 15;
  return (((it * 8 + (j >> 1)) * 64) + m + 16 * q) * 2 + (j & 1);
}

// exact split: high part = x with the low 16 bits cleared (as a bfloat16 pattern in the low
// half of the result), remainder = x - high, rounded to nearest bfloat16 by the caller
__device__ __forceinline__ float mf_hi(float x) { return __uint_as_float(__float_as_uint(x) & 0xFFFF0000u); }

// packed bfloat16 pair: high parts of x0, x1 (one byte permute) / nearest of y0, y1
__device__ __forceinline__ uint32_t mf_pack_hi(float x0, float x1) {
  return __builtin_amdgcn_perm(__float_as_uint(x1), __float_as_uint(x0), 0x07060302u);
}
__device__ __forceinline__ uint32_t mf_pack_rne(float y0, float y1) {
  const mf_bf16x2 v = {(__bf16)y0, (__bf16)y1};
  return __builtin_bit_cast(uint32_t, v);
}

// max over each aligned 8-lane group: three v_max_f32 with a DPP source (quad swaps, then the
// half-row mirror).  Written as instructions (through fmaxf the compiler would first quiet a
// possible signalling NaN of every DPP-moved operand); a DPP read of a VGPR needs two wait
// states after the VALU write of it, which the compiler does not insert inside or before an
// asm block, hence the s_nop 1 before each.
__device__ __forceinline__ float mf_max8(float v) {
  float r;
  asm volatile(
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf"
      : "=&v"(r)
      : "v"(v));
  return r;
}

template <bool IL, bool PAGED>
__global__ __launch_bounds__(kScoreWaves * 64) void score_mfma_kernel(const ScoreParams P) {
  constexpr int NW = kScoreWaves;
  constexpr int NT = NW * 64;
  constexpr int STEPS = kChunk / kMfKeys;       // wave steps per chunk
  constexpr int PF = 2;                         // steps of loads in flight
  constexpr int ROW = kHeadDim * 2;
  static_assert(STEPS % PF == 0, "chunk geometry");

  __shared__ float4 tab[kChunk * kBands / 2];
  __shared__ float2 stepc[kBands];             // e^{-i kChunk theta_f}
  __shared__ float2 anc[NW][kBands];           // per-wave anchors

  const int tid = threadIdx.x;
  {  // phase table: float64 recurrence per (band, run of offsets), rounded once
    constexpr int RL = kChunk * kBands / NT;
    const int f = tid & 63, run = tid >> 6;
    const double th = P.theta[f];
    double s1, c1, zr, zi;
    sincos(-th, &s1, &c1);
    sincos(-double(run * RL) * th, &zi, &zr);
    float2* t2 = reinterpret_cast<float2*>(tab);
    for (int m = 0; m < RL; ++m) {
      t2[mf_tab_index(run * RL + m, f)] = make_float2(float(zr), float(zi));
      const double nr = zr * c1 - zi * s1;
      zi = zr * s1 + zi * c1;
      zr = nr;
    }
    if (tid < kBands) {
      double ss, cc;
      sincos(-double(kChunk) * th, &ss, &cc);
      stepc[tid] = make_float2(float(cc), float(ss));
    }
  }
  __syncthreads();

  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int km = lane & 15;     // key of the step (A row), and weight column (B)
  const int q = lane >> 4;      // lane group: bands 8q..8q+7, 32+8q..32+8q+7
  const int head = km & 7;      // head of this lane's weight column
  const bool lo_col = km >= 8;  // column holds the weights' remainders
  const float col_mask = km < P.group ? 0.0f : -INFINITY;   // columns past the group drop out of the max
  const int ups = P.n_layer * P.n_kvh;
  const int n_qh = P.n_kvh * P.group;
  // per-lane byte offsets of the four 16-byte pieces of the lane's key row
  uint32_t off[4];
  if constexpr (IL) {
    off[0] = km * ROW + 32 * q;
    off[1] = off[0] + 16;
    off[2] = km * ROW + 128 + 32 * q;
    off[3] = off[2] + 16;
  } else {
    off[0] = km * ROW + 16 * q;
    off[1] = km * ROW + 64 + 16 * q;
    off[2] = km * ROW + 128 + 16 * q;
    off[3] = km * ROW + 192 + 16 * q;
  }

  // work division shared with score_kernel.h, in 16-key steps
  const int64_t n_waves = int64_t(gridDim.x) * NW;
  const int64_t w_id = int64_t(blockIdx.x) * NW + wave;
  for_each_segment<kMfKeys>(P, lane, w_id, n_waves, [&](const int s, const int u_in, const int st0,
                                                        const int n_steps) __attribute__((always_inline)) {
    const int64_t unit = int64_t(s) * ups + u_in;
    const int l = u_in / P.n_kvh;
    const int h = u_in - l * P.n_kvh;
    const int L = min(max(P.seq_len[s], 0), int(P.score_stride));
    const int p0 = kMfKeys * st0;                 // a multiple of 16: one page per step
    const int nkeys = min(L - p0, kMfKeys * n_steps);
    const int64_t Q = P.query_pos ? P.query_pos[s] : int64_t(L) - 1;

    // ---- key stream ------------------------------------------------------------------
    const char* kbase = static_cast<const char*>(P.k);
    typedef __attribute__((address_space(4))) const int32_t* mf_const_i32_ptr;
    const mf_const_i32_ptr bt = PAGED ? (mf_const_i32_ptr)(P.block_table + int64_t(s) * P.max_pages) : nullptr;
    // paged: bytes per page id (all layers and heads) and this unit's slice of a page
    const uint64_t pg_bytes = uint64_t(P.n_layer) * uint64_t(P.n_kvh) * uint64_t(kPage * ROW);
    const char* ubase = kbase + (int64_t(l) * P.n_kvh + h) * int64_t(kPage * ROW);
    uint4 ring[PF][4];
    auto load_step = [&](int n, int sl) __attribute__((always_inline)) {
      if (n >= n_steps) return;
      const int key0 = p0 + kMfKeys * n;
      const char* base;
      if constexpr (PAGED) {
        base = ubase + uint64_t(uint32_t(bt[key0 >> 4])) * pg_bytes;
      } else {
        base = kbase + (unit * P.max_len + key0) * ROW;
      }
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, min(kMfKeys, nkeys - kMfKeys * n) * ROW, 0x00020000);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ring[sl][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off[i], 0, kStreamPolicy));
    };
#pragma unroll
    for (int i = 0; i < PF; ++i) load_step(i, i);

    // ---- weights of this lane's column: head `head` of the group (0 beyond G) ----------
    // feature order of a lane: Re x_j, Im x_j at 2j, 2j + 1 (products 0..3 take bands 4p..4p+3),
    // |k_j| at 32 + j (products 4, 5); w[] multiplies the feature at the same index
    float w[kMfFeat];
    const int64_t hrow = int64_t(l) * n_qh + int64_t(h) * P.group + head;
    const bool live_col = head < P.group;
    {
      const float2* c2 = reinterpret_cast<const float2*>(P.center);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int64_t idx = hrow * kBands + mf_band(q, j);
        const float2 c = live_col ? c2[idx] : make_float2(0.0f, 0.0f);
        const float m = live_col ? P.mean_abs[idx] : 0.0f;
        w[2 * j] = c.x;
        w[2 * j + 1] = c.y;
        w[32 + j] = m;
      }
    }
    {  // anchor of this segment (float64), one band per lane
      const double ang = double(Q - p0) * P.theta[lane];
      double sa, ca;
      sincos(ang, &sa, &ca);
      const double cr = P.c_re[lane], ci = P.c_im[lane];
      anc[wave][lane] = make_float2(float(cr * ca - ci * sa), float(cr * sa + ci * ca));
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < 16; ++j) {   // W = c A, N = m - |c| (a band with m = 0 has no norm term)
      const float2 A = anc[wave][mf_band(q, j)];
      const float cx = w[2 * j], cy = w[2 * j + 1], m = w[32 + j];
      w[2 * j] = cx * A.x - cy * A.y;
      w[2 * j + 1] = -(cx * A.y + cy * A.x);
      w[32 + j] = (m > 0.0f) ? m - __builtin_sqrtf(cx * cx + cy * cy) : 0.0f;
    }
    // the B operands: the column's high parts, or its remainders
    mf_u32x4 bm[kMfProducts];
    auto pack_weights = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int p = 0; p < kMfProducts; ++p)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float w0 = w[8 * p + 2 * e], w1 = w[8 * p + 2 * e + 1];
          bm[p][e] = lo_col ? mf_pack_rne(w0 - mf_hi(w0), w1 - mf_hi(w1)) : mf_pack_hi(w0, w1);
        }
    };
    pack_weights();

    float* out = P.scores + unit * P.score_stride + p0;
    int n = 0;
    for (int c = 0; n < n_steps; ++c) {
      int tz = lane;
      asm volatile("" : "+v"(tz));
      if (c > 0) {  // next chunk: W <- W e^{-i kChunk theta_f}, then new B operands
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float2 R = stepc[mf_band(q, j)];
          const float a = w[2 * j], b = w[2 * j + 1];
          w[2 * j] = fmaf(a, R.x, b * R.y);
          w[2 * j + 1] = fmaf(b, R.x, -(a * R.y));
        }
        pack_weights();
      }
#pragma unroll
      for (int it = 0; it < STEPS; ++it) {
        if (n < n_steps) {
          const uint4* cur = ring[it % PF];
          const float4* tp = tab + it * 8 * 64 + tz;
          float x[kMfFeat];
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            const float4 t = tp[jj * 64];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int j = 2 * jj + e;
              float a, b;
              if constexpr (IL) {
                const uint32_t wv = word(cur[j >> 2], j & 3);
                a = bf16_lo(wv);
                b = bf16_hi(wv);
              } else {
                const uint32_t wr = word(cur[j < 8 ? 0 : 1], (j & 7) >> 1);
                const uint32_t wi = word(cur[j < 8 ? 2 : 3], (j & 7) >> 1);
                a = (j & 1) ? bf16_hi(wr) : bf16_lo(wr);
                b = (j & 1) ? bf16_hi(wi) : bf16_lo(wi);
              }
              const float tc = e ? t.z : t.x, ts = e ? t.w : t.y;
              x[2 * j] = fmaf(tc, a, ts * b);           // Re(e^{-i r theta} conj(k))
              x[2 * j + 1] = fmaf(ts, a, -(tc * b));    // Im(...)
              x[32 + j] = __builtin_amdgcn_sqrtf(fmaf(a, a, b * b));
            }
          }
          load_step(n + PF, it % PF);
          // the high parts and the remainders of each group of 8 features against the same B
          mf_f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int p = 0; p < kMfProducts; ++p) {
            mf_u32x4 ah, al;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float x0 = x[8 * p + 2 * e], x1 = x[8 * p + 2 * e + 1];
              ah[e] = mf_pack_hi(x0, x1);
              al[e] = mf_pack_rne(x0 - mf_hi(x0), x1 - mf_hi(x1));
            }
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mf_bf16x8, ah),
                                                           __builtin_bit_cast(mf_bf16x8, bm[p]), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mf_bf16x8, al),
                                                           __builtin_bit_cast(mf_bf16x8, bm[p]), acc, 0, 0, 0);
          }
          // C[key][h] + C[key][8 + h], then the max over the live heads (columns 0..G-1)
          float sc[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = acc[i];
            v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
            sc[i] = mf_max8(v + col_mask);
          }
          // lanes 0, 16, 32, 48 hold keys 4(l / 16) .. 4(l / 16) + 3 of the step
          const int key = kMfKeys * n + 4 * q;
          if (km == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (key + i < nkeys) __builtin_nontemporal_store(sc[i], out + key + i);
          }
          ++n;
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  });
}

template <bool IL, bool PAGED>
hipError_t launch_mfma_case(const ScoreParams& p, int grid, hipStream_t st) {
  hipLaunchKernelGGL((score_mfma_kernel<IL, PAGED>), dim3(grid), dim3(kScoreWaves * 64), 0, st, p);
  return hipGetLastError();
}

}  // namespace
}  // namespace tri
