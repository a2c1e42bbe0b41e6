// Key scoring with the head contraction on the bf16 matrix cores, weights as the row operand
// (gfx950): bfloat16 keys before RoPE at consecutive positions, or bfloat16, fp8 and int8 keys
// cached after RoPE (POST; DT = 1, 2, 3), additive form, max over a group of G query heads.
//
// It computes what the vector kernel in score_kernel.h computes (the same exact rewrite:
// s_h(j) = sum_f Re(W_hf x_f) + N_hf |k_f|, x_f = e^{-i r theta_f} conj(k_f); "TriAttention:
// Trigonometric KV Compression for Efficient Long Reasoning", sections "Core Mechanism" and "Key
// Concepts", and the norm term of "TriAttention: How a Geometric Trick Cuts LLM Memory Use by 10x
// Without Losing Accuracy", section "The Core Idea: Q/K Concentration in Pre-RoPE Space").
// Per key the three real features of each band (Re x_f, Im x_f, |k_f|) are formed in float32 on
// the vector ALUs; the contraction with the heads' weights is a 16-row x 16-key x 384 product on
// v_mfma_f32_16x16x32_bf16 with an exact two-part split of both factors:
//   - a feature x is x_hi + x_lo, x_hi = x with its low 16 bits cleared (a bfloat16), x_lo =
//     x - x_hi rounded to the nearest bfloat16 (together 16 significand bits, relative error
//     below 2^-16); a weight w is split the same way;
//   - row 2h of the weight operand holds head h's w_hi, row 2h + 1 its w_lo (heads >= G are 0);
//   - each group of 8 features is multiplied twice, with x_hi and with x_lo as the key operand,
//     into one float32 accumulator, so rows 2h and 2h + 1 sum to (w_hi + w_lo)(x_hi + x_lo) up
//     to the w_lo x_lo term (relative 2^-16 of the product).
// The bf16 matrix cores run beside the vector ALUs when a wave interleaves its products with its
// vector work (about 30 vector instructions per product hide it); a wave issues the two products
// of each feature group as soon as that group is packed, and reduces a step's accumulator only
// during the next step.
//
// Mapping: a wave step is 16 keys.  Lane l holds key m = l % 16 and bands 8q..8q+7 and
// 32+8q..32+8q+7 (q = l / 16), four 16-byte pieces of the key's row; in the product it supplies column m
// of the key operand (its own features, as 8 values of the k-range of lane group q) and row m of
// the weight operand (the same bands' weights of head m / 2, part m % 2), and receives rows
// 4q..4q+3 of column m: both parts of heads 2q and 2q + 1 of key m.  So the sum of the parts and
// the max over a lane's two heads stay in the lane (a step's accumulator starts at -inf in the
// rows of heads past the group); the max over the four lane groups is taken for two steps at
// once: a swap of the 32-lane halves between the two steps' values (v_permlane32_swap) and a
// swap of 16-lane rows within the result (v_permlane16_swap) leave the even step's scores in
// rows 0 and 1 and the odd step's in rows 2 and 3.  Two such pairs give each lane one of 64
// consecutive keys to store.
//
// Key stream: in that layout 16 consecutive lanes hold 16 different keys, so loading it directly
// would make every group of consecutive lanes read 16 bytes of 16 different rows.  Instead the
// wave reads each step's 16 rows whole (16 consecutive lanes per 256-byte row, a plain streaming
// pattern), two steps ahead, writes them to its own staging area in LDS and reads them back in
// the product layout one step ahead of their use.  In the staging area 16-byte piece p of row r
// sits in slot 16 r + (p xor r): the 16 lanes writing one row and the 16 lanes reading one piece
// of 16 rows both hit 16 distinct slots modulo 16, so neither access has bank conflicts.  The
// phase table, anchors, chunk re-anchoring and work division follow score_kernel.h; this kernel's
// chunk is 224 offsets (14 steps), so that the table (112 KB) and the eight waves' staging rows
// (32 KB) share the CU's 160 KB of LDS.
//
// Keys cached after RoPE (POST): k'_f = k_f e^{i p_j theta_f}, so x_f = conj(k'_f) and the weights
// are anchored at Q once per segment (W_f = c_f C_f e^{i Q theta_f}); there is no phase table and
// no re-anchoring.  Re(W x) = Re W Re k' + Im W Im k' is linear in the raw key, whose bfloat16
// values are exact operands: the four trig products per step take the four staged 16-byte pieces
// of the lane's row as they are (one product each, the weight rows still split in two parts),
// and only |k_f| is formed and split on the vector ALUs.  8-bit keys (fp8 OCP E4M3, int8; a row is
// 128 bytes, loaded in two 16-byte instructions per lane and step) are converted exactly to float32
// for |k_f| and packed as bfloat16 for the products (their values have at most 8 significant bits);
// a per-(layer, KV head) key scale multiplies the weights once per segment.
#pragma once
#include "score_kernel.h"   // for_each_segment, uniform64, kStreamPolicy

namespace tri {
namespace {

typedef __bf16 mx_bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 mx_bf16x2 __attribute__((ext_vector_type(2)));
typedef float mx_f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t mx_u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMxKeys = 16;                 // keys per wave step
constexpr int kMxSteps = 14;                // wave steps per chunk
constexpr int kMxChunk = kMxSteps * kMxKeys;   // phase-table offsets (224)
constexpr int kMxRow16 = 16;                // 16-byte slots per staged key row
constexpr int kMxFeat = 48;                 // features per lane: 16 bands x (Re x, Im x, |k|)
constexpr int kMxProducts = kMxFeat / 8;    // 16x16x32 products per operand part

// band of local band j (0..15) of lane group q (0..3)
__device__ __forceinline__ int mx_band(int q, int j) { return j < 8 ? 8 * q + j : 24 + 8 * q + j; }

// float2 index of the phase table entry (r, f), r < kMxChunk: the 64 lanes of step r / 16 read
// 64 consecutive 16-byte slots per instruction (instruction jj: the lane's local bands 2jj and
// 2jj + 1)
__device__ __forceinline__ int mx_tab_index(int r, int f) {
  const int q = (f & 31) >> 3, j = (f & 7) + (f >= 32 ? 8 : 0);
  const int it = r >> 4, m = r & 15;
  return (((it * 8 + (j >> 1)) * 64) + m + 16 * q) * 2 + (j & 1);
}

// high part of x (low 16 bits cleared) as a float
__device__ __forceinline__ float mx_hi(float x) { return __uint_as_float(__float_as_uint(x) & 0xFFFF0000u); }
// packed bfloat16 pair: high parts of x0, x1 (one byte permute) / nearest of y0, y1
__device__ __forceinline__ uint32_t mx_pack_hi(float x0, float x1) {
  return __builtin_amdgcn_perm(__float_as_uint(x1), __float_as_uint(x0), 0x07060302u);
}
__device__ __forceinline__ uint32_t mx_pack_rne(float y0, float y1) {
  const mx_bf16x2 v = {(__bf16)y0, (__bf16)y1};
  return __builtin_bit_cast(uint32_t, v);
}

// The two operand parts of 8 features x[0..7]: high parts by truncation (one byte permute per
// pair), remainders x - high (exact) rounded to the nearest bfloat16.
__device__ __forceinline__ void mx_split8(const float (&x)[8], mx_u32x4& bh, mx_u32x4& bl) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float x0 = x[2 * e], x1 = x[2 * e + 1];
    bh[e] = mx_pack_hi(x0, x1);
    bl[e] = mx_pack_rne(x0 - mx_hi(x0), x1 - mx_hi(x1));
  }
}

// Index into w[] (Re W of local band j at 2j, -Im W at 2j + 1) of the weight that multiplies element
// e of raw key piece p (0..3) in the products of keys cached after RoPE; an odd index (an imaginary
// part) takes the weight negated.  The half split's pieces hold the real parts of local bands 0..7
// and 8..15, then their imaginary parts; the interleaved pieces hold (re, im) of local bands
// 4p..4p+3.
__device__ __forceinline__ constexpr int mx_post_index(bool il, int p, int e) {
  return il ? 2 * (4 * p + (e >> 1)) + (e & 1) : 2 * ((p & 1) * 8 + e) + (p >> 1);
}

// (re, im) of local bands 0..15 of a lane's 8-bit key piece words cw(0..7), exactly (DT 2: OCP E4M3
// codes, two per conversion; DT 3: int8 codes): half split, words 0..3 hold the real codes of local
// bands 0..15 and words 4..7 the imaginary ones; interleaved, word k holds (re, im) of local bands
// 2k and 2k + 1
template <int DT, bool IL, typename CW>
__device__ __forceinline__ void mx_decode8(const CW& cw, float (&re)[16], float (&im)[16]) {
#pragma unroll
  for (int j = 0; j < 16; j += 2) {
    if constexpr (DT == 2) {
      if constexpr (IL) {
        const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(int(cw(j >> 1)), false);
        const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(int(cw(j >> 1)), true);
        re[j] = a[0]; im[j] = a[1]; re[j + 1] = b[0]; im[j + 1] = b[1];
      } else {
        const bool hi = (j & 2) != 0;
        const auto a = hi ? __builtin_amdgcn_cvt_pk_f32_fp8(int(cw(j >> 2)), true)
                          : __builtin_amdgcn_cvt_pk_f32_fp8(int(cw(j >> 2)), false);
        const auto b = hi ? __builtin_amdgcn_cvt_pk_f32_fp8(int(cw(4 + (j >> 2))), true)
                          : __builtin_amdgcn_cvt_pk_f32_fp8(int(cw(4 + (j >> 2))), false);
        re[j] = a[0]; re[j + 1] = a[1]; im[j] = b[0]; im[j + 1] = b[1];
      }
    } else {
      if constexpr (IL) {
        const uint32_t w = cw(j >> 1);
        re[j] = float(int8_t(w)); im[j] = float(int8_t(w >> 8));
        re[j + 1] = float(int8_t(w >> 16)); im[j + 1] = float(int8_t(w >> 24));
      } else {
        const uint32_t wr = cw(j >> 2), wi = cw(4 + (j >> 2));
        const int sh = 8 * (j & 3);
        re[j] = float(int8_t(wr >> sh)); re[j + 1] = float(int8_t(wr >> (sh + 8)));
        im[j] = float(int8_t(wi >> sh)); im[j + 1] = float(int8_t(wi >> (sh + 8)));
      }
    }
  }
}

template <int G, bool IL, bool PAGED, bool POST, int DT = 1>
__global__ __launch_bounds__(kScoreWaves * 64) void score_mx_kernel(const ScoreParams P) {
  constexpr int NW = kScoreWaves;
  constexpr int NT = NW * 64;
  // wave steps per chunk (keys after RoPE have no table: there the chunk is only the unrolled
  // loop), and steps of loads in flight (3 or 4 steps for keys after RoPE measured the same, and so
  // did 8 for 8-bit keys and 12 waves per CU)
  constexpr int STEPS = kMxSteps;
  constexpr int PF = 2;
  // DT 1: bfloat16 keys; DT 2 / 3: fp8 (OCP E4M3) / int8 codes, keys cached after RoPE only.  An
  // 8-bit row is 128 bytes: 8 pieces of 16 bytes, loaded in 2 instructions per step instead of 4.
  static_assert(DT == 1 || (POST && (DT == 2 || DT == 3)), "8-bit keys: after RoPE");
  constexpr bool E8 = DT != 1;
  constexpr int ROW = kHeadDim * (E8 ? 1 : 2);
  constexpr int NLD = E8 ? 2 : 4;               // 16-byte load instructions per step
  constexpr int RPC = E8 ? 8 : kMxRow16;        // 16-byte pieces per row
  static_assert(STEPS % 2 == 0 && STEPS % PF == 0, "chunk geometry");
  static_assert(G >= 1 && G <= 8, "group");

  __shared__ float4 tab[POST ? 1 : kMxChunk * kBands / 2];   // keys after RoPE need no table
  __shared__ float2 stepc[kBands];             // e^{-i kMxChunk theta_f}
  __shared__ float2 anc[NW][kBands];           // per-wave anchors
  __shared__ uint4 stage[NW][kMxKeys * RPC];        // per-wave staging rows of one step

  const int tid = threadIdx.x;
  if constexpr (!POST) {  // phase table: float64 recurrence per (band, run of offsets), rounded once
    constexpr int RL = kMxChunk * kBands / NT;
    const int f = tid & 63, run = tid >> 6;
    const double th = P.theta[f];
    double s1, c1, zr, zi;
    sincos(-th, &s1, &c1);
    sincos(-double(run * RL) * th, &zi, &zr);
    float2* t2 = reinterpret_cast<float2*>(tab);
    for (int m = 0; m < RL; ++m) {
      t2[mx_tab_index(run * RL + m, f)] = make_float2(float(zr), float(zi));
      const double nr = zr * c1 - zi * s1;
      zi = zr * s1 + zi * c1;
      zr = nr;
    }
    if (tid < kBands) {
      double ss, cc;
      sincos(-double(kMxChunk) * th, &ss, &cc);
      stepc[tid] = make_float2(float(cc), float(ss));
    }
  }
  __syncthreads();

  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int km = lane & 15;       // key of the step (column), and weight row
  const int q = lane >> 4;        // lane group: bands 8q..8q+7, 32+8q..32+8q+7
  const int head = km >> 1;       // head of this lane's weight row
  const bool lo_row = km & 1;     // the row holds the weights' remainders
  const bool live_row = head < G;
  // heads 2q and 2q + 1 of the lane's output rows: -inf drops a head past the group from the max
  const float mask_a = (2 * q < G) ? 0.0f : -INFINITY;
  const float mask_b = (2 * q + 1 < G) ? 0.0f : -INFINITY;
  const mx_f32x4 init = {mask_a, 0.0f, mask_b, 0.0f};   // a step's accumulator before its products
  const int ups = P.n_layer * P.n_kvh;
  const int n_qh = P.n_kvh * P.group;
  // whole-row loads: load i, lane l reads 16-byte piece l % 16 of row 4i + l / 16 (8-bit rows:
  // piece l % 8 of row 8i + l / 8)
  const int ld_p = lane & (RPC - 1), ld_r = lane / RPC;
  uint32_t off[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) off[i] = ((64 / RPC) * i + ld_r) * ROW + 16 * ld_p;
  // Staging slots, in 16-byte units: piece p of row r sits at 16 r + (p xor r); for 8-bit rows at
  // 8 r + (p xor (r / 2)), so that the 16 rows read back at one piece or 8-byte half fall on 16
  // distinct bank groups (r / 2 and r mod 2 tell them apart).  st_w: the slots of the loaded pieces.
  // st_r: the pieces this lane reads back, from row km.  Half split: pieces q, 4 + q, 8 + q, 12 + q
  // (re of bands 8q.., re of 32+8q.., im, im); interleaved: pieces 2q, 2q + 1, 8 + 2q, 9 + 2q.
  // 8-bit rows, half split: the 8-byte halves q % 2 of pieces 2i + q / 2 (the same bands' codes),
  // indexed in 8-byte units; interleaved: pieces q and 4 + q.
  uint4* const st = stage[wave];
  int st_w[NLD], st_r[4];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int r = (64 / RPC) * i + ld_r;
    st_w[i] = r * RPC + (ld_p ^ (E8 ? r >> 1 : r));
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (E8) {
      const int pc = IL ? (i == 0 ? q : 4 + q) : 2 * i + (q >> 1);
      const int slot = km * RPC + (pc ^ (km >> 1));
      st_r[i] = IL ? slot : 2 * slot + (q & 1);
    } else {
      const int pc = IL ? (i < 2 ? 2 * q + i : 8 + 2 * q + (i - 2)) : 4 * i + q;
      st_r[i] = km * kMxRow16 + (pc ^ km);
    }
  }
  const int64_t n_waves = int64_t(gridDim.x) * NW;
  const int64_t w_id = int64_t(blockIdx.x) * NW + wave;
  for_each_segment<kMxKeys>(P, lane, w_id, n_waves, [&](const int s, const int u_in, const int st0,
                                                        const int n_steps) __attribute__((always_inline)) {
    const int64_t unit = int64_t(s) * ups + u_in;
    const int l = u_in / P.n_kvh;
    const int h = u_in - l * P.n_kvh;
    const int L = min(max(P.seq_len[s], 0), int(P.score_stride));
    const int p0 = kMxKeys * st0;                 // a multiple of 16: one page per step
    const int nkeys = min(L - p0, kMxKeys * n_steps);
    const int64_t Q = P.query_pos ? P.query_pos[s] : int64_t(L) - 1;

    // ---- key stream ------------------------------------------------------------------
    const char* kbase = static_cast<const char*>(P.k);
    typedef __attribute__((address_space(4))) const int32_t* mx_const_i32_ptr;
    const mx_const_i32_ptr bt = PAGED ? (mx_const_i32_ptr)(P.block_table + int64_t(s) * P.max_pages) : nullptr;
    const uint64_t pg_bytes = uint64_t(P.n_layer) * uint64_t(P.n_kvh) * uint64_t(kPage * ROW);
    const char* ubase = kbase + (int64_t(l) * P.n_kvh + h) * int64_t(kPage * ROW);
    uint4 ring[PF][NLD];
    // Loads of step n into ring slot sl.  They are issued whatever n is (past the segment's last
    // step the range is empty: the loads return zeros and touch no memory), so that a ring
    // register never merges with an older value under a branch; such a merge makes the compiler
    // wait for every load in flight instead of the one step it needs.
    auto load_step = [&](int n, int sl) __attribute__((always_inline)) {
      const int nc = min(n, n_steps - 1);                    // a valid page-table entry
      const int key0 = p0 + kMxKeys * nc;
      const char* base;
      if constexpr (PAGED) {
        base = ubase + uint64_t(uint32_t(bt[key0 >> 4])) * pg_bytes;
      } else {
        base = kbase + (unit * P.max_len + key0) * ROW;
      }
      const int rem = nkeys - kMxKeys * n;
      const int rows = __builtin_amdgcn_readfirstlane(n < n_steps ? (rem < kMxKeys ? rem : kMxKeys) : 0);
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, rows * ROW, 0x00020000);
#pragma unroll
      for (int i = 0; i < NLD; ++i)
        ring[sl][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off[i], 0, kStreamPolicy));
    };
    // rows of a loaded step into the staging area, and back in the product layout (the wave's own
    // area: LDS operations of one wave run in order, the fence keeps the compiler's order)
    auto stage_write = [&](const uint4 (&r)[NLD]) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < NLD; ++i) st[st_w[i]] = r[i];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    uint4 cur[4];                                  // the current step's pieces, product layout
    auto stage_read = [&]() __attribute__((always_inline)) {
      if constexpr (E8 && IL) {                    // 8-bit: the lane's 32 bytes in cur[0], cur[1]
        cur[0] = st[st_r[0]];
        cur[1] = st[st_r[1]];
      } else if constexpr (E8) {
        const uint2* st2 = reinterpret_cast<const uint2*>(st);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint2 v = st2[st_r[i]];
          if (i & 1) {
            cur[i >> 1].z = v.x;
            cur[i >> 1].w = v.y;
          } else {
            cur[i >> 1].x = v.x;
            cur[i >> 1].y = v.y;
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) cur[i] = st[st_r[i]];
      }
    };
#pragma unroll
    for (int i = 0; i < PF; ++i) load_step(i, i);
    stage_write(ring[0]);                           // step 0 into the product layout
    load_step(PF, 0);
    stage_read();

    // ---- weights of this lane's row: head `head` of the group (0 beyond G) ----------------
    // feature order of a lane: Re x_j, Im x_j at 2j, 2j + 1 (products 0..3 take bands 4p..4p+3),
    // |k_j| at 32 + j (products 4, 5); w[] multiplies the feature at the same index
    float w[kMxFeat];
    {
      const int64_t hrow = int64_t(l) * n_qh + int64_t(h) * P.group + (live_row ? head : 0);
      const float2* c2 = reinterpret_cast<const float2*>(P.center);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int64_t idx = hrow * kBands + mx_band(q, j);
        const float2 c = live_row ? c2[idx] : make_float2(0.0f, 0.0f);
        const float mm = live_row ? P.mean_abs[idx] : 0.0f;
        w[2 * j] = c.x;
        w[2 * j + 1] = c.y;
        w[32 + j] = mm;
      }
    }
    {  // anchor of this segment (float64), one band per lane; after RoPE the key carries its own phase
      const double ang = double(POST ? Q : Q - p0) * P.theta[lane];
      double sa, ca;
      sincos(ang, &sa, &ca);
      const double cr = P.c_re[lane], ci = P.c_im[lane];
      anc[wave][lane] = make_float2(float(cr * ca - ci * sa), float(cr * sa + ci * ca));
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < 16; ++j) {   // W = c A, N = m - |c| (a band with m = 0 has no norm term)
      const float2 A = anc[wave][mx_band(q, j)];
      const float cx = w[2 * j], cy = w[2 * j + 1], mm = w[32 + j];
      w[2 * j] = cx * A.x - cy * A.y;
      w[2 * j + 1] = -(cx * A.y + cy * A.x);
      w[32 + j] = (mm > 0.0f) ? mm - __builtin_sqrtf(cx * cx + cy * cy) : 0.0f;
    }
    if constexpr (E8) {
      if (P.k_scale) {   // stored key = true key / scale: both terms are linear in the key
        const float ks = P.k_scale[int64_t(l) * P.n_kvh + h];
#pragma unroll
        for (int i = 0; i < kMxFeat; ++i) w[i] *= ks;
      }
    }
    // the weight operands: the row's high parts, or its remainders
    mx_u32x4 am[kMxProducts];
    auto pack_weights = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int p = 0; p < kMxProducts; ++p)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // keys after RoPE: the trig products take the raw key pieces, so their weights follow the
          // pieces' element order, Re W for a real part and Im W (= -w[2j + 1]) for an imaginary one
          float w0 = w[8 * p + 2 * e], w1 = w[8 * p + 2 * e + 1];
          if (POST && p < 4) {
            const int i0 = mx_post_index(IL, p, 2 * e), i1 = mx_post_index(IL, p, 2 * e + 1);
            w0 = (i0 & 1) ? -w[i0] : w[i0];
            w1 = (i1 & 1) ? -w[i1] : w[i1];
          }
          am[p][e] = lo_row ? mx_pack_rne(w0 - mx_hi(w0), w1 - mx_hi(w1)) : mx_pack_hi(w0, w1);
        }
    };
    pack_weights();

    float* out = P.scores + unit * P.score_stride + p0;
    mx_f32x4 acc[2];
    float te = 0.0f, pa = 0.0f;      // the even step of a pair; the first pair of a 4-step group
    // lane (q, km) stores key km of step so of each 4-step group, so = 0, 2, 1, 3 for q = 0..3
    const int so = ((q & 1) << 1) | (q >> 1);
    // reduction of step n's accumulator (rows 4q..4q+3 of column km; the initial value drops
    // heads past the group): the lane's two heads' maximum, then, for a pair of steps at once,
    // the maximum over the four lane groups by a 32-lane swap of the two steps' values and a
    // 16-lane swap of the result (rows 0, 1 then hold the even step's scores, rows 2, 3 the odd
    // one's); every second pair completes a group of 64 consecutive keys, one per lane
    auto finish = [&](const mx_f32x4& c, int n, bool last) __attribute__((always_inline)) {
      const float t = __builtin_fmaxf(c[0] + c[1], c[2] + c[3]);
      if ((n & 1) == 0 && !last) {
        te = t;
        return;
      }
      const float e = (n & 1) ? te : t;   // an even last step pairs with itself
      const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(e), __float_as_uint(t), false, false);
      const float a = __builtin_fmaxf(__uint_as_float(x[0]), __uint_as_float(x[1]));
      const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
      const float pr = __builtin_fmaxf(__uint_as_float(y[0]), __uint_as_float(y[1]));
      if ((n & 2) == 0) {
        pa = pr;
        if (!last) return;
      }
      const float v = (q & 1) ? pr : pa;
      const int key = kMxKeys * ((n & ~3) + so) + km;
      if (so <= (n & 3) && key < nkeys) __builtin_nontemporal_store(v, out + key);
    };
    // n0: first step of the current chunk; steps n0 + it >= n_steps of the last chunk compute
    // nothing, but still issue their (empty) loads
    for (int n0 = 0; n0 < n_steps; n0 += STEPS) {
      int tz = lane;
      asm volatile("" : "+v"(tz));
      if (!POST && n0 > 0) {  // next chunk: W <- W e^{-i kMxChunk theta_f}, then new weight operands
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float2 R = stepc[mx_band(q, j)];
          const float a = w[2 * j], b = w[2 * j + 1];
          w[2 * j] = fmaf(a, R.x, b * R.y);
          w[2 * j + 1] = fmaf(b, R.x, -(a * R.y));
        }
        pack_weights();
      }
#pragma unroll
      for (int it = 0; it < STEPS; ++it) {
        const int n = n0 + it;
        const bool live = n < n_steps;                        // wave-uniform
        const float4* tp = tab + it * 8 * 64 + tz;
        mx_f32x4& ac = acc[it & 1];
        float kabs[16];
        if (E8 && live) {
          // 8-bit keys after RoPE: the codes' values (exact in float32, and in bfloat16: at most 8
          // significant bits) give |k_f| and, packed as bfloat16 in the raw pieces' element order,
          // the trig products' key operand
          ac = init;
          float re[16], im[16];
          mx_decode8<DT, IL>([&](int k) { return word(cur[k >> 2], k & 3); }, re, im);
#pragma unroll
          for (int j = 0; j < 16; ++j) kabs[j] = __builtin_amdgcn_sqrtf(fmaf(re[j], re[j], im[j] * im[j]));
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            mx_u32x4 bk;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i0 = mx_post_index(IL, p, 2 * e), i1 = mx_post_index(IL, p, 2 * e + 1);
              bk[e] = mx_pack_hi((i0 & 1) ? im[i0 >> 1] : re[i0 >> 1], (i1 & 1) ? im[i1 >> 1] : re[i1 >> 1]);
            }
            ac = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mx_bf16x8, am[p]),
                                                          __builtin_bit_cast(mx_bf16x8, bk), ac, 0, 0, 0);
          }
        } else if (!E8 && POST && live) {
          // keys after RoPE: x_f = conj(k'_f), so Re(W x) = Re W Re k' + Im W Im k' and the trig
          // products take the raw bfloat16 pieces (exact) as the key operand, one product per piece;
          // |k_f| = |k'_f| from the same words
          ac = init;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
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
            kabs[j] = __builtin_amdgcn_sqrtf(fmaf(a, a, b * b));
          }
#pragma unroll
          for (int p = 0; p < 4; ++p)
            ac = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mx_bf16x8, am[p]),
                                                          __builtin_bit_cast(mx_bf16x8, cur[p]), ac, 0, 0, 0);
        } else if (!POST && live) {
          ac = init;
#pragma unroll
          for (int p = 0; p < 4; ++p) {            // trig features of bands 4p..4p+3
            float x[8];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
              const float4 t = tp[(2 * p + jj) * 64];
#pragma unroll
              for (int e = 0; e < 2; ++e) {
                const int j = 4 * p + 2 * jj + e;
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
                x[4 * jj + 2 * e] = fmaf(tc, a, ts * b);           // Re(e^{-i r theta} conj(k))
                x[4 * jj + 2 * e + 1] = fmaf(ts, a, -(tc * b));    // Im(...)
                kabs[j] = __builtin_amdgcn_sqrtf(fmaf(a, a, b * b));
              }
            }
            mx_u32x4 bh, bl;
            mx_split8(x, bh, bl);
            ac = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mx_bf16x8, am[p]),
                                                          __builtin_bit_cast(mx_bf16x8, bh), ac, 0, 0, 0);
            ac = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mx_bf16x8, am[p]),
                                                          __builtin_bit_cast(mx_bf16x8, bl), ac, 0, 0, 0);
          }
        }
        // the next step: its rows (loaded two steps ago) through the staging area into cur (free
        // now: this step's features are formed), and its ring slot refilled
        stage_write(ring[(it + 1) % PF]);
        load_step(n + 1 + PF, (it + 1) % PF);
        stage_read();
        if (live) {
#pragma unroll
          for (int p = 4; p < 6; ++p) {            // |k| of bands 8(p - 4)..8(p - 4) + 7
            mx_u32x4 bh, bl;
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = kabs[8 * (p - 4) + e];
            mx_split8(x, bh, bl);
            ac = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mx_bf16x8, am[p]),
                                                          __builtin_bit_cast(mx_bf16x8, bh), ac, 0, 0, 0);
            ac = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mx_bf16x8, am[p]),
                                                          __builtin_bit_cast(mx_bf16x8, bl), ac, 0, 0, 0);
          }
          if (n > 0) finish(acc[(it & 1) ^ 1], n - 1, false);   // the previous step's products are done by now
        }
      }
    }
    if (n_steps > 0) finish(acc[(n_steps - 1) & 1], n_steps - 1, true);
  });
}

template <int G, bool IL, bool PAGED, bool POST, int DT = 1>
hipError_t launch_mx_case(const ScoreParams& p, int grid, hipStream_t st) {
  hipLaunchKernelGGL((score_mx_kernel<G, IL, PAGED, POST, DT>), dim3(grid), dim3(kScoreWaves * 64), 0, st, p);
  return hipGetLastError();
}

}  // namespace
}  // namespace tri
