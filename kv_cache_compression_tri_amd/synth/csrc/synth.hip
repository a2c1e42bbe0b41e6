// Device implementation of the seeded key/value generator (test and benchmark
// infrastructure; holds no step of the compression method).
//
// Same definition as the numpy implementation in synth/__init__.py, bit for bit:
//   hash   = SplitMix64 output function mix64 (Steele, Lea & Flood, OOPSLA 2014) at
//            stream index n: mix64(key + n * 0x9E3779B97F4A7C15), key = mix64(seed<<8|tag)
//   normal = (sum of twelve 16-bit fields of the hashes at n = 3c+1, 3c+2, 3c+3) - 393210,
//            times 2^-16 (Irwin-Hall(12) - 6, exact in float32)
//   value  = mu[col] + sigma[col] * normal, each float32 operation rounded once (no FMA),
//            times 20 on a sink row (row 0), then RNE to bfloat16, kept as float32, or
//            (fp8, int8) times a power-of-two inverse scale and encoded as OCP E4M3 with
//            round-to-nearest-even, saturating at +-448, or as int8 with round-to-nearest-
//            even, clamped to [-127, 127]
//   counter c = unit << 27 | row << 7 | col
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float element(uint64_t key, uint64_t unit, uint32_t row, uint32_t col,
                                         float mu, float sigma, bool sink_row) {
  // each float32 operation must round on its own, as on the host: no contraction into FMA
#pragma clang fp contract(off)
  const uint64_t c = (unit << 27) | (uint64_t(row) << 7) | col;
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const uint64_t h = mix64(key + (3ull * c + uint64_t(i + 1)) * kGamma);
    s += uint32_t(h & 0xFFFF) + uint32_t((h >> 16) & 0xFFFF) + uint32_t((h >> 32) & 0xFFFF) +
         uint32_t(h >> 48);
  }
  const float n = float(int32_t(s) - 393210) * (1.0f / 65536.0f);
  float x = __fadd_rn(mu, __fmul_rn(sigma, n));
  if (sink_row) x = __fmul_rn(20.0f, x);
  return x;
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
  const uint32_t u = __float_as_uint(x);
  return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// OCP E4M3: round to nearest even on the float32 bits; normal codes for |x| >= 2^-6,
// subnormal steps of 2^-9 below; magnitudes rounding past 448 saturate to 448; NaN -> S.1111.111
__device__ __forceinline__ uint32_t to_fp8_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;
  int e = int(a >> 23) - 127;
  uint32_t code;
  if (e >= -6) {
    uint32_t r = (a >> 20) & 7u;
    const uint32_t rem = a & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ++r;
    if (r == 8u) {
      r = 0u;
      ++e;
    }
    code = e > 8 ? 0x7Eu : ((uint32_t(e + 7) << 3) | r);
    if (code > 0x7Eu) code = 0x7Eu;
  } else {
    code = uint32_t(rintf(__uint_as_float(a) * 512.0f));   // exact scaling, then RNE: 0..8
  }
  return sign | code;
}

// int8: round to nearest even, clamp to [-127, 127]
__device__ __forceinline__ uint32_t to_int8(float x) {
  const float r = fminf(fmaxf(rintf(x), -127.0f), 127.0f);
  return uint32_t(int32_t(r)) & 0xFFu;
}

// 8 consecutive columns per thread; DT 0 = float32, 1 = bfloat16, 2 = fp8 E4M3, 3 = int8.
template <int DT>
__device__ __forceinline__ void write8(void* dst, uint64_t key, uint64_t unit, uint32_t row,
                                       uint32_t col0, const float* mu, const float* sigma,
                                       bool sink_row, float inv_scale) {
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    v[e] = element(key, unit, row, col0 + e, mu[col0 + e], sigma[col0 + e], sink_row);
  if (DT >= 2) {
    uint32_t c[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      c[e] = DT == 2 ? to_fp8_e4m3(__fmul_rn(v[e], inv_scale)) : to_int8(__fmul_rn(v[e], inv_scale));
    uint2 w;
    w.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
    w.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
    *reinterpret_cast<uint2*>(dst) = w;
  } else if (DT == 1) {
    uint4 w;
    w.x = uint32_t(to_bf16(v[0])) | (uint32_t(to_bf16(v[1])) << 16);
    w.y = uint32_t(to_bf16(v[2])) | (uint32_t(to_bf16(v[3])) << 16);
    w.z = uint32_t(to_bf16(v[4])) | (uint32_t(to_bf16(v[5])) << 16);
    w.w = uint32_t(to_bf16(v[6])) | (uint32_t(to_bf16(v[7])) << 16);
    *reinterpret_cast<uint4*>(dst) = w;
  } else {
    float4* d = reinterpret_cast<float4*>(dst);
    d[0] = make_float4(v[0], v[1], v[2], v[3]);
    d[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

template <int DT>
__global__ void fill_dense_kernel(void* out, int64_t n_units, int64_t max_len, int32_t n_model_units,
                                  const float* __restrict__ mu, const float* __restrict__ sigma,
                                  int32_t sink, uint64_t key, const float* __restrict__ inv_scale) {
  const int64_t total = n_units * max_len * 16;  // 16 groups of 8 columns per row
  const size_t esz = DT >= 2 ? 1 : (DT == 1 ? 2 : 4);
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * blockDim.x) {
    const uint32_t cg = uint32_t(i & 15);
    const int64_t r = i >> 4;
    const uint32_t row = uint32_t(r % max_len);
    const int64_t unit = r / max_len;
    const float* m = mu + int64_t(unit % n_model_units) * 128;
    char* dst = static_cast<char*>(out) + (r * 128 + cg * 8) * esz;
    const float isc = inv_scale ? inv_scale[unit % n_model_units] : 1.0f;
    write8<DT>(dst, key, uint64_t(unit), row, cg * 8, m, sigma, sink && row == 0, isc);
  }
}

template <int DT>
__global__ void fill_paged_kernel(void* pool, int32_t n_seq, int32_t n_layer, int32_t n_kvh,
                                  int32_t page, int32_t max_pages,
                                  const int32_t* __restrict__ block_table,
                                  const int32_t* __restrict__ seq_len,
                                  const float* __restrict__ mu, const float* __restrict__ sigma,
                                  int32_t sink, uint64_t key, const float* __restrict__ inv_scale) {
  // one work index per (seq, page slot, layer, head, row-in-page, column group)
  const int64_t per_page = int64_t(n_layer) * n_kvh * page * 16;
  const int64_t total = int64_t(n_seq) * max_pages * per_page;
  const size_t esz = DT >= 2 ? 1 : (DT == 1 ? 2 : 4);
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * blockDim.x) {
    const uint32_t cg = uint32_t(i & 15);
    int64_t r = i >> 4;
    const int32_t prow = int32_t(r % page);
    r /= page;
    const int32_t h = int32_t(r % n_kvh);
    r /= n_kvh;
    const int32_t l = int32_t(r % n_layer);
    r /= n_layer;
    const int32_t pslot = int32_t(r % max_pages);
    const int32_t s = int32_t(r / max_pages);
    const int32_t slot = pslot * page + prow;
    if (slot >= seq_len[s]) continue;
    const int64_t pg = block_table[int64_t(s) * max_pages + pslot];
    const uint64_t unit = (uint64_t(s) * n_layer + l) * n_kvh + h;
    const float* m = mu + (int64_t(l) * n_kvh + h) * 128;
    const int64_t elem = (((pg * n_layer + l) * n_kvh + h) * page + prow) * 128 + cg * 8;
    const float isc = inv_scale ? inv_scale[int64_t(l) * n_kvh + h] : 1.0f;
    write8<DT>(static_cast<char*>(pool) + elem * esz, key, unit, uint32_t(slot), cg * 8, m,
               sigma, sink && slot == 0, isc);
  }
}

uint64_t host_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

int grid_for(int64_t work) {
  int64_t g = (work + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return int(g);
}

}  // namespace

extern "C" {

// Fill a dense [n_units][max_len][128] cache (dtype 0 = float32, 1 = bfloat16, 2 = fp8 E4M3,
// 3 = int8).
// mu: device [n_model_units][128] float32 (unit u uses row u % n_model_units);
// sigma: device [128] float32; inv_scale: 8-bit only, device [n_model_units] float32 powers of
// two (NULL = 1).  Returns 0, -1 on a bad argument, -4 on a HIP error.
int tri_synth_fill_dense(void* out, int32_t dtype, int64_t n_units, int64_t max_len,
                         int32_t n_model_units, const float* mu, const float* sigma,
                         int32_t sink, uint64_t seed, uint32_t tag, const float* inv_scale,
                         void* stream) {
  if (!out || !mu || !sigma || n_units <= 0 || max_len <= 0 || max_len > (1 << 20) ||
      n_model_units <= 0 || dtype < 0 || dtype > 3 || seed >= (1ull << 56) || tag > 255)
    return -1;
  const uint64_t key = host_mix64((seed << 8) | tag);
  const int grid = grid_for(n_units * max_len * 16);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == 3)
    hipLaunchKernelGGL(fill_dense_kernel<3>, dim3(grid), dim3(256), 0, st, out, n_units, max_len,
                       n_model_units, mu, sigma, sink, key, inv_scale);
  else if (dtype == 2)
    hipLaunchKernelGGL(fill_dense_kernel<2>, dim3(grid), dim3(256), 0, st, out, n_units, max_len,
                       n_model_units, mu, sigma, sink, key, inv_scale);
  else if (dtype == 1)
    hipLaunchKernelGGL(fill_dense_kernel<1>, dim3(grid), dim3(256), 0, st, out, n_units, max_len,
                       n_model_units, mu, sigma, sink, key, inv_scale);
  else
    hipLaunchKernelGGL(fill_dense_kernel<0>, dim3(grid), dim3(256), 0, st, out, n_units, max_len,
                       n_model_units, mu, sigma, sink, key, inv_scale);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Fill a paged pool [n_pages][n_layer][n_kvh][page][128] through per-sequence block tables
// (device [n_seq][max_pages]) for slots < seq_len[s] (device [n_seq]).  mu: device
// [n_layer][n_kvh][128]; unit index of (s, l, h) is (s * n_layer + l) * n_kvh + h;
// inv_scale: 8-bit only, device [n_layer][n_kvh] (NULL = 1).
int tri_synth_fill_paged(void* pool, int32_t dtype, int32_t n_seq, int32_t n_layer, int32_t n_kvh,
                         int32_t page, int32_t max_pages, const int32_t* block_table,
                         const int32_t* seq_len, const float* mu, const float* sigma,
                         int32_t sink, uint64_t seed, uint32_t tag, const float* inv_scale,
                         void* stream) {
  if (!pool || !block_table || !seq_len || !mu || !sigma || n_seq <= 0 || n_layer <= 0 ||
      n_kvh <= 0 || page <= 0 || max_pages <= 0 || int64_t(page) * max_pages > (1 << 20) ||
      dtype < 0 || dtype > 3 || seed >= (1ull << 56) || tag > 255)
    return -1;
  const uint64_t key = host_mix64((seed << 8) | tag);
  const int64_t work = int64_t(n_seq) * max_pages * n_layer * n_kvh * page * 16;
  const int grid = grid_for(work);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == 3)
    hipLaunchKernelGGL(fill_paged_kernel<3>, dim3(grid), dim3(256), 0, st, pool, n_seq, n_layer, n_kvh,
                       page, max_pages, block_table, seq_len, mu, sigma, sink, key, inv_scale);
  else if (dtype == 2)
    hipLaunchKernelGGL(fill_paged_kernel<2>, dim3(grid), dim3(256), 0, st, pool, n_seq, n_layer, n_kvh,
                       page, max_pages, block_table, seq_len, mu, sigma, sink, key, inv_scale);
  else if (dtype == 1)
    hipLaunchKernelGGL(fill_paged_kernel<1>, dim3(grid), dim3(256), 0, st, pool, n_seq, n_layer, n_kvh,
                       page, max_pages, block_table, seq_len, mu, sigma, sink, key, inv_scale);
  else
    hipLaunchKernelGGL(fill_paged_kernel<0>, dim3(grid), dim3(256), 0, st, pool, n_seq, n_layer, n_kvh,
                       page, max_pages, block_table, seq_len, mu, sigma, sink, key, inv_scale);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
