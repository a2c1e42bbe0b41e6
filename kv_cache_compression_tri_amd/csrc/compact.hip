// Forward-packing compaction kernels of the TriAttention compression pass (gfx950).
//
// Survivors are moved forward so that they fill as few blocks as possible and the tail
// blocks become empty and reclaimable ("TriAttention: How a Geometric Trick Cuts LLM Memory
// Use by 10x Without Losing Accuracy", sections "Solving the Memory Fragmentation Problem"
// and "Why Existing KV Cache Compression Breaks in Production": a paged allocator can only
// free a block that is completely empty).
//
// Dense (out of place): one workgroup of kDenseCopyThreads threads per (unit, group of
// output rows).  ROW/16 lanes copy one row (128 B fp8, 256 B bf16, 512 B float32) with
// 16-byte loads and stores, so a workgroup moves 16, 8 or 4 rows of K and of V and each
// thread one piece of each.  Many small workgroups keep every CU busy with some loading
// while others store: same-process timing of the 32K pass's compaction (288 units x 2048
// bf16 rows of K and V) gave 0.113 ms with 256 threads moving 64 rows, 0.105 ms with 16
// rows, 0.102 ms with 128 threads moving 8 rows (5.9 TB/s).
//
// Paged (in place): one workgroup per unit walks its destination slots in chunks of 64,
// in increasing order; each chunk loads all of its source rows into registers, waits for
// the loads, synchronises, then stores.  Safety: kept[] is strictly ascending, so
// kept[i] >= i.  A source row read for destination i is overwritten only by destination
// kept[i] >= i, i.e. in the same chunk (after the barrier) or a later one; rows with
// kept[i] == i are not touched.  Units of one sequence own disjoint (layer, head) slices of
// each page, so workgroups never touch the same bytes.
#include "tri_internal.h"

namespace tri {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kRowsPerChunk = 64;

// Rows are moved exactly once, so the loads and stores carry the non-temporal hint (the
// copy then streams instead of filling the caches with rows nobody reads again).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_row_piece(const char* p) {
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ void store_row_piece(char* p, const uint4& v) {
  const u32x4 t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<u32x4*>(p));
}

template <int ESZ>
__global__ __launch_bounds__(kDenseCopyThreads) void compact_dense_kernel(const CompactParams P,
                                                                           bool with_v) {
  constexpr int ROW = kHeadDim * ESZ;
  constexpr int TPR = ROW / 16;                    // lanes per row
  constexpr int RPB = kDenseCopyThreads / TPR;     // rows per workgroup
  static_assert(RPB == dense_copy_rows(ESZ), "row geometry");
  const int64_t unit = blockIdx.x / P.chunks_per_unit;
  const int chunk = int(blockIdx.x - unit * P.chunks_per_unit);
  const int s = int(unit / P.units_per_seq);
  const int L = min(max(P.seq_len[s], 0), int(P.pos_stride));
  const int n = min(min(P.kept_n[s], L), P.budget);
  const int tid = threadIdx.x;
  if (P.new_len && chunk == 0 && tid == 0 && unit % P.units_per_seq == 0) P.new_len[s] = n;
  const int i = chunk * RPB + tid / TPR;
  if (i >= n) return;
  const int src = P.kept[unit * P.budget + i];
  if (src < 0 || src >= L) return;
  const int part = tid % TPR;
  const int64_t so = (unit * P.max_len + src) * ROW + part * 16;
  const uint4 kb = load_row_piece(static_cast<const char*>(P.k) + so);
  uint4 vb;
  if (with_v) vb = load_row_piece(static_cast<const char*>(P.v) + so);
  const int64_t dof = (unit * P.budget + i) * ROW + part * 16;
  store_row_piece(static_cast<char*>(P.k_out) + dof, kb);
  if (with_v) store_row_piece(static_cast<char*>(P.v_out) + dof, vb);
  if (P.pos_out && part == 0) P.pos_out[unit * P.budget + i] = P.pos ? P.pos[unit * P.pos_stride + src] : src;
}

template <int ESZ>
__global__ __launch_bounds__(kCopyThreads) void compact_paged_kernel(const CompactParams P,
                                                                      bool with_v) {
  constexpr int ROW = kHeadDim * ESZ;
  constexpr int TPR = ROW / 16;
  constexpr int RPP = kCopyThreads / TPR;
  constexpr int PASSES = kRowsPerChunk / RPP;
  const int64_t unit = blockIdx.x;
  const int s = int(unit / P.units_per_seq);
  const int rem = int(unit - int64_t(s) * P.units_per_seq);
  const int l = rem / P.n_kvh, h = rem - l * P.n_kvh;
  const int L = min(max(P.seq_len[s], 0), int(P.pos_stride));
  const int n = min(min(P.kept_n[s], L), P.budget);
  const int tid = threadIdx.x;
  const int32_t* kp = P.kept + unit * P.budget;
  const int32_t* bt = P.block_table + int64_t(s) * P.max_pages;
  const int part = tid % TPR;
  char* kpool = const_cast<char*>(static_cast<const char*>(P.k));
  char* vpool = const_cast<char*>(static_cast<const char*>(P.v));
  auto row_off = [&](int slot) -> int64_t {
    const int64_t page = bt[slot >> 4];
    return ((((page * P.n_layer + l) * P.n_kvh + h) * kPage) + (slot & 15)) * ROW + part * 16;
  };

  for (int i0 = 0; i0 < n; i0 += kRowsPerChunk) {
    uint4 kb[PASSES], vb[PASSES];
    int dst[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int i = i0 + p * RPP + tid / TPR;
      dst[p] = -1;
      if (i < n) {
        const int src = kp[i];
        if (src != i && src >= 0 && src < L) {
          const int64_t so = row_off(src);
          kb[p] = load_row_piece(kpool + so);
          if (with_v) vb[p] = load_row_piece(vpool + so);
          dst[p] = i;
        }
      }
    }
    // every source row of this chunk is in registers before any destination is written
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      if (dst[p] >= 0) {
        const int64_t d = row_off(dst[p]);
        store_row_piece(kpool + d, kb[p]);
        if (with_v) store_row_piece(vpool + d, vb[p]);
      }
    }
  }
  if (P.pos_out)
    for (int i = tid; i < n; i += kCopyThreads)
      P.pos_out[unit * P.budget + i] =
          (P.pos && kp[i] >= 0 && kp[i] < L) ? P.pos[unit * P.pos_stride + kp[i]] : kp[i];
  if (rem == 0) {  // once per sequence: the emptied tail pages and the new length
    const int used_before = (L + kPage - 1) / kPage;
    const int used_after = (n + kPage - 1) / kPage;
    const int nf = used_before - used_after;
    if (P.n_freed && tid == 0) P.n_freed[s] = nf;
    if (P.freed)
      for (int m = tid; m < nf; m += kCopyThreads) P.freed[int64_t(s) * P.max_pages + m] = bt[used_after + m];
    if (P.new_len && tid == 0) P.new_len[s] = n;
  }
}

template <int ESZ>
void launch_compact_esz(const CompactParams& p, int64_t n_units, bool paged, bool with_v,
                        hipStream_t stream) {
  if (paged)
    hipLaunchKernelGGL(compact_paged_kernel<ESZ>, dim3(unsigned(n_units)), dim3(kCopyThreads), 0, stream, p,
                       with_v);
  else
    hipLaunchKernelGGL(compact_dense_kernel<ESZ>, dim3(unsigned(n_units * p.chunks_per_unit)),
                       dim3(kDenseCopyThreads), 0, stream, p, with_v);
}

}  // namespace

hipError_t launch_compact(const CompactParams& p, int64_t n_units, int elem_bytes, bool paged,
                          bool with_v, hipStream_t stream) {
  switch (elem_bytes) {
    case 1: launch_compact_esz<1>(p, n_units, paged, with_v, stream); break;
    case 2: launch_compact_esz<2>(p, n_units, paged, with_v, stream); break;
    case 4: launch_compact_esz<4>(p, n_units, paged, with_v, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace tri
