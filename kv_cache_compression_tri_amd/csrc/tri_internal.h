// Internal launch descriptors shared by the host API and the kernels of libtri.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tri {

constexpr int kHeadDim = 128;
constexpr int kBands = 64;          // F = head_dim / 2 RoPE frequency bands
constexpr int kPage = 16;           // paged-cache block size (tokens)
constexpr int kMaxGroup = 8;        // query heads per KV head
constexpr int kMaxOffsets = 64;
constexpr int64_t kMaxUnitLen = 1 << 20;

// Score kernel geometry: 8 lanes per key (8 bands each), 8 keys per wave per step, phase
// table of kChunk consecutive offsets in LDS, weights re-anchored every kChunk keys, one
// persistent workgroup of kScoreWaves waves per CU, at least kMinWaveSteps 8-key steps per
// wave (so that the per-segment set-up stays small next to the streaming).
constexpr int kChunk = 256;
constexpr int kScoreWaves = 8;      // waves per workgroup
constexpr int kMinWaveSteps = 32;

struct ScoreParams {
  const void* k;
  const int32_t* seq_len;
  const int64_t* query_pos;
  const int32_t* block_table;
  const float* center;       // [n_layer][n_qh][64][2]
  const float* mean_abs;     // [n_layer][n_qh][64]
  const float* k_scale;      // optional [n_layer][n_kvh] (8-bit keys): key = code * scale
  const int32_t* pos;        // optional [units][score_stride] key positions (pre-RoPE keys)
  float* scores;
  int64_t max_len;           // dense token stride
  int64_t score_stride;      // slots per unit in `scores`
  int32_t n_seq, n_layer, n_kvh, group, max_pages;
  int32_t reduce_mean;
  double theta[kBands];      // theta_f, float64
  double c_re[kBands];       // C_f = mean over offsets of exp(i Delta theta_f), float64
  double c_im[kBands];
};

struct SelectParams {
  const float* scores;
  int64_t score_stride;
  const int32_t* seq_len;
  int32_t* kept;
  int32_t* kept_n;
  int32_t budget;
  int32_t window;
  int32_t units_per_seq;
};

struct CompactParams {
  const void* k;             // dense source or paged pool
  const void* v;
  void* k_out;               // dense only
  void* v_out;
  const int32_t* kept;
  const int32_t* kept_n;
  const int32_t* seq_len;
  const int32_t* block_table;
  const int32_t* pos;
  int32_t* pos_out;
  int32_t* freed;
  int32_t* n_freed;
  int32_t* new_len;
  int64_t max_len;           // dense token stride
  int64_t pos_stride;        // slots per unit of `pos`
  int32_t budget;
  int32_t units_per_seq;
  int32_t n_layer, n_kvh, max_pages;
  int32_t chunks_per_unit;   // dense: ceil(budget / dense_copy_rows(element bytes))
};

// Dense compaction: each thread of a kDenseCopyThreads-thread workgroup moves one 16-byte
// piece of a kept row of K and of V, so a workgroup covers this many output rows.
constexpr int kDenseCopyThreads = 128;
constexpr int dense_copy_rows(int elem_bytes) { return kDenseCopyThreads * 16 / (kHeadDim * elem_bytes); }

struct CalibParams {
  const void* q;
  int64_t n;
  int32_t n_layer, n_qh;
  float* center;
  float* mean_abs;
};

// launchers (return hipError_t of the launch)
hipError_t launch_score(const ScoreParams& p, int G_eff, int dtype, bool interleaved, bool paged,
                        bool post, bool mult, int grid, hipStream_t stream);
hipError_t launch_score_pos(const ScoreParams& p, int G_eff, int dtype, bool interleaved, bool paged, int grid,
                            hipStream_t stream);
// fused scoring and selection, one workgroup per unit of at most kFuseMaxSlots slots (float32 /
// bfloat16 keys before RoPE at their slots, additive form; dense or paged)
constexpr int kFuseMaxSlots = 32768;
hipError_t launch_score_select(const ScoreParams& p, const SelectParams& s, int G_eff, int dtype, bool interleaved,
                               bool paged, int64_t units, hipStream_t stream);
hipError_t launch_score_select_f32(const ScoreParams& p, const SelectParams& s, int G_eff, bool interleaved,
                                   int64_t units, hipStream_t stream);
hipError_t launch_score_select_bf16_paged(const ScoreParams& p, const SelectParams& s, int G_eff, bool interleaved,
                                          int64_t units, hipStream_t stream);
hipError_t launch_score_select_f32_paged(const ScoreParams& p, const SelectParams& s, int G_eff, bool interleaved,
                                         int64_t units, hipStream_t stream);
// the matrix-core scoring kernel (bfloat16 keys, additive form, max over the group's heads;
// before RoPE at consecutive positions, or cached after RoPE) and the shapes it takes
bool score_mx_applies(int G_eff, int dtype, bool post, bool mult, bool positions, bool reduce_mean);
hipError_t launch_score_mx(const ScoreParams& p, int G_eff, int dtype, bool interleaved, bool paged, bool post,
                           int grid, hipStream_t stream);
hipError_t launch_score_mx_paged(const ScoreParams& p, int G_eff, bool interleaved, int grid, hipStream_t stream);
hipError_t launch_score_mx_post(const ScoreParams& p, int G_eff, bool interleaved, int grid, hipStream_t stream);
hipError_t launch_score_mx_post_paged(const ScoreParams& p, int G_eff, bool interleaved, int grid,
                                      hipStream_t stream);
hipError_t launch_score_mx_post_8bit(const ScoreParams& p, int G_eff, int dtype, bool interleaved, bool paged,
                                     int grid, hipStream_t stream);
hipError_t launch_score_pos_8bit(const ScoreParams& p, int G_eff, int dtype, bool interleaved, bool paged,
                                 int grid, hipStream_t stream);
hipError_t launch_score_mult(const ScoreParams& p, int G_eff, int dtype, bool interleaved, bool paged,
                            int grid, hipStream_t stream);
hipError_t launch_score_post_mult(const ScoreParams& p, int G_eff, int dtype, bool interleaved, bool paged,
                                 int grid, hipStream_t stream);
hipError_t launch_score_mult_8bit(const ScoreParams& p, int G_eff, int dtype, bool interleaved, bool paged,
                                 int grid, hipStream_t stream);
hipError_t launch_score_post_mult_8bit(const ScoreParams& p, int G_eff, int dtype, bool interleaved, bool paged,
                                      int grid, hipStream_t stream);
hipError_t launch_score_post(const ScoreParams& p, int G_eff, int dtype, bool interleaved, bool paged,
                             int grid, hipStream_t stream);
hipError_t launch_score_8bit(const ScoreParams& p, int G_eff, int dtype, bool interleaved, bool paged,
                             int grid, hipStream_t stream);
hipError_t launch_score_post_8bit(const ScoreParams& p, int G_eff, int dtype, bool interleaved, bool paged,
                                  int grid, hipStream_t stream);
// Attention of the newest query over a compressed cache (decode.hip).
struct DecodeParams {
  double theta_turns[kBands];   // theta_f / (2 pi), float64
  const void* k;
  const void* v;
  const int32_t* seq_len;
  const int32_t* block_table;
  const int32_t* pos;           // [n_seq][n_layer][n_kvh][pos_stride] or NULL (position = slot)
  const int64_t* query_pos;     // [n_seq]
  const float* q;               // [n_seq][n_layers][n_qh][128]
  float* out;                   // [n_seq][n_layers][n_qh][128]
  int64_t max_len, slots, pos_stride;
  int32_t n_seq, n_layer, n_kvh, group, max_pages, layer0, n_layers;
  int32_t n_pass;               // passes over the keys (4 query heads each); set by the launcher
  // Split over the key slots: n_split workgroups per (sequence, layer, KV head, pass), each
  // over split_len slots, write partial softmax states that a second kernel merges.
  // n_split == 1: one workgroup writes out directly (no workspace).
  int32_t n_split;
  int64_t split_len;            // multiple of 64
  float* part_ml;               // [units * n_pass][n_split][4][2]   (reference max, base 2; sum)
  float* part_acc;              // [units * n_pass][n_split][4][128] (unnormalised value sums)
};
// Slot splits for the attention kernel.  A CU holds four of its (bfloat16) workgroups at once;
// the kernel streams best with several per CU, so groups are split (a power of two ways)
// until every CU has kDecodeMinGroupsPerCU of them, keeping kDecodeMinSplitLen slots or more
// per split (fitted to same-process timings on MI355X, 256 CUs).  The partial states then
// stay under 2 * 4 * 256 groups x 4 heads x 520 bytes (4.3 MB).
constexpr int kDecodeCUs = 256;
constexpr int kDecodeMinGroupsPerCU = 4;
constexpr int kDecodeMinSplitLen = 128;
constexpr int kDecodeMaxSplits = 16;
constexpr int kDecodeHeadsPerPass = 4;
// slot splits the attention kernel uses for this many (sequence, layer, KV head, pass)
// groups, and the workspace they need (0 for one split)
int decode_splits(int64_t unit_passes, int64_t slots);
int64_t decode_workspace_bytes(int64_t unit_passes, int n_split);
hipError_t launch_decode_attention(const DecodeParams& p, bool bf16, bool interleaved, bool paged, bool post,
                                   hipStream_t stream);

// selection; with a workspace of select_workspace_bytes (> 0 only for units longer than the
// register-resident capacity), the two-stage tournament, otherwise one workgroup per unit
size_t select_workspace_bytes(const SelectParams& p, int64_t n_units);
hipError_t launch_select(const SelectParams& p, int64_t n_units, void* ws, hipStream_t stream);
hipError_t launch_compact(const CompactParams& p, int64_t n_units, int elem_bytes, bool paged,
                          bool with_v, hipStream_t stream);
hipError_t launch_calib(const CalibParams& p, bool bf16, bool interleaved, hipStream_t stream);

}  // namespace tri
