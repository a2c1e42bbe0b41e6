// C ABI of libtri.so: argument validation, float64 coefficient preparation and kernel
// dispatch for the TriAttention KV-cache compression pass.  The entry points and their
// contracts are declared and documented in include/tri.h.
#include "tri.h"
#include "tri_internal.h"

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

namespace {

thread_local std::string g_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(TRI_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// Compute units of the current device (cached per device id; calls may come from several
// host threads at once).
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

int64_t slots_of(const tri_kv* kv) {
  return kv->layout == TRI_PAGED ? int64_t(kv->max_pages) * kv->page : kv->max_len;
}

int elem_bytes(int32_t dtype) { return dtype == TRI_F32 ? 4 : (dtype == TRI_BF16 ? 2 : 1); }

int check_dims(int32_t head_dim) {
  if (head_dim < 2 || (head_dim & 1)) return fail(TRI_EINVAL, "head_dim must be even and >= 2 (got %d)", head_dim);
  if (head_dim != tri::kHeadDim) return fail(TRI_ENOTSUP, "head_dim %d is not supported (only 128)", head_dim);
  return TRI_OK;
}

int check_kv(const tri_kv* kv, bool need_k) {
  if (!kv) return fail(TRI_EINVAL, "kv descriptor is NULL");
  if (kv->layout != TRI_DENSE && kv->layout != TRI_PAGED) return fail(TRI_EINVAL, "unknown kv layout %d", kv->layout);
  if (kv->dtype != TRI_F32 && kv->dtype != TRI_BF16 && kv->dtype != TRI_FP8_E4M3 && kv->dtype != TRI_INT8)
    return fail(TRI_EINVAL, "unknown dtype %d", kv->dtype);
  if (kv->k_scale && kv->dtype != TRI_FP8_E4M3 && kv->dtype != TRI_INT8)
    return fail(TRI_EINVAL, "k_scale is only valid with 8-bit keys");
  if (kv->n_seq < 1 || kv->n_layer < 1 || kv->n_kvh < 1)
    return fail(TRI_EINVAL, "n_seq, n_layer and n_kvh must be >= 1");
  if (int rc = check_dims(kv->head_dim)) return rc;
  if (!kv->seq_len) return fail(TRI_EINVAL, "seq_len is NULL");
  if (need_k && !kv->k) return fail(TRI_EINVAL, "k is NULL");
  if (kv->layout == TRI_DENSE) {
    if (kv->max_len < 1) return fail(TRI_EINVAL, "max_len must be >= 1");
  } else {
    if (kv->page < 1 || kv->max_pages < 1) return fail(TRI_EINVAL, "page and max_pages must be >= 1");
    if (kv->page != tri::kPage) return fail(TRI_ENOTSUP, "page size %d is not supported (only 16)", kv->page);
    if (!kv->block_table) return fail(TRI_EINVAL, "block_table is NULL");
  }
  if (slots_of(kv) > tri::kMaxUnitLen)
    return fail(TRI_ENOTSUP, "per-unit capacity %lld exceeds %lld slots", (long long)slots_of(kv),
                (long long)tri::kMaxUnitLen);
  const int64_t units = int64_t(kv->n_seq) * kv->n_layer * kv->n_kvh;
  if (units > 0x7FFFFFFF) return fail(TRI_ENOTSUP, "too many units (%lld)", (long long)units);
  return TRI_OK;
}

// 1: size query answered; 0: proceed; <0: error.
int workspace(void* ws, size_t* ws_bytes, size_t need) {
  if (ws_bytes && !ws) {
    *ws_bytes = need;
    return 1;
  }
  if (need == 0) return 0;
  if (!ws || !ws_bytes) return fail(TRI_EWORKSPACE, "workspace of %zu bytes required", need);
  if (*ws_bytes < need) return fail(TRI_EWORKSPACE, "workspace of %zu bytes required (%zu given)", need, *ws_bytes);
  return 0;
}

// Validation and launch parameters of the attention consumer (shared by its two entry points).
int decode_setup(const tri_kv* kv, int32_t layer0, int32_t n_layers, const float* q, const int64_t* query_pos,
                 const int32_t* pos, int64_t pos_stride, double rope_base, int32_t rope_layout, int32_t key_space,
                 int32_t group, float* out, tri::DecodeParams& p, int64_t& unit_passes) {
  if (int rc = check_kv(kv, true)) return rc;
  if (kv->dtype != TRI_F32 && kv->dtype != TRI_BF16)
    return fail(TRI_ENOTSUP, "attention reads float32 or bfloat16 caches");
  if (!kv->v) return fail(TRI_EINVAL, "v is NULL");
  if (!q || !query_pos || !out) return fail(TRI_EINVAL, "q, query_pos and out must be non-NULL");
  if (n_layers < 1 || layer0 < 0 || int64_t(layer0) + n_layers > kv->n_layer)
    return fail(TRI_EINVAL, "layers [%d, %d) outside [0, %d)", layer0, layer0 + n_layers, kv->n_layer);
  if (group < 1) return fail(TRI_EINVAL, "group must be >= 1");
  if (group > tri::kMaxGroup) return fail(TRI_ENOTSUP, "group %d > %d", group, tri::kMaxGroup);
  if (!std::isfinite(rope_base) || rope_base <= 0.0) return fail(TRI_EINVAL, "rope_base must be finite and > 0");
  if (rope_layout != TRI_ROPE_HALF && rope_layout != TRI_ROPE_INTERLEAVED)
    return fail(TRI_EINVAL, "unknown rope layout %d", rope_layout);
  if (key_space != TRI_KEYS_PRE_ROPE && key_space != TRI_KEYS_POST_ROPE)
    return fail(TRI_EINVAL, "unknown key space %d", key_space);
  const int64_t slots = slots_of(kv);
  if (pos && pos_stride < slots) return fail(TRI_EINVAL, "pos_stride %lld < %lld slots", (long long)pos_stride,
                                             (long long)slots);
  unit_passes = int64_t(kv->n_seq) * n_layers * kv->n_kvh *
                ((group + tri::kDecodeHeadsPerPass - 1) / tri::kDecodeHeadsPerPass);
  for (int f = 0; f < tri::kBands; ++f)
    p.theta_turns[f] = std::pow(rope_base, -2.0 * f / double(tri::kHeadDim)) / (2.0 * M_PI);
  p.k = kv->k;
  p.v = kv->v;
  p.seq_len = kv->seq_len;
  p.block_table = kv->layout == TRI_PAGED ? kv->block_table : nullptr;
  p.pos = pos;
  p.query_pos = query_pos;
  p.q = q;
  p.out = out;
  p.max_len = kv->max_len;
  p.slots = slots;
  p.pos_stride = pos ? pos_stride : 0;
  p.n_seq = kv->n_seq;
  p.n_layer = kv->n_layer;
  p.n_kvh = kv->n_kvh;
  p.group = group;
  p.max_pages = kv->max_pages;
  p.layer0 = layer0;
  p.n_layers = n_layers;
  return TRI_OK;
}

// Launch with n_split slot splits; their partial softmax states go to `parts_buf` (256-byte
// aligned, decode_workspace_bytes(unit_passes, n_split) bytes) when n_split > 1.
int decode_launch(const tri_kv* kv, tri::DecodeParams& p, int64_t unit_passes, int n_split, void* parts_buf,
                  int32_t rope_layout, int32_t key_space, void* stream) {
  if (unit_passes * n_split > 0x7FFFFFFF) return fail(TRI_ENOTSUP, "too many units");
  p.n_split = n_split;
  if (n_split > 1) {
    p.split_len = ((p.slots + n_split - 1) / n_split + 63) / 64 * 64;
    const int64_t parts = unit_passes * n_split * tri::kDecodeHeadsPerPass;
    p.part_ml = static_cast<float*>(parts_buf);
    p.part_acc = reinterpret_cast<float*>(static_cast<char*>(parts_buf) + ((parts * 2 * 4 + 255) / 256) * 256);
  }
  (void)hipGetLastError();
  hipError_t e = tri::launch_decode_attention(p, kv->dtype == TRI_BF16, rope_layout == TRI_ROPE_INTERLEAVED,
                                              kv->layout == TRI_PAGED, key_space == TRI_KEYS_POST_ROPE,
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TRI_OK : hip_fail(e, "attention launch");
}

// Static scratch of tri_decode_attention_noalloc: a file-scope device array, one copy per GPU,
// held until the process ends.  In host code `scratch` names a host-side stand-in, so its
// device address is looked up once per device (with that device current) and only that
// address is passed to kernels.
constexpr size_t kStaticScratchBytes = size_t(8) << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];

}  // namespace

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

int static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(TRI_ENOTSUP, "device %d: the static scratch covers devices 0..%d", dev,
                                                 kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr || reinterpret_cast<uintptr_t>(ptr) % 256 != 0)
      return fail(TRI_EHIP, "static scratch of device %d is not 256-byte aligned", dev);
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return TRI_OK;
}

}  // namespace

namespace {

// Checks of a scoring configuration and the kernel parameters it gives (shared by
// tri_score_keys and tri_score_select).  scores may be NULL here; each caller decides.
int score_setup(const tri_score_cfg* cfg, const float* center, const float* mean_abs, const tri_kv* kv,
                const int64_t* query_pos, float* scores, tri::ScoreParams& p) {
  if (!cfg) return fail(TRI_EINVAL, "cfg is NULL");
  if (int rc = check_kv(kv, true)) return rc;
  if (!std::isfinite(cfg->rope_base) || cfg->rope_base <= 0.0)
    return fail(TRI_EINVAL, "rope_base must be finite and > 0");
  if (cfg->rope_layout != TRI_ROPE_HALF && cfg->rope_layout != TRI_ROPE_INTERLEAVED)
    return fail(TRI_EINVAL, "unknown rope layout %d", cfg->rope_layout);
  if (cfg->reduce != TRI_REDUCE_MAX && cfg->reduce != TRI_REDUCE_MEAN)
    return fail(TRI_EINVAL, "unknown reduce %d", cfg->reduce);
  if (cfg->key_space != TRI_KEYS_PRE_ROPE && cfg->key_space != TRI_KEYS_POST_ROPE)
    return fail(TRI_EINVAL, "unknown key space %d", cfg->key_space);
  if (cfg->form != TRI_SCORE_ADDITIVE && cfg->form != TRI_SCORE_MULTIPLICATIVE)
    return fail(TRI_EINVAL, "unknown score form %d", cfg->form);
  const bool mult = cfg->form == TRI_SCORE_MULTIPLICATIVE;
  if (cfg->group < 1) return fail(TRI_EINVAL, "group must be >= 1");
  if (cfg->group > tri::kMaxGroup) return fail(TRI_ENOTSUP, "group %d > %d", cfg->group, tri::kMaxGroup);
  if (cfg->n_offsets < 1 || !cfg->offsets) return fail(TRI_EINVAL, "at least one offset is required");
  if (cfg->n_offsets > tri::kMaxOffsets)
    return fail(TRI_ENOTSUP, "%d offsets > %d", cfg->n_offsets, tri::kMaxOffsets);
  for (int i = 0; i < cfg->n_offsets; ++i)
    if (cfg->offsets[i] < 0) return fail(TRI_EINVAL, "offsets must be >= 0");
  if (!center) return fail(TRI_EINVAL, "center must be non-NULL");
  if (!mean_abs && !mult) return fail(TRI_EINVAL, "mean_abs must be non-NULL for the additive form");
  // keys at explicit positions: pre-RoPE keys are rotated at them (additive form); keys cached
  // after RoPE already carry their rotation, so their positions are not needed
  if (kv->pos && mult && cfg->key_space == TRI_KEYS_PRE_ROPE)
    return fail(TRI_ENOTSUP, "explicit key positions with the multiplicative form are not supported");

  p = tri::ScoreParams{};
  // theta_f = base^(-2f/d) and C_f = mean over offsets of e^{i Delta theta_f}, in float64
  for (int f = 0; f < tri::kBands; ++f) {
    const double th = std::pow(cfg->rope_base, -2.0 * f / double(tri::kHeadDim));
    double cr = 0.0, ci = 0.0;
    for (int i = 0; i < cfg->n_offsets; ++i) {
      const double a = double(cfg->offsets[i]) * th;
      cr += std::cos(a);
      ci += std::sin(a);
    }
    p.theta[f] = th;
    p.c_re[f] = cr / cfg->n_offsets;
    p.c_im[f] = ci / cfg->n_offsets;
  }
  p.k = kv->k;
  p.seq_len = kv->seq_len;
  p.query_pos = query_pos;
  p.block_table = kv->layout == TRI_PAGED ? kv->block_table : nullptr;
  p.center = center;
  p.mean_abs = mean_abs;
  p.k_scale = kv->k_scale;
  p.pos = cfg->key_space == TRI_KEYS_PRE_ROPE ? kv->pos : nullptr;
  p.scores = scores;
  p.max_len = kv->max_len;
  p.score_stride = slots_of(kv);
  p.n_layer = kv->n_layer;
  p.n_kvh = kv->n_kvh;
  p.group = cfg->group;
  p.max_pages = kv->max_pages;
  p.reduce_mean = cfg->reduce == TRI_REDUCE_MEAN;
  p.n_seq = kv->n_seq;
  return TRI_OK;
}

int select_setup(const tri_kv* kv, int32_t budget, int32_t window, int32_t* kept, int32_t* kept_n,
                 tri::SelectParams& p) {
  if (budget < 1) return fail(TRI_EINVAL, "budget must be >= 1");
  if (window < 0) return fail(TRI_EINVAL, "window must be >= 0");
  if (!kept || !kept_n) return fail(TRI_EINVAL, "kept and kept_n must be non-NULL");
  p = tri::SelectParams{};
  p.score_stride = slots_of(kv);
  p.seq_len = kv->seq_len;
  p.kept = kept;
  p.kept_n = kept_n;
  p.budget = budget;
  p.window = window;
  p.units_per_seq = kv->n_layer * kv->n_kvh;
  return TRI_OK;
}

}  // namespace

extern "C" {

const char* tri_last_error(void) { return g_error.c_str(); }

int tri_decode_attention(const tri_kv* kv, int32_t layer0, int32_t n_layers, const float* q,
                         const int64_t* query_pos, const int32_t* pos, int64_t pos_stride, double rope_base,
                         int32_t rope_layout, int32_t key_space, int32_t group, float* out, void* ws,
                         size_t* ws_bytes, void* stream) {
  try {
    g_error.clear();
    tri::DecodeParams p{};
    int64_t unit_passes = 0;
    if (int rc = decode_setup(kv, layer0, n_layers, q, query_pos, pos, pos_stride, rope_base, rope_layout,
                              key_space, group, out, p, unit_passes))
      return rc;
    // optional workspace: it lets few, long units split their slots over several workgroups
    const int n_split = tri::decode_splits(unit_passes, p.slots);
    const size_t need = size_t(tri::decode_workspace_bytes(unit_passes, n_split));
    if (ws_bytes && !ws) {
      *ws_bytes = need;
      return TRI_OK;
    }
    const bool split = ws && ws_bytes && need > 0;
    if (split && *ws_bytes < need)
      return fail(TRI_EWORKSPACE, "workspace of %zu bytes required (%zu given)", need, *ws_bytes);
    if (split && reinterpret_cast<uintptr_t>(ws) % 256 != 0) return fail(TRI_EINVAL, "workspace must be 256-byte aligned");
    return decode_launch(kv, p, unit_passes, split ? n_split : 1, split ? ws : nullptr, rope_layout, key_space,
                         stream);
  } catch (...) {
    return fail(TRI_EHIP, "unexpected host exception in tri_decode_attention");
  }
}

int tri_decode_attention_noalloc(const tri_kv* kv, int32_t layer0, int32_t n_layers, const float* q,
                                 const int64_t* query_pos, const int32_t* pos, int64_t pos_stride,
                                 double rope_base, int32_t rope_layout, int32_t key_space, int32_t group,
                                 float* out, void* stream) {
  try {
    g_error.clear();
    tri::DecodeParams p{};
    int64_t unit_passes = 0;
    if (int rc = decode_setup(kv, layer0, n_layers, q, query_pos, pos, pos_stride, rope_base, rope_layout,
                              key_space, group, out, p, unit_passes))
      return rc;
    // the split tri_decode_attention takes with a workspace, its partial results in the
    // library's static scratch of this device
    const int n_split = tri::decode_splits(unit_passes, p.slots);
    const size_t need = size_t(tri::decode_workspace_bytes(unit_passes, n_split));
    if (need > kStaticScratchBytes)
      return fail(TRI_EWORKSPACE,
                  "this shape splits its slots %d ways and needs %zu bytes of scratch; the static scratch "
                  "holds %zu (call tri_decode_attention with a workspace, or without one)",
                  n_split, need, kStaticScratchBytes);
    void* scr = nullptr;
    if (need > 0)
      if (int rc = static_scratch(&scr)) return rc;
    return decode_launch(kv, p, unit_passes, need > 0 ? n_split : 1, scr, rope_layout, key_space, stream);
  } catch (...) {
    return fail(TRI_EHIP, "unexpected host exception in tri_decode_attention_noalloc");
  }
}

int tri_version(void) { return TRI_VERSION; }

int tri_calibrate_stats(const void* q, int32_t dtype, int64_t n, int32_t n_layer, int32_t n_qh,
                        int32_t head_dim, int32_t rope_layout, float* center, float* mean_abs,
                        void* ws, size_t* ws_bytes, void* stream) {
  try {
    g_error.clear();
    if (!q || !center || !mean_abs) return fail(TRI_EINVAL, "q, center and mean_abs must be non-NULL");
    if (dtype == TRI_FP8_E4M3 || dtype == TRI_INT8)
      return fail(TRI_ENOTSUP, "calibration takes float32 or bfloat16 queries");
    if (dtype != TRI_F32 && dtype != TRI_BF16) return fail(TRI_EINVAL, "unknown dtype %d", dtype);
    if (rope_layout != TRI_ROPE_HALF && rope_layout != TRI_ROPE_INTERLEAVED)
      return fail(TRI_EINVAL, "unknown rope layout %d", rope_layout);
    if (n < 1 || n_layer < 1 || n_qh < 1) return fail(TRI_EINVAL, "n, n_layer and n_qh must be >= 1");
    if (int rc = check_dims(head_dim)) return rc;
    if (int64_t(n_layer) * n_qh > 0x7FFFFFFF) return fail(TRI_ENOTSUP, "too many heads");
    if (int rc = workspace(ws, ws_bytes, 0)) return rc > 0 ? TRI_OK : rc;
    tri::CalibParams p{};
    p.q = q;
    p.n = n;
    p.n_layer = n_layer;
    p.n_qh = n_qh;
    p.center = center;
    p.mean_abs = mean_abs;
    (void)hipGetLastError();
    hipError_t e = tri::launch_calib(p, dtype == TRI_BF16, rope_layout == TRI_ROPE_INTERLEAVED,
                                     static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TRI_OK : hip_fail(e, "calibration launch");
  } catch (...) {
    return fail(TRI_EHIP, "unexpected host exception in tri_calibrate_stats");
  }
}

int tri_score_keys(const tri_score_cfg* cfg, const float* center, const float* mean_abs,
                   const tri_kv* kv, const int64_t* query_pos, float* scores, void* ws,
                   size_t* ws_bytes, void* stream) {
  try {
    g_error.clear();
    tri::ScoreParams p;
    if (int rc = score_setup(cfg, center, mean_abs, kv, query_pos, scores, p)) return rc;
    if (!scores) return fail(TRI_EINVAL, "scores must be non-NULL");
    if (int rc = workspace(ws, ws_bytes, 0)) return rc > 0 ? TRI_OK : rc;
    const bool mult = cfg->form == TRI_SCORE_MULTIPLICATIVE;
    const int64_t slots = p.score_stride;
    const int64_t units = int64_t(kv->n_seq) * kv->n_layer * kv->n_kvh;
    // persistent grid: one workgroup per CU builds the 128 KB phase table once; fewer
    // workgroups when there are not kMinWaveSteps steps per wave even at full length
    const int64_t max_steps = units * ((slots + 7) / 8);
    const int64_t waves = (max_steps + tri::kMinWaveSteps - 1) / tri::kMinWaveSteps;
    int64_t grid = (waves + tri::kScoreWaves - 1) / tri::kScoreWaves;
    const int64_t resident = int64_t(cu_count());
    if (grid > resident) grid = resident;
    if (grid < 1) grid = 1;
    const int g_eff = p.reduce_mean ? 1 : cfg->group;
    (void)hipGetLastError();
    hipError_t e = tri::launch_score(p, g_eff, kv->dtype,
                                     cfg->rope_layout == TRI_ROPE_INTERLEAVED,
                                     kv->layout == TRI_PAGED, cfg->key_space == TRI_KEYS_POST_ROPE, mult, int(grid),
                                     static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TRI_OK : hip_fail(e, "score launch");
  } catch (...) {
    return fail(TRI_EHIP, "unexpected host exception in tri_score_keys");
  }
}

int tri_score_select(const tri_score_cfg* cfg, const float* center, const float* mean_abs, const tri_kv* kv,
                     const int64_t* query_pos, int32_t budget, int32_t window, float* scores, int32_t* kept,
                     int32_t* kept_n, void* ws, size_t* ws_bytes, void* stream) {
  try {
    g_error.clear();
    tri::ScoreParams p;
    tri::SelectParams sp;
    if (int rc = score_setup(cfg, center, mean_abs, kv, query_pos, scores, p)) return rc;
    if (int rc = select_setup(kv, budget, window, kept, kept_n, sp)) return rc;
    if (kv->dtype != TRI_F32 && kv->dtype != TRI_BF16)
      return fail(TRI_ENOTSUP, "fused scoring and selection takes float32 or bfloat16 keys only");
    if (cfg->key_space != TRI_KEYS_PRE_ROPE || cfg->form != TRI_SCORE_ADDITIVE || kv->pos)
      return fail(TRI_ENOTSUP, "fused scoring and selection takes pre-RoPE keys at their slots, additive form");
    if (p.score_stride > tri::kFuseMaxSlots)
      return fail(TRI_ENOTSUP, "fused scoring and selection holds at most %d slots per unit (%lld)",
                  tri::kFuseMaxSlots, (long long)p.score_stride);
    const int64_t units = int64_t(kv->n_seq) * kv->n_layer * kv->n_kvh;
    if (units > 0x7FFFFFFF) return fail(TRI_ENOTSUP, "grid too large");
    if (int rc = workspace(ws, ws_bytes, 0)) return rc > 0 ? TRI_OK : rc;
    if (units == 0) return TRI_OK;
    const int g_eff = p.reduce_mean ? 1 : cfg->group;
    (void)hipGetLastError();
    hipError_t e = tri::launch_score_select(p, sp, g_eff, kv->dtype, cfg->rope_layout == TRI_ROPE_INTERLEAVED,
                                            kv->layout == TRI_PAGED, units, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TRI_OK : hip_fail(e, "fused score/select launch");
  } catch (...) {
    return fail(TRI_EHIP, "unexpected host exception in tri_score_select");
  }
}

int tri_select_topb(const float* scores, const tri_kv* kv, int32_t budget, int32_t window,
                    int32_t* kept, int32_t* kept_n, void* ws, size_t* ws_bytes, void* stream) {
  try {
    g_error.clear();
    if (int rc = check_kv(kv, false)) return rc;
    tri::SelectParams p;
    if (int rc = select_setup(kv, budget, window, kept, kept_n, p)) return rc;
    if (!scores) return fail(TRI_EINVAL, "scores, kept and kept_n must be non-NULL");
    p.scores = scores;
    const int64_t units = int64_t(kv->n_seq) * p.units_per_seq;
    // optional workspace: units longer than 32768 slots are then selected by the two-stage
    // tournament instead of one workgroup each
    const size_t need = tri::select_workspace_bytes(p, units);
    if (ws_bytes && !ws) {
      *ws_bytes = need;
      return TRI_OK;
    }
    const bool tour = ws && ws_bytes && need > 0;
    if (tour && *ws_bytes < need)
      return fail(TRI_EWORKSPACE, "workspace of %zu bytes required (%zu given)", need, *ws_bytes);
    if (tour && units * ((p.score_stride + 32767) / 32768) > 0x7FFFFFFF) return fail(TRI_ENOTSUP, "grid too large");
    (void)hipGetLastError();
    hipError_t e = tri::launch_select(p, units, tour ? ws : nullptr, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TRI_OK : hip_fail(e, "select launch");
  } catch (...) {
    return fail(TRI_EHIP, "unexpected host exception in tri_select_topb");
  }
}

int tri_compact_kv(const tri_kv* kv, const int32_t* kept, const int32_t* kept_n, int32_t budget,
                   void* k_out, void* v_out, int32_t* pos_out, int32_t* freed, int32_t* n_freed,
                   int32_t* new_len, void* stream) {
  try {
    g_error.clear();
    if (int rc = check_kv(kv, true)) return rc;
    if (!kept || !kept_n) return fail(TRI_EINVAL, "kept and kept_n must be non-NULL");
    if (budget < 1) return fail(TRI_EINVAL, "budget must be >= 1");
    const bool paged = kv->layout == TRI_PAGED;
    const bool with_v = kv->v != nullptr;
    if (paged) {
      if (k_out || v_out) return fail(TRI_ENOTSUP, "paged compaction is in place: k_out and v_out must be NULL");
      if ((freed == nullptr) != (n_freed == nullptr))
        return fail(TRI_EINVAL, "freed and n_freed must both be given or both be NULL");
    } else {
      if (!k_out) return fail(TRI_EINVAL, "dense compaction needs k_out");
      if (with_v != (v_out != nullptr)) return fail(TRI_EINVAL, "v_out must be given exactly when kv->v is");
      if (freed || n_freed) return fail(TRI_EINVAL, "freed / n_freed apply to the paged layout only");
    }
    tri::CompactParams p{};
    p.k = kv->k;
    p.v = kv->v;
    p.k_out = k_out;
    p.v_out = v_out;
    p.kept = kept;
    p.kept_n = kept_n;
    p.seq_len = kv->seq_len;
    p.block_table = paged ? kv->block_table : nullptr;
    p.pos = kv->pos;
    p.pos_out = pos_out;
    p.freed = freed;
    p.n_freed = n_freed;
    p.new_len = new_len;
    p.max_len = kv->max_len;
    p.pos_stride = slots_of(kv);
    p.budget = budget;
    p.units_per_seq = kv->n_layer * kv->n_kvh;
    p.n_layer = kv->n_layer;
    p.n_kvh = kv->n_kvh;
    p.max_pages = kv->max_pages;
    const int copy_rows = tri::dense_copy_rows(elem_bytes(kv->dtype));
    p.chunks_per_unit = (budget + copy_rows - 1) / copy_rows;
    const int64_t units = int64_t(kv->n_seq) * p.units_per_seq;
    if (!paged && units * p.chunks_per_unit > 0x7FFFFFFF) return fail(TRI_ENOTSUP, "grid too large");
    (void)hipGetLastError();
    hipError_t e = tri::launch_compact(p, units, elem_bytes(kv->dtype), paged, with_v,
                                       static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TRI_OK : hip_fail(e, "compaction launch");
  } catch (...) {
    return fail(TRI_EHIP, "unexpected host exception in tri_compact_kv");
  }
}

}  // extern "C"
