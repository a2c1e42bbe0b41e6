/*
 * tri.h - C ABI of the TriAttention KV-cache compression pass for AMD Instinct MI355X
 * (gfx950).  One shared library, libtri.so; every entry point is extern "C" and takes
 * plain pointers and sizes.
 *
 * Sources (web pages about "TriAttention: Efficient Long Reasoning with Trigonometric KV
 * Compression", Mao et al.):
 *   [Review]  "TriAttention: Trigonometric KV Compression for Efficient Long Reasoning"
 *             (alanhou.org review): sections "Core Mechanism", "Key Concepts".
 *   [DevTo]   "TriAttention: How a Geometric Trick Cuts LLM Memory Use by 10x Without
 *             Losing Accuracy" (dev.to): sections "Why Existing KV Cache Compression
 *             Breaks in Production", "The Core Idea: Q/K Concentration in Pre-RoPE Space",
 *             "Solving the Memory Fragmentation Problem", "What the Numbers Look Like".
 *   [Project] "TriAttention: trigonometric KV cache compression for long reasoning"
 *             (hysenlabs.com): sections "Pre-RoPE centres decide which keys are worth
 *             keeping", "The KV budget is a runtime knob that chat sessions should
 *             raise", "Calibration statistics are tied to a specific model".
 *
 * The pass, per unit = (sequence, layer, KV head) holding L cached pre-RoPE keys:
 *   1. tri_score_keys   score every key from calibrated query statistics
 *   2. tri_select_topb  keep the top-B keys (the recent window always kept)
 *   3. tri_compact_kv   pack the survivors forward (dense out-of-place or paged in place)
 * and, once per model, tri_calibrate_stats builds the statistics from query samples.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller unless a parameter says
 *     "host".  The library never frees or retains them, allocates no device memory, and
 *     keeps no state between calls (re-entrant; calls on different streams may overlap as
 *     long as their output buffers are disjoint).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls are asynchronous: they
 *     return once their kernels are enqueued.  Argument errors are reported synchronously
 *     before anything is launched; a device fault shows at the caller's next
 *     synchronisation (and as TRI_EHIP from the next call that sees it).
 *   - Workspace: if `ws_bytes != NULL` and `ws == NULL`, the call writes the bytes it needs
 *     to *ws_bytes and returns TRI_OK without launching.  If both are non-NULL, *ws_bytes
 *     is the capacity of `ws` (device memory, 256-byte aligned).  If `ws_bytes == NULL`
 *     the call runs without workspace and fails with TRI_EWORKSPACE if it needs one.
 *   - Return values are tri_status codes; tri_last_error() gives the text of the last
 *     failure on the calling thread.
 *   - Supported set: head_dim == 128 (F = 64 RoPE bands), dtype TRI_F32, TRI_BF16,
 *     TRI_FP8_E4M3 or TRI_INT8 (tri_calibrate_stats: TRI_F32 or TRI_BF16), page
 *     size 16, group (query heads per KV head) 1..8, up to 64 future offsets, per-unit
 *     length up to 1,048,576 keys.  Other valid values return TRI_ENOTSUP.
 */
#ifndef TRI_H_
#define TRI_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tri_status {
  TRI_OK = 0,
  TRI_EINVAL = -1,     /* bad argument or shape                       */
  TRI_ENOTSUP = -2,    /* valid but outside the supported set          */
  TRI_EWORKSPACE = -3, /* workspace missing or too small               */
  TRI_EHIP = -4        /* HIP launch or runtime error                  */
} tri_status;

/* Element type of k and v.  The two 8-bit types let the pass run on a quantised KV cache
 * ([Project] "The same compression idea now runs on four different backends": the method
 * composes with KV quantisation); their key codes may carry a scale (tri_kv.k_scale).
 *   TRI_FP8_E4M3: the OCP 8-bit float E4M3 (1 sign bit, 4 exponent bits with bias 7, 3
 *                 mantissa bits, subnormals, no infinities, S.1111.111 = NaN, largest
 *                 finite 448), one byte per element.
 *   TRI_INT8:     two's-complement signed bytes (symmetric quantisation: value = code). */
typedef enum tri_dtype { TRI_F32 = 0, TRI_BF16 = 1, TRI_FP8_E4M3 = 2, TRI_INT8 = 3 } tri_dtype;

/* Pairing of the RoPE frequency bands inside a head vector x[0..d):
 *   TRI_ROPE_HALF:        band f = (x[f], x[f + d/2])   (rotate-half pairing)
 *   TRI_ROPE_INTERLEAVED: band f = (x[2f], x[2f + 1])
 * The pages do not fix the pairing; it must match the model's RoPE. */
typedef enum tri_rope_layout { TRI_ROPE_HALF = 0, TRI_ROPE_INTERLEAVED = 1 } tri_rope_layout;

/* Reduction of the per-query-head scores over the G query heads reading one KV head. */
typedef enum tri_reduce { TRI_REDUCE_MAX = 0, TRI_REDUCE_MEAN = 1 } tri_reduce;

typedef enum tri_kv_layout { TRI_DENSE = 0, TRI_PAGED = 1 } tri_kv_layout;

/* What the cache holds.  The score is defined on pre-RoPE keys ([DevTo] "The Core Idea:
 * Q/K Concentration in Pre-RoPE Space"; [Review] "Framework Shift").  A serving cache may
 * instead hold keys already rotated by RoPE at their positions; with
 * TRI_KEYS_POST_ROPE the same score is computed from those keys (slot j rotated at
 * position j) without rotating them back. */
typedef enum tri_key_space { TRI_KEYS_PRE_ROPE = 0, TRI_KEYS_POST_ROPE = 1 } tri_key_space;

/* Form of the score.
 *   TRI_SCORE_ADDITIVE (default): the offset-averaged cosine series of the centre/key band
 *     pairs, sum_f |c_f||k_f| cos(d theta_f + arg c_f - arg k_f), plus the concentration-
 *     weighted norm term sum_f (1 - R_f) E|q_f| |k_f| ([Review] "Key Concepts"; [DevTo] "The
 *     Core Idea: Q/K Concentration in Pre-RoPE Space").
 *   TRI_SCORE_MULTIPLICATIVE: the phase-only series sum_f cos(d theta_f + arg c_f - arg k_f)
 *     (a band whose centre or key part is 0 contributes 0), offset-averaged, times ||c|| ||k||
 *     ([Review] "Core Mechanism": a trigonometric series in the distance, then weighted by
 *     the query and key norms).  ||c|| is the L2 norm of the query head's centre and ||k||
 *     the key's; mean_abs is not read and may be NULL.  A key band with |k_f|^2 below the
 *     float32 range (|k_f| < about 1e-19) counts as 0. */
typedef enum tri_score_form { TRI_SCORE_ADDITIVE = 0, TRI_SCORE_MULTIPLICATIVE = 1 } tri_score_form;

/* Description of a pre-RoPE KV cache (all pointers device, caller-owned).
 *   dense: k, v are [n_seq][n_layer][n_kvh][max_len][head_dim]; slot j of unit (s,l,h) is
 *          row j; the unit holds seq_len[s] <= max_len keys.
 *   paged: k, v are pools [n_pages][n_layer][n_kvh][page][head_dim]; slot j of sequence s
 *          lives in page block_table[s * max_pages + j / page], row j % page.  Every page
 *          holds all layers and KV heads of its 16 tokens, so it can be freed only when it
 *          is empty for all of them ([DevTo] "Why Existing KV Cache Compression Breaks in
 *          Production").  max_len is ignored; the per-unit slot capacity is
 *          max_pages * page.
 *   seq_len: [n_seq] int32 number of cached keys per sequence.
 *   pos:     optional [n_seq][n_layer][n_kvh][slots] int32 RoPE positions of the cached
 *            keys (slots = max_len dense, max_pages * page paged); NULL means the position
 *            of slot j is j.  A cache compacted before holds keys whose slots no longer
 *            equal their positions, and the next compression must score them at pos:
 *              tri_score_keys, pre-RoPE keys, additive form: each key is scored at pos[j];
 *              tri_score_keys, pre-RoPE keys, multiplicative form: TRI_ENOTSUP;
 *              tri_score_keys, TRI_KEYS_POST_ROPE: pos is not read (the cached keys
 *                already carry their rotation);
 *              tri_compact_kv: pos is gathered into pos_out.
 *   k_scale: optional device [n_layer][n_kvh] float32, dtype TRI_FP8_E4M3 or TRI_INT8 only
 *            (must be NULL otherwise): the key of head (l, h) is its decoded code times
 *            k_scale[l * n_kvh + h] (NULL = 1).  Scores are computed from the scaled keys;
 *            compaction copies codes unchanged, so the scale still applies to k_out.
 *            Values must be finite and > 0. */
typedef struct tri_kv {
  int32_t layout;   /* tri_kv_layout */
  int32_t dtype;    /* tri_dtype of k and v */
  int32_t n_seq;
  int32_t n_layer;
  int32_t n_kvh;
  int32_t head_dim;
  int64_t max_len;
  const int32_t *seq_len;
  void *k;
  void *v;          /* may be NULL (keys only) */
  int32_t page;
  int32_t max_pages;
  const int32_t *block_table;
  const int32_t *pos;
  const float *k_scale;   /* 8-bit dtypes only, optional: [n_layer][n_kvh] float32 */
} tri_kv;

/* Scoring configuration.
 *   rope_base: RoPE base; theta_f = rope_base^(-2f/head_dim).
 *   offsets:   HOST array of n_offsets future query offsets Delta >= 0 (the score is the
 *              mean over these offsets of the predicted logit at query_pos + Delta).
 *   group:     G, query heads per KV head; query head hq reads KV head hq / G. */
typedef struct tri_score_cfg {
  double rope_base;
  int32_t rope_layout;      /* tri_rope_layout */
  int32_t n_offsets;
  const int32_t *offsets;   /* host */
  int32_t group;
  int32_t reduce;           /* tri_reduce */
  int32_t key_space;        /* tri_key_space (0 = pre-RoPE keys) */
  int32_t form;             /* tri_score_form (0 = additive) */
} tri_score_cfg;

/* Calibration of the query statistics ([Review] "Key Concepts": the centre is the mean of
 * the pre-RoPE queries over a calibration set; [Project] "Calibration statistics are tied
 * to a specific model").
 *   q:        [n][n_layer][n_qh][head_dim] pre-RoPE query samples (dtype TRI_F32/TRI_BF16)
 *   center:   out [n_layer][n_qh][head_dim/2][2] float32, E[q_f] = mean_n q_{n,f} (re, im)
 *   mean_abs: out [n_layer][n_qh][head_dim/2] float32, E|q_f| = mean_n |q_{n,f}|
 * Sums are accumulated in float64.  n >= 1.  Needs no workspace. */
int tri_calibrate_stats(const void *q, int32_t dtype, int64_t n, int32_t n_layer, int32_t n_qh,
                        int32_t head_dim, int32_t rope_layout, float *center, float *mean_abs,
                        void *ws, size_t *ws_bytes, void *stream);

/* Score every cached key ([Review] "Core Mechanism" and "Key Concepts": a trigonometric
 * series in the query-key distance set by the pre-RoPE centres, plus norms; [DevTo] "The
 * Core Idea": weakly concentrated heads blend in a norm signal weighted by the measured
 * concentration).  For unit (s, l, h), key slot j with band values k_f and position p_j,
 * and each query head hq of the group with statistics c_f = center[l][hq][f] (complex)
 * and m_f = mean_abs[l][hq][f]:
 *
 *   R_f     = |c_f| / m_f                         (R_f = 0 where m_f = 0)
 *   s_hq(j) = mean_{Delta in offsets} sum_f |c_f| |k_f| cos((Q - p_j + Delta) theta_f
 *                                                       + arg c_f - arg k_f)
 *           + sum_f (1 - R_f) m_f |k_f|
 *   score(j) = max_hq s_hq(j)  (TRI_REDUCE_MAX)   or   mean_hq s_hq(j)  (TRI_REDUCE_MEAN)
 *
 * with Q = query_pos[s] (int64; NULL means seq_len[s] - 1) and p_j = kv->pos[...][j] when
 * kv->pos is given (pre-RoPE keys, additive form), else p_j = j.  With cfg->key_space ==
 * TRI_KEYS_POST_ROPE the cached vector of slot j is k'_f = k_f e^{i j theta_f} (RoPE
 * applied at position j) and the score is that of k_f; since
 * conj(k_f) e^{-i p_j theta_f} = conj(k'_f), it is evaluated as
 * sum_f Re(c_f C_f e^{i Q theta_f} conj(k'_f)) + (1 - R_f) m_f |k'_f|.
 *   center:   [n_layer][n_kvh * group][head_dim/2][2] float32
 *   mean_abs: [n_layer][n_kvh * group][head_dim/2] float32
 *   scores:   out float32 [n_seq][n_layer][n_kvh][slots] (slots = max_len dense,
 *             max_pages * page paged); entries at j >= seq_len[s] are not written.
 * Computed in float32 from float64-derived phase tables; needs no workspace. */
int tri_score_keys(const tri_score_cfg *cfg, const float *center, const float *mean_abs,
                   const tri_kv *kv, const int64_t *query_pos, float *scores, void *ws,
                   size_t *ws_bytes, void *stream);

/* Top-B selection per unit ([Review] "Core Mechanism": keep only the top-scoring keys;
 * [Project] "The KV budget is a runtime knob": the budget bounds the whole kept cache).
 * With L = seq_len[s]:
 *   L <= budget: every slot is kept.
 *   otherwise:   the last W' = min(window, budget) slots are kept, plus the best
 *                budget - W' of the other slots ranked by (score descending, slot
 *                ascending); a NaN score ranks as -inf and -0.0 equals +0.0.
 *   scores: [n_seq][n_layer][n_kvh][slots] float32 as written by tri_score_keys
 *   kept:   out int32 [n_seq][n_layer][n_kvh][budget], kept slots in ascending order;
 *           entries past the kept count are set to -1
 *   kept_n: out int32 [n_seq], min(budget, seq_len[s]) (same for every unit of s)
 * Workspace (optional): ws == NULL with ws_bytes != NULL stores the size that lets units of
 * more than 32768 slots be selected in two stages over many workgroups (0 when that does not
 * apply: shorter units, or budget - min(window, budget) too large for it); given a
 * workspace of that size, the call uses it, and returns TRI_EWORKSPACE if it is smaller.
 * Without one (ws_bytes == NULL) every unit is selected by one workgroup.  The result is
 * the same either way. */
int tri_select_topb(const float *scores, const tri_kv *kv, int32_t budget, int32_t window,
                    int32_t *kept, int32_t *kept_n, void *ws, size_t *ws_bytes, void *stream);

/* Scoring and selection in one launch ([Review] "Core Mechanism": every key is scored and
 * only the top-scoring ones are kept), one workgroup per unit: the unit's scores stay in
 * on-chip memory between the two steps instead of going to memory and back.  It computes
 * exactly what tri_score_keys followed by tri_select_topb compute, for the cases it takes:
 *   dense or paged caches of TRI_F32 or TRI_BF16 keys before RoPE (cfg->key_space
 *   TRI_KEYS_PRE_ROPE) at their slot positions (kv->pos NULL), additive form, at most 32768
 *   slots per unit (dense: max_len; paged: max_pages * page); anything else returns
 *   TRI_ENOTSUP.
 * Arguments as for tri_score_keys and tri_select_topb; scores may be NULL (then no score is
 * written) or, as for tri_score_keys, [n_seq][n_layer][n_kvh][slots] float32 to receive them
 * as well.  kept and kept_n as for tri_select_topb.  Needs no workspace. */
int tri_score_select(const tri_score_cfg *cfg, const float *center, const float *mean_abs,
                     const tri_kv *kv, const int64_t *query_pos, int32_t budget, int32_t window,
                     float *scores, int32_t *kept, int32_t *kept_n, void *ws, size_t *ws_bytes,
                     void *stream);

/* Forward-packing compaction ([DevTo] "Solving the Memory Fragmentation Problem": the
 * survivors are moved into as few blocks as possible so that the emptied tail blocks can
 * be reclaimed).  Row kept[i] of each unit moves to slot i, i < kept_n[s] (bit copy).
 *   dense: k_out (and v_out iff kv->v != NULL) are [n_seq][n_layer][n_kvh][budget][d],
 *          written out of place; freed / n_freed must be NULL.
 *   paged: k_out = v_out = NULL (in place through the block tables; kv->k and kv->v are
 *          modified).  Because every unit of a sequence keeps kept_n[s] rows, pages
 *          block_table[s][ceil(kept_n/page) .. ceil(seq_len/page)) become empty for every
 *          layer and head; they are written to freed[s * max_pages + 0 ..] with their
 *          count in n_freed[s] (both optional, both or neither).  Rows of the last kept
 *          page past kept_n are left as they were.  The block table is not modified.
 *   pos_out: optional out int32 [n_seq][n_layer][n_kvh][budget], RoPE position of the row
 *            now in slot i (kv->pos gathered, or kept[i] when kv->pos == NULL).
 *   new_len: optional out int32 [n_seq], = kept_n.
 * kept must be ascending per unit (as written by tri_select_topb); the in-place order of
 * the paged path relies on kept[i] >= i.  The dense path launches one workgroup per
 * (unit, 4 / 8 / 16 output rows) for float32 / bf16 / 8-bit rows and returns TRI_ENOTSUP
 * when that exceeds 2^31 - 1 workgroups. */
int tri_compact_kv(const tri_kv *kv, const int32_t *kept, const int32_t *kept_n, int32_t budget,
                   void *k_out, void *v_out, int32_t *pos_out, int32_t *freed, int32_t *n_freed,
                   int32_t *new_len, void *stream);

/* Attention of the newest token over a compressed cache: the consumer of the compaction
 * outputs.  After compression the kept keys are rotated by RoPE at their own positions and
 * read by standard attention ([Review] "Core Mechanism"; [DevTo] "Solving the Memory
 * Fragmentation Problem": packing keeps the survivors but not their slot indices).
 *   kv:         the (compacted) cache: dense [n_seq][n_layer][n_kvh][max_len][head_dim] or
 *               paged; seq_len = the lengths after compaction (new_len); dtype TRI_F32 or
 *               TRI_BF16 (other dtypes: TRI_ENOTSUP); v is required.
 *   layer0, n_layers: the layers [layer0, layer0 + n_layers) to process.
 *   q:          device [n_seq][n_layers][n_kvh * group][head_dim] float32 pre-RoPE queries of
 *               the newest token of each sequence.
 *   query_pos:  device [n_seq] int64 position of that token.
 *   pos:        device [n_seq][n_layer][n_kvh][pos_stride] int32 positions of the cached keys
 *               (e.g. tri_compact_kv's pos_out with pos_stride = budget), or NULL for
 *               position = slot; pos_stride >= the per-unit slot capacity when pos is given.
 *   key_space:  TRI_KEYS_PRE_ROPE (keys rotated here at their positions) or
 *               TRI_KEYS_POST_ROPE (keys already rotated).
 *   group:      query heads per KV head (1..8).
 *   out:        device [n_seq][n_layers][n_kvh * group][head_dim] float32:
 *               softmax_j((R(Q) q) . (R(p_j) k_j) / sqrt(head_dim)) weighted sum of v_j over
 *               the seq_len[s] cached keys (zeros when there are none).
 *   ws, ws_bytes: optional workspace (convention above).  Without one (ws_bytes == NULL)
 *               each (sequence, layer, KV head) is one workgroup.  With one, shapes with
 *               fewer than 1024 (sequence, layer, KV head, pass of 4 heads) groups split their
 *               slots over 2-16 workgroups (a power of two, >= 128 slots each) and merge the
 *               partial softmax states in a second kernel; the size query returns 0 when the
 *               shape is not split, and never more than 4.3 MB.  A workspace smaller than the query's answer: TRI_EWORKSPACE.  The
 *               results of the two paths agree to float32 rounding (the summation order
 *               differs).
 * Errors as for the other calls. */
int tri_decode_attention(const tri_kv *kv, int32_t layer0, int32_t n_layers, const float *q,
                         const int64_t *query_pos, const int32_t *pos, int64_t pos_stride, double rope_base,
                         int32_t rope_layout, int32_t key_space, int32_t group, float *out, void *ws,
                         size_t *ws_bytes, void *stream);

/* tri_decode_attention without any allocation, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, results and errors as tri_decode_attention with a workspace, except:
 *   - the partial softmax states of a split shape go to a scratch array the library holds in
 *     device memory, 8 MiB per GPU, until the process ends (it is set up on the first call
 *     on each device); nothing is allocated or freed by the call;
 *   - a shape whose split needs more than those 8 MiB (tri_decode_attention's workspace size
 *     query returns the need) is refused with TRI_EWORKSPACE before anything is launched; the
 *     split rule above keeps every need under 4.3 MB, so this is a guard;
 *   - every call on one GPU shares that GPU's scratch: calls that overlap on one GPU (other
 *     streams or threads) race on it and must be serialised by the caller.  Each call writes
 *     every scratch entry it reads, so nothing has to be cleared between calls. */
int tri_decode_attention_noalloc(const tri_kv *kv, int32_t layer0, int32_t n_layers, const float *q,
                                 const int64_t *query_pos, const int32_t *pos, int64_t pos_stride,
                                 double rope_base, int32_t rope_layout, int32_t key_space, int32_t group,
                                 float *out, void *stream);

/* Text of the last failure on the calling thread ("" if none).  Owned by the library;
 * valid until the next call on this thread. */
const char *tri_last_error(void);

/* ABI version of this header: major * 10000 + minor * 100 + patch. */
int tri_version(void);

#define TRI_VERSION 10900

#ifdef __cplusplus
}
#endif

#endif /* TRI_H_ */
