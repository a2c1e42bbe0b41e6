"""Float64 CPU oracle of TriAttention's KV-cache compression step.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct statement of what
the compression pass computes.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the HIP library never does, and this
module imports nothing from the HIP library or its binding.  It shares no code, tables or
constants with the GPU path.

Sources (web pages about the paper "TriAttention: Efficient Long Reasoning with
Trigonometric KV Compression", Mao et al.), cited below by tag:

  [Review]   "TriAttention: Trigonometric KV Compression for Efficient Long Reasoning"
             (alanhou.org paper review): sections "Core Mechanism", "Key Concepts".
  [Abstract] "TriAttention: Efficient Long Reasoning with Trigonometric KV Compression"
             (chatpaper.ai abstract page), English abstract.
  [DevTo]    "TriAttention: How a Geometric Trick Cuts LLM Memory Use by 10x Without Losing
             Accuracy" (dev.to): sections "Why Existing KV Cache Compression Breaks in
             Production", "The Core Idea: Q/K Concentration in Pre-RoPE Space", "Solving
             the Memory Fragmentation Problem", "What the Numbers Look Like".
  [Project]  "TriAttention: trigonometric KV cache compression for long reasoning"
             (hysenlabs.com project page): sections "Pre-RoPE centres decide which keys
             are worth keeping", "The KV budget is a runtime knob that chat sessions
             should raise", "Calibration statistics are tied to a specific model".

The scoring contract (the pages give its parts; the exact additive form is the build's
documented reading of them).  For a pre-RoPE key k with RoPE bands k_f, f = 0..F-1
(F = d/2, theta_f = base^(-2f/d)), calibrated query statistics E[q_f] (complex centre) and
E|q_f| with concentration R_f = |E[q_f]| / E|q_f|, and future offsets Delta in D giving the
distance d = query_pos - key_pos + Delta:

    score(k) = mean_Delta sum_f |E[q_f]| |k_f| cos(d theta_f + arg E[q_f] - arg k_f)
             + sum_f (1 - R_f) E|q_f| |k_f|

A second, multiplicative form follows [Review] "Core Mechanism" (a trigonometric series
in the distance, then scaled by ||Q|| ||K||): the series keeps only the phases,

    score_mult(k) = mean_Delta sum_f cos(d theta_f + arg E[q_f] - arg k_f) * ||E q|| * ||k||

with ||E q|| the L2 norm of the query centre and ||k|| that of the key (bands where E[q_f]
or k_f is 0 have no phase and contribute 0 to the series).

Scores are reduced over the query heads of a GQA group (max or mean), the top-B keys of
each KV head are kept with the most recent window always kept, and the survivors are
packed forward into dense or paged storage.

Parity status: each public function is pinned by a CPU test against something other than
itself (tests/test_oracle_pins.py, tests/test_oracle_golden.py; planted mistakes in
tests/test_oracle_mutations.py must each fail one of them):
  rope_theta, split_bands, score_keys (additive)   exact-centre identity against textbook
        2x2 RoPE rotations, R = 0 limit, single-band hand values, invariants (shift,
        scaling, mean fold, identical heads, zero key)
  concentration            hand values, including the 0/0 band (read as 0)
  unit_heads               hand values of the contiguous GQA groups, and a score of KV head 1
                           that only its own query heads can produce
  score_magnitude_bound    equality with the score where every band is phase-aligned at
                           R = 1, hand values under max and mean with R < 1 and R > 1, and
                           |score| <= bound on random units
  score_keys (multiplicative)   hand value, aligned-phase closed form, the single-band
                           identity with the additive series, scaling by the key norm
  rope_apply               textbook rotation, inverse, post-RoPE keys score like pre-RoPE keys
  decode_fp8_e4m3          values the E4M3 format fixes (subnormals, normals, 448, NaN)
  decode_bf16, decode_stored   values the bfloat16 format fixes, and every one of the 65536
                           patterns against torch's own bfloat16 widening; int8 codes
  select_top_b             brute force over all subsets on tiny inputs, edge cases
  compact_dense, compact_paged_sequence   bit copies, forward packing, freed pages
  calibrate                closed forms (identical samples, rotating samples, scaling)
  decode_attention         one key, equal logits, a 3:1 hand weighting, relative positions
No function here is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "decode_fp8_e4m3",
    "decode_bf16",
    "decode_stored",
    "rope_theta",
    "rope_apply",
    "split_bands",
    "concentration",
    "score_keys",
    "score_magnitude_bound",
    "select_top_b",
    "compact_dense",
    "compact_paged_sequence",
    "calibrate",
    "unit_heads",
    "decode_attention",
]


# ---------------------------------------------------------------------------------------
# fp8 keys (OCP 8-bit floating point, E4M3 "fn" encoding)
# ---------------------------------------------------------------------------------------

def decode_fp8_e4m3(codes) -> np.ndarray:
    """Exact float64 values of OCP E4M3 codes (1 sign, 4 exponent bits with bias 7, 3
    mantissa bits; exponent field 0 is subnormal; S.1111.111 is NaN; there is no infinity).

    A cache may hold its keys as such codes times a positive scale, which composes the
    compression with KV quantisation ([Project], the project's news entries).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = sign * val
    out[(c & 0x7F) == 0x7F] = np.nan
    return out


def decode_bf16(bits) -> np.ndarray:
    """Exact float64 values of bfloat16 bit patterns (1 sign, 8 exponent bits with bias 127,
    7 mantissa bits; exponent field 0 is subnormal, 255 is infinity or NaN)."""
    b = np.asarray(bits).astype(np.int64) & 0xFFFF
    sign = np.where(b & 0x8000, -1.0, 1.0)
    e = (b >> 7) & 0xFF
    m = (b & 0x7F).astype(np.float64)
    with np.errstate(over="ignore"):
        val = np.where(e == 0, m * 2.0 ** -133, (1.0 + m / 128.0) * np.exp2(e - 127.0))
    val = np.where(e == 0xFF, np.where(m == 0, np.inf, np.nan), val)
    return sign * val


def decode_stored(raw, dtype: str, scale: float = 1.0) -> np.ndarray:
    """The float64 values a cache stores: float32 as is, bfloat16 bits decoded, and 8-bit
    codes (OCP E4M3 or two's-complement int8) decoded and multiplied by the head's scale
    (stored key = true key / scale).  This is the key the score is defined on."""
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return decode_bf16(np.asarray(raw).view(np.uint16))
    if dtype == "fp8":
        return decode_fp8_e4m3(np.asarray(raw).view(np.uint8)) * np.float64(scale)
    if dtype == "int8":
        return np.asarray(raw).view(np.int8).astype(np.float64) * np.float64(scale)
    raise ValueError(f"unknown cache dtype {dtype!r}")


# ---------------------------------------------------------------------------------------
# RoPE frequency bands
# ---------------------------------------------------------------------------------------

def rope_theta(base: float, head_dim: int) -> np.ndarray:
    """theta_f = base^(-2f/d) for f = 0 .. d/2-1, in float64.

    RoPE rotates each frequency pair by an angle proportional to position
    ([Review] "Key Concepts", trigonometric distance preference).
    """
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    f = np.arange(head_dim // 2, dtype=np.float64)
    return np.float64(base) ** (-2.0 * f / head_dim)


def rope_apply(x, positions, *, base: float, layout: str = "half", inverse: bool = False) -> np.ndarray:
    """Rotate every RoPE pair of the vectors x[L, d] by the angle p_j theta_f (float64).

    RoPE turns each frequency pair by an angle proportional to the token's position
    ([Review] "Key Concepts"): the pair (a, b) of a vector at position p becomes
    (a cos(p theta_f) - b sin(p theta_f), a sin(p theta_f) + b cos(p theta_f)).
    inverse=True turns by the opposite angle, which undoes the rotation.
    """
    x = np.asarray(x, dtype=np.float64)
    L, d = x.shape
    ang = np.asarray(positions, dtype=np.float64).reshape(L, 1) * rope_theta(base, d)[None, :]
    if inverse:
        ang = -ang
    c, s = np.cos(ang), np.sin(ang)
    if layout == "half":
        ia, ib = np.arange(d // 2), np.arange(d // 2, d)
    elif layout == "interleaved":
        ia, ib = np.arange(0, d, 2), np.arange(1, d, 2)
    else:
        raise ValueError(f"unknown layout {layout!r}")
    a, b = x[:, ia], x[:, ib]
    out = np.empty_like(x)
    out[:, ia] = a * c - b * s
    out[:, ib] = a * s + b * c
    return out


def split_bands(x, layout: str = "half") -> np.ndarray:
    """The complex RoPE bands x_f of vectors x[..., d] (exact float64 upcast).

    layout "half":        x_f = x[f] + i x[f + d/2]   (rotate-half pairing)
    layout "interleaved": x_f = x[2f] + i x[2f + 1]
    The pages do not say which pairing the models use; both are supported.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if layout == "half":
        return x[..., : d // 2] + 1j * x[..., d // 2:]
    if layout == "interleaved":
        return x[..., 0::2] + 1j * x[..., 1::2]
    raise ValueError(f"unknown layout {layout!r}")


# ---------------------------------------------------------------------------------------
# Calibration ([Review] "Key Concepts": the centre is the mean pre-RoPE query over a
# calibration set; [Project] "Calibration statistics are tied to a specific model")
# ---------------------------------------------------------------------------------------

def calibrate(q, layout: str = "half"):
    """Per-band query statistics from pre-RoPE query samples.

    q: [N, n_layer, n_qh, d].  Returns (center [n_layer, n_qh, F] complex128,
    mean_abs [n_layer, n_qh, F] float64): E[q_f] = mean_n q_{n,f} and
    E|q_f| = mean_n |q_{n,f}|.
    """
    qb = split_bands(q, layout)
    center = qb.mean(axis=0)
    mean_abs = np.abs(qb).mean(axis=0)
    return center, mean_abs


def concentration(center, mean_abs) -> np.ndarray:
    """R_f = |E[q_f]| / E|q_f| ([DevTo] "The Core Idea": a measured concentration metric).

    A band with E|q_f| = 0 has no query energy at all; R_f is read as 0 there (0/0 -> 0).
    No clamp is applied: statistics with R_f > 1 are used as given.
    """
    center = np.asarray(center, dtype=np.complex128)
    mean_abs = np.asarray(mean_abs, dtype=np.float64)
    mag = np.abs(center)
    out = np.zeros(np.broadcast(mag, mean_abs).shape, dtype=np.float64)
    np.divide(mag, mean_abs, out=out, where=mean_abs > 0)
    return out


# ---------------------------------------------------------------------------------------
# Scoring
# ---------------------------------------------------------------------------------------

def _trig_term(k_bands, key_pos, query_pos, center_h, theta, offsets):
    """mean_Delta sum_f |E q_f| |k_f| cos(d theta_f + arg E q_f - arg k_f), d = Q - p + Delta.

    The dot product of fixed centres after RoPE is a cosine series in the relative
    distance ([Review] "Core Mechanism" and "Key Concepts"; [Abstract]); it is evaluated
    at each future query position Q + Delta and averaged over the offsets.
    """
    q_abs = np.abs(center_h)                                  # |E[q_f]|        [F]
    q_arg = np.arctan2(center_h.imag, center_h.real)          # arg E[q_f]      [F]
    k_abs = np.abs(k_bands)                                   # |k_f|           [L, F]
    k_arg = np.arctan2(k_bands.imag, k_bands.real)            # arg k_f         [L, F]
    total = np.zeros(k_bands.shape[0], dtype=np.float64)
    for delta in offsets:
        dist = (np.float64(query_pos) - key_pos.astype(np.float64)) + np.float64(delta)
        phase = dist[:, None] * theta[None, :] + q_arg[None, :] - k_arg
        total += np.sum(q_abs[None, :] * k_abs * np.cos(phase), axis=1)
    return total / len(offsets)


def _trig_unit_term(k_bands, key_pos, query_pos, center_h, theta, offsets):
    """mean_Delta sum_f cos(d theta_f + arg E q_f - arg k_f), d = Q - p + Delta (phases only).

    The review's series in the distance ([Review] "Core Mechanism": one cosine per frequency
    band, summed, before the norm weighting): each band contributes the cosine of its
    phase difference at the distance, with unit amplitude.  A band whose centre or key part is 0
    has no phase and contributes 0.
    """
    q_arg = np.arctan2(center_h.imag, center_h.real)          # arg E[q_f]      [F]
    k_arg = np.arctan2(k_bands.imag, k_bands.real)            # arg k_f         [L, F]
    live = (np.abs(center_h)[None, :] > 0) & (np.abs(k_bands) > 0)
    total = np.zeros(k_bands.shape[0], dtype=np.float64)
    for delta in offsets:
        dist = (np.float64(query_pos) - key_pos.astype(np.float64)) + np.float64(delta)
        phase = dist[:, None] * theta[None, :] + q_arg[None, :] - k_arg
        total += np.sum(np.where(live, np.cos(phase), 0.0), axis=1)
    return total / len(offsets)


def _l2_norm(bands):
    """||x|| = sqrt(sum_f |x_f|^2) over the bands of each row (the vector's L2 norm)."""
    return np.sqrt(np.sum(np.abs(bands) ** 2, axis=-1))


def _norm_term(k_bands, center_h, mean_abs_h):
    """sum_f (1 - R_f) E|q_f| |k_f|.

    Norms carry importance ([Review] "Key Concepts", norm as importance signal); weakly
    concentrated heads lean on this norm-only signal in proportion to 1 - R_f ([DevTo]
    "The Core Idea").  For a band with E|q_f| = 0 the product is read as 0.
    """
    R = concentration(center_h, mean_abs_h)
    coef = (1.0 - R) * np.asarray(mean_abs_h, dtype=np.float64)
    return np.sum(coef[None, :] * np.abs(k_bands), axis=1)


def score_keys(keys, center, mean_abs, *, base: float, offsets, key_pos=None,
               query_pos=None, layout: str = "half", reduce: str = "max",
               return_heads: bool = False, key_space: str = "pre", form: str = "additive"):
    """Score every cached key of one (layer, KV head) unit.

    keys:     [L, d] cached keys (any float dtype; upcast exactly to float64): pre-RoPE
              (key_space "pre"), or already rotated by RoPE at key_pos (key_space
              "post"), in which case they are turned back to pre-RoPE first: the score
              is defined on pre-RoPE keys ([Review] "Framework Shift"; [DevTo] "The Core
              Idea: Q/K Concentration in Pre-RoPE Space")
    center:   [G, F] complex E[q_f] of the G query heads of the group
              (or [G, F, 2] real/imaginary pairs)
    mean_abs: [G, F] E|q_f|
    key_pos:  [L] RoPE positions of the keys (default: slot index 0..L-1)
    query_pos: position of the newest query (default: L - 1)
    reduce:   "max" or "mean" over the G query heads of the group
    form:     "additive" (the trig series of centre/key band pairs plus the
              concentration-weighted norm term) or "multiplicative" (the phase-only
              series times ||E q|| ||k||, [Review] "Core Mechanism"; mean_abs is unused)

    Returns float64 scores [L] (and the per-head scores [G, L] if return_heads).
    The series is position-aware: the keys are scored at their positions relative to
    the queries that will read them ([Review] "Framework Shift").
    """
    keys = np.asarray(keys, dtype=np.float64)
    L, d = keys.shape
    center = _as_complex(center)
    mean_abs = np.asarray(mean_abs, dtype=np.float64)
    if center.ndim == 1:
        center = center[None, :]
        mean_abs = mean_abs[None, :]
    if key_pos is None:
        key_pos = np.arange(L, dtype=np.int64)
    key_pos = np.asarray(key_pos, dtype=np.int64)
    if query_pos is None:
        query_pos = L - 1
    if key_space == "post":
        keys = rope_apply(keys, key_pos, base=base, layout=layout, inverse=True)
    elif key_space != "pre":
        raise ValueError(f"unknown key_space {key_space!r}")
    theta = rope_theta(base, d)
    kb = split_bands(keys, layout)

    if form not in ("additive", "multiplicative"):
        raise ValueError(f"unknown score form {form!r}")
    heads = []
    for h in range(center.shape[0]):
        if form == "multiplicative":
            series = _trig_unit_term(kb, key_pos, query_pos, center[h], theta, offsets)
            heads.append(series * _l2_norm(center[h][None, :])[0] * _l2_norm(kb))
            continue
        trig = _trig_term(kb, key_pos, query_pos, center[h], theta, offsets)
        norm = _norm_term(kb, center[h], mean_abs[h])
        heads.append(trig + norm)
    heads = np.stack(heads, axis=0) if heads else np.zeros((0, L))
    scores = _reduce_heads(heads, reduce)
    if return_heads:
        return scores, heads
    return scores


def score_magnitude_bound(keys, center, mean_abs, *, layout: str = "half",
                          reduce: str = "max", form: str = "additive") -> np.ndarray:
    """S_j = sum_f |k_f| (|E q_f| + |(1 - R_f) E|q_f||), reduced over heads like the score
    (multiplicative form: n_j ||E q|| ||k_j||, n_j = bands where both parts are non-zero).

    |score_j| <= S_j for every key; it is the scale against which score errors are
    measured (a plain |error| / |score| is unbounded where a signed score crosses 0).
    """
    if form == "multiplicative":
        kb = split_bands(np.asarray(keys, dtype=np.float64), layout)
        center = _as_complex(center)
        if center.ndim == 1:
            center = center[None, :]
        k_norm = np.sqrt(np.sum(np.abs(kb) ** 2, axis=1))
        heads = []
        for h in range(center.shape[0]):
            live = (np.abs(center[h])[None, :] > 0) & (np.abs(kb) > 0)
            heads.append(live.sum(axis=1) * np.sqrt(np.sum(np.abs(center[h]) ** 2)) * k_norm)
        return _reduce_heads(np.stack(heads, axis=0), reduce)
    keys = np.asarray(keys, dtype=np.float64)
    center = _as_complex(center)
    mean_abs = np.asarray(mean_abs, dtype=np.float64)
    if center.ndim == 1:
        center = center[None, :]
        mean_abs = mean_abs[None, :]
    k_abs = np.abs(split_bands(keys, layout))
    heads = []
    for h in range(center.shape[0]):
        R = concentration(center[h], mean_abs[h])
        coef = np.abs(center[h]) + np.abs((1.0 - R) * mean_abs[h])
        heads.append(np.sum(coef[None, :] * k_abs, axis=1))
    return _reduce_heads(np.stack(heads, axis=0), reduce)


def _reduce_heads(heads, reduce):
    if reduce == "max":
        return np.max(heads, axis=0)
    if reduce == "mean":
        return np.mean(heads, axis=0)
    raise ValueError(f"unknown reduce {reduce!r}")


def _as_complex(c):
    c = np.asarray(c)
    if np.iscomplexobj(c):
        return c.astype(np.complex128)
    c = c.astype(np.float64)
    if c.shape[-1] != 2:
        raise ValueError("real center arrays must end in a (re, im) axis of size 2")
    return c[..., 0] + 1j * c[..., 1]


def unit_heads(center, mean_abs, layer: int, kv_head: int, group: int):
    """Statistics of the query heads that read KV head ``kv_head``.

    center [n_layer, n_qh, F(,2)], mean_abs [n_layer, n_qh, F].  Query head h reads
    KV head h // group (contiguous GQA groups).
    """
    n_qh = np.asarray(mean_abs).shape[1]
    if group < 1 or kv_head < 0 or (kv_head + 1) * group > n_qh:
        raise ValueError(f"KV head {kv_head} with {group} query heads each needs more than {n_qh} query heads")
    hs = slice(kv_head * group, (kv_head + 1) * group)
    return _as_complex(np.asarray(center)[layer, hs]), np.asarray(mean_abs, np.float64)[layer, hs]


# ---------------------------------------------------------------------------------------
# Selection ([Review] "Core Mechanism": keep only the top-scoring keys; [Project] "The KV
# budget is a runtime knob": the budget bounds the whole kept cache; [DevTo] "What the
# Numbers Look Like": a 3,072-token budget for 32K-token generations)
# ---------------------------------------------------------------------------------------

def select_top_b(scores, length: int, budget: int, window: int) -> np.ndarray:
    """Kept slot indices of one unit, ascending.

    If length <= budget every slot is kept.  Otherwise the last W' = min(window, budget)
    slots are always kept, and the remaining B - W' slots are the best of the other
    candidates ranked by (score descending, slot ascending); a NaN score ranks as -inf.
    """
    if budget < 1 or window < 0:
        raise ValueError("budget must be >= 1 and window >= 0")
    L = int(length)
    if L <= budget:
        return np.arange(L, dtype=np.int64)
    w = min(window, budget)
    n_cand = L - w
    s = np.asarray(scores, dtype=np.float64)[:n_cand].copy()
    s[np.isnan(s)] = -np.inf
    slots = np.arange(n_cand, dtype=np.int64)
    order = np.lexsort((slots, -s))        # last key is primary: -score asc, then slot asc
    top = slots[order[: budget - w]]
    return np.sort(np.concatenate([top, np.arange(n_cand, L, dtype=np.int64)]))


# ---------------------------------------------------------------------------------------
# Compaction ([DevTo] "Solving the Memory Fragmentation Problem": survivors are moved
# forward into as few blocks as possible so the emptied tail blocks can be reclaimed;
# "Why Existing KV Cache Compression Breaks in Production": a paged allocator can only
# free a block that is completely empty)
# ---------------------------------------------------------------------------------------

def compact_dense(k, v, kept, pos=None):
    """Dense compaction of one unit: rows kept[i] move to slot i (bit copy).

    Returns (k_out, v_out or None, pos_out) where pos_out[i] is the RoPE position of the
    row now in slot i (the slot index itself when ``pos`` is None).
    """
    kept = np.asarray(kept, dtype=np.int64)
    k_out = np.asarray(k)[kept]
    v_out = None if v is None else np.asarray(v)[kept]
    pos_out = kept.copy() if pos is None else np.asarray(pos)[kept]
    return k_out, v_out, pos_out


def compact_paged_sequence(pool_k, pool_v, block_table_row, length: int, kept_by_unit,
                           page: int = 16):
    """Forward-pack one sequence of a paged cache.

    pool_k, pool_v: [n_pages, n_layer, n_kvh, page, d] (copies are returned, inputs are
      not modified; pool_v may be None)
    block_table_row: [max_pages] page ids of the sequence (slot j lives in page
      block_table_row[j // page], row j % page)
    kept_by_unit: dict {(layer, kv_head): kept slots (ascending)}; every unit of the
      sequence keeps the same number of rows.

    Returns (pool_k', pool_v', freed_pages, new_len): row kept[i] of each unit is moved to
    slot i, new_len = number kept, and the pages past ceil(new_len / page) that held the
    sequence before are returned as freed (each is now empty).
    """
    bt = np.asarray(block_table_row, dtype=np.int64)
    out_k = np.array(pool_k, copy=True)
    out_v = None if pool_v is None else np.array(pool_v, copy=True)
    counts = {len(np.asarray(v)) for v in kept_by_unit.values()}
    if len(counts) > 1:
        raise ValueError("every unit of a sequence must keep the same number of rows")
    new_len = counts.pop() if counts else min(int(length), 0)
    for (layer, head), kept in kept_by_unit.items():
        kept = np.asarray(kept, dtype=np.int64)
        src_page, src_row = bt[kept // page], kept % page
        dst = np.arange(len(kept), dtype=np.int64)
        dst_page, dst_row = bt[dst // page], dst % page
        # gather from the pre-compaction snapshot, then scatter forward
        rows_k = np.asarray(pool_k)[src_page, layer, head, src_row]
        out_k[dst_page, layer, head, dst_row] = rows_k
        if out_v is not None:
            rows_v = np.asarray(pool_v)[src_page, layer, head, src_row]
            out_v[dst_page, layer, head, dst_row] = rows_v
    used_before = -(-int(length) // page)
    used_after = -(-int(new_len) // page)
    freed = bt[used_after:used_before].copy()
    return out_k, out_v, freed, int(new_len)


# ---------------------------------------------------------------------------------------
# The consumer of the compressed cache: RoPE at the kept keys' positions, then attention
# ---------------------------------------------------------------------------------------

def decode_attention(q, keys, values, *, base: float, key_pos, query_pos: int,
                     layout: str = "half", key_space: str = "pre") -> np.ndarray:
    """Attention of the newest token's query heads over a (compressed) cache.

    After compression the surviving keys are rotated by RoPE at their own positions and
    read by standard attention ([Review] "Core Mechanism": apply RoPE, then attention on
    the compressed cache); compacted slots no longer equal positions, so the positions
    come from the compaction's position output.

    q:        [G, d] pre-RoPE query vectors of the query heads reading this KV head,
              at position query_pos
    keys:     [L, d] cached keys, pre-RoPE (key_space "pre", rotated here at key_pos) or
              already rotated at their positions (key_space "post")
    values:   [L, d]
    key_pos:  [L] RoPE positions of the cached keys

    Returns float64 [G, d]: softmax_j((R(Q) q) . (R(p_j) k_j) / sqrt(d)) weighted sum of the
    values (zeros when L = 0).
    """
    q = np.atleast_2d(np.asarray(q, dtype=np.float64))
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    G, d = q.shape
    L = keys.shape[0]
    if L == 0:
        return np.zeros((G, d))
    key_pos = np.asarray(key_pos, dtype=np.int64)
    q_rot = rope_apply(q, np.full(G, query_pos), base=base, layout=layout)
    k_rot = keys if key_space == "post" else rope_apply(keys, key_pos, base=base, layout=layout)
    logits = q_rot @ k_rot.T / np.sqrt(d)                                   # [G, L]
    logits = logits - logits.max(axis=1, keepdims=True)
    w = np.exp(logits)
    w /= w.sum(axis=1, keepdims=True)
    return w @ values
