"""Shared helpers of the GPU parity tests: oracle inputs, comparisons and tolerances.

The oracle's inputs are regenerated on the host from the workload seed (the host half of
the counter-based generator), never read back from the GPU path.  Tolerances:
  * scores: |s_gpu - s_oracle| <= 2e-3 * S_j, S_j = sum_f |k_f| (|E q_f| + |(1-R_f) E|q_f||)
    reduced over the group like the score (a bound on |s_j|; the scores are computed in
    float32 from the stored keys, the oracle in float64); for the multiplicative form
    S_j = n_j ||E q|| ||k_j|| (n_j = bands where centre and key parts are non-zero);
  * selection: exact against the oracle's selection applied to the GPU's own scores, and
    equal to the oracle's selection on oracle scores except for keys whose oracle score is
    within 2e-3 * S_j of the threshold score;
  * compaction: bit-exact given the kept indices.
"""

from __future__ import annotations

import numpy as np

import oracle
from kv_cache_compression_tri_amd import synth
from kv_cache_compression_tri_amd.synth import workloads as W

SCORE_TOL = 2e-3


# numpy view of a cache element's raw bits
BITS_VIEW = {"f32": np.int32, "bf16": np.int16, "fp8": np.uint8, "int8": np.int8}


def host_rows(w, hp, s, layer, kv_head, tag=synth.TAG_K, as_float=True):
    """One unit's rows from the host generator: the stored elements as the oracle decodes
    them (float64; 8-bit key codes times their head's scale), or the raw stored elements."""
    unit = W.unit_index(w, s, layer, kv_head)
    L = int(hp.lengths[s])
    scale = 1.0
    if tag == synth.TAG_K:
        mu, sig, sink = hp.mu_k[layer, kv_head], hp.sigma, w.sink
        if w.dtype in ("fp8", "int8"):
            scale = float(hp.k_scale[layer, kv_head])
    else:
        mu, sig, sink = np.zeros(w.head_dim, np.float32), np.ones(w.head_dim, np.float32), False
    raw = synth.rows(w.seed, tag, unit, L, mu, sig, sink, w.dtype, scale=scale)
    return oracle.decode_stored(raw, w.dtype, scale) if as_float else raw


def host_bits(w, hp, s, layer, kv_head, tag=synth.TAG_K):
    """Raw stored elements of one unit, viewed as the integer type of the cache element."""
    return host_rows(w, hp, s, layer, kv_head, tag, as_float=False).view(BITS_VIEW[w.dtype])


def oracle_scores(w, hp, s, layer, kv_head, keys, key_space="pre", form="additive"):
    center, mean_abs = oracle.unit_heads(hp.center, hp.mean_abs, layer, kv_head, w.group)
    sc = oracle.score_keys(keys, center, mean_abs, base=w.base, offsets=w.offsets,
                           layout=w.layout, reduce=w.reduce, key_space=key_space, form=form)
    S = oracle.score_magnitude_bound(keys, center, mean_abs, layout=w.layout, reduce=w.reduce, form=form)
    return sc, S


def check_scores(gpu, orc, S, tol=SCORE_TOL):
    gpu = np.asarray(gpu, dtype=np.float64)
    err = np.abs(gpu - orc) / S
    worst = float(err.max()) if err.size else 0.0
    big = np.abs(orc) >= 0.01 * S
    rel = float((np.abs(gpu - orc)[big] / np.abs(orc[big])).max()) if big.any() else 0.0
    assert np.all(np.isfinite(gpu)), "non-finite GPU score"
    assert worst <= tol, f"score error {worst:.3e} of the magnitude bound exceeds {tol}"
    return worst, rel


def check_kept(gpu_kept, gpu_scores, orc_scores, S, L, budget, window, tol=SCORE_TOL):
    n = min(L, budget)
    gk = np.asarray(gpu_kept[:n], dtype=np.int64)
    assert np.all(np.asarray(gpu_kept[n:]) == -1), "entries past kept_n must be -1"
    # exact: selection is a definition of the scores it is given
    exact = oracle.select_top_b(np.asarray(gpu_scores[:L], dtype=np.float64), L, budget, window)
    assert np.array_equal(gk, exact), "kept set differs from the oracle's selection of the GPU scores"
    # against oracle scores, outside the threshold band
    ok = oracle.select_top_b(orc_scores, L, budget, window)
    if L <= budget:
        assert np.array_equal(gk, ok)
        return 0
    w = min(window, budget)
    cand = L - w
    need = budget - w
    if need == 0:
        assert np.array_equal(gk, ok)
        return 0
    s = orc_scores[:cand].copy()
    s[np.isnan(s)] = -np.inf
    order = np.lexsort((np.arange(cand), -s))
    tau = s[order[need - 1]]
    excused = set(np.nonzero(np.abs(orc_scores - tau) <= tol * S)[0].tolist())
    a, b = set(gk.tolist()) - excused, set(ok.tolist()) - excused
    assert a == b, f"kept sets differ outside the threshold band: {sorted(a ^ b)[:10]}"
    return len(excused)
