"""Pins of the float64 oracle against facts fixed outside the oracle itself.

Each test states what it pins.  Nothing here calls the HIP library.
  P1  exact-centre identity: with E[q] = q the trig series equals the mean over the
      offsets of the post-RoPE dot product, computed with textbook 2x2 rotations
  P2  R = 0 limit: zero centre leaves the pure norm term
  P3  single-band hand values (3-4-5 triangle) and theta_f hand values
  P4  invariants: position shift, key scaling, mean-fold linearity, identical heads, k = 0
  P5  brute-force top-B on tiny inputs (all subsets), plus window / budget edge cases
  P6  calibration closed forms
  P7  compaction invariants
  P9  keys cached after RoPE: the oracle's rotation equals textbook RoPE, undoes itself,
      and scoring rotated keys equals scoring the pre-RoPE keys
  P10 fp8 (OCP E4M3) key codes: values the format definition fixes; bfloat16 patterns:
      values the format fixes and all 65536 patterns against torch's widening; int8 codes
  P11 multiplicative form: hand value, aligned-phase closed form, the single-band
      identity with the amplitude series, and scaling by the key norm
  P12 attention over the compressed cache: one key returns its value, equal logits
      average the values, a hand-made 3:1 weighting, the relative-position property
      against textbook RoPE, and post-RoPE keys give the same result
  P13 the statistics a KV head reads (contiguous GQA groups) and the magnitude bound S_j:
      hand values for the group of KV head 1, equality s_j = S_j where every band is
      phase-aligned at R = 1, hand values of S_j under max and mean, and a band with no
      query energy (E|q_f| = E[q_f] = 0, concentration 0/0 read as 0)
"""

import itertools
import math

import numpy as np
import pytest

import oracle
from oracle import triattention as T

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------------------------------
# helpers that are independent of the oracle's formula
# ---------------------------------------------------------------------------------------

def rope_rotate(x, position, base, layout):
    """Textbook RoPE: rotate each frequency pair of x by position * theta_f with an
    explicit 2x2 rotation matrix.  theta_f = base ** (-2 f / d) written out per f."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    out = np.empty_like(x)
    for f in range(d // 2):
        theta = base ** (-(2.0 * f) / d)
        ang = position * theta
        c, s = math.cos(ang), math.sin(ang)
        if layout == "half":
            i0, i1 = f, f + d // 2
        else:
            i0, i1 = 2 * f, 2 * f + 1
        rot = np.array([[c, -s], [s, c]])
        out[..., [i0, i1]] = np.stack([x[..., i0], x[..., i1]], -1) @ rot.T
    return out


def bands_of(x, layout):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if layout == "half":
        re, im = x[..., : d // 2], x[..., d // 2:]
    else:
        re, im = x[..., 0::2], x[..., 1::2]
    return np.stack([re, im], axis=-1)          # [..., F, 2] real pairs


# ---------------------------------------------------------------------------------------
# P1 exact-centre identity
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("layout", ["half", "interleaved"])
@pytest.mark.parametrize("d,base,qpos,offsets", [
    (128, 1e4, 2047, [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024]),
    (128, 1e6, 131071, [2 ** i for i in range(15)]),
    (16, 500.0, 37, [1, 3, 9]),
])
def test_p1_exact_centre_identity(layout, d, base, qpos, offsets):
    rng = np.random.default_rng(7)
    q = rng.standard_normal(d)
    L = 24
    keys = rng.standard_normal((L, d)) * rng.uniform(0.2, 3.0, (L, 1))
    key_pos = np.sort(rng.choice(qpos + 1, size=L, replace=False))
    key_pos[-1] = qpos
    center = bands_of(q, layout)[None]                                   # E[q] = q
    mag = np.hypot(center[..., 0], center[..., 1])                       # E|q_f| = |q_f|
    got = oracle.score_keys(keys, center, mag, base=base, offsets=offsets,
                            key_pos=key_pos, query_pos=qpos, layout=layout)
    want = np.zeros(L)
    for delta in offsets:
        rq = rope_rotate(q, qpos + delta, base, layout)
        for j in range(L):
            want[j] += rope_rotate(keys[j], key_pos[j], base, layout) @ rq
    want /= len(offsets)
    bound = oracle.score_magnitude_bound(keys, center, mag, layout=layout)
    assert np.all(np.abs(got - want) <= 1e-9 * bound)


# ---------------------------------------------------------------------------------------
# P2 R = 0 limit
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("layout", ["half", "interleaved"])
def test_p2_zero_centre_is_pure_norm(layout):
    rng = np.random.default_rng(3)
    d, L = 128, 50
    keys = rng.standard_normal((L, d))
    mean_abs = rng.uniform(0.1, 2.0, (1, d // 2))
    center = np.zeros((1, d // 2, 2))
    got = oracle.score_keys(keys, center, mean_abs, base=1e4, offsets=[1, 2, 4], layout=layout)
    kb = bands_of(keys, layout)
    k_abs = np.hypot(kb[..., 0], kb[..., 1])
    want = (k_abs * mean_abs[0][None, :]).sum(axis=1)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=0)


def test_p2_partial_concentration_norm_coefficient():
    # one band (d = 2, theta_0 = 1), E q = 0.6 (arg 0) against E|q| = 2: R = 0.3, so the
    # norm coefficient is (1 - 0.3) * 2 = 1.4.  k = 2i (|k| = 2, arg pi/2), distance Delta:
    # trig = 0.6 * 2 * cos(Delta - pi/2) = 1.2 sin(Delta);  norm = 1.4 * 2
    keys = np.array([[0.0, 2.0]])
    center = np.array([[[0.6, 0.0]]])
    mean_abs = np.array([[2.0]])
    delta = 5
    got = oracle.score_keys(keys, center, mean_abs, base=10.0, offsets=[delta],
                            key_pos=[0], query_pos=0)
    want = 1.2 * math.sin(delta) + 2.8
    assert abs(got[0] - want) < 1e-14


# ---------------------------------------------------------------------------------------
# P3 hand values
# ---------------------------------------------------------------------------------------

def test_p3_theta_hand_values():
    th = oracle.rope_theta(10000.0, 4)
    assert th[0] == 1.0
    assert abs(th[1] - 0.01) < 1e-18
    th = oracle.rope_theta(1e6, 128)
    assert abs(th[32] - 1e-3) < 1e-18            # 1e6 ** (-64/128) = 1e-3
    assert abs(th[63] - 1e6 ** (-126 / 128)) < 1e-20


@pytest.mark.parametrize("delta", [1, 7, 1000, 147455])
def test_p3_single_band_345(delta):
    # d = 2 (one band), theta_0 = 1.  E q = 2i (|Eq| = 2, E|q| = 2, R = 1, no norm term),
    # k = 3 + 4i (|k| = 5, arg k = phi with cos phi = 0.6, sin phi = 0.8).
    # score = 10 cos(delta + pi/2 - phi) = 10 (sin(phi) cos(delta) - cos(phi) sin(delta))
    #       = 8 cos(delta) - 6 sin(delta)
    keys = np.array([[3.0, 4.0]])
    center = np.array([[[0.0, 2.0]]])
    got = oracle.score_keys(keys, center, np.array([[2.0]]), base=10.0, offsets=[delta],
                            key_pos=[0], query_pos=0)
    want = 8.0 * math.cos(delta) - 6.0 * math.sin(delta)
    # the phase argument is ~delta in size: allow a few ulps of it, times |Eq||k| = 10
    assert abs(got[0] - want) < 10 * 4 * np.spacing(float(delta) + 4.0)


def test_p3_zero_distance_quarter_turn():
    # E q = i, k = 1, distance 0: cos(pi/2) = 0
    keys = np.array([[1.0, 0.0]])
    got = oracle.score_keys(keys, np.array([[[0.0, 1.0]]]), np.array([[1.0]]), base=10.0,
                            offsets=[0], key_pos=[0], query_pos=0)
    assert abs(got[0]) < 1e-15


def test_p3_offsets_are_averaged():
    # E q = 1, k = 1, theta_0 = 1, Q = p: each offset contributes cos(Delta); the score is
    # their mean, not their sum
    keys = np.array([[1.0, 0.0]])
    c = np.array([[[1.0, 0.0]]])
    m = np.array([[1.0]])
    one = oracle.score_keys(keys, c, m, base=10.0, offsets=[0], key_pos=[0], query_pos=0)
    two = oracle.score_keys(keys, c, m, base=10.0, offsets=[0, 2], key_pos=[0], query_pos=0)
    assert abs(one[0] - 1.0) < 1e-15
    assert abs(two[0] - 0.5 * (1.0 + (1.0 - 2.0 * math.sin(1.0) ** 2))) < 1e-15   # cos 2 = 1 - 2 sin^2 1


# ---------------------------------------------------------------------------------------
# P4 invariants
# ---------------------------------------------------------------------------------------

def _random_unit(rng, G=3, L=40, d=32):
    keys = rng.standard_normal((L, d)) + rng.standard_normal(d)
    center = rng.standard_normal((G, d // 2, 2))
    mag = np.hypot(center[..., 0], center[..., 1])
    mean_abs = mag * rng.uniform(1.0, 3.0, mag.shape)
    return keys, center, mean_abs


def test_p4_shift_invariance():
    rng = np.random.default_rng(11)
    keys, center, mean_abs = _random_unit(rng)
    pos = np.arange(keys.shape[0])
    kw = dict(base=1e4, offsets=[1, 4, 16, 64])
    a = oracle.score_keys(keys, center, mean_abs, key_pos=pos, query_pos=39, **kw)
    b = oracle.score_keys(keys, center, mean_abs, key_pos=pos + 100003, query_pos=39 + 100003, **kw)
    S = oracle.score_magnitude_bound(keys, center, mean_abs)
    assert np.all(np.abs(a - b) <= 1e-9 * S)


def test_p4_key_scaling():
    rng = np.random.default_rng(12)
    keys, center, mean_abs = _random_unit(rng)
    kw = dict(base=1e4, offsets=[1, 2, 3])
    a = oracle.score_keys(keys, center, mean_abs, **kw)
    b = oracle.score_keys(2.5 * keys, center, mean_abs, **kw)
    np.testing.assert_allclose(b, 2.5 * a, rtol=1e-12, atol=1e-12)
    assert np.array_equal(oracle.select_top_b(a, 40, 12, 4), oracle.select_top_b(b, 40, 12, 4))


def test_p4_mean_fold_linearity():
    # mean over heads == one head whose E q is the head-mean of E q and whose norm
    # coefficient E|q| - |E q| is the head-mean of the heads' coefficients
    rng = np.random.default_rng(13)
    keys, center, mean_abs = _random_unit(rng, G=4)
    cq = center[..., 0] + 1j * center[..., 1]
    c_bar = cq.mean(axis=0)
    n_bar = (mean_abs - np.abs(cq)).mean(axis=0)
    m_bar = np.abs(c_bar) + n_bar
    kw = dict(base=1e4, offsets=[1, 2, 4, 8])
    a = oracle.score_keys(keys, center, mean_abs, reduce="mean", **kw)
    b = oracle.score_keys(keys, c_bar[None], m_bar[None], reduce="max", **kw)
    S = oracle.score_magnitude_bound(keys, center, mean_abs, reduce="mean")
    assert np.all(np.abs(a - b) <= 1e-12 * S)


def test_p4_identical_heads_and_max():
    rng = np.random.default_rng(14)
    keys, center, mean_abs = _random_unit(rng, G=1)
    kw = dict(base=1e4, offsets=[1, 2, 4])
    one = oracle.score_keys(keys, center, mean_abs, **kw)
    c3 = np.repeat(center, 3, axis=0)
    m3 = np.repeat(mean_abs, 3, axis=0)
    np.testing.assert_allclose(oracle.score_keys(keys, c3, m3, reduce="max", **kw), one, rtol=1e-14)
    np.testing.assert_allclose(oracle.score_keys(keys, c3, m3, reduce="mean", **kw), one, rtol=1e-13)
    # max over distinct heads equals the elementwise max of single-head scores
    keys, center, mean_abs = _random_unit(rng, G=3)
    s, heads = oracle.score_keys(keys, center, mean_abs, return_heads=True, **kw)
    for h in range(3):
        single = oracle.score_keys(keys, center[h:h + 1], mean_abs[h:h + 1], **kw)
        np.testing.assert_array_equal(heads[h], single)
    np.testing.assert_array_equal(s, heads.max(axis=0))


def test_p4_zero_key_scores_zero():
    rng = np.random.default_rng(15)
    keys, center, mean_abs = _random_unit(rng)
    keys[5] = 0.0
    s = oracle.score_keys(keys, center, mean_abs, base=1e4, offsets=[1, 2])
    assert s[5] == 0.0


def test_p4_bound_dominates_score():
    rng = np.random.default_rng(16)
    keys, center, mean_abs = _random_unit(rng, G=4, L=200)
    mean_abs[1] *= 0.5                       # some R > 1 bands too
    for reduce in ("max", "mean"):
        s = oracle.score_keys(keys, center, mean_abs, base=1e6, offsets=[1, 2, 4], reduce=reduce)
        S = oracle.score_magnitude_bound(keys, center, mean_abs, reduce=reduce)
        assert np.all(np.abs(s) <= S * (1 + 1e-12))


def test_p4_r_above_one_not_clamped():
    # E|q| < |E q| gives a negative norm coefficient, used as written
    keys = np.array([[0.0, 1.0]])                      # |k| = 1
    center = np.array([[[2.0, 0.0]]])                  # |Eq| = 2
    mean_abs = np.array([[1.0]])                       # R = 2
    got = oracle.score_keys(keys, center, mean_abs, base=10.0, offsets=[0], key_pos=[0], query_pos=0)
    # trig: 2 * 1 * cos(0 + 0 - pi/2) = 0 ; norm: (1 - 2) * 1 * 1 = -1
    assert abs(got[0] - (-1.0)) < 1e-15


# ---------------------------------------------------------------------------------------
# P5 selection vs brute force
# ---------------------------------------------------------------------------------------

def brute_force_kept(scores, L, B, W):
    """All subsets: keep the window, then among the candidate subsets of the right size
    take the one whose descending score vector is largest, ties to the smallest slots."""
    if L <= B:
        return list(range(L))
    w = min(W, B)
    cand = list(range(L - w))
    s = [(-math.inf if math.isnan(x) else x) for x in scores]
    best = None
    for sub in itertools.combinations(cand, B - w):
        key = (tuple(sorted((s[j] for j in sub), reverse=True)), tuple(-j for j in sub))
        if best is None or key > best[0]:
            best = (key, sub)
    return sorted(list(best[1]) + list(range(L - w, L)))


@pytest.mark.parametrize("trial", range(60))
def test_p5_select_matches_brute_force(trial):
    rng = np.random.default_rng(1000 + trial)
    L = int(rng.integers(1, 12))
    B = int(rng.integers(1, 12))
    W = int(rng.integers(0, 6))
    kind = trial % 4
    if kind == 0:
        s = rng.standard_normal(L)
    elif kind == 1:
        s = rng.integers(-2, 3, L).astype(float)          # many ties
    elif kind == 2:
        s = rng.standard_normal(L)
        s[rng.integers(0, L)] = np.nan
        s[rng.integers(0, L)] = -np.inf
    else:
        s = np.zeros(L)
        s[rng.integers(0, L)] = -0.0
    got = oracle.select_top_b(s, L, B, W)
    assert list(got) == brute_force_kept(list(s), L, B, W)


def test_p5_edge_cases():
    s = np.arange(10.0)[::-1]          # slot 0 best
    assert list(oracle.select_top_b(s, 10, 10, 3)) == list(range(10))      # L <= B
    assert list(oracle.select_top_b(s, 10, 4, 8)) == [6, 7, 8, 9]          # W >= B: window only
    assert list(oracle.select_top_b(s, 10, 4, 0)) == [0, 1, 2, 3]          # W = 0
    assert list(oracle.select_top_b(s, 10, 9, 2)) == [0, 1, 2, 3, 4, 5, 6, 8, 9]   # B = L - 1
    assert list(oracle.select_top_b(np.zeros(6), 6, 3, 1)) == [0, 1, 5]    # ties -> low slots
    assert list(oracle.select_top_b(np.full(6, np.nan), 6, 3, 1)) == [0, 1, 5]


# ---------------------------------------------------------------------------------------
# P6 calibration closed forms
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("layout", ["half", "interleaved"])
def test_p6_identical_samples(layout):
    rng = np.random.default_rng(21)
    q = rng.standard_normal((2, 3, 16))
    samples = np.broadcast_to(q, (7, 2, 3, 16))
    center, mean_abs = oracle.calibrate(samples, layout)
    qb = bands_of(q, layout)
    np.testing.assert_allclose(center.real, qb[..., 0], rtol=1e-15)
    np.testing.assert_allclose(center.imag, qb[..., 1], rtol=1e-15)
    np.testing.assert_allclose(mean_abs, np.hypot(qb[..., 0], qb[..., 1]), rtol=1e-15)
    np.testing.assert_allclose(oracle.concentration(center, mean_abs), 1.0, rtol=1e-15)


def test_p6_rotating_samples_have_zero_centre():
    N, r = 12, 1.7
    ang = 2 * np.pi * np.arange(N) / N + 0.3
    q = np.zeros((N, 1, 1, 4))
    q[:, 0, 0, 0] = r * np.cos(ang)       # band 0 (half layout: re = x[0], im = x[2])
    q[:, 0, 0, 2] = r * np.sin(ang)
    q[:, 0, 0, 1] = 2.0                   # band 1 constant: centre 2 + 0i
    center, mean_abs = oracle.calibrate(q, "half")
    assert abs(center[0, 0, 0]) < 1e-15
    assert abs(mean_abs[0, 0, 0] - r) < 1e-15
    assert abs(center[0, 0, 1] - 2.0) < 1e-15
    assert oracle.concentration(center, mean_abs)[0, 0, 0] < 1e-15


def test_p6_scaling_and_permutation():
    rng = np.random.default_rng(22)
    q = rng.standard_normal((9, 2, 2, 8))
    c1, m1 = oracle.calibrate(q)
    c2, m2 = oracle.calibrate(3.0 * q[rng.permutation(9)])
    np.testing.assert_allclose(c2, 3.0 * c1, rtol=1e-13)
    np.testing.assert_allclose(m2, 3.0 * m1, rtol=1e-13)


# ---------------------------------------------------------------------------------------
# P7 compaction invariants
# ---------------------------------------------------------------------------------------

def test_p7_dense_rows_are_bit_copies():
    rng = np.random.default_rng(31)
    k = rng.standard_normal((50, 8)).astype(np.float32)
    v = rng.standard_normal((50, 8)).astype(np.float32)
    kept = np.sort(rng.choice(50, 13, replace=False))
    ko, vo, po = oracle.compact_dense(k, v, kept)
    assert ko.tobytes() == b"".join(k[j].tobytes() for j in kept)
    assert vo.tobytes() == b"".join(v[j].tobytes() for j in kept)
    assert list(po) == list(kept)
    pos = rng.integers(0, 10 ** 6, 50)
    _, _, po = oracle.compact_dense(k, None, kept, pos=pos)
    assert list(po) == list(pos[kept])


def test_p7_paged_forward_packing():
    rng = np.random.default_rng(32)
    page, n_layer, n_kvh, d = 4, 2, 3, 5
    L, B, W = 37, 14, 3
    n_used = -(-L // page)
    n_pages = n_used + 5
    pool = rng.standard_normal((n_pages, n_layer, n_kvh, page, d))
    pool_v = rng.standard_normal((n_pages, n_layer, n_kvh, page, d))
    bt = rng.permutation(n_pages)[:n_used]
    kept = {}
    for l in range(n_layer):
        for h in range(n_kvh):
            kept[(l, h)] = oracle.select_top_b(rng.standard_normal(L), L, B, W)
    pk, pv, freed, new_len = oracle.compact_paged_sequence(pool, pool_v, bt, L, kept, page)
    assert new_len == min(B, L)
    kept_pages = bt[: -(-new_len // page)]
    assert set(freed) | set(kept_pages) == set(bt)
    assert not (set(freed) & set(kept_pages))
    assert len(set(freed)) == len(freed)
    for (l, h), kk in kept.items():
        for i, j in enumerate(kk):
            got = pk[bt[i // page], l, h, i % page]
            src = pool[bt[j // page], l, h, j % page]
            assert got.tobytes() == src.tobytes()
            assert pv[bt[i // page], l, h, i % page].tobytes() == pool_v[bt[j // page], l, h, j % page].tobytes()
    # pages outside the sequence are untouched
    others = sorted(set(range(n_pages)) - set(bt))
    assert pk[others].tobytes() == pool[others].tobytes()


# ---------------------------------------------------------------------------------------
# P9 keys cached after RoPE
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("layout", ["half", "interleaved"])
def test_p9_rope_apply_is_textbook_rope(layout):
    rng = np.random.default_rng(21)
    x = rng.standard_normal((9, 128))
    pos = np.array([0, 1, 2, 17, 255, 4096, 32767, 131071, 147455])
    got = oracle.rope_apply(x, pos, base=1e6, layout=layout)
    want = np.stack([rope_rotate(x[i], int(pos[i]), 1e6, layout) for i in range(len(pos))])
    # the two compute theta_f with different rounding; the angle error grows with p
    tol = 1e-14 * (pos[:, None] + 1.0)
    assert np.all(np.abs(got - want) <= tol)
    back = oracle.rope_apply(got, pos, base=1e6, layout=layout, inverse=True)
    assert np.all(np.abs(back - x) <= tol)
    assert np.array_equal(oracle.rope_apply(x[:1], [0], base=1e6, layout=layout), x[:1])


@pytest.mark.parametrize("layout", ["half", "interleaved"])
@pytest.mark.parametrize("reduce", ["max", "mean"])
def test_p9_post_rope_keys_score_like_pre_rope_keys(layout, reduce):
    rng = np.random.default_rng(22)
    d, G, L, qpos, base = 128, 3, 40, 50000, 1e6
    offsets = [2 ** i for i in range(13)]
    keys = rng.standard_normal((L, d)) + rng.standard_normal(d)
    key_pos = np.sort(rng.choice(qpos + 1, size=L, replace=False))
    center = rng.standard_normal((G, d // 2, 2))
    mean_abs = np.hypot(center[..., 0], center[..., 1]) * rng.uniform(1.0, 3.0, (G, d // 2))
    rotated = np.stack([rope_rotate(keys[i], int(key_pos[i]), base, layout) for i in range(L)])
    pre = oracle.score_keys(keys, center, mean_abs, base=base, offsets=offsets, key_pos=key_pos,
                            query_pos=qpos, layout=layout, reduce=reduce)
    post = oracle.score_keys(rotated, center, mean_abs, base=base, offsets=offsets, key_pos=key_pos,
                             query_pos=qpos, layout=layout, reduce=reduce, key_space="post")
    S = oracle.score_magnitude_bound(keys, center, mean_abs, layout=layout, reduce=reduce)
    assert np.all(np.abs(post - pre) <= 1e-9 * S)


@pytest.mark.parametrize("layout", ["half", "interleaved"])
def test_p9_post_rope_exact_centre_identity(layout):
    # with E[q] = q the score of a rotated key is the mean over the offsets of the dot
    # product of the rotated query with the key exactly as cached
    rng = np.random.default_rng(23)
    d, L, qpos, base = 128, 16, 9000, 1e4
    offsets = [1, 2, 4, 8, 16, 32]
    q = rng.standard_normal(d)
    cached = rng.standard_normal((L, d))
    key_pos = np.sort(rng.choice(qpos + 1, size=L, replace=False))
    center = bands_of(q, layout)[None]
    mag = np.hypot(center[..., 0], center[..., 1])
    got = oracle.score_keys(cached, center, mag, base=base, offsets=offsets, key_pos=key_pos,
                            query_pos=qpos, layout=layout, key_space="post")
    want = np.array([np.mean([rope_rotate(q, qpos + o, base, layout) @ cached[j] for o in offsets])
                     for j in range(L)])
    S = oracle.score_magnitude_bound(cached, center, mag, layout=layout)
    assert np.all(np.abs(got - want) <= 1e-9 * S)


# ---------------------------------------------------------------------------------------
# P10 fp8 (OCP E4M3) key codes
# ---------------------------------------------------------------------------------------

def test_p10_fp8_e4m3_values_fixed_by_the_format():
    v = oracle.decode_fp8_e4m3
    # zero, smallest subnormal 2^-9, largest subnormal 7 * 2^-9, smallest normal 2^-6, one,
    # the largest finite value 448, its negation, and the NaN codes
    assert v([0x00])[0] == 0.0 and math.copysign(1.0, v([0x80])[0]) == -1.0
    assert v([0x01])[0] == 2.0 ** -9
    assert v([0x07])[0] == 7 * 2.0 ** -9
    assert v([0x08])[0] == 2.0 ** -6
    assert v([0x38])[0] == 1.0 and v([0xB8])[0] == -1.0
    assert v([0x7E])[0] == 448.0 and v([0xFE])[0] == -448.0
    assert np.isnan(v([0x7F, 0xFF])).all()
    assert v([0x3C])[0] == 1.5 and v([0x40])[0] == 2.0 and v([0x46])[0] == 3.5 and v([0x4B])[0] == 5.5
    # every other code is finite, and the positive codes increase with the code
    c = np.arange(256)
    fin = (c & 0x7F) != 0x7F
    assert np.isfinite(v(c[fin])).all()
    pos = v(np.arange(0x00, 0x7F))
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(v(np.arange(0x80, 0xFF)), -pos)


# ---------------------------------------------------------------------------------------
# P11 multiplicative form: phase-only series times ||E q|| ||k||
# ---------------------------------------------------------------------------------------

def _bands_to_vector(bands, layout):
    """Real head vector [.., d] from complex bands [.., F] (written out per layout)."""
    F = bands.shape[-1]
    x = np.empty(bands.shape[:-1] + (2 * F,))
    if layout == "half":
        x[..., :F], x[..., F:] = bands.real, bands.imag
    else:
        x[..., 0::2], x[..., 1::2] = bands.real, bands.imag
    return x


def test_p11_hand_value_two_bands():
    # d = 4: bands f = 0, 1 with theta = 1 and base^-1/2; one offset; Q - p = 3 for key 0
    base, qpos, delta = 100.0, 3, 2
    c = np.array([[3.0 + 4.0j, 0.0 - 2.0j]])                 # |c| = 5, 2 -> ||c|| = sqrt(29)
    kb = np.array([[1.0 + 1.0j, -2.0 + 0.0j]])                # |k| = sqrt2, 2 -> ||k|| = sqrt6
    keys = _bands_to_vector(kb, "half")
    got = oracle.score_keys(keys, c, np.abs(c), base=base, offsets=[delta], query_pos=qpos,
                            form="multiplicative")[0]
    dist = qpos - 0 + delta
    th = [1.0, base ** -0.5]
    want = (math.cos(dist * th[0] + math.atan2(4, 3) - math.atan2(1, 1))
            + math.cos(dist * th[1] + math.atan2(-2, 0) - math.atan2(0, -2))) * math.sqrt(29) * math.sqrt(6)
    assert abs(got - want) <= 1e-12 * abs(want)


@pytest.mark.parametrize("layout", ["half", "interleaved"])
def test_p11_aligned_phases_closed_form(layout):
    # key bands rotated so every band's phase difference is 0 at the one offset: the series
    # counts the live bands, so the score is n_live * ||c|| * ||k||
    rng = np.random.default_rng(41)
    d, base, qpos, delta, L = 128, 1e4, 900, 8, 6
    F = d // 2
    c = rng.standard_normal(F) + 1j * rng.standard_normal(F)
    pos = np.array([0, 1, 5, 100, 640, 900])
    theta = np.array([base ** (-(2.0 * f) / d) for f in range(F)])
    r = rng.uniform(0.2, 3.0, (L, F))
    r[2, 10:20] = 0.0                                        # dead key bands: no phase
    kb = r * np.exp(1j * (np.angle(c)[None, :] + (qpos - pos[:, None] + delta) * theta[None, :]))
    keys = _bands_to_vector(kb, layout)
    got = oracle.score_keys(keys, c, np.abs(c), base=base, offsets=[delta], key_pos=pos, query_pos=qpos,
                            layout=layout, form="multiplicative")
    n_live = (r > 0).sum(axis=1)
    want = n_live * np.sqrt(np.sum(np.abs(c) ** 2)) * np.sqrt(np.sum(r ** 2, axis=1))
    assert np.allclose(got, want, rtol=1e-9, atol=0)


@pytest.mark.parametrize("layout", ["half", "interleaved"])
def test_p11_single_band_centre_matches_amplitude_series(layout):
    # with one live centre band f0 the phase-only series times |c| |k_f0| is the amplitude
    # series of the additive form (pinned by P1); R = 1 leaves that form no norm term
    rng = np.random.default_rng(42)
    d, base, qpos, L = 128, 1e6, 3000, 30
    offsets = [2 ** i for i in range(9)]
    F, f0 = d // 2, 23
    c = np.zeros(F, complex)
    c[f0] = 1.7 - 0.4j
    keys = rng.standard_normal((L, d))
    kb = (keys[:, :F] + 1j * keys[:, F:]) if layout == "half" else (keys[:, 0::2] + 1j * keys[:, 1::2])
    mult = oracle.score_keys(keys, c, np.abs(c), base=base, offsets=offsets, query_pos=qpos, layout=layout,
                             form="multiplicative")
    add = oracle.score_keys(keys, c, np.abs(c), base=base, offsets=offsets, query_pos=qpos, layout=layout)
    k_norm = np.sqrt(np.sum(keys ** 2, axis=1))
    assert np.allclose(mult * np.abs(kb[:, f0]), add * k_norm, rtol=1e-9, atol=1e-12)


def test_p11_band_magnitudes_enter_only_through_the_key_norm():
    rng = np.random.default_rng(43)
    d, L = 128, 12
    c = rng.standard_normal((2, d // 2, 2))
    keys = rng.standard_normal((L, d))
    kw = dict(base=1e4, offsets=[1, 2, 4, 8], reduce="mean", form="multiplicative")
    s0 = oracle.score_keys(keys, c, np.ones((2, d // 2)), **kw)
    scaled = keys.copy()
    scaled[:, [3, 3 + 64, 40, 40 + 64]] *= 5.0                  # two bands, phases unchanged
    s1 = oracle.score_keys(scaled, c, np.ones((2, d // 2)), **kw)
    ratio = np.sqrt(np.sum(scaled ** 2, axis=1)) / np.sqrt(np.sum(keys ** 2, axis=1))
    assert np.allclose(s1, s0 * ratio, rtol=1e-10, atol=1e-12)
    S = oracle.score_magnitude_bound(keys, c, np.ones((2, d // 2)), reduce="mean", form="multiplicative")
    assert np.all(np.abs(s0) <= S)


# ---------------------------------------------------------------------------------------
# P12 attention over the compressed cache (RoPE at the kept positions, then softmax)
# ---------------------------------------------------------------------------------------

def test_p12_one_key_returns_its_value():
    rng = np.random.default_rng(51)
    q, k, v = rng.standard_normal((3, 128)), rng.standard_normal((1, 128)), rng.standard_normal((1, 128))
    out = oracle.decode_attention(q, k, v, base=1e6, key_pos=[777], query_pos=5000)
    assert np.allclose(out, np.repeat(v, 3, axis=0), rtol=0, atol=1e-14)


def test_p12_equal_logits_average_the_values():
    rng = np.random.default_rng(52)
    k = np.repeat(rng.standard_normal((1, 128)), 5, axis=0)
    v = rng.standard_normal((5, 128))
    out = oracle.decode_attention(rng.standard_normal((2, 128)), k, v, base=1e4, key_pos=[40] * 5, query_pos=90)
    assert np.allclose(out, np.repeat(v.mean(axis=0, keepdims=True), 2, axis=0), atol=1e-13)
    assert np.array_equal(oracle.decode_attention(np.ones((2, 128)), k[:0], v[:0], base=1e4, key_pos=[],
                                                  query_pos=3), np.zeros((2, 128)))


@pytest.mark.parametrize("layout", ["half", "interleaved"])
def test_p12_hand_weighting_three_to_one(layout):
    # at zero distance RoPE cancels: logits are q.k / sqrt(d); two keys along q whose logits
    # differ by ln 3 get weights 3/4 and 1/4
    d = 128
    q = np.zeros((1, d))
    q[0, 5] = 2.0
    a = 1.0
    b = a - math.log(3.0) * math.sqrt(d) / 2.0
    k = np.zeros((2, d))
    k[0, 5], k[1, 5] = a, b
    v = np.stack([np.full(d, 4.0), np.full(d, -8.0)])
    out = oracle.decode_attention(q, k, v, base=1e6, key_pos=[321, 321], query_pos=321, layout=layout)
    assert np.allclose(out, 0.75 * 4.0 + 0.25 * -8.0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("layout", ["half", "interleaved"])
def test_p12_relative_positions_and_post_rope_keys(layout):
    # logits depend on the query-key distance only (textbook RoPE), and keys cached after
    # RoPE at their positions give the same attention
    rng = np.random.default_rng(53)
    d, L, base = 128, 40, 1e4
    q = rng.standard_normal((2, d))
    k = rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    pos = np.sort(rng.choice(6000, L, replace=False))
    Q = 7000
    out = oracle.decode_attention(q, k, v, base=base, key_pos=pos, query_pos=Q, layout=layout)
    shifted = oracle.decode_attention(q, k, v, base=base, key_pos=pos + 12345, query_pos=Q + 12345, layout=layout)
    assert np.allclose(out, shifted, atol=1e-9)
    # the same logits from explicit 2x2 rotations of the distance only (query at Q - p, key at 0)
    logits = np.stack([[rope_rotate(q[h], Q - int(p), base, layout) @ k[j] for j, p in enumerate(pos)]
                       for h in range(2)]) / np.sqrt(d)
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    want = (w / w.sum(axis=1, keepdims=True)) @ v
    assert np.allclose(out, want, atol=1e-9)
    k_post = np.stack([rope_rotate(k[j], int(pos[j]), base, layout) for j in range(L)])
    post = oracle.decode_attention(q, k_post, v, base=base, key_pos=pos, query_pos=Q, layout=layout,
                                   key_space="post")
    assert np.allclose(out, post, atol=1e-9)


# ---------------------------------------------------------------------------------------
# P13 GQA mapping, the magnitude bound and the 0/0 band
# ---------------------------------------------------------------------------------------

def _stats_table(n_layer=2, n_qh=6, F=2):
    """Statistics where query head q of layer l has centre (10 l + q + 1) on band 0 only
    (0 elsewhere) and mean magnitude 2 (10 l + q + 1) on every band: every head is
    told apart by its values."""
    center = np.zeros((n_layer, n_qh, F, 2))
    mean_abs = np.zeros((n_layer, n_qh, F))
    for l in range(n_layer):
        for q in range(n_qh):
            center[l, q, 0, 0] = 10 * l + q + 1
            mean_abs[l, q, :] = 2 * (10 * l + q + 1)
    return center, mean_abs


def test_p13_kv_head_reads_its_contiguous_query_heads():
    # 6 query heads, G = 2: KV head h is read by query heads 2h and 2h + 1
    center, mean_abs = _stats_table()
    c, m = oracle.unit_heads(center, mean_abs, 1, 1, 2)
    # layer 1, query heads 2 and 3: centres 13 and 14, magnitudes 26 and 28
    np.testing.assert_array_equal(c, np.array([[13.0 + 0j, 0.0], [14.0 + 0j, 0.0]]))
    np.testing.assert_array_equal(m, np.array([[26.0, 26.0], [28.0, 28.0]]))
    c, m = oracle.unit_heads(center, mean_abs, 0, 1, 3)      # G = 3: heads 3, 4, 5 of layer 0
    np.testing.assert_array_equal(c[:, 0].real, [4.0, 5.0, 6.0])
    with pytest.raises(ValueError):                          # there is no KV head 2 at G = 3
        oracle.unit_heads(center, mean_abs, 0, 2, 3)
    c, m = oracle.unit_heads(center, mean_abs, 0, 0, 6)      # one KV head: all six
    np.testing.assert_array_equal(c[:, 0].real, [1.0, 2.0, 3.0, 4.0, 5.0, 6.0])


def test_p13_score_of_kv_head_one_hand_value():
    # Only query heads 2 and 3 of layer 1 have a centre; every other head is all zeros (and
    # E|q| = 0 there, so it adds nothing).  d = 4 (two bands, theta_0 = 1), key band 0 = 1,
    # band 1 = 0, query at the key's position, one offset Delta = 1:
    #   head 2: E q_0 = 3       -> 3 cos(1)
    #   head 3: E q_0 = 5i      -> 5 cos(1 + pi/2) = -5 sin(1)
    # both with E|q_0| = |E q_0| (R = 1, no norm term).
    n_layer, n_qh, F, G = 2, 6, 2, 2
    center = np.zeros((n_layer, n_qh, F, 2))
    mean_abs = np.zeros((n_layer, n_qh, F))
    center[1, 2, 0] = [3.0, 0.0]
    center[1, 3, 0] = [0.0, 5.0]
    mean_abs[1, 2, 0], mean_abs[1, 3, 0] = 3.0, 5.0
    key = np.array([[1.0, 0.0, 0.0, 0.0]])
    kw = dict(base=100.0, offsets=[1], key_pos=[0], query_pos=0)
    got = {}
    for h in range(n_qh // G):
        c, m = oracle.unit_heads(center, mean_abs, 1, h, G)
        got[h] = (oracle.score_keys(key, c, m, reduce="max", **kw)[0],
                  oracle.score_keys(key, c, m, reduce="mean", **kw)[0])
    assert abs(got[1][0] - 3.0 * math.cos(1.0)) < 1e-14
    assert abs(got[1][1] - (3.0 * math.cos(1.0) - 5.0 * math.sin(1.0)) / 2.0) < 1e-14
    assert got[0] == (0.0, 0.0) and got[2] == (0.0, 0.0)


@pytest.mark.parametrize("layout", ["half", "interleaved"])
@pytest.mark.parametrize("reduce", ["max", "mean"])
def test_p13_bound_is_reached_by_aligned_phases(layout, reduce):
    # R = 1 on every band (E|q_f| = |E q_f|: no norm term).  Choose each key band's phase so
    # that d theta_f + arg E q_f - arg k_f = 0 at the one offset: every cosine is 1 and
    # s_j = sum_f |E q_f| |k_f|, which is exactly S_j (the same for identical heads).
    rng = np.random.default_rng(21)
    d, F, L = 16, 8, 5
    base, Q, delta = 300.0, 40, 3
    cq = rng.standard_normal(F) + 1j * rng.standard_normal(F)
    theta = np.array([base ** (-2.0 * f / d) for f in range(F)])
    pos = np.array([0, 7, 19, 33, 40])
    mags = rng.uniform(0.5, 2.0, (L, F))
    kb = mags * np.exp(1j * ((Q - pos[:, None] + delta) * theta[None, :] + np.angle(cq)[None, :]))
    keys = np.empty((L, d))
    if layout == "half":
        keys[:, :F], keys[:, F:] = kb.real, kb.imag
    else:
        keys[:, 0::2], keys[:, 1::2] = kb.real, kb.imag
    center = np.stack([cq.real, cq.imag], -1)[None].repeat(2, axis=0)      # two identical heads
    mean_abs = np.abs(cq)[None].repeat(2, axis=0)
    s = oracle.score_keys(keys, center, mean_abs, base=base, offsets=[delta], key_pos=pos, query_pos=Q,
                          layout=layout, reduce=reduce)
    S = oracle.score_magnitude_bound(keys, center, mean_abs, layout=layout, reduce=reduce)
    want = (mags * np.abs(cq)[None, :]).sum(axis=1)
    np.testing.assert_allclose(S, want, rtol=1e-13, atol=0)
    np.testing.assert_allclose(s, S, rtol=1e-12, atol=0)


def test_p13_bound_hand_values_two_heads():
    # d = 4: bands k_0 = 3, k_1 = 4i (|k| = 3, 4).  Coefficient of band f in S:
    # |E q_f| + |(1 - R_f) E|q_f||.
    #   head 0: E q = (1, 0),  E|q| = (2, 1)    R = (0.5, 0)  coef = (1 + 1,   0 + 1)   = (2, 1)
    #   head 1: E q = (2i, 1), E|q| = (2, 0.5)  R = (1, 2)    coef = (2 + 0,   1 + 0.5) = (2, 1.5)
    # S_head0 = 2*3 + 1*4 = 10, S_head1 = 2*3 + 1.5*4 = 12: max 12, mean 11.
    keys = np.array([[3.0, 0.0, 0.0, 4.0]])
    center = np.array([[[1.0, 0.0], [0.0, 0.0]], [[0.0, 2.0], [1.0, 0.0]]])
    mean_abs = np.array([[2.0, 1.0], [2.0, 0.5]])
    assert oracle.score_magnitude_bound(keys, center, mean_abs, reduce="max")[0] == pytest.approx(12.0, abs=1e-14)
    assert oracle.score_magnitude_bound(keys, center, mean_abs, reduce="mean")[0] == pytest.approx(11.0, abs=1e-14)
    # and the scores lie inside it (any offsets)
    for reduce, S in (("max", 12.0), ("mean", 11.0)):
        s = oracle.score_keys(keys, center, mean_abs, base=10.0, offsets=[1, 2, 5], reduce=reduce)
        assert abs(s[0]) <= S


def test_p13_band_without_query_energy_adds_nothing():
    # concentration of a band with E|q_f| = 0 (and so E q_f = 0) is read as 0, and the band
    # adds nothing to the score or to the bound.  d = 4: band 0 has E q = 0.6, E|q| = 2
    # (R = 0.3); band 1 has neither.  k = (2i, 7 + 7i), query at the key, Delta = 5,
    # theta_0 = 1: s = 0.6 * 2 cos(5 - pi/2) + (1 - 0.3) * 2 * 2 = 1.2 sin 5 + 2.8, and
    # S = 2 (0.6 + 1.4) = 4.
    np.testing.assert_array_equal(oracle.concentration(np.array([0.6 + 0j, 0j]), np.array([2.0, 0.0])),
                                  [0.3, 0.0])
    assert oracle.concentration(np.array([0j]), np.array([0.0]))[0] == 0.0
    keys = np.array([[0.0, 7.0, 2.0, 7.0]])
    center = np.array([[[0.6, 0.0], [0.0, 0.0]]])
    mean_abs = np.array([[2.0, 0.0]])
    s = oracle.score_keys(keys, center, mean_abs, base=10.0, offsets=[5], key_pos=[0], query_pos=0)
    assert abs(s[0] - (1.2 * math.sin(5.0) + 2.8)) < 1e-14
    S = oracle.score_magnitude_bound(keys, center, mean_abs)
    assert abs(S[0] - 4.0) < 1e-14


# ---------------------------------------------------------------------------------------
# P10 (continued): bfloat16 patterns and the stored-key decoding
# ---------------------------------------------------------------------------------------

def test_p10_bf16_values_fixed_by_the_format():
    dec = lambda b: float(oracle.decode_bf16(np.array([b], dtype=np.uint16))[0])
    assert dec(0x3F80) == 1.0 and dec(0xBF80) == -1.0 and dec(0x4000) == 2.0
    assert dec(0x3FC0) == 1.5 and dec(0x4049) == 3.140625 and dec(0x0000) == 0.0
    assert dec(0x8000) == 0.0 and math.copysign(1.0, dec(0x8000)) == -1.0
    assert dec(0x0001) == 2.0 ** -133                       # smallest subnormal
    assert dec(0x007F) == 127 * 2.0 ** -133                 # largest subnormal
    assert dec(0x0080) == 2.0 ** -126                       # smallest normal
    assert dec(0x7F7F) == (2.0 - 2.0 ** -7) * 2.0 ** 127    # largest finite
    assert dec(0x7F80) == math.inf and dec(0xFF80) == -math.inf
    assert math.isnan(dec(0x7FC0)) and math.isnan(dec(0xFF81))


def test_p10_bf16_all_patterns_match_torch():
    torch = pytest.importorskip("torch")
    bits = np.arange(1 << 16, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.decode_bf16(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_p10_stored_keys_decode_with_their_scale():
    codes = np.array([0x38, 0xB8, 0x01, 0x7E], dtype=np.uint8)          # 1, -1, 2^-9, 448
    np.testing.assert_array_equal(oracle.decode_stored(codes, "fp8", 0.5), [0.5, -0.5, 2.0 ** -10, 224.0])
    i8 = np.array([-128, -127, -1, 0, 1, 127], dtype=np.int8)
    np.testing.assert_array_equal(oracle.decode_stored(i8, "int8", 0.125),
                                  [-16.0, -15.875, -0.125, 0.0, 0.125, 15.875])
    bf = np.array([0x3F80, 0xC040], dtype=np.uint16)                     # 1, -3
    np.testing.assert_array_equal(oracle.decode_stored(bf.view(np.int16), "bf16"), [1.0, -3.0])
    f = np.array([0.1, -2.5], dtype=np.float32)
    np.testing.assert_array_equal(oracle.decode_stored(f, "f32"), f.astype(np.float64))
