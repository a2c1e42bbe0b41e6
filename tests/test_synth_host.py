"""Host side of the seeded input generator and the workload parameters (no GPU)."""

import numpy as np
import pytest
import torch

import oracle
from kv_cache_compression_tri_amd import synth
from kv_cache_compression_tri_amd.synth import workloads as W


def test_mix64_known_values():
    # SplitMix64 seeded with 0: first outputs are mix64(k * gamma), published reference values
    g = np.uint64(synth.GAMMA)
    with np.errstate(over="ignore"):
        outs = synth.mix64(np.array([g, g * np.uint64(2), g * np.uint64(3)], dtype=np.uint64))
    assert [int(x) for x in outs] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_normals_moments_and_range():
    n = synth.normals(7, 0, 3, np.arange(4000), 128).ravel()
    assert abs(n.mean()) < 0.01
    assert abs(n.var() - 1.0) < 0.02
    assert n.min() >= -6.0 and n.max() <= 6.0
    assert n.dtype == np.float32
    # exact multiples of 2^-16
    assert np.all((n * 65536.0) == np.round(n * 65536.0))


def test_normals_deterministic_and_stream_separated():
    a = synth.normals(1, 0, 5, np.arange(64))
    b = synth.normals(1, 0, 5, np.arange(64))
    assert np.array_equal(a, b)
    c = synth.normals(1, 1, 5, np.arange(64))
    d = synth.normals(2, 0, 5, np.arange(64))
    e = synth.normals(1, 0, 6, np.arange(64))
    for other in (c, d, e):
        assert abs(np.corrcoef(a.ravel(), other.ravel())[0, 1]) < 0.05
    # a row range starting mid-unit equals the same rows of the full range
    full = synth.normals(1, 0, 5, np.arange(100))
    assert np.array_equal(full[40:60], synth.normals(1, 0, 5, np.arange(40, 60)))


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000).astype(np.float32) * 10
    # add exact ties: values halfway between two bf16 numbers
    ties = (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(oracle.decode_bf16(ours), torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).double().numpy())


def test_rows_sink_and_center():
    mu = np.linspace(-1, 1, 128).astype(np.float32)
    sig = np.full(128, 0.3, np.float32)
    r = synth.rows(3, 0, 2, 8, mu, sig, sink=True, dtype="f32")
    n = synth.normals(3, 0, 2, np.arange(8))
    np.testing.assert_array_equal(r[1:], mu + sig * n[1:])
    np.testing.assert_array_equal(r[0], np.float32(20) * (mu + sig * n[0]))
    rb = synth.rows(3, 0, 2, 8, mu, sig, sink=True, dtype="bf16")
    assert np.array_equal(rb, synth.f32_to_bf16_bits(r))


@pytest.mark.parametrize("name", sorted(W.WORKLOADS))
def test_workload_params(name):
    w = W.WORKLOADS[name]
    hp = W.make_params(w)
    F = w.head_dim // 2
    assert hp.center.shape == (w.n_layer, w.n_qh, F, 2) and hp.center.dtype == np.float32
    assert hp.mean_abs.shape == (w.n_layer, w.n_qh, F)
    assert hp.mu_k.shape == (w.n_layer, w.n_kvh, w.head_dim)
    assert int(hp.low_r.sum()) == int(round(w.low_r_frac * w.n_layer * w.n_kvh))
    mag = np.hypot(hp.center[..., 0].astype(np.float64), hp.center[..., 1].astype(np.float64))
    R = mag / hp.mean_abs
    low = np.repeat(hp.low_r, w.group, axis=1)
    if low.any():
        assert np.allclose(R[low], 0.3, rtol=1e-6)
    assert np.allclose(R[~low], 1 / 1.1, rtol=1e-6)
    if w.paged:
        lo, hi = w.len_range
        assert hp.lengths.min() >= lo and hp.lengths.max() <= hi
        pages = -(-hp.lengths.astype(np.int64) // w.page)
        assert hp.n_pages == pages.sum()
        used = np.concatenate([hp.block_table[s, : pages[s]] for s in range(w.n_seq)])
        assert np.array_equal(np.sort(used), np.arange(hp.n_pages))
    else:
        assert np.all(hp.lengths == w.max_len)
    # deterministic
    hp2 = W.make_params(w)
    assert np.array_equal(hp.center, hp2.center) and np.array_equal(hp.mu_k, hp2.mu_k)


def test_heteroscedastic_sigma_by_band():
    w = W.WORKLOADS["long_128k_bf16"]
    s = W.make_params(w).sigma
    assert np.all(s[:32] == np.float32(0.1)) and np.all(s[64:96] == np.float32(0.1))
    assert np.all(s[32:64] == np.float32(1.0)) and np.all(s[96:] == np.float32(1.0))


# ---------------------------------------------------------------------------------------
# fp8 (OCP E4M3) encoding of the generator
# ---------------------------------------------------------------------------------------

def _fp8_nearest_even(x):
    """Brute force: the finite E4M3 value nearest to x (ties to the even code), or the
    saturated code when |x| rounds past 448."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = oracle.decode_fp8_e4m3(codes)
    out = []
    for v in np.asarray(x, dtype=np.float64):
        if abs(v) >= 464.0:                     # past the midpoint of 448 and 480
            out.append(0x7E | (0x80 if v < 0 else 0))
            continue
        d = np.abs(vals - v)
        best = np.nonzero(d == d.min())[0]
        cand = codes[best]
        if len(cand) > 1:
            # +0 and -0 tie for zero: the sign of x decides; otherwise the even mantissa wins
            same_sign = [c for c in cand if ((c & 0x80) != 0) == (np.signbit(v))]
            cand = same_sign or list(cand)
            even = [c for c in cand if (c & 1) == 0]
            cand = even or cand
        out.append(int(cand[0]))
    return np.array(out, dtype=np.uint8)


def test_fp8_encoder_is_round_to_nearest_even():
    rng = np.random.default_rng(31)
    x = np.concatenate([
        rng.standard_normal(3000) * 10.0,
        rng.standard_normal(1000) * 2.0 ** -7,                 # subnormal range
        np.exp(rng.uniform(-12, 6.5, 2000)) * rng.choice([-1, 1], 2000),
    ]).astype(np.float32)
    assert np.array_equal(synth.f32_to_fp8_e4m3(x), _fp8_nearest_even(x))


def test_fp8_encoder_ties_saturation_and_specials():
    enc = lambda v: int(synth.f32_to_fp8_e4m3(np.float32([v]))[0])
    assert enc(1.0625) == 0x38 and enc(1.1875) == 0x3A          # ties go to the even mantissa
    assert enc(2.0 ** -10) == 0x00 and enc(3 * 2.0 ** -10) == 0x02   # subnormal ties
    assert enc(7.5 * 2.0 ** -9) == 0x08                          # rounds up into the normals
    assert enc(448.0) == 0x7E and enc(463.9) == 0x7E and enc(464.0) == 0x7E and enc(1e9) == 0x7E
    assert enc(float("inf")) == 0x7E and enc(-float("inf")) == 0xFE
    assert enc(float("nan")) & 0x7F == 0x7F
    assert enc(-0.0) == 0x80 and enc(0.0) == 0x00


def test_fp8_rows_are_codes_of_scaled_values():
    w = W.scaled(W.WORKLOADS["gqa8b_32k_bf16"], dtype="fp8", n_layer=2, n_kvh=2, max_len=64)
    hp = W.make_params(w)
    assert set(np.unique(hp.k_scale)) == {0.5, 1.0}
    for l in range(2):
        for h in range(2):
            unit = W.unit_index(w, 0, l, h)
            sc = float(hp.k_scale[l, h])
            codes = synth.rows(w.seed, synth.TAG_K, unit, 64, hp.mu_k[l, h], hp.sigma, True, "fp8", scale=sc)
            x = synth.rows(w.seed, synth.TAG_K, unit, 64, hp.mu_k[l, h], hp.sigma, True, "f32")
            assert codes.dtype == np.uint8
            assert np.array_equal(codes, synth.f32_to_fp8_e4m3(x / np.float32(sc)))
            # the decoded cache is within half a code step (plus saturation) of the true keys
            vals = oracle.decode_stored(codes, "fp8", sc)
            ok = np.abs(x) < 448 * sc
            assert np.all(np.abs(vals - x)[ok] <= np.abs(x)[ok] * 2.0 ** -4 + 2.0 ** -10 * sc)


# ---------------------------------------------------------------------------------------
# int8 encoding of the generator
# ---------------------------------------------------------------------------------------

def _int8_nearest_even(x):
    """Brute force: the nearest of the codes -127..127, ties to the even code."""
    codes = np.arange(-127, 128)
    out = []
    for v in np.asarray(x, dtype=np.float64):
        d = np.abs(codes - v)
        cand = codes[d == d.min()]
        even = [c for c in cand if c % 2 == 0]
        out.append(int(even[0] if even else cand[0]))
    return np.array(out, dtype=np.int8)


def test_int8_encoder_is_round_to_nearest_even_and_clamps():
    rng = np.random.default_rng(32)
    x = np.concatenate([rng.standard_normal(3000) * 40.0, rng.uniform(-3, 3, 1000),
                        np.arange(-130, 131) + 0.5, [127.4, 127.5, 200.0, -127.5, -1e9, 1e9]]).astype(np.float32)
    assert np.array_equal(synth.f32_to_int8(x), _int8_nearest_even(x))
    enc = lambda v: int(synth.f32_to_int8(np.float32([v]))[0])
    assert enc(0.5) == 0 and enc(1.5) == 2 and enc(2.5) == 2 and enc(-0.5) == 0 and enc(-1.5) == -2
    assert enc(126.5) == 126 and enc(127.5) == 127 and enc(300.0) == 127 and enc(-300.0) == -127


def test_int8_rows_are_codes_of_scaled_values():
    w = W.scaled(W.WORKLOADS["gqa8b_32k_bf16"], dtype="int8", n_layer=2, n_kvh=2, max_len=64)
    hp = W.make_params(w)
    assert set(np.unique(hp.k_scale)) == {1.0 / 16, 1.0 / 8}
    for l in range(2):
        for h in range(2):
            unit = W.unit_index(w, 0, l, h)
            sc = float(hp.k_scale[l, h])
            codes = synth.rows(w.seed, synth.TAG_K, unit, 64, hp.mu_k[l, h], hp.sigma, True, "int8", scale=sc)
            x = synth.rows(w.seed, synth.TAG_K, unit, 64, hp.mu_k[l, h], hp.sigma, True, "f32")
            assert codes.dtype == np.int8
            assert np.array_equal(codes, synth.f32_to_int8(x / np.float32(sc)))
            assert np.abs(codes[1:]).max() < 127          # only the sink row may clamp
            vals = oracle.decode_stored(codes, "int8", sc)
            assert np.all(np.abs(vals - x)[1:] <= 0.5 * sc)
