"""GPU parity of the HIP path (through the C ABI) against the float64 oracle.

Small cases compare every unit (several 128-key chunks, ragged tails, lengths below the
budget); the full-size workloads run exactly as the benchmark launches them and compare
sampled units (first, last, low-concentration, random, shortest/longest paged sequence).
Oracle inputs are regenerated on the host from the seed.  Tolerances: see parity.py.
"""

import numpy as np
import pytest
import torch

import oracle
import kv_cache_compression_tri_amd as tri
from kv_cache_compression_tri_amd import synth
from kv_cache_compression_tri_amd.synth import device as SD
from kv_cache_compression_tri_amd.synth import workloads as W

import parity as P

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def bits(t):
    """Raw element bits of a device tensor as a host numpy array."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).cpu().numpy()
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    return t.cpu().numpy()


def run_pass(dw, key_space="pre", form="additive"):
    w = dw.w
    kv = dw.kv()
    mean_abs = None if form == "multiplicative" else dw.mean_abs    # not read by that form
    scores = tri.tri_score_keys(kv, dw.center, mean_abs, rope_base=w.base, offsets=w.offsets,
                                group=w.group, reduce=w.reduce, rope_layout=w.layout, key_space=key_space,
                                form=form)
    kept, kept_n = tri.tri_select_topb(scores, kv, w.budget, w.window)
    out = tri.tri_compact_kv(kv, kept, kept_n, w.budget)
    torch.cuda.synchronize()
    return scores, kept, kept_n, out


def check_dense_unit(dw, s, l, h, sc_h, kept_h, kept_n_h, out_h, key_space="pre", form="additive"):
    """sc_h etc. are host copies; checks one unit of a dense workload."""
    w, hp = dw.w, dw.hp
    L = int(hp.lengths[s])
    keys = P.host_rows(w, hp, s, l, h)
    orc, S = P.oracle_scores(w, hp, s, l, h, keys, key_space, form)
    worst, rel = P.check_scores(sc_h[s, l, h, :L], orc, S)
    P.check_kept(kept_h[s, l, h], sc_h[s, l, h], orc, S, L, w.budget, w.window)
    n = min(L, w.budget)
    assert kept_n_h[s] == n
    kk = kept_h[s, l, h, :n]
    kbits = P.host_bits(w, hp, s, l, h)
    assert np.array_equal(out_h["k_out"][s, l, h, :n], kbits[kk]), "compacted K rows differ"
    if w.with_values:
        vbits = P.host_bits(w, hp, s, l, h, tag=synth.TAG_V)
        assert np.array_equal(out_h["v_out"][s, l, h, :n], vbits[kk]), "compacted V rows differ"
    assert np.array_equal(out_h["pos_out"][s, l, h, :n], kk)
    assert out_h["new_len"][s] == n
    return worst, rel


def host_outputs(scores, kept, kept_n, out):
    o = {k: (bits(v) if v is not None else None) for k, v in out.items()}
    return scores.cpu().numpy(), kept.cpu().numpy(), kept_n.cpu().numpy(), o


# ---------------------------------------------------------------------------------------
# generator: device == host, bit for bit
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32", "fp8", "int8"])
def test_device_generator_matches_host(dtype):
    w = W.scaled(W.WORKLOADS["gqa8b_32k_bf16"], n_seq=2, n_layer=2, n_kvh=2, max_len=300, dtype=dtype)
    log(f"generator dense {dtype}")
    dw = SD.build(w)
    kb, vb = bits(dw.k), bits(dw.v)
    for s in range(2):
        for l in range(2):
            for h in range(2):
                assert np.array_equal(kb[s, l, h], P.host_bits(w, dw.hp, s, l, h))
                assert np.array_equal(vb[s, l, h], P.host_bits(w, dw.hp, s, l, h, tag=synth.TAG_V))
    wp = W.scaled(W.WORKLOADS["paged_ragged64_bf16"], n_seq=3, n_layer=2, n_kvh=2, max_len=700,
                  len_range=(10, 700), dtype=dtype)
    log(f"generator paged {dtype}")
    dp = SD.build(wp)
    pk = bits(dp.k)
    bt = dp.hp.block_table
    for s in range(3):
        L = int(dp.hp.lengths[s])
        for l in range(2):
            for h in range(2):
                got = np.stack([pk[bt[s, j // 16], l, h, j % 16] for j in range(L)])
                assert np.array_equal(got, P.host_bits(wp, dp.hp, s, l, h))


# ---------------------------------------------------------------------------------------
# small dense cases: every unit, several chunks, ragged tails, L < B
# ---------------------------------------------------------------------------------------

BASE = W.WORKLOADS["gqa8b_32k_bf16"]
SMALL_DENSE = {
    "g4_max_half_bf16": (dict(n_seq=2, n_layer=2, n_kvh=2, group=4, max_len=3000, budget=700, window=64),
                         [3000, 1777]),
    "g3_mean_interleaved_bf16": (dict(n_seq=2, n_layer=1, n_kvh=3, group=3, reduce="mean", layout="interleaved",
                                      max_len=2100, budget=500, window=100), [2100, 333]),
    "g1_half_f32": (dict(n_seq=1, n_layer=2, n_kvh=2, group=1, dtype="f32", max_len=2500, budget=256,
                         window=64, base=1e4, offsets=W.geometric_offsets(10)), [2500]),
    "g8_max_bf16": (dict(n_seq=1, n_layer=1, n_kvh=2, group=8, max_len=1500, budget=300, window=0), [1500]),
    "g7_max_interleaved_f32": (dict(n_seq=2, n_layer=1, n_kvh=1, group=7, dtype="f32", layout="interleaved",
                                    max_len=1100, budget=1000, window=1200, sigma_low=0.1, sigma_high=1.0,
                                    offsets=W.geometric_offsets(14)), [1100, 1001]),
    "g2_mean_half_f32": (dict(n_seq=1, n_layer=1, n_kvh=2, group=2, dtype="f32", reduce="mean",
                              max_len=1025, budget=1024, window=8), [1025]),
    "g5_max_half_bf16_lowR": (dict(n_seq=1, n_layer=2, n_kvh=2, group=5, max_len=2049, budget=129,
                                   window=1, low_r_frac=0.5), [2049]),
    "g6_max_half_bf16_short": (dict(n_seq=3, n_layer=1, n_kvh=1, group=6, max_len=900, budget=64,
                                    window=16), [900, 1, 65]),
    # G = 4..8 with bf16 keys run on the matrix-core kernel: several 224-key chunks, tails that
    # are not a multiple of its 16-key step, interleaved layout
    "g7_max_interleaved_bf16": (dict(n_seq=2, n_layer=2, n_kvh=1, group=7, layout="interleaved", max_len=2300,
                                     budget=333, window=20), [2300, 1201]),
    # matrix-core scoring (G >= 4, bfloat16): lengths at its 224-key chunk, 16-key step and
    # 64-key store-group boundaries, on either side of them
    "g5_max_half_bf16_chunk_edges": (dict(n_seq=8, n_layer=1, n_kvh=2, group=5, max_len=1100, budget=100,
                                          window=8), [223, 224, 225, 447, 448, 449, 1100, 1087]),
    "g8_max_interleaved_bf16_step_edges": (dict(n_seq=8, n_layer=2, n_kvh=1, group=8, layout="interleaved",
                                                max_len=320, budget=40, window=4), [1, 15, 16, 17, 63, 64, 65, 320]),
    "g4_max_half_bf16_one_step": (dict(n_seq=3, n_layer=3, n_kvh=2, group=4, max_len=16, budget=9, window=2),
                                  [16, 2, 9]),
    # empty sequences between non-empty ones: the score grid divides only real keys
    "g4_max_half_bf16_empty_seqs": (dict(n_seq=5, n_layer=2, n_kvh=2, group=4, max_len=2600, budget=300,
                                         window=32), [0, 2600, 0, 0, 1031]),
    # fp8 (OCP E4M3) keys with per-(layer, KV head) scales 1 and 1/2
    "g4_max_half_fp8": (dict(n_seq=2, n_layer=2, n_kvh=2, group=4, dtype="fp8", max_len=2600, budget=500,
                             window=32), [2600, 1111]),
    "g8_max_interleaved_fp8": (dict(n_seq=1, n_layer=1, n_kvh=2, group=8, dtype="fp8", layout="interleaved",
                                    max_len=1300, budget=200, window=16), [1300]),
    "g2_mean_half_fp8_wide": (dict(n_seq=2, n_layer=1, n_kvh=3, group=2, dtype="fp8", reduce="mean",
                                   max_len=1100, budget=1024, window=8, sigma_low=0.01, sigma_high=2.0),
                              [1100, 57]),
    # int8 keys with per-(layer, KV head) scales 1/16 and 1/8
    "g4_max_half_int8": (dict(n_seq=2, n_layer=2, n_kvh=2, group=4, dtype="int8", max_len=2300, budget=400,
                              window=64), [2300, 700]),
    "g7_max_interleaved_int8": (dict(n_seq=1, n_layer=2, n_kvh=1, group=7, dtype="int8", layout="interleaved",
                                     max_len=1800, budget=256, window=0), [1800]),
}


@pytest.mark.parametrize("name", sorted(SMALL_DENSE))
def test_small_dense_parity(name):
    over, lengths = SMALL_DENSE[name]
    w = W.scaled(BASE, name=name, **over)
    log(f"small dense {name}: {over} lengths={lengths}")
    dw = SD.build(w, hp=W.make_params(w, lengths=lengths))
    sc, kept, kept_n, out = host_outputs(*run_pass(dw))
    worst = 0.0
    for s in range(w.n_seq):
        for l in range(w.n_layer):
            for h in range(w.n_kvh):
                e, _ = check_dense_unit(dw, s, l, h, sc, kept, kept_n, out)
                worst = max(worst, e)
    log(f"  max score error / bound = {worst:.3e}")


# bfloat16, fp8 and int8 caches read as keys cached after RoPE, max over G >= 4 heads: the
# matrix-core kernel with the raw keys (8-bit: their values packed as bfloat16) as the trig
# products' operand, at the step, store-group and chunk edges above and with per-head key scales
# (8-bit keys from G = 2); and bfloat16 at G = 2, 3 (the vector kernel)
POST_MX = ["g4_max_half_bf16", "g8_max_bf16", "g5_max_half_bf16_lowR", "g6_max_half_bf16_short",
           "g7_max_interleaved_bf16", "g5_max_half_bf16_chunk_edges", "g8_max_interleaved_bf16_step_edges",
           "g4_max_half_bf16_one_step", "g4_max_half_bf16_empty_seqs", "g4_max_half_fp8",
           "g8_max_interleaved_fp8", "g4_max_half_int8", "g7_max_interleaved_int8"]
POST_MX_EXTRA = {
    "g2_max_half_bf16": (dict(n_seq=2, n_layer=2, n_kvh=2, group=2, max_len=1700, budget=300, window=16),
                         [1700, 1041]),
    "g3_max_interleaved_bf16": (dict(n_seq=3, n_layer=1, n_kvh=2, group=3, layout="interleaved", max_len=700,
                                     budget=90, window=0), [700, 17, 241]),
    "g5_max_half_fp8_step_edges": (dict(n_seq=8, n_layer=2, n_kvh=1, group=5, dtype="fp8", max_len=320,
                                        budget=40, window=4), [1, 15, 16, 17, 63, 64, 65, 320]),
    "g6_max_interleaved_fp8_chunk_edges": (dict(n_seq=8, n_layer=1, n_kvh=2, group=6, dtype="fp8",
                                                layout="interleaved", max_len=1100, budget=100, window=8),
                                           [223, 224, 225, 447, 448, 449, 1100, 1087]),
    "g8_max_half_int8_step_edges": (dict(n_seq=8, n_layer=1, n_kvh=2, group=8, dtype="int8", max_len=320,
                                         budget=40, window=0), [1, 15, 16, 17, 63, 64, 65, 320]),
    "g2_max_half_fp8": (dict(n_seq=2, n_layer=2, n_kvh=2, group=2, dtype="fp8", max_len=1700, budget=300,
                             window=16), [1700, 1041]),
    "g3_max_interleaved_int8": (dict(n_seq=3, n_layer=1, n_kvh=2, group=3, dtype="int8", layout="interleaved",
                                     max_len=700, budget=90, window=0), [700, 17, 241]),
    "g5_max_interleaved_int8_empty_seqs": (dict(n_seq=5, n_layer=2, n_kvh=2, group=5, dtype="int8",
                                                layout="interleaved", max_len=2600, budget=300, window=32),
                                           [0, 2600, 0, 0, 1031]),
}


@pytest.mark.parametrize("name", POST_MX + sorted(POST_MX_EXTRA))
def test_small_dense_parity_post_rope(name):
    over, lengths = SMALL_DENSE[name] if name in SMALL_DENSE else POST_MX_EXTRA[name]
    w = W.scaled(BASE, name=name + "_post", **over)
    log(f"small dense post-RoPE {name}: {over} lengths={lengths}")
    dw = SD.build(w, hp=W.make_params(w, lengths=lengths))
    sc, kept, kept_n, out = host_outputs(*run_pass(dw, "post"))
    worst = 0.0
    for s in range(w.n_seq):
        for l in range(w.n_layer):
            for h in range(w.n_kvh):
                e, _ = check_dense_unit(dw, s, l, h, sc, kept, kept_n, out, "post")
                worst = max(worst, e)
    log(f"  max score error / bound = {worst:.3e}")


# ---------------------------------------------------------------------------------------
# small paged case: every unit, in-place packing, freed pages
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("lengths,key_space,extra", [
    ([5000, 70, 1300, 1024], "pre", {}),
    ([1025, 4096, 16, 2047], "pre", {}),
    ([3000, 17, 4096, 900], "post", {}),
    ([2222, 4000, 1, 513], "pre", dict(dtype="f32", layout="interleaved", group=2)),
    ([700, 4100, 1500, 33], "post", dict(layout="interleaved", group=3, reduce="mean")),
    ([3000, 17, 4096, 900], "pre", dict(dtype="fp8")),
    ([1200, 4111, 64, 2000], "post", dict(dtype="fp8", layout="interleaved", group=5)),
    ([2500, 33, 4096, 1000], "pre", dict(dtype="int8", layout="interleaved", reduce="mean")),
    ([3000, 17, 4096, 905], "pre", dict(group=7)),                       # matrix-core scoring, paged
    ([1200, 4111, 64, 2001], "pre", dict(layout="interleaved", group=8)),
    ([1200, 4111, 64, 2001], "post", dict(layout="interleaved", group=8)),   # matrix cores, keys after RoPE
    ([333, 4096, 17, 1600], "post", dict(group=2)),                         # vector kernel, keys after RoPE
    ([2500, 33, 4096, 1000], "post", dict(dtype="int8")),                   # matrix cores, 8-bit after RoPE
    ([1025, 4096, 16, 2047], "post", dict(dtype="fp8", group=7)),
    ([700, 4100, 1500, 33], "post", dict(dtype="int8", layout="interleaved", group=3)),
])
def test_small_paged_parity(lengths, key_space, extra):
    w = W.scaled(W.WORKLOADS["paged_ragged64_bf16"], n_seq=4, n_layer=2, n_kvh=2, max_len=5120,
                 len_range=(16, 5120), **extra)
    log(f"small paged lengths={lengths} keys {key_space}-RoPE {extra}")
    dw = SD.build(w, hp=W.make_params(w, lengths=lengths))
    k_before, v_before = bits(dw.k), bits(dw.v)
    sc, kept, kept_n, out = host_outputs(*run_pass(dw, key_space))
    k_after, v_after = bits(dw.k), bits(dw.v)
    bt = dw.hp.block_table
    exp_k, exp_v = k_before.copy(), v_before.copy()
    for s in range(w.n_seq):
        L = int(lengths[s])
        kept_units = {}
        for l in range(w.n_layer):
            for h in range(w.n_kvh):
                keys = P.host_rows(w, dw.hp, s, l, h)
                orc, S = P.oracle_scores(w, dw.hp, s, l, h, keys, key_space)
                P.check_scores(sc[s, l, h, :L], orc, S)
                P.check_kept(kept[s, l, h], sc[s, l, h], orc, S, L, w.budget, w.window)
                kept_units[(l, h)] = kept[s, l, h, : min(L, w.budget)]
                assert np.array_equal(out["pos_out"][s, l, h, : min(L, w.budget)], kept_units[(l, h)])
        # oracle forward packing of this sequence on the pre-compaction snapshot
        ek, ev, freed, new_len = oracle.compact_paged_sequence(exp_k, exp_v, bt[s], L, kept_units, 16)
        exp_k, exp_v = ek, ev
        assert kept_n[s] == new_len == out["new_len"][s]
        nf = int(out["n_freed"][s])
        assert nf == len(freed) and np.array_equal(out["freed"][s, :nf], freed)
    assert np.array_equal(k_after, exp_k), "paged K pool differs from the oracle's forward packing"
    assert np.array_equal(v_after, exp_v), "paged V pool differs from the oracle's forward packing"


def test_paged_in_place_every_row_moves():
    """Hand-made kept sets where every survivor moves (by one slot, and to the far end)."""
    w = W.scaled(W.WORKLOADS["paged_ragged64_bf16"], n_seq=2, n_layer=3, n_kvh=2, max_len=4096,
                 len_range=(16, 4096))
    lengths = [4096, 3001]
    B = 1000
    dw = SD.build(w, hp=W.make_params(w, lengths=lengths))
    kv = dw.kv()
    kept = np.zeros((2, 3, 2, B), np.int32)
    for s, L in enumerate(lengths):
        for l in range(3):
            for h in range(2):
                if (l + h) % 2 == 0:
                    kept[s, l, h] = np.arange(1, B + 1)            # every row moves by one slot
                else:
                    kept[s, l, h] = np.arange(L - B, L)            # every row moves far forward
    kept_n = np.full(2, B, np.int32)
    k_before, v_before = bits(dw.k), bits(dw.v)
    out = tri.tri_compact_kv(kv, torch.from_numpy(kept).cuda(), torch.from_numpy(kept_n).cuda(), B)
    torch.cuda.synchronize()
    ek, ev = k_before, v_before
    for s, L in enumerate(lengths):
        units = {(l, h): kept[s, l, h] for l in range(3) for h in range(2)}
        ek, ev, freed, new_len = oracle.compact_paged_sequence(ek, ev, dw.hp.block_table[s], L, units, 16)
        assert int(bits(out["n_freed"])[s]) == len(freed)
    assert np.array_equal(bits(dw.k), ek) and np.array_equal(bits(dw.v), ev)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8", "int8"])
@pytest.mark.parametrize("budget", [1, 7, 13, 33])
@pytest.mark.parametrize("with_pos", [False, True])
def test_dense_compaction_row_groups(dtype, budget, with_pos):
    """Dense compaction of hand-made kept sets: budgets that leave a partial last group for
    each of the kernel's 4-, 8- and 16-row sizes, sequences shorter than the budget and an empty one;
    K, V bit for bit, positions (slot ids or explicit positions) and new lengths."""
    rng = np.random.default_rng(1000 * budget + len(dtype) + (7 if with_pos else 0))
    lengths = [37, 5, 0, 100]
    n_seq, n_layer, n_kvh, max_len = len(lengths), 2, 3, 100
    shape = (n_seq, n_layer, n_kvh, max_len, 128)
    raw = {"f32": (np.int32, torch.float32), "bf16": (np.int16, torch.bfloat16),
           "fp8": (np.uint8, torch.float8_e4m3fn), "int8": (np.int8, torch.int8)}[dtype]
    info = np.iinfo(raw[0])
    kb = rng.integers(info.min, info.max, size=shape, dtype=raw[0], endpoint=True)
    vb = rng.integers(info.min, info.max, size=shape, dtype=raw[0], endpoint=True)
    k = torch.from_numpy(kb).cuda().view(raw[1])
    v = torch.from_numpy(vb).cuda().view(raw[1])
    pos = rng.integers(0, 1 << 20, size=(n_seq, n_layer, n_kvh, max_len), dtype=np.int32) if with_pos else None
    kv = tri.KVCache.dense(k, v, torch.tensor(lengths, dtype=torch.int32, device="cuda"),
                           pos=torch.from_numpy(pos).cuda() if with_pos else None)
    kept = np.full((n_seq, n_layer, n_kvh, budget), -1, np.int32)
    for s, L in enumerate(lengths):
        n = min(L, budget)
        for l in range(n_layer):
            for h in range(n_kvh):
                kept[s, l, h, :n] = np.sort(rng.choice(L, size=n, replace=False)) if n else []
    kept_n = np.array([min(L, budget) for L in lengths], np.int32)
    out = tri.tri_compact_kv(kv, torch.from_numpy(kept).cuda(), torch.from_numpy(kept_n).cuda(), budget)
    torch.cuda.synchronize()
    ko, vo, po, nl = bits(out["k_out"]), bits(out["v_out"]), bits(out["pos_out"]), bits(out["new_len"])
    for s, L in enumerate(lengths):
        n = min(L, budget)
        assert nl[s] == n
        for l in range(n_layer):
            for h in range(n_kvh):
                ek, ev, ep = oracle.compact_dense(kb[s, l, h], vb[s, l, h], kept[s, l, h, :n],
                                                  pos=pos[s, l, h] if with_pos else None)
                assert np.array_equal(ko[s, l, h, :n], ek), (s, l, h)
                assert np.array_equal(vo[s, l, h, :n], ev), (s, l, h)
                assert np.array_equal(po[s, l, h, :n], ep), (s, l, h)


# ---------------------------------------------------------------------------------------
# selection edge cases on hand-made scores
# ---------------------------------------------------------------------------------------

def _select_case(scores_list, budget, window):
    n_seq = len(scores_list)
    max_len = max(len(x) for x in scores_list)
    sc = np.zeros((n_seq, 1, 1, max_len), np.float32)
    for i, x in enumerate(scores_list):
        sc[i, 0, 0, : len(x)] = x
    lengths = torch.tensor([len(x) for x in scores_list], dtype=torch.int32, device="cuda")
    k = torch.empty((n_seq, 1, 1, max_len, 128), dtype=torch.bfloat16, device="cuda")
    kv = tri.KVCache.dense(k, None, lengths)
    dsc = torch.from_numpy(sc).cuda()
    # both ways: with the workspace (units over 32768 slots: two-stage selection) and without
    for ws in ("auto", None):
        kept, kept_n = tri.tri_select_topb(dsc, kv, budget, window, workspace=ws)
        kept, kept_n = kept.cpu().numpy(), kept_n.cpu().numpy()
        for i, x in enumerate(scores_list):
            L = len(x)
            want = oracle.select_top_b(np.asarray(x, np.float64), L, budget, window)
            n = min(L, budget)
            assert kept_n[i] == n
            assert np.array_equal(kept[i, 0, 0, :n], want), f"case {i} (L={L}, B={budget}, W={window}, ws={ws})"
            assert np.all(kept[i, 0, 0, n:] == -1)


def test_select_edge_cases():
    rng = np.random.default_rng(5)
    mixed = rng.standard_normal(3000).astype(np.float32)
    mixed[rng.choice(3000, 200, replace=False)] = np.nan
    mixed[rng.choice(3000, 200, replace=False)] = -np.inf
    mixed[rng.choice(3000, 50, replace=False)] = np.inf
    mixed[rng.choice(3000, 300, replace=False)] = 0.0
    mixed[rng.choice(3000, 300, replace=False)] = -0.0
    cases = [
        np.zeros(3000, np.float32),                                   # all ties
        mixed,
        rng.integers(-3, 4, 3000).astype(np.float32),                 # heavy ties at the threshold
        rng.standard_normal(500).astype(np.float32),                  # L <= B
        rng.standard_normal(1001).astype(np.float32),                 # B = L - 1
        np.full(2000, np.nan, np.float32),                            # all NaN
        (rng.standard_normal(4000) * 1e-30).astype(np.float32),       # tiny magnitudes
        (rng.standard_normal(3000) * 1e-40).astype(np.float32),       # subnormals
        np.exp(rng.standard_normal(3000) * 20).astype(np.float32),    # wide dynamic range
        np.float32([5.0]),                                            # L = 1
    ]
    log("select edge cases B=1000 W=100")
    _select_case(cases, 1000, 100)
    log("select edge cases B=1000 W=0 / W=2000 / B=1")
    _select_case(cases, 1000, 0)
    _select_case(cases, 1000, 2000)
    _select_case(cases, 1, 0)
    _select_case(cases, 1, 1)


def test_select_register_resident_boundary():
    # units of up to 32768 slots keep their keys in registers; longer ones stream
    rng = np.random.default_rng(7)
    heavy = rng.integers(0, 100, 32768).astype(np.float32)        # ties at the threshold
    normal = rng.standard_normal(32768).astype(np.float32)
    ragged = rng.standard_normal(24577).astype(np.float32)
    ragged[rng.choice(24577, 3000, replace=False)] = 0.5
    log("select resident units (32768, 32768, 24577), B=2048 W=128")
    _select_case([heavy, normal, ragged], 2048, 128)
    log("select streamed units (32769, 40000), B=2048 W=128")
    _select_case([rng.standard_normal(32769).astype(np.float32),
                  rng.integers(-5, 5, 40000).astype(np.float32)], 2048, 128)


def test_select_long_unit_multiple_segments():
    rng = np.random.default_rng(6)
    x = rng.standard_normal(140000).astype(np.float32)
    x[::7] = 1.25                              # ties spread over both segments
    y = rng.integers(0, 50, 70001).astype(np.float32)
    log("select long units (140000, 70001), B=5000 W=256")
    _select_case([x, y], 5000, 256)


def test_select_two_stage_runs():
    # units over 32768 slots with a workspace: each run of 32768 candidates keeps its best B',
    # then the unit keeps its best B' of those; lengths around the runs' edges, ties across
    # runs, special values, units at or below the budget and at the register capacity
    rng = np.random.default_rng(8)
    special = rng.standard_normal(65553).astype(np.float32)
    special[rng.choice(65553, 3000, replace=False)] = np.nan
    special[rng.choice(65553, 3000, replace=False)] = -np.inf
    special[rng.choice(65553, 500, replace=False)] = np.inf
    special[rng.choice(65553, 2000, replace=False)] = -0.0
    ties = np.full(98310, 0.75, np.float32)
    ties[rng.choice(98310, 20000, replace=False)] = 2.0
    cases = [
        rng.standard_normal(131072).astype(np.float32),
        rng.integers(0, 40, 32769).astype(np.float32),                # 1 candidate in the second run
        rng.standard_normal(500).astype(np.float32),                  # L <= B
        rng.standard_normal(32768).astype(np.float32),                # one run
        special,
        ties,                                                         # ties across three runs
        np.zeros(0, np.float32),                                      # empty
    ]
    for budget, window in ((3840, 256), (1000, 0), (4097, 4096), (8200, 8), (8201, 8), (2048, 2048)):
        log(f"two-stage selection B={budget} W={window}")
        _select_case(cases, budget, window)


# ---------------------------------------------------------------------------------------
# calibration
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,layout", [("bf16", "half"), ("f32", "interleaved"), ("f32", "half")])
def test_calibration_parity(dtype, layout):
    g = torch.Generator().manual_seed(3)
    n, n_layer, n_qh = 777, 3, 5
    q = torch.randn((n, n_layer, n_qh, 128), generator=g) * 0.7 + torch.randn((1, n_layer, n_qh, 128), generator=g)
    q = q.to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    log(f"calibration {dtype} {layout}")
    center, mean_abs = tri.tri_calibrate_stats(q.cuda(), rope_layout=layout)
    oc, om = oracle.calibrate(q.float().numpy(), layout)
    c = center.cpu().numpy()
    m = mean_abs.cpu().numpy()
    tol = 1e-6 * om + 1e-30
    assert np.all(np.abs(c[..., 0] - oc.real) <= tol)
    assert np.all(np.abs(c[..., 1] - oc.imag) <= tol)
    assert np.all(np.abs(m - om) <= tol)


# ---------------------------------------------------------------------------------------
# full-size workloads, sampled units
# ---------------------------------------------------------------------------------------

ATT_TOL = 2e-3     # |out_gpu - out_oracle| <= ATT_TOL * max_j |v_j| (per query head)


def _check_consumer(w, hp, cache, kept, picks, pos, seed):
    """Attention of a new query of every sequence over the cache the pass compressed, as
    bench.py times it (the no-allocation entry point: the same kernels and slot split as with a
    workspace), against the oracle on sampled (sequence, layer, KV head) units."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((w.n_seq, w.n_layer, w.n_qh, w.head_dim)).astype(np.float32)
    qpos = np.asarray(hp.lengths, np.int64)                 # the next token of each sequence
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    tri.tri_decode_attention_noalloc(cache, torch.from_numpy(q).cuda(), torch.from_numpy(qpos).cuda(),
                                     rope_base=w.base, group=w.group, pos=pos, rope_layout=w.layout, out=out)
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got)), "non-finite attention output"
    g = w.group
    worst = 0.0
    for s, l, h in picks:
        n = min(int(hp.lengths[s]), w.budget)
        kk = kept[s, l, h, :n]
        k = P.host_rows(w, hp, s, l, h)[kk]
        v = P.host_rows(w, hp, s, l, h, tag=synth.TAG_V)[kk]
        want = oracle.decode_attention(q[s, l, h * g:(h + 1) * g], k, v, base=w.base, key_pos=kk,
                                       query_pos=int(qpos[s]), layout=w.layout)
        err = float(np.abs(got[s, l, h * g:(h + 1) * g] - want).max()) / max(float(np.abs(v).max()), 1e-30)
        assert err <= ATT_TOL, f"attention (seq {s}, layer {l}, head {h}): error {err:.3e} of max |v|"
        worst = max(worst, err)
    log(f"  attention over the compressed cache, {len(picks)} sampled units: max error / max|v| = {worst:.3e}")


def _full_dense(name, units, key_space="pre"):
    w = W.WORKLOADS[name]
    log(f"full size {name}: building")
    dw = SD.build(w)
    log(f"full size {name}: running the pass (keys {key_space}-RoPE)")
    scores, kept, kept_n, out = run_pass(dw, key_space)
    kn = kept_n.cpu().numpy()
    if out["v_out"] is not None and key_space == "pre" and w.dtype in ("f32", "bf16"):
        log(f"full size {name}: attention over the compressed cache")
        cache = tri.KVCache.dense(out["k_out"], out["v_out"], out["new_len"])
        _check_consumer(w, dw.hp, cache, kept.cpu().numpy(), [W.unit_coords(w, u) for u in units],
                        out["pos_out"], seed=200 + len(units))
    worst = 0.0
    for u in units:
        s, l, h = W.unit_coords(w, u)
        log(f"  unit {u} (seq {s}, layer {l}, head {h}, lowR={bool(dw.hp.low_r[l, h])})")
        sc_h = scores[s:s + 1, l:l + 1, h:h + 1].cpu().numpy()
        kp_h = kept[s:s + 1, l:l + 1, h:h + 1].cpu().numpy()
        o = {"k_out": bits(out["k_out"][s:s + 1, l:l + 1, h:h + 1]),
             "v_out": bits(out["v_out"][s:s + 1, l:l + 1, h:h + 1]) if out["v_out"] is not None else None,
             "pos_out": out["pos_out"][s:s + 1, l:l + 1, h:h + 1].cpu().numpy(),
             "new_len": out["new_len"][s:s + 1].cpu().numpy()}
        # re-index the sampled unit as unit (0, 0, 0) of a one-unit view
        sub = SD.DeviceWorkload(w, dw.hp, None, None, None, None, None, None)
        worst = max(worst, _check_sampled(sub, s, l, h, sc_h, kp_h, kn[s:s + 1], o, key_space))
    # the generator itself: device K rows of the sampled units equal the host rows
    for u in units[:2]:
        s, l, h = W.unit_coords(w, u)
        assert np.array_equal(bits(dw.k[s, l, h]), P.host_bits(w, dw.hp, s, l, h))
    log(f"  max score error / bound = {worst:.3e}")


def _check_sampled(dw, s, l, h, sc_h, kp_h, kn_h, o, key_space="pre"):
    w, hp = dw.w, dw.hp
    L = int(hp.lengths[s])
    keys = P.host_rows(w, hp, s, l, h)
    orc, S = P.oracle_scores(w, hp, s, l, h, keys, key_space)
    worst, _ = P.check_scores(sc_h[0, 0, 0, :L], orc, S)
    P.check_kept(kp_h[0, 0, 0], sc_h[0, 0, 0], orc, S, L, w.budget, w.window)
    n = min(L, w.budget)
    assert kn_h[0] == n and o["new_len"][0] == n
    kk = kp_h[0, 0, 0, :n]
    assert np.array_equal(o["k_out"][0, 0, 0, :n], P.host_bits(w, hp, s, l, h)[kk])
    if o["v_out"] is not None:
        hv = P.host_bits(w, hp, s, l, h, tag=synth.TAG_V)
        assert np.array_equal(o["v_out"][0, 0, 0, :n], hv[kk])
    assert np.array_equal(o["pos_out"][0, 0, 0, :n], kk)
    return worst


def _low_r_units(w, hp, count):
    idx = [W.unit_index(w, 0, int(l), int(h)) for l, h in zip(*np.nonzero(hp.low_r))]
    return idx[:count]


def test_full_single_head_2k_f32():
    w = W.WORKLOADS["single_head_2k_f32"]
    log("full size single_head_2k_f32")
    dw = SD.build(w)
    scores, kept, kept_n, out = run_pass(dw)
    sc, kp, kn, o = host_outputs(scores, kept, kept_n, out)
    e, rel = check_dense_unit(dw, 0, 0, 0, sc, kp, kn, o)
    log(f"  score error / bound = {e:.3e}, plain relative error (|s| >= 1% of bound) = {rel:.3e}")


def test_full_gqa8b_32k_bf16():
    w = W.WORKLOADS["gqa8b_32k_bf16"]
    hp = W.make_params(w)
    rng = np.random.default_rng(100)
    units = [0, w.n_units - 1] + _low_r_units(w, hp, 2) + [int(x) for x in rng.choice(w.n_units, 2, replace=False)]
    _full_dense("gqa8b_32k_bf16", units)


def test_full_gqa8b_batch16_16k_bf16():
    w = W.WORKLOADS["gqa8b_batch16_16k_bf16"]
    hp = W.make_params(w)
    rng = np.random.default_rng(101)
    low = _low_r_units(w, hp, 1)
    units = [0, w.n_units - 1] + [u + 9 * w.n_layer * w.n_kvh for u in low] + \
        [int(x) for x in rng.choice(w.n_units, 3, replace=False)]
    _full_dense("gqa8b_batch16_16k_bf16", units)


def test_full_long_128k_bf16():
    w = W.WORKLOADS["long_128k_bf16"]
    hp = W.make_params(w)
    rng = np.random.default_rng(103)
    # every unit spans many waves' shares; unit 0 starts a share, units 1 and the last start in
    # the middle of one (the wave finishes the previous unit first)
    units = [0, 1, w.n_units - 1] + _low_r_units(w, hp, 1) + [int(rng.integers(2, w.n_units - 1))]
    _full_dense("long_128k_bf16", units)


def test_full_paged_ragged64_bf16():
    w = W.WORKLOADS["paged_ragged64_bf16"]
    log("full size paged_ragged64_bf16: building")
    dw = SD.build(w)
    hp = dw.hp
    rng = np.random.default_rng(102)
    seqs = [int(np.argmin(hp.lengths)), int(np.argmax(hp.lengths))] + [int(x) for x in rng.choice(w.n_seq, 2, replace=False)]
    picks = [(s, int(rng.integers(w.n_layer)), int(rng.integers(w.n_kvh))) for s in seqs]
    # units where a wave's share of the scoring grid starts inside the unit: the matrix-core kernel
    # runs one 8-wave workgroup per CU and splits the 16-key steps of all units, in (sequence,
    # layer, head) order, into equal shares (the first total % waves shares one step longer)
    unit_steps = np.repeat((hp.lengths.astype(np.int64) + 15) // 16, w.n_layer * w.n_kvh)
    ends = np.cumsum(unit_steps)
    n_waves = torch.cuda.get_device_properties(0).multi_processor_count * 8
    share, extra = divmod(int(ends[-1]), n_waves)
    for wv in (n_waves // 3, n_waves // 2, (2 * n_waves) // 3):
        g0 = wv * share + min(wv, extra)
        u = int(np.searchsorted(ends, g0, side="right"))
        if g0 > (ends[u - 1] if u else 0):           # the share starts after the unit's first step
            picks.append(W.unit_coords(w, u))
    # the pool is compacted in place: the oracle's rows come from the host generator
    pk = dw.k
    for s, l, h in picks[:2]:
        L = int(hp.lengths[s])
        pages = torch.from_numpy(hp.block_table[s, : -(-L // 16)].astype(np.int64)).cuda()
        got = bits(pk.index_select(0, pages)[:, l, h].reshape(-1, 128)[:L])
        assert np.array_equal(got, P.host_rows(w, hp, s, l, h, as_float=False).view(np.int16))
    log("full size paged_ragged64_bf16: running the pass")
    scores, kept, kept_n, out = run_pass(dw)
    kn = kept_n.cpu().numpy()
    nf = out["n_freed"].cpu().numpy()
    freed = out["freed"].cpu().numpy()
    for s, l, h in picks:
        L = int(hp.lengths[s])
        log(f"  seq {s} (L={L}), layer {l}, head {h}")
        keys = P.host_rows(w, hp, s, l, h)
        orc, S = P.oracle_scores(w, hp, s, l, h, keys)
        sc_h = scores[s, l, h].cpu().numpy()
        kp_h = kept[s, l, h].cpu().numpy()
        P.check_scores(sc_h[:L], orc, S)
        P.check_kept(kp_h, sc_h, orc, S, L, w.budget, w.window)
        n = min(L, w.budget)
        assert kn[s] == n
        # packed rows: slot i of the unit holds original row kept[i]
        pages = torch.from_numpy(hp.block_table[s, : -(-n // 16)].astype(np.int64)).cuda()
        packed = bits(pk.index_select(0, pages)[:, l, h].reshape(-1, 128)[:n])
        hk = P.host_rows(w, hp, s, l, h, as_float=False).view(np.int16)
        assert np.array_equal(packed, hk[kp_h[:n]])
        hv = P.host_rows(w, hp, s, l, h, tag=synth.TAG_V, as_float=False).view(np.int16)
        packed_v = bits(dw.v.index_select(0, pages)[:, l, h].reshape(-1, 128)[:n])
        assert np.array_equal(packed_v, hv[kp_h[:n]])
        want_freed = hp.block_table[s, -(-n // 16): -(-L // 16)]
        assert nf[s] == len(want_freed) and np.array_equal(freed[s, : nf[s]], want_freed)
    # attention over the pool packed in place, with the kept keys' positions at the pool's slot
    # stride (as bench.py runs it)
    log("full size paged_ragged64_bf16: attention over the compressed cache")
    pos = torch.zeros((w.n_seq, w.n_layer, w.n_kvh, dw.kv().slots), dtype=torch.int32, device="cuda")
    pos[..., :w.budget] = out["pos_out"]
    cache = tri.KVCache.paged(dw.k, dw.v, dw.block_table, out["new_len"], pos=pos)
    _check_consumer(w, hp, cache, kept.cpu().numpy(), picks, pos, seed=210)
    # freed-page accounting over the whole batch
    total_before = int(sum(-(-int(L) // 16) for L in hp.lengths))
    total_after = int(sum(-(-min(int(L), w.budget) // 16) for L in hp.lengths))
    assert int(nf.sum()) == total_before - total_after


# ---------------------------------------------------------------------------------------
# binding: buffers whose shape does not match the descriptor are rejected before launch
# ---------------------------------------------------------------------------------------

@pytest.mark.gpu
def test_binding_rejects_mismatched_shapes():
    import torch
    lengths = torch.tensor([100, 80], dtype=torch.int32, device="cuda")
    k = torch.zeros((2, 3, 2, 128, 128), dtype=torch.bfloat16, device="cuda")
    kv = tri.KVCache.dense(k, k.clone(), lengths)
    center = torch.zeros((3, 4, 64, 2), dtype=torch.float32, device="cuda")
    mean_abs = torch.zeros((3, 4, 64), dtype=torch.float32, device="cuda")
    kw = dict(rope_base=1e4, offsets=(1, 2), group=2)
    bad = [
        lambda: tri.tri_score_keys(kv, center[:2], mean_abs, **kw),
        lambda: tri.tri_score_keys(kv, center, mean_abs, scores=torch.empty((2, 3, 2, 100), device="cuda"), **kw),
        lambda: tri.tri_select_topb(torch.empty((2, 3, 2, 64), device="cuda"), kv, 16, 4),
        lambda: tri.tri_select_topb(torch.empty((2, 3, 2, 128), device="cuda"), kv, 16, 4,
                                    kept=torch.empty((2, 3, 2, 8), dtype=torch.int32, device="cuda")),
        lambda: tri.tri_compact_kv(kv, torch.zeros((2, 3, 2, 16), dtype=torch.int32, device="cuda"),
                                   torch.zeros((2,), dtype=torch.int32, device="cuda"), 16,
                                   k_out=torch.empty((2, 3, 2, 8, 128), dtype=torch.bfloat16, device="cuda")),
    ]
    for i, fn in enumerate(bad):
        with pytest.raises(ValueError):
            fn()
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------------------
# adversarial keys through the whole pass: exact score ties (zero keys score exactly 0 at any
# position), near-ties (one row repeated at many positions) and a NaN row
# ---------------------------------------------------------------------------------------

@pytest.mark.gpu
def test_zero_duplicated_and_nan_key_rows():
    w = W.scaled(BASE, name="adversarial", n_seq=1, n_layer=1, n_kvh=2, group=4, max_len=1500,
                 budget=300, window=16)
    hp = W.make_params(w)
    L = w.max_len
    raw = np.stack([P.host_rows(w, hp, 0, 0, h, as_float=False) for h in range(w.n_kvh)])  # [2, L, 128] bf16 bits
    rng = np.random.default_rng(11)
    live = np.zeros(L, bool)
    live[rng.choice(L, 150, replace=False)] = True
    raw[0, ~live] = 0                          # head 0: mostly zero keys, so the threshold sits in a tie at 0
    raw[0, 300] = 0x7FC0                       # and a NaN key row (scores as -inf)
    raw[1, 100:200] = raw[1, 50:51]            # head 1: one row repeated at 100 positions
    raw[1, 700:1000:3] = raw[1, 699:700]
    log("adversarial rows: zero keys (exact ties at the threshold), repeated rows, a NaN row; B=300 W=16")
    k = torch.from_numpy(raw.view(np.int16).reshape(1, 1, 2, L, 128).copy()).cuda().view(torch.bfloat16)
    v = torch.from_numpy(raw[::-1].copy().view(np.int16).reshape(1, 1, 2, L, 128)).cuda().view(torch.bfloat16)
    lengths = torch.tensor([L], dtype=torch.int32, device="cuda")
    kv = tri.KVCache.dense(k, v, lengths)
    center = torch.from_numpy(hp.center).cuda()
    mean_abs = torch.from_numpy(hp.mean_abs).cuda()
    sc = tri.tri_score_keys(kv, center, mean_abs, rope_base=w.base, offsets=w.offsets, group=w.group)
    kept, kept_n = tri.tri_select_topb(sc, kv, w.budget, w.window)
    out = tri.tri_compact_kv(kv, kept, kept_n, w.budget)
    torch.cuda.synchronize()
    sc_h, kept_h = sc.cpu().numpy()[0, 0], kept.cpu().numpy()[0, 0]
    k_out, v_out = bits(out["k_out"])[0, 0], bits(out["v_out"])[0, 0]
    for h in range(w.n_kvh):
        keys = oracle.decode_stored(raw[h], "bf16")
        center_h, mean_abs_h = oracle.unit_heads(hp.center, hp.mean_abs, 0, h, w.group)
        orc = oracle.score_keys(keys, center_h, mean_abs_h, base=w.base, offsets=w.offsets)
        S = oracle.score_magnitude_bound(keys, center_h, mean_abs_h)
        bad = ~np.isfinite(orc)
        assert np.array_equal(~np.isfinite(sc_h[h, :L]), bad), "non-finite scores differ from the oracle's"
        fin = ~bad
        assert np.all(np.abs(sc_h[h, :L][fin] - orc[fin]) <= P.SCORE_TOL * S[fin])
        want = oracle.select_top_b(sc_h[h, :L].astype(np.float64), L, w.budget, w.window)
        assert np.array_equal(kept_h[h, : len(want)], want)
        if h == 0:
            zero = (raw[0] == 0).all(axis=1)
            assert np.all(sc_h[0, :L][zero] == 0.0), "zero keys must score exactly 0"
            cand = np.arange(L - w.window)
            kept_zero = np.intersect1d(want, cand[zero[: L - w.window]])
            assert 0 < kept_zero.size < zero[: L - w.window].sum(), "the threshold must fall inside the zero tie"
            assert 300 not in set(want.tolist()), "a NaN-scored key must rank last"
            # both selections agree exactly here: ties are exact in both score sets
            assert np.array_equal(want, oracle.select_top_b(orc, L, w.budget, w.window))
        assert np.array_equal(k_out[h, : len(want)], raw[h].view(np.int16)[want])
        assert np.array_equal(v_out[h, : len(want)], raw[::-1][h].view(np.int16)[want])



# ---------------------------------------------------------------------------------------
# keys cached after RoPE
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,layout,group,reduce", [("bf16", "half", 4, "max"), ("f32", "interleaved", 3, "mean"),
                                                       ("bf16", "interleaved", 7, "max"), ("fp8", "half", 4, "max"),
                                                       ("int8", "interleaved", 2, "mean")])
def test_post_rope_small_dense(dtype, layout, group, reduce):
    # a post-RoPE cache built on the host: the generator's keys rotated by RoPE at their
    # slots in float64 (the oracle's rotation), then stored in the cache dtype (fp8: the
    # codes of key / scale, with the head's power-of-two scale)
    w = W.scaled(BASE, name="post_rope", n_seq=2, n_layer=2, n_kvh=2, group=group, reduce=reduce, dtype=dtype,
                 layout=layout, max_len=2600, budget=500, window=32)
    lengths = [2600, 1111]
    hp = W.make_params(w, lengths=lengths)
    log(f"post-RoPE small dense {dtype} {layout} G={group} {reduce}")
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32, "fp8": torch.float8_e4m3fn, "int8": torch.int8}[dtype]
    k = torch.zeros((2, 2, 2, w.max_len, 128), dtype=tdt)
    cached, stored = {}, {}
    for s in range(2):
        L = lengths[s]
        for l in range(2):
            for h in range(2):
                pre = P.host_rows(w, hp, s, l, h)
                post = oracle.rope_apply(pre, np.arange(L), base=w.base, layout=layout).astype(np.float32)
                if dtype == "bf16":
                    raw = synth.f32_to_bf16_bits(post).view(np.int16)
                    cached[(s, l, h)] = oracle.decode_stored(raw, "bf16")
                elif dtype == "fp8":
                    sc_lh = np.float32(hp.k_scale[l, h])
                    raw = synth.f32_to_fp8_e4m3(post / sc_lh)
                    cached[(s, l, h)] = oracle.decode_stored(raw, "fp8", sc_lh)
                elif dtype == "int8":
                    sc_lh = np.float32(hp.k_scale[l, h])
                    raw = synth.f32_to_int8(post / sc_lh)
                    cached[(s, l, h)] = oracle.decode_stored(raw, "int8", sc_lh)
                else:
                    raw = post.view(np.int32)
                    cached[(s, l, h)] = post
                stored[(s, l, h)] = raw
                k[s, l, h, :L] = torch.from_numpy(raw.copy()).view(tdt)
    k = k.cuda()
    k_scale = torch.from_numpy(hp.k_scale).cuda() if dtype in ("fp8", "int8") else None
    kv = tri.KVCache.dense(k, None, torch.tensor(lengths, dtype=torch.int32, device="cuda"), k_scale=k_scale)
    center, mean_abs = torch.from_numpy(hp.center).cuda(), torch.from_numpy(hp.mean_abs).cuda()
    out = tri.compress(kv, center, mean_abs, rope_base=w.base, offsets=w.offsets, group=group, budget=w.budget,
                       window=w.window, reduce=reduce, rope_layout=layout, key_space="post")
    torch.cuda.synchronize()
    sc, kp, kn = out["scores"].cpu().numpy(), out["kept"].cpu().numpy(), out["kept_n"].cpu().numpy()
    ko = bits(out["k_out"])
    worst = 0.0
    for (s, l, h), keys in cached.items():
        L = lengths[s]
        orc, S = P.oracle_scores(w, hp, s, l, h, keys, "post")
        e, _ = P.check_scores(sc[s, l, h, :L], orc, S)
        worst = max(worst, e)
        P.check_kept(kp[s, l, h], sc[s, l, h], orc, S, L, w.budget, w.window)
        n = min(L, w.budget)
        assert kn[s] == n
        assert np.array_equal(ko[s, l, h, :n], stored[(s, l, h)][kp[s, l, h, :n]])
    log(f"  max score error / bound = {worst:.3e}")


def test_full_gqa8b_32k_bf16_post_rope():
    # the full-size cache read as a post-RoPE cache (the synthetic keys stand for rotated keys)
    w = W.WORKLOADS["gqa8b_32k_bf16"]
    hp = W.make_params(w)
    rng = np.random.default_rng(105)
    units = [0, w.n_units - 1] + _low_r_units(w, hp, 1) + [int(x) for x in rng.choice(w.n_units, 1, replace=False)]
    _full_dense("gqa8b_32k_bf16", units, key_space="post")


@pytest.mark.parametrize("dtype,layout,group,key_space", [("fp8", "half", 4, "post"), ("int8", "interleaved", 3, "post"),
                                                           ("fp8", "interleaved", 4, "pre"), ("int8", "half", 6, "pre")])
def test_8bit_without_key_scales(dtype, layout, group, key_space):
    # 8-bit codes passed without per-head scales: each key is its codes' values (scale 1); post-RoPE
    # max takes the matrix-core kernel, pre-RoPE the vector kernel
    w = W.scaled(BASE, name="noscale", n_seq=2, n_layer=2, n_kvh=2, group=group, dtype=dtype, layout=layout,
                 max_len=1300, budget=200, window=16)
    lengths = [1300, 517]
    hp = W.make_params(w, lengths=lengths)
    log(f"8-bit keys without scales: {dtype} {layout} G={group} keys {key_space}-RoPE")
    dw = SD.build(w, hp=hp)
    kv = tri.KVCache.dense(dw.k, dw.v, dw.seq_len)
    sc = tri.tri_score_keys(kv, dw.center, dw.mean_abs, rope_base=w.base, offsets=w.offsets, group=w.group,
                            reduce=w.reduce, rope_layout=w.layout, key_space=key_space)
    torch.cuda.synchronize()
    sc = sc.cpu().numpy()
    worst = 0.0
    for s in range(w.n_seq):
        L = lengths[s]
        for l in range(w.n_layer):
            for h in range(w.n_kvh):
                codes = P.host_rows(w, hp, s, l, h, as_float=False)
                keys = oracle.decode_stored(codes, dtype, 1.0)
                orc, S = P.oracle_scores(w, hp, s, l, h, keys, key_space)
                e, _ = P.check_scores(sc[s, l, h, :L], orc, S)
                worst = max(worst, e)
    log(f"  max score error / bound = {worst:.3e}")


@pytest.mark.parametrize("name", ["gqa8b_32k_fp8", "gqa8b_32k_int8"])
def test_full_gqa8b_32k_8bit_post_rope(name):
    # the full-size 8-bit caches read as post-RoPE caches: matrix cores, codes times per-head scales
    w = W.WORKLOADS[name]
    hp = W.make_params(w)
    rng = np.random.default_rng(109)
    units = [0, w.n_units - 1] + _low_r_units(w, hp, 1) + [int(x) for x in rng.choice(w.n_units, 1, replace=False)]
    _full_dense(name, units, key_space="post")


def test_full_long_128k_bf16_post_rope():
    # the 128K cache read as a post-RoPE cache: G = 7 on the matrix cores, raw keys in the products
    w = W.WORKLOADS["long_128k_bf16"]
    hp = W.make_params(w)
    rng = np.random.default_rng(107)
    units = [1, w.n_units - 1] + _low_r_units(w, hp, 1) + [int(rng.integers(2, w.n_units - 1))]
    _full_dense("long_128k_bf16", units, key_space="post")


def test_full_gqa8b_32k_fp8():
    w = W.WORKLOADS["gqa8b_32k_fp8"]
    hp = W.make_params(w)
    rng = np.random.default_rng(106)
    units = [0, 1, w.n_units - 1] + _low_r_units(w, hp, 1) + [int(x) for x in rng.choice(w.n_units, 2, replace=False)]
    _full_dense("gqa8b_32k_fp8", units)


def test_full_gqa8b_32k_int8():
    w = W.WORKLOADS["gqa8b_32k_int8"]
    hp = W.make_params(w)
    rng = np.random.default_rng(107)
    units = [0, 1, w.n_units - 1] + _low_r_units(w, hp, 1) + [int(x) for x in rng.choice(w.n_units, 2, replace=False)]
    _full_dense("gqa8b_32k_int8", units)


# ---------------------------------------------------------------------------------------
# multiplicative score form: phase-only series times the centre and key norms
# ---------------------------------------------------------------------------------------

MULT_DENSE = {
    "g4_max_half_bf16": (dict(n_seq=2, n_layer=2, n_kvh=2, group=4, max_len=2700, budget=600, window=64),
                         [2700, 1500], "pre"),
    "g3_mean_interleaved_f32": (dict(n_seq=1, n_layer=2, n_kvh=2, group=3, reduce="mean", layout="interleaved",
                                     dtype="f32", max_len=1700, budget=300, window=16), [1700], "pre"),
    "g8_max_half_fp8": (dict(n_seq=1, n_layer=1, n_kvh=2, group=8, dtype="fp8", max_len=1300, budget=200,
                             window=8), [1300], "pre"),
    "g1_half_int8": (dict(n_seq=2, n_layer=1, n_kvh=2, group=1, dtype="int8", max_len=1100, budget=128,
                          window=32), [1100, 450], "pre"),
    "g4_max_half_bf16_post": (dict(n_seq=1, n_layer=2, n_kvh=2, group=4, max_len=2100, budget=500, window=32),
                              [2100], "post"),
    "g6_max_interleaved_bf16_post": (dict(n_seq=2, n_layer=1, n_kvh=1, group=6, layout="interleaved",
                                          max_len=1500, budget=256, window=0), [1500, 999], "post"),
}


@pytest.mark.parametrize("name", sorted(MULT_DENSE))
def test_multiplicative_small_dense(name):
    over, lengths, key_space = MULT_DENSE[name]
    w = W.scaled(BASE, name="mult_" + name, **over)
    log(f"multiplicative small dense {name}: {over} lengths={lengths} keys {key_space}-RoPE")
    dw = SD.build(w, hp=W.make_params(w, lengths=lengths))
    sc, kept, kept_n, out = host_outputs(*run_pass(dw, key_space, "multiplicative"))
    worst = 0.0
    for s in range(w.n_seq):
        for l in range(w.n_layer):
            for h in range(w.n_kvh):
                e, _ = check_dense_unit(dw, s, l, h, sc, kept, kept_n, out, key_space, "multiplicative")
                worst = max(worst, e)
    log(f"  max score error / bound = {worst:.3e}")


def test_multiplicative_small_paged():
    w = W.scaled(W.WORKLOADS["paged_ragged64_bf16"], n_seq=3, n_layer=2, n_kvh=2, max_len=4200,
                 len_range=(16, 4200))
    lengths = [4200, 40, 2049]
    log(f"multiplicative small paged lengths={lengths}")
    dw = SD.build(w, hp=W.make_params(w, lengths=lengths))
    sc, kept, kept_n, out = host_outputs(*run_pass(dw, "pre", "multiplicative"))
    for s in range(w.n_seq):
        L = lengths[s]
        for l in range(w.n_layer):
            for h in range(w.n_kvh):
                keys = P.host_rows(w, dw.hp, s, l, h)
                orc, S = P.oracle_scores(w, dw.hp, s, l, h, keys, "pre", "multiplicative")
                P.check_scores(sc[s, l, h, :L], orc, S)
                P.check_kept(kept[s, l, h], sc[s, l, h], orc, S, L, w.budget, w.window)
        assert kept_n[s] == min(L, w.budget)


def test_multiplicative_zero_and_nan_key_rows():
    # zero keys score exactly 0 (no live band, ||k|| = 0); a NaN key scores NaN
    w = W.scaled(BASE, name="mult_adv", n_seq=1, n_layer=1, n_kvh=1, group=4, max_len=600, budget=100, window=8)
    hp = W.make_params(w)
    keys = P.host_rows(w, hp, 0, 0, 0).copy()
    keys[[5, 77, 300]] = 0.0
    keys[400, 9] = np.nan
    k = torch.from_numpy(synth.f32_to_bf16_bits(keys).view(np.int16).reshape(1, 1, 1, 600, 128).copy())
    k = k.cuda().view(torch.bfloat16)
    kv = tri.KVCache.dense(k, None, torch.tensor([600], dtype=torch.int32, device="cuda"))
    sc = tri.tri_score_keys(kv, torch.from_numpy(hp.center).cuda(), None, rope_base=w.base, offsets=w.offsets,
                            group=4, form="multiplicative").cpu().numpy()[0, 0, 0]
    assert np.all(sc[[5, 77, 300]] == 0.0) and np.isnan(sc[400])
    ok = np.ones(600, bool)
    ok[[5, 77, 300, 400]] = False          # checked above; their bound S is 0
    orc, S = P.oracle_scores(w, hp, 0, 0, 0, oracle.decode_stored(synth.f32_to_bf16_bits(keys), "bf16"), "pre",
                             "multiplicative")
    P.check_scores(sc[ok], orc[ok], S[ok])


def test_full_gqa8b_32k_bf16_multiplicative():
    w = W.WORKLOADS["gqa8b_32k_bf16"]
    hp = W.make_params(w)
    log("full size gqa8b_32k_bf16, multiplicative form: building")
    dw = SD.build(w)
    scores, kept, kept_n, out = run_pass(dw, "pre", "multiplicative")
    rng = np.random.default_rng(108)
    units = [0, w.n_units - 1] + _low_r_units(w, hp, 1) + [int(x) for x in rng.choice(w.n_units, 2, replace=False)]
    for u in units:
        s, l, h = W.unit_coords(w, u)
        log(f"  unit {u} (seq {s}, layer {l}, head {h})")
        L = int(hp.lengths[s])
        keys = P.host_rows(w, hp, s, l, h)
        orc, S = P.oracle_scores(w, hp, s, l, h, keys, "pre", "multiplicative")
        sc_h = scores[s, l, h].cpu().numpy()
        P.check_scores(sc_h[:L], orc, S)
        P.check_kept(kept[s, l, h].cpu().numpy(), sc_h, orc, S, L, w.budget, w.window)


# ---------------------------------------------------------------------------------------
# seeded random combinations of every option, small enough for the oracle on every unit
# ---------------------------------------------------------------------------------------

def _random_case(seed):
    rng = np.random.default_rng(1000 + seed)
    dtype = ["f32", "bf16", "fp8", "int8"][rng.integers(4)]
    paged = bool(rng.integers(2))
    group = int(rng.integers(1, 9))
    over = dict(name=f"mix{seed}", n_seq=int(rng.integers(1, 4)), n_layer=int(rng.integers(1, 3)),
                n_kvh=int(rng.integers(1, 3)), group=group, dtype=dtype,
                layout=["half", "interleaved"][rng.integers(2)], reduce=["max", "mean"][rng.integers(2)],
                max_len=int(rng.integers(300, 2600)), budget=int(16 * rng.integers(2, 40)),
                window=int(rng.integers(0, 200)), base=float([1e4, 5e5, 1e6][rng.integers(3)]),
                offsets=W.geometric_offsets(int(rng.integers(0, 15))), seed=int(50 + seed),
                low_r_frac=float(rng.uniform(0, 0.5)), sink=bool(rng.integers(2)))
    if paged:
        w = W.scaled(W.WORKLOADS["paged_ragged64_bf16"], len_range=(1, over["max_len"]), **over)
    else:
        w = W.scaled(BASE, **over)
    lengths = [int(x) for x in rng.integers(0, w.max_len + 1, w.n_seq)]
    lengths[int(rng.integers(w.n_seq))] = w.max_len
    key_space = ["pre", "post"][rng.integers(2)]
    form = ["additive", "multiplicative"][rng.integers(2)]
    return w, lengths, key_space, form


@pytest.mark.parametrize("seed", range(16))
def test_random_option_mix(seed):
    w, lengths, key_space, form = _random_case(seed)
    log(f"mix {seed}: {w.dtype} {'paged' if w.paged else 'dense'} {w.layout} G={w.group} {w.reduce} "
        f"B={w.budget} W={w.window} |D|={len(w.offsets)} base={w.base:g} keys {key_space}-RoPE {form} "
        f"lengths={lengths}")
    dw = SD.build(w, hp=W.make_params(w, lengths=lengths))
    k_before, v_before = bits(dw.k), bits(dw.v)
    sc, kept, kept_n, out = host_outputs(*run_pass(dw, key_space, form))
    exp_k, exp_v = k_before.copy(), v_before.copy()
    for s in range(w.n_seq):
        L = lengths[s]
        n = min(L, w.budget)
        assert kept_n[s] == n and out["new_len"][s] == n
        kept_units = {}
        for l in range(w.n_layer):
            for h in range(w.n_kvh):
                keys = P.host_rows(w, dw.hp, s, l, h)
                orc, S = P.oracle_scores(w, dw.hp, s, l, h, keys, key_space, form)
                live = S > 0
                P.check_scores(sc[s, l, h, :L][live], orc[live], S[live])
                assert np.all(sc[s, l, h, :L][~live] == 0.0)
                P.check_kept(kept[s, l, h], sc[s, l, h], orc, S, L, w.budget, w.window)
                kk = kept[s, l, h, :n]
                assert np.array_equal(out["pos_out"][s, l, h, :n], kk)
                if w.paged:
                    kept_units[(l, h)] = kk
                else:
                    assert np.array_equal(out["k_out"][s, l, h, :n], P.host_bits(w, dw.hp, s, l, h)[kk])
                    assert np.array_equal(out["v_out"][s, l, h, :n],
                                          P.host_bits(w, dw.hp, s, l, h, tag=synth.TAG_V)[kk])
        if w.paged:
            ek, ev, freed, new_len = oracle.compact_paged_sequence(exp_k, exp_v, dw.hp.block_table[s], L,
                                                                   kept_units, 16)
            exp_k, exp_v = ek, ev
            nf = int(out["n_freed"][s])
            assert new_len == n and nf == len(freed) and np.array_equal(out["freed"][s, :nf], freed)
    if w.paged:
        assert np.array_equal(bits(dw.k), exp_k) and np.array_equal(bits(dw.v), exp_v)


# ---------------------------------------------------------------------------------------
# explicit query positions, and the longest supported unit
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("key_space", ["pre", "post"])
def test_explicit_query_positions(key_space):
    # the newest query ahead of the cache (tokens generated since the last pass) and behind it
    w = W.scaled(BASE, name="qpos", n_seq=3, n_layer=1, n_kvh=2, group=4, max_len=1500, budget=256, window=16)
    lengths = [1500, 900, 1200]
    qpos = [1500 + 3000, 950, 700]
    hp = W.make_params(w, lengths=lengths)
    log(f"explicit query positions {qpos} (lengths {lengths}), keys {key_space}-RoPE")
    dw = SD.build(w, hp=hp)
    kv = dw.kv()
    q = torch.tensor(qpos, dtype=torch.int64, device="cuda")
    sc = tri.tri_score_keys(kv, dw.center, dw.mean_abs, rope_base=w.base, offsets=w.offsets, group=w.group,
                            reduce=w.reduce, query_pos=q, key_space=key_space)
    kept, kept_n = tri.tri_select_topb(sc, kv, w.budget, w.window)
    torch.cuda.synchronize()
    sc, kept = sc.cpu().numpy(), kept.cpu().numpy()
    for s in range(w.n_seq):
        L = lengths[s]
        for h in range(w.n_kvh):
            keys = P.host_rows(w, hp, s, 0, h)
            center, mean_abs = oracle.unit_heads(hp.center, hp.mean_abs, 0, h, w.group)
            orc = oracle.score_keys(keys, center, mean_abs, base=w.base, offsets=w.offsets, query_pos=qpos[s],
                                    layout=w.layout, reduce=w.reduce, key_space=key_space)
            S = oracle.score_magnitude_bound(keys, center, mean_abs, layout=w.layout, reduce=w.reduce)
            P.check_scores(sc[s, 0, h, :L], orc, S)
            P.check_kept(kept[s, 0, h], sc[s, 0, h], orc, S, L, w.budget, w.window)


def test_longest_supported_unit_sampled():
    # one unit of 2^20 keys (the largest per-unit length the library accepts): float64
    # anchors keep the phase exact at large positions; scores are checked on sampled row
    # blocks, the selection exactly against the GPU's own scores and, outside the threshold
    # band, against the sampled oracle scores
    L = 1 << 20
    w = W.scaled(BASE, name="max_unit", n_seq=1, n_layer=1, n_kvh=1, group=4, max_len=L, budget=4096,
                 window=256, offsets=W.geometric_offsets(14))
    hp = W.make_params(w)
    log("longest unit: 1 x 1048576 keys, building")
    dw = SD.build(w, hp=hp)
    sc, kept, kept_n, _ = run_pass(dw)
    sc, kept = sc.cpu().numpy()[0, 0, 0], kept.cpu().numpy()[0, 0, 0]
    assert int(kept_n.cpu()[0]) == w.budget
    exact = oracle.select_top_b(sc.astype(np.float64), L, w.budget, w.window)
    assert np.array_equal(kept, exact)
    center, mean_abs = oracle.unit_heads(hp.center, hp.mean_abs, 0, 0, w.group)
    cand = L - w.window
    tau = np.sort(sc[:cand])[::-1][w.budget - w.window - 1]
    kept_set = set(kept.tolist())
    worst = 0.0
    for r0 in [0, 4096, 131072 - 32, 524288 + 7, 1000000, L - 1024, L - 300]:
        n = min(256, L - r0)
        rows = oracle.decode_stored(synth.rows(w.seed, synth.TAG_K, 0, n, hp.mu_k[0, 0], hp.sigma, w.sink, w.dtype,
                                               row_start=r0), w.dtype)
        pos = np.arange(r0, r0 + n)
        orc = oracle.score_keys(rows, center, mean_abs, base=w.base, offsets=w.offsets, key_pos=pos,
                                query_pos=L - 1, layout=w.layout, reduce=w.reduce)
        S = oracle.score_magnitude_bound(rows, center, mean_abs, layout=w.layout, reduce=w.reduce)
        e, _ = P.check_scores(sc[r0:r0 + n], orc, S)
        worst = max(worst, e)
        for j in range(n):
            p = r0 + j
            if p >= cand:
                assert p in kept_set                      # the window is always kept
            elif orc[j] > tau + P.SCORE_TOL * S[j]:
                assert p in kept_set
            elif orc[j] < tau - P.SCORE_TOL * S[j]:
                assert p not in kept_set
    log(f"  max score error / bound over sampled blocks = {worst:.3e}")


# ---------------------------------------------------------------------------------------
# the three calls captured in a HIP graph: the library allocates nothing and issues no
# memsets, so a captured pass replays to the eager results (also with scoring and selection
# in one launch, and with the two-stage selection of units over 32768 slots, whose
# workspace is allocated before the capture)
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("mode", ["dense", "paged", "fused", "long"])
def test_graph_capture_replays_match_eager(mode):
    paged = mode == "paged"
    if paged:
        w = W.scaled(W.WORKLOADS["paged_ragged64_bf16"], name="graph_paged", n_seq=3, n_layer=2, n_kvh=2,
                     max_len=3000, len_range=(16, 3000), budget=512, window=32)
        lengths = [3000, 700, 2049]
    elif mode == "long":
        w = W.scaled(BASE, name="graph_long", n_seq=2, n_layer=1, n_kvh=2, max_len=40000, budget=2048, window=64)
        lengths = [40000, 33000]
    else:
        w = W.scaled(BASE, name="graph_dense", n_seq=2, n_layer=2, n_kvh=2, max_len=2500, budget=400, window=32)
        lengths = [2500, 1333]
    log(f"graph capture, {mode} lengths={lengths}")
    dw = SD.build(w, hp=W.make_params(w, lengths=lengths))
    kv = dw.kv()
    dev = dw.k.device
    slots = kv.slots
    scores = torch.empty((w.n_seq, w.n_layer, w.n_kvh, slots), dtype=torch.float32, device=dev)
    kept = torch.empty((w.n_seq, w.n_layer, w.n_kvh, w.budget), dtype=torch.int32, device=dev)
    kept_n = torch.empty((w.n_seq,), dtype=torch.int32, device=dev)
    pos_out = torch.empty((w.n_seq, w.n_layer, w.n_kvh, w.budget), dtype=torch.int32, device=dev)
    new_len = torch.empty((w.n_seq,), dtype=torch.int32, device=dev)
    if paged:
        k_out = v_out = None
        freed = torch.empty((w.n_seq, w.max_pages), dtype=torch.int32, device=dev)
        n_freed = torch.empty((w.n_seq,), dtype=torch.int32, device=dev)
    else:
        k_out = torch.empty((w.n_seq, w.n_layer, w.n_kvh, w.budget, 128), dtype=dw.k.dtype, device=dev)
        v_out = torch.empty_like(k_out)
        freed = n_freed = None

    sel_ws = tri.select_workspace(scores, kv, w.budget, w.window, kept, kept_n)
    assert (sel_ws is not None) == (mode == "long")

    def one_pass(stream):
        if mode == "fused":
            tri.tri_score_select(kv, dw.center, dw.mean_abs, w.budget, w.window, rope_base=w.base,
                                 offsets=w.offsets, group=w.group, reduce=w.reduce, scores=scores, kept=kept,
                                 kept_n=kept_n, stream=stream)
        else:
            tri.tri_score_keys(kv, dw.center, dw.mean_abs, rope_base=w.base, offsets=w.offsets, group=w.group,
                               reduce=w.reduce, scores=scores, stream=stream)
            tri.tri_select_topb(scores, kv, w.budget, w.window, kept=kept, kept_n=kept_n, stream=stream,
                                workspace=sel_ws)
        tri.tri_compact_kv(kv, kept, kept_n, w.budget, k_out=k_out, v_out=v_out, pos_out=pos_out, freed=freed,
                           n_freed=n_freed, new_len=new_len, stream=stream)

    def snapshot():
        torch.cuda.synchronize()
        out = [scores.clone(), kept.clone(), kept_n.clone(), pos_out.clone(), new_len.clone()]
        if paged:
            out += [freed.clone(), n_freed.clone(), dw.k.clone(), dw.v.clone()]
        else:
            out += [k_out.clone(), v_out.clone()]
        return out

    def restore():
        if paged:   # in-place compaction rewrote the pools
            SD.fill(w, dw.hp, dw.k, dw.v, dw.seq_len, dw.block_table)
        torch.cuda.synchronize()

    restore()
    one_pass(torch.cuda.current_stream())
    ref = snapshot()
    restore()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            one_pass(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        restore()
        scores.fill_(-1.0)      # eager work between replays
        kept.fill_(-7)
        graph.replay()
        got = snapshot()
        for i, (a, b) in enumerate(zip(ref, got)):
            if i == 0:   # only slots < seq_len hold scores
                for s, L in enumerate(lengths):
                    assert torch.equal(a[s, ..., :L], b[s, ..., :L]), f"replay {rep}: scores differ"
            elif not paged and i >= 5:
                for s, L in enumerate(lengths):
                    n = min(L, w.budget)
                    assert torch.equal(a[s, :, :, :n].view(torch.int16), b[s, :, :, :n].view(torch.int16))
            elif paged and i == 5:
                for s in range(w.n_seq):
                    nf = int(ref[6][s])
                    assert torch.equal(a[s, :nf], b[s, :nf])
            elif i == 3:
                for s, L in enumerate(lengths):
                    n = min(L, w.budget)
                    assert torch.equal(a[s, :, :, :n], b[s, :, :, :n])
            else:
                assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else
                                   (a.view(torch.int16) if a.dtype == torch.bfloat16 else a),
                                   b.view(torch.int32) if b.dtype == torch.float32 else
                                   (b.view(torch.int16) if b.dtype == torch.bfloat16 else b)), \
                    f"replay {rep}: output {i} differs"


# ---------------------------------------------------------------------------------------
# calls enqueued on a non-default stream give the default stream's results
# ---------------------------------------------------------------------------------------

def test_side_stream_matches_default_stream():
    w = W.scaled(BASE, name="streams", n_seq=2, n_layer=2, n_kvh=2, max_len=2000, budget=300, window=32)
    dw = SD.build(w, hp=W.make_params(w, lengths=[2000, 1234]))
    log("same pass on the default stream and on a side stream")
    ref = run_pass(dw)
    side = torch.cuda.Stream()
    kv = dw.kv()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        sc = tri.tri_score_keys(kv, dw.center, dw.mean_abs, rope_base=w.base, offsets=w.offsets,
                                group=w.group, reduce=w.reduce, stream=side)
        kept, kept_n = tri.tri_select_topb(sc, kv, w.budget, w.window, stream=side)
        out = tri.tri_compact_kv(kv, kept, kept_n, w.budget, stream=side)
    side.synchronize()
    assert torch.equal(kept, ref[1]) and torch.equal(kept_n, ref[2])
    # only slots < seq_len hold scores and only rows < kept_n are written
    for s, L in enumerate([2000, 1234]):
        n = min(L, w.budget)
        assert torch.equal(sc[s, ..., :L].view(torch.int32), ref[0][s, ..., :L].view(torch.int32))
        for name in ("k_out", "v_out"):
            assert torch.equal(out[name][s, :, :, :n].view(torch.int16), ref[3][name][s, :, :, :n].view(torch.int16))
