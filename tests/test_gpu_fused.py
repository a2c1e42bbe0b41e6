"""GPU parity of the fused scoring + selection entry point (tri_score_select).

Two checks, through the C ABI:
- exact: the kept slots of the fused launch equal those tri_select_topb picks from the
  scores the fused launch itself wrote (the same selection, once over LDS, once over memory);
- against the float64 oracle: those scores within the score tolerance and the kept set valid
  up to ties within it (parity.py), for every unit of the small dense and paged cases and
  sampled units of the full-size 32K (288 units), batch-16 (4608 units) and paged 64-sequence
  (18432 units) workloads.
"""

import numpy as np
import pytest
import torch

import kv_cache_compression_tri_amd as tri
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


def fused(dw, with_scores=True):
    w = dw.w
    kv = dw.kv()
    scores = None
    if with_scores:
        scores = torch.full((w.n_seq, w.n_layer, w.n_kvh, kv.slots), float("nan"), dtype=torch.float32,
                            device=dw.k.device)
    kept, kept_n = tri.tri_score_select(kv, dw.center, dw.mean_abs, w.budget, w.window, rope_base=w.base,
                                        offsets=w.offsets, group=w.group, reduce=w.reduce, rope_layout=w.layout,
                                        scores=scores)
    torch.cuda.synchronize()
    return kv, scores, kept, kept_n


def check_against_select(dw, kv, scores, kept, kept_n):
    """The fused selection equals the standalone one on the fused launch's own scores."""
    w = dw.w
    k2, n2 = tri.tri_select_topb(scores, kv, w.budget, w.window)
    torch.cuda.synchronize()
    assert torch.equal(kept, k2), "fused kept slots differ from tri_select_topb on the same scores"
    assert torch.equal(kept_n, n2)


def check_unit(dw, s, l, h, sc, kp, kn):
    w, hp = dw.w, dw.hp
    L = int(hp.lengths[s])
    keys = P.host_rows(w, hp, s, l, h)
    orc, S = P.oracle_scores(w, hp, s, l, h, keys)
    worst, _ = P.check_scores(sc[:L], orc, S)
    P.check_kept(kp, sc, orc, S, L, w.budget, w.window)
    assert kn == min(L, w.budget)
    return worst


BASE = W.WORKLOADS["gqa8b_32k_bf16"]
SMALL = {
    # max over 4 heads, ragged lengths around the 64-key groups and the per-wave shares
    "g4_max_half_bf16": (dict(n_seq=4, n_layer=2, n_kvh=2, group=4, max_len=3000, budget=500, window=64),
                         [3000, 1777, 513, 64]),
    # mean over the group (one effective head), interleaved pairs
    "g4_mean_interleaved_bf16": (dict(n_seq=2, n_layer=2, n_kvh=2, group=4, reduce="mean", layout="interleaved",
                                      max_len=2100, budget=333, window=32), [2100, 1000]),
    # float32 keys, G = 1; lengths at and below the budget, a single key, an empty sequence
    "g1_max_half_f32": (dict(n_seq=5, n_layer=1, n_kvh=2, group=1, dtype="f32", max_len=1200, budget=256,
                             window=16, base=1e4, offsets=W.geometric_offsets(10)), [1200, 256, 100, 1, 0]),
    # G = 8, window larger than the budget, low-concentration heads
    "g8_max_interleaved_bf16": (dict(n_seq=1, n_layer=2, n_kvh=2, group=8, layout="interleaved", max_len=1500,
                                     budget=200, window=300, low_r_frac=0.5), [1500]),
    # the largest unit the fused launch takes: 32768 slots, and one that is one 8-key step short
    "g2_max_half_bf16_max_len": (dict(n_seq=2, n_layer=1, n_kvh=1, group=2, max_len=32768, budget=2048,
                                      window=128), [32768, 32761]),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_fused_small(name):
    over, lengths = SMALL[name]
    w = W.scaled(BASE, name=name, **over)
    log(f"fused small {name}: {over} lengths={lengths}")
    dw = SD.build(w, hp=W.make_params(w, lengths=lengths))
    kv, scores, kept, kept_n = fused(dw)
    check_against_select(dw, kv, scores, kept, kept_n)
    sc, kp, kn = scores.cpu().numpy(), kept.cpu().numpy(), kept_n.cpu().numpy()
    worst = 0.0
    for s in range(w.n_seq):
        for l in range(w.n_layer):
            for h in range(w.n_kvh):
                worst = max(worst, check_unit(dw, s, l, h, sc[s, l, h], kp[s, l, h], kn[s]))
    # without a score buffer the kept slots are the same
    _, _, kept2, kept_n2 = fused(dw, with_scores=False)
    assert torch.equal(kept, kept2) and torch.equal(kept_n, kept_n2)
    log(f"  max score error / bound = {worst:.3e}")


@pytest.mark.parametrize("lengths,extra", [
    ([5000, 70, 1300, 1024], {}),                                            # bf16, max over 4 heads
    ([2222, 4000, 1, 513], dict(dtype="f32", layout="interleaved", group=2)),
    ([700, 4100, 1500, 33], dict(layout="interleaved", group=3, reduce="mean")),
    ([5120, 5105, 17, 4096], dict(group=8, window=0)),
])
def test_fused_small_paged(lengths, extra):
    w = W.scaled(W.WORKLOADS["paged_ragged64_bf16"], n_seq=4, n_layer=2, n_kvh=2, max_len=5120,
                 len_range=(16, 5120), **extra)
    log(f"fused small paged lengths={lengths} {extra}")
    dw = SD.build(w, hp=W.make_params(w, lengths=lengths))
    kv, scores, kept, kept_n = fused(dw)
    check_against_select(dw, kv, scores, kept, kept_n)
    sc, kp, kn = scores.cpu().numpy(), kept.cpu().numpy(), kept_n.cpu().numpy()
    for s in range(w.n_seq):
        for l in range(w.n_layer):
            for h in range(w.n_kvh):
                check_unit(dw, s, l, h, sc[s, l, h], kp[s, l, h], kn[s])


@pytest.mark.parametrize("name,units", [
    ("gqa8b_32k_bf16", [0, 1, 287, 150]),
    ("gqa8b_batch16_16k_bf16", [0, 4607, 2000]),
    ("paged_ragged64_bf16", [0, 18431, 9000]),
])
def test_fused_full_size(name, units):
    w = W.WORKLOADS[name]
    log(f"fused full size {name}")
    dw = SD.build(w)
    kv, scores, kept, kept_n = fused(dw)
    check_against_select(dw, kv, scores, kept, kept_n)
    worst = 0.0
    for u in units:
        s, l, h = W.unit_coords(w, u)
        log(f"  unit {u} (seq {s}, layer {l}, head {h})")
        worst = max(worst, check_unit(dw, s, l, h, scores[s, l, h].cpu().numpy(), kept[s, l, h].cpu().numpy(),
                                      int(kept_n[s].item())))
    log(f"  max score error / bound = {worst:.3e}")


def test_fused_explicit_query_positions():
    # the newest query ahead of the cache and behind it (query_pos given), max over 4 heads and
    # the mean over them
    import oracle
    for reduce in ("max", "mean"):
        w = W.scaled(BASE, name=f"fused_qpos_{reduce}", n_seq=3, n_layer=1, n_kvh=2, group=4, reduce=reduce,
                     max_len=1500, budget=256, window=16)
        lengths = [1500, 900, 1200]
        qpos = [1500 + 3000, 950, 700]
        hp = W.make_params(w, lengths=lengths)
        log(f"fused, explicit query positions {qpos} (lengths {lengths}), reduce {reduce}")
        dw = SD.build(w, hp=hp)
        kv = dw.kv()
        q = torch.tensor(qpos, dtype=torch.int64, device="cuda")
        scores = torch.full((w.n_seq, w.n_layer, w.n_kvh, kv.slots), float("nan"), device="cuda")
        kept, kept_n = tri.tri_score_select(kv, dw.center, dw.mean_abs, w.budget, w.window, rope_base=w.base,
                                            offsets=w.offsets, group=w.group, reduce=w.reduce, query_pos=q,
                                            scores=scores)
        torch.cuda.synchronize()
        check_against_select(dw, kv, scores, kept, kept_n)
        sc, kp = scores.cpu().numpy(), kept.cpu().numpy()
        for s in range(w.n_seq):
            L = lengths[s]
            for h in range(w.n_kvh):
                keys = P.host_rows(w, hp, s, 0, h)
                center, mean_abs = oracle.unit_heads(hp.center, hp.mean_abs, 0, h, w.group)
                orc = oracle.score_keys(keys, center, mean_abs, base=w.base, offsets=w.offsets, query_pos=qpos[s],
                                        layout=w.layout, reduce=w.reduce)
                S = oracle.score_magnitude_bound(keys, center, mean_abs, layout=w.layout, reduce=w.reduce)
                P.check_scores(sc[s, 0, h, :L], orc, S)
                P.check_kept(kp[s, 0, h], sc[s, 0, h], orc, S, L, w.budget, w.window)


def _fused_random_case(seed):
    rng = np.random.default_rng(2000 + seed)
    paged = bool(rng.integers(2))
    over = dict(name=f"fmix{seed}", n_seq=int(rng.integers(1, 4)), n_layer=int(rng.integers(1, 3)),
                n_kvh=int(rng.integers(1, 3)), group=int(rng.integers(1, 9)), dtype=["f32", "bf16"][rng.integers(2)],
                layout=["half", "interleaved"][rng.integers(2)], reduce=["max", "mean"][rng.integers(2)],
                max_len=int(rng.integers(300, 2600)), budget=int(16 * rng.integers(2, 40)),
                window=int(rng.integers(0, 200)), base=float([1e4, 5e5, 1e6][rng.integers(3)]),
                offsets=W.geometric_offsets(int(rng.integers(0, 15))), seed=int(80 + seed),
                low_r_frac=float(rng.uniform(0, 0.5)), sink=bool(rng.integers(2)))
    if paged:
        w = W.scaled(W.WORKLOADS["paged_ragged64_bf16"], len_range=(1, over["max_len"]), **over)
    else:
        w = W.scaled(BASE, **over)
    lengths = [int(x) for x in rng.integers(0, w.max_len + 1, w.n_seq)]
    lengths[int(rng.integers(w.n_seq))] = w.max_len
    return w, lengths


@pytest.mark.parametrize("seed", range(12))
def test_fused_random_option_mix(seed):
    w, lengths = _fused_random_case(seed)
    log(f"fused mix {seed}: {w.dtype} {'paged' if w.paged else 'dense'} {w.layout} G={w.group} {w.reduce} "
        f"B={w.budget} W={w.window} |D|={len(w.offsets)} base={w.base:g} lengths={lengths}")
    dw = SD.build(w, hp=W.make_params(w, lengths=lengths))
    kv, scores, kept, kept_n = fused(dw)
    check_against_select(dw, kv, scores, kept, kept_n)
    sc, kp, kn = scores.cpu().numpy(), kept.cpu().numpy(), kept_n.cpu().numpy()
    for s in range(w.n_seq):
        L = lengths[s]
        for l in range(w.n_layer):
            for h in range(w.n_kvh):
                keys = P.host_rows(w, dw.hp, s, l, h)
                orc, S = P.oracle_scores(w, dw.hp, s, l, h, keys)
                live = S > 0
                P.check_scores(sc[s, l, h, :L][live], orc[live], S[live])
                assert np.all(sc[s, l, h, :L][~live] == 0.0)
                P.check_kept(kp[s, l, h], sc[s, l, h], orc, S, L, w.budget, w.window)
                assert kn[s] == min(L, w.budget)
