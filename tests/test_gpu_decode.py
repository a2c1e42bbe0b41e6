"""GPU parity of the steps either side of compaction: attention over the compressed cache
(RoPE at the kept keys' positions), scoring keys at explicit positions, and a decode loop on
a synthetic token stream.

The decode loop follows the pages' serving picture: prompts arrive in prefill chunks of at most
1024 tokens (a chunk can overshoot the budget before compression runs, so the budget is a soft
target), decoding appends one token per step, and every 128 decode steps the cache is
compressed and packed forward in its pages, whose emptied tail pages go back to the pool.
Oracle inputs are regenerated on the host from the generator's seed; the host tracks which
positions each unit still holds.
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

ATT_TOL = 2e-3     # |out_gpu - out_oracle| <= ATT_TOL * max_j |v_j| (per query head)


def log(msg):
    print(msg, flush=True)


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def check_attention(got, want, values):
    scale = max(float(np.abs(values).max()), 1e-30) if values.size else 1.0
    err = float(np.abs(got - want).max()) / scale
    assert np.all(np.isfinite(got)), "non-finite attention output"
    assert err <= ATT_TOL, f"attention error {err:.3e} of max |v| exceeds {ATT_TOL}"
    return err


def unit_rows(w, hp, s, l, h, n, tag=synth.TAG_K):
    unit = W.unit_index(w, s, l, h)
    if tag == synth.TAG_K:
        return synth.rows(w.seed, tag, unit, n, hp.mu_k[l, h], hp.sigma, w.sink, w.dtype)
    return synth.rows(w.seed, tag, unit, n, np.zeros(128, np.float32), np.ones(128, np.float32), False, w.dtype)


def as_float(bits, dtype):
    return oracle.decode_stored(bits, dtype)


# ---------------------------------------------------------------------------------------
# attention over a cache
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("workspace", ["auto", None])
@pytest.mark.parametrize("dtype,layout,key_space,group", [("bf16", "half", "pre", 4), ("f32", "interleaved", "pre", 7),
                                                          ("bf16", "interleaved", "post", 2),
                                                          ("f32", "half", "post", 8), ("bf16", "half", "pre", 1)])
def test_attention_dense(dtype, layout, key_space, group, workspace):
    # workspace "auto": the units split their 1300 slots over 8 workgroups each (splits past a
    # unit's length, and a unit with no keys, included); None: one workgroup per unit
    w = W.scaled(W.WORKLOADS["gqa8b_32k_bf16"], name="att", n_seq=3, n_layer=2, n_kvh=2, group=group, dtype=dtype,
                 layout=layout, max_len=1300)
    lengths = [1300, 517, 0]
    hp = W.make_params(w, lengths=lengths)
    log(f"attention dense {dtype} {layout} keys {key_space}-RoPE G={group} lengths={lengths} workspace={workspace}")
    dw = SD.build(w, hp=hp)
    rng = np.random.default_rng(61)
    n_qh = w.n_kvh * group
    q = rng.standard_normal((w.n_seq, w.n_layer, n_qh, 128)).astype(np.float32)
    qpos = np.array([1300 + 40, 517, 9], np.int64)
    out = tri.tri_decode_attention(dw.kv(), torch.from_numpy(q).cuda(), torch.from_numpy(qpos).cuda(),
                                   rope_base=w.base, group=group, rope_layout=layout, key_space=key_space,
                                   workspace=workspace)
    out = out.cpu().numpy()
    worst = 0.0
    for s in range(w.n_seq):
        L = lengths[s]
        for l in range(w.n_layer):
            for h in range(w.n_kvh):
                k = as_float(unit_rows(w, hp, s, l, h, L), dtype)
                v = as_float(unit_rows(w, hp, s, l, h, L, synth.TAG_V), dtype)
                want = oracle.decode_attention(q[s, l, h * group:(h + 1) * group], k, v, base=w.base,
                                               key_pos=np.arange(L), query_pos=int(qpos[s]), layout=layout,
                                               key_space=key_space)
                worst = max(worst, check_attention(out[s, l, h * group:(h + 1) * group], want, v))
    log(f"  max attention error / max|v| = {worst:.3e}")


@pytest.mark.parametrize("workspace", ["auto", None])
@pytest.mark.parametrize("dtype,layout,key_space,group", [("f32", "interleaved", "pre", 3),
                                                          ("bf16", "interleaved", "post", 8),
                                                          ("f32", "half", "post", 5), ("bf16", "half", "pre", 6)])
def test_attention_paged(dtype, layout, key_space, group, workspace):
    # a paged pool (pages at a random permutation of the pool), positions = slots; lengths
    # that end inside a page, one page, and no keys; with the workspace the units split their
    # slots (splits past a unit's length included), without it one workgroup per unit
    w = W.scaled(W.WORKLOADS["paged_ragged64_bf16"], name="att_paged", n_seq=4, n_layer=2, n_kvh=2, group=group,
                 dtype=dtype, layout=layout, max_len=1300, len_range=(1, 1300))
    lengths = [1300, 517, 0, 16]
    hp = W.make_params(w, lengths=lengths)
    log(f"attention paged {dtype} {layout} keys {key_space}-RoPE G={group} lengths={lengths} workspace={workspace}")
    dw = SD.build(w, hp=hp)
    kv = dw.kv()
    assert kv.layout == "paged"
    rng = np.random.default_rng(63)
    n_qh = w.n_kvh * group
    q = rng.standard_normal((w.n_seq, w.n_layer, n_qh, 128)).astype(np.float32)
    qpos = np.array([1300 + 7, 517 + 300, 5, 16], np.int64)
    out = tri.tri_decode_attention(kv, torch.from_numpy(q).cuda(), torch.from_numpy(qpos).cuda(),
                                   rope_base=w.base, group=group, rope_layout=layout, key_space=key_space,
                                   workspace=workspace)
    out = out.cpu().numpy()
    worst = 0.0
    for s in range(w.n_seq):
        L = lengths[s]
        for l in range(w.n_layer):
            for h in range(w.n_kvh):
                k = as_float(unit_rows(w, hp, s, l, h, L), dtype)
                v = as_float(unit_rows(w, hp, s, l, h, L, synth.TAG_V), dtype)
                want = oracle.decode_attention(q[s, l, h * group:(h + 1) * group], k, v, base=w.base,
                                               key_pos=np.arange(L), query_pos=int(qpos[s]), layout=layout,
                                               key_space=key_space)
                worst = max(worst, check_attention(out[s, l, h * group:(h + 1) * group], want, v))
    log(f"  max attention error / max|v| = {worst:.3e}")


@pytest.mark.parametrize("paged,group", [(False, 4), (True, 7)])
def test_noalloc_attention_under_graph_capture(paged, group):
    # the no-allocation entry point captured in a HIP graph (its intended caller); every replay,
    # after eager calls that reuse the static scratch with other queries, equals the eager call
    name = "paged_ragged64_bf16" if paged else "gqa8b_32k_bf16"
    extra = dict(len_range=(1, 3000)) if paged else {}
    w = W.scaled(W.WORKLOADS[name], name="att_graph", n_seq=2, n_layer=2, n_kvh=2, group=group, max_len=3000,
                 **extra)
    lengths = [3000, 1111]
    hp = W.make_params(w, lengths=lengths)
    log(f"no-allocation attention under graph capture, paged={paged} G={group} lengths={lengths}")
    dw = SD.build(w, hp=hp)
    kv = dw.kv()
    rng = np.random.default_rng(64)
    n_qh = w.n_kvh * group
    q = torch.from_numpy(rng.standard_normal((w.n_seq, w.n_layer, n_qh, 128)).astype(np.float32)).cuda()
    q_other = torch.from_numpy(rng.standard_normal((w.n_seq, w.n_layer, n_qh, 128)).astype(np.float32)).cuda()
    qpos = torch.tensor([3000 + 5, 1111], dtype=torch.int64, device="cuda")
    out = torch.empty_like(q)
    out_other = torch.empty_like(q)

    def call(stream, qq, oo):
        tri.tri_decode_attention_noalloc(kv, qq, qpos, rope_base=w.base, group=group, out=oo, stream=stream)

    call(None, q, out)
    torch.cuda.synchronize()
    ref = out.clone()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            call(side, q, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        call(None, q_other, out_other)     # eager work that rewrites the static scratch
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), f"replay {rep} differs from the eager call"
    # and the eager result itself against the oracle on one unit per sequence
    got = ref.cpu().numpy()
    for s, L in enumerate(lengths):
        k = as_float(unit_rows(w, hp, s, 1, 1, L), w.dtype)
        v = as_float(unit_rows(w, hp, s, 1, 1, L, synth.TAG_V), w.dtype)
        want = oracle.decode_attention(q.cpu().numpy()[s, 1, group:2 * group], k, v, base=w.base,
                                       key_pos=np.arange(L), query_pos=int(qpos[s]), layout=w.layout)
        check_attention(got[s, 1, group:2 * group], want, v)


@pytest.mark.parametrize("paged", [False, True])
def test_attention_over_a_layer_slice(paged):
    # one layer at a time (as a decode loop calls it) and a slice of two layers: queries and
    # outputs cover only the slice, keys, values and positions are read at the absolute layer;
    # explicit positions (not the slot index), with and without the split workspace, and the
    # no-allocation entry point
    name = "paged_ragged64_bf16" if paged else "gqa8b_32k_bf16"
    extra = dict(len_range=(1, 1500)) if paged else {}
    w = W.scaled(W.WORKLOADS[name], name="att_slice", n_seq=2, n_layer=3, n_kvh=2, group=4, max_len=1500, **extra)
    lengths = [1500, 611]
    hp = W.make_params(w, lengths=lengths)
    log(f"attention over layer slices, paged={paged} lengths={lengths}")
    dw = SD.build(w, hp=hp)
    kv0 = dw.kv()
    slots = kv0.slots
    rng = np.random.default_rng(65)
    # strictly increasing positions with gaps, as a compacted cache holds them
    pos_h = np.zeros((w.n_seq, w.n_layer, w.n_kvh, slots), np.int32)
    for s, L in enumerate(lengths):
        for l in range(w.n_layer):
            for h in range(w.n_kvh):
                pos_h[s, l, h, :L] = np.cumsum(rng.integers(1, 9, size=L))
    pos = torch.from_numpy(pos_h).cuda()
    kv = tri.KVCache.paged(dw.k, dw.v, dw.block_table, dw.seq_len, pos=pos) if paged else \
        tri.KVCache.dense(dw.k, dw.v, dw.seq_len, pos=pos)
    qpos = torch.from_numpy(np.array([int(pos_h[s, :, :, max(L - 1, 0)].max()) + 3 for s, L in enumerate(lengths)],
                                     np.int64)).cuda()
    n_qh = w.n_kvh * w.group
    for layer0, n_layers in ((2, 1), (0, 1), (1, 2)):
        q = rng.standard_normal((w.n_seq, n_layers, n_qh, 128)).astype(np.float32)
        qd = torch.from_numpy(q).cuda()
        outs = {ws: tri.tri_decode_attention(kv, qd, qpos, rope_base=w.base, group=w.group, pos=pos, layer0=layer0,
                                             n_layers=n_layers, workspace=ws).cpu().numpy() for ws in ("auto", None)}
        out_na = torch.empty_like(qd)
        tri.tri_decode_attention_noalloc(kv, qd, qpos, rope_base=w.base, group=w.group, pos=pos, layer0=layer0,
                                         n_layers=n_layers, out=out_na)
        assert np.array_equal(out_na.cpu().numpy(), outs["auto"])   # same kernels, same split
        worst = 0.0
        for s, L in enumerate(lengths):
            for lr in range(n_layers):
                l = layer0 + lr
                for h in range(w.n_kvh):
                    k = as_float(unit_rows(w, hp, s, l, h, L), w.dtype)
                    v = as_float(unit_rows(w, hp, s, l, h, L, synth.TAG_V), w.dtype)
                    want = oracle.decode_attention(q[s, lr, h * w.group:(h + 1) * w.group], k, v, base=w.base,
                                                   key_pos=pos_h[s, l, h, :L], query_pos=int(qpos[s]))
                    for ws, out in outs.items():
                        worst = max(worst, check_attention(out[s, lr, h * w.group:(h + 1) * w.group], want, v))
        log(f"  layers [{layer0}, {layer0 + n_layers}): max attention error / max|v| = {worst:.3e}")


def test_attention_over_a_compressed_cache():
    # compress a dense cache, then attend over k_out / v_out with the kept keys' positions
    w = W.scaled(W.WORKLOADS["gqa8b_32k_bf16"], name="att_comp", n_seq=2, n_layer=2, n_kvh=2, max_len=3000,
                 budget=640, window=64)
    lengths = [3000, 1900]
    hp = W.make_params(w, lengths=lengths)
    dw = SD.build(w, hp=hp)
    kv = dw.kv()
    res = tri.compress(kv, dw.center, dw.mean_abs, rope_base=w.base, offsets=w.offsets, group=w.group,
                       budget=w.budget, window=w.window)
    packed = tri.KVCache.dense(res["k_out"], res["v_out"], res["new_len"])
    rng = np.random.default_rng(62)
    q = rng.standard_normal((w.n_seq, w.n_layer, w.n_qh, 128)).astype(np.float32)
    qpos = np.array(lengths, np.int64)            # the next token
    out = tri.tri_decode_attention(packed, torch.from_numpy(q).cuda(), torch.from_numpy(qpos).cuda(),
                                   rope_base=w.base, group=w.group, pos=res["pos_out"]).cpu().numpy()
    # a caller-owned workspace (larger than needed), and no workspace: the same result to rounding
    ws = torch.empty((1 << 22,), dtype=torch.uint8, device="cuda")
    out_ws = tri.tri_decode_attention(packed, torch.from_numpy(q).cuda(), torch.from_numpy(qpos).cuda(),
                                      rope_base=w.base, group=w.group, pos=res["pos_out"], workspace=ws).cpu().numpy()
    out_one = tri.tri_decode_attention(packed, torch.from_numpy(q).cuda(), torch.from_numpy(qpos).cuda(),
                                       rope_base=w.base, group=w.group, pos=res["pos_out"],
                                       workspace=None).cpu().numpy()
    assert np.array_equal(out_ws, out)
    assert np.allclose(out_one, out, rtol=0, atol=1e-5 * float(np.abs(out).max()))
    kept = res["kept"].cpu().numpy()
    worst = 0.0
    for s in range(w.n_seq):
        n = min(lengths[s], w.budget)
        for l in range(w.n_layer):
            for h in range(w.n_kvh):
                kk = kept[s, l, h, :n]
                k = as_float(unit_rows(w, hp, s, l, h, lengths[s]), w.dtype)[kk]
                v = as_float(unit_rows(w, hp, s, l, h, lengths[s], synth.TAG_V), w.dtype)[kk]
                want = oracle.decode_attention(q[s, l, h * w.group:(h + 1) * w.group], k, v, base=w.base,
                                               key_pos=kk, query_pos=int(qpos[s]))
                worst = max(worst, check_attention(out[s, l, h * w.group:(h + 1) * w.group], want, v))
    log(f"attention over the compressed cache: max error / max|v| = {worst:.3e}")


# ---------------------------------------------------------------------------------------
# scoring keys at explicit positions
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,layout,group,reduce", [("bf16", "half", 4, "max"), ("f32", "interleaved", 3, "mean"),
                                                       ("fp8", "half", 7, "max"), ("int8", "interleaved", 1, "max")])
def test_scores_at_explicit_positions(dtype, layout, group, reduce):
    w = W.scaled(W.WORKLOADS["gqa8b_32k_bf16"], name="xpos", n_seq=2, n_layer=1, n_kvh=2, group=group,
                 reduce=reduce, dtype=dtype, layout=layout, max_len=1800, budget=300, window=16)
    lengths = [1800, 1011]
    hp = W.make_params(w, lengths=lengths)
    dw = SD.build(w, hp=hp)
    rng = np.random.default_rng(63)
    # sparse, ascending positions far beyond the slot index (a cache compacted before)
    pos = np.zeros((w.n_seq, w.n_layer, w.n_kvh, w.max_len), np.int32)
    for s in range(w.n_seq):
        for h in range(w.n_kvh):
            pos[s, 0, h] = np.sort(rng.choice(200000, w.max_len, replace=False))
    qpos = np.array([200500, 200017], np.int64)
    log(f"scores at explicit positions {dtype} {layout} G={group} {reduce}")
    kv = dw.kv()
    kv.pos = torch.from_numpy(pos).cuda()
    sc = tri.tri_score_keys(kv, dw.center, dw.mean_abs, rope_base=w.base, offsets=w.offsets, group=group,
                            reduce=reduce, rope_layout=layout, query_pos=torch.from_numpy(qpos).cuda())
    kept, _ = tri.tri_select_topb(sc, kv, w.budget, w.window)
    sc, kept = sc.cpu().numpy(), kept.cpu().numpy()
    for s in range(w.n_seq):
        L = lengths[s]
        for h in range(w.n_kvh):
            keys = P.host_rows(w, hp, s, 0, h)
            center, mean_abs = oracle.unit_heads(hp.center, hp.mean_abs, 0, h, group)
            orc = oracle.score_keys(keys, center, mean_abs, base=w.base, offsets=w.offsets, key_pos=pos[s, 0, h, :L],
                                    query_pos=int(qpos[s]), layout=layout, reduce=reduce)
            S = oracle.score_magnitude_bound(keys, center, mean_abs, layout=layout, reduce=reduce)
            P.check_scores(sc[s, 0, h, :L], orc, S)
            P.check_kept(kept[s, 0, h], sc[s, 0, h], orc, S, L, w.budget, w.window)


# ---------------------------------------------------------------------------------------
# decode loop on a synthetic token stream
# ---------------------------------------------------------------------------------------

PREFILL_CHUNK = 1024
TRIGGER = 128


class PagedStream:
    """A paged K/V pool fed token by token from the generator, with a host page allocator."""

    def __init__(self, w, hp, total_tokens, max_pages):
        self.w, self.hp = w, hp
        n_pool = w.n_seq * max_pages
        self.k = torch.zeros((n_pool, w.n_layer, w.n_kvh, 16, 128), dtype=torch.bfloat16, device="cuda")
        self.v = torch.zeros_like(self.k)
        self.free = list(range(n_pool))[::-1]
        self.bt = np.full((w.n_seq, max_pages), -1, np.int32)
        self.max_pages = max_pages
        self.length = np.zeros(w.n_seq, np.int64)          # cached keys per sequence
        self.next_pos = np.zeros(w.n_seq, np.int64)        # position of the next token
        self.pos = torch.zeros((w.n_seq, w.n_layer, w.n_kvh, max_pages * 16), dtype=torch.int32, device="cuda")
        self.held = {(s, l, h): np.zeros(0, np.int64) for s in range(w.n_seq) for l in range(w.n_layer)
                     for h in range(w.n_kvh)}                # host: positions held, in slot order
        # the stream's rows by absolute position, per unit
        self.kbits = {u: unit_rows(w, hp, *u, total_tokens) for u in self.held}
        self.vbits = {u: unit_rows(w, hp, *u, total_tokens, synth.TAG_V) for u in self.held}
        self.peak = 0

    def append(self, s, n):
        L, t0 = int(self.length[s]), int(self.next_pos[s])
        for pg in range(L // 16, -(-(L + n) // 16)):
            if self.bt[s, pg] < 0:
                self.bt[s, pg] = self.free.pop()
        slots = np.arange(L, L + n)
        pages = torch.from_numpy(self.bt[s, slots // 16].astype(np.int64)).cuda()
        rows = torch.from_numpy((slots % 16).astype(np.int64)).cuda()
        for (ss, l, h), held in self.held.items():
            if ss != s:
                continue
            kb = torch.from_numpy(self.kbits[(s, l, h)][t0:t0 + n].view(np.int16).copy()).cuda().view(torch.bfloat16)
            vb = torch.from_numpy(self.vbits[(s, l, h)][t0:t0 + n].view(np.int16).copy()).cuda().view(torch.bfloat16)
            self.k[pages, l, h, rows] = kb
            self.v[pages, l, h, rows] = vb
            self.held[(s, l, h)] = np.concatenate([held, np.arange(t0, t0 + n)])
        self.pos[s, :, :, L:L + n] = torch.arange(t0, t0 + n, dtype=torch.int32, device="cuda")
        self.length[s] += n
        self.next_pos[s] += n
        self.peak = max(self.peak, int(self.length.max()))

    def kv(self):
        return tri.KVCache.paged(self.k, self.v, torch.from_numpy(self.bt).cuda(),
                                 torch.from_numpy(self.length.astype(np.int32)).cuda(), pos=self.pos)

    def compress(self, dw, budget, window):
        w, hp = self.w, self.hp
        kv = self.kv()
        qpos = torch.from_numpy(self.next_pos - 1).cuda()     # the newest token's position
        res = tri.compress(kv, dw.center, dw.mean_abs, rope_base=w.base, offsets=w.offsets, group=w.group,
                           budget=budget, window=window, query_pos=qpos)
        torch.cuda.synchronize()
        sc, kept = res["scores"].cpu().numpy(), res["kept"].cpu().numpy()
        new_len = res["new_len"].cpu().numpy()
        n_freed, freed = res["n_freed"].cpu().numpy(), res["freed"].cpu().numpy()
        for (s, l, h), held in self.held.items():
            L = int(self.length[s])
            keys = as_float(self.kbits[(s, l, h)][held], w.dtype)
            center, mean_abs = oracle.unit_heads(hp.center, hp.mean_abs, l, h, w.group)
            orc = oracle.score_keys(keys, center, mean_abs, base=w.base, offsets=w.offsets, key_pos=held,
                                    query_pos=int(self.next_pos[s] - 1))
            S = oracle.score_magnitude_bound(keys, center, mean_abs)
            P.check_scores(sc[s, l, h, :L], orc, S)
            P.check_kept(kept[s, l, h], sc[s, l, h], orc, S, L, budget, window)
            n = min(L, budget)
            self.held[(s, l, h)] = held[kept[s, l, h, :n]]
        for s in range(w.n_seq):
            L, n = int(self.length[s]), int(new_len[s])
            assert n == min(L, budget)
            used_after, used_before = -(-n // 16), -(-L // 16)
            assert int(n_freed[s]) == used_before - used_after
            assert np.array_equal(freed[s, :n_freed[s]], self.bt[s, used_after:used_before])
            self.free.extend(int(x) for x in freed[s, :n_freed[s]])
            self.bt[s, used_after:used_before] = -1
            self.length[s] = n
        self.pos[..., :budget] = res["pos_out"]
        # the packed pages hold exactly the stream's rows of the kept positions
        k_now = self.k.view(torch.int16).cpu().numpy()
        for (s, l, h), held in self.held.items():
            n = len(held)
            slots = np.arange(n)
            got = k_now[self.bt[s, slots // 16], l, h, slots % 16]
            assert np.array_equal(got, self.kbits[(s, l, h)][held].view(np.int16)), "packed rows differ"
            assert np.array_equal(self.pos[s, l, h, :n].cpu().numpy(), held)


def test_decode_loop_on_a_synthetic_stream():
    budget, window = 512, 64
    prompts, decode_steps = [1500, 2300], 600
    total = max(prompts) + decode_steps + 1
    w = W.scaled(W.WORKLOADS["paged_ragged64_bf16"], name="stream", n_seq=2, n_layer=2, n_kvh=2, budget=budget,
                 window=window, max_len=total, len_range=(1, total))
    hp = W.make_params(w, lengths=[1, 1])
    dw = SD.build(w, hp=hp)                      # statistics only; the pool is fed below
    max_pages = -(-(budget + PREFILL_CHUNK + TRIGGER) // 16) + 2
    st = PagedStream(w, hp, total, max_pages)
    n_compress = 0
    # prefill in chunks; a chunk can overshoot the budget before compression runs
    for s, plen in enumerate(prompts):
        done = 0
        while done < plen:
            c = min(PREFILL_CHUNK, plen - done)
            st.append(s, c)
            done += c
            if st.length.max() > budget:
                st.compress(dw, budget, window)
                n_compress += 1
    log(f"prefill done: lengths {st.length.tolist()}, {n_compress} compressions")
    for step in range(1, decode_steps + 1):
        for s in range(w.n_seq):
            st.append(s, 1)
        if step % TRIGGER == 0 and st.length.max() > budget:
            st.compress(dw, budget, window)
            n_compress += 1
    log(f"decode done: lengths {st.length.tolist()}, {n_compress} compressions, peak {st.peak} keys, "
        f"{len(st.free)} free pages")
    assert st.peak <= budget + PREFILL_CHUNK + TRIGGER            # the soft budget
    assert len(st.free) + int(sum(-(-int(L) // 16) for L in st.length)) == st.k.shape[0]   # no page leaks
    # the consumer: attention of the newest token over the compressed paged cache
    rng = np.random.default_rng(64)
    q = rng.standard_normal((w.n_seq, w.n_layer, w.n_qh, 128)).astype(np.float32)
    qpos = st.next_pos - 1
    out = tri.tri_decode_attention(st.kv(), torch.from_numpy(q).cuda(), torch.from_numpy(qpos).cuda(),
                                   rope_base=w.base, group=w.group, pos=st.pos).cpu().numpy()
    worst = 0.0
    for (s, l, h), held in st.held.items():
        k = as_float(st.kbits[(s, l, h)][held], w.dtype)
        v = as_float(st.vbits[(s, l, h)][held], w.dtype)
        want = oracle.decode_attention(q[s, l, h * w.group:(h + 1) * w.group], k, v, base=w.base, key_pos=held,
                                       query_pos=int(qpos[s]))
        worst = max(worst, check_attention(out[s, l, h * w.group:(h + 1) * w.group], want, v))
    log(f"  attention over the compressed stream: max error / max|v| = {worst:.3e}")
