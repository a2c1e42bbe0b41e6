"""The no-allocation attention entry point against the one that takes a workspace.

tri_decode_attention_noalloc keeps the partial softmax states of a split shape in the
library's static per-GPU scratch instead of a caller workspace.  Two calls in a row over the
same scratch, the second on a smaller input with another split count (and a third that is
not split at all), must each equal tri_decode_attention with a workspace bit for bit (the
same kernels and the same split), and agree with the oracle.  The split rule keeps the
partial states of every shape under the scratch (tests/test_abi.py checks the bound); a
larger need would be refused before any launch.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import kv_cache_compression_tri_amd as tri
from kv_cache_compression_tri_amd import _abi
from kv_cache_compression_tri_amd import synth
from kv_cache_compression_tri_amd.synth import device as SD
from kv_cache_compression_tri_amd.synth import workloads as W

pytestmark = pytest.mark.gpu

ATT_TOL = 2e-3     # |out_gpu - out_oracle| <= ATT_TOL * max_j |v_j| (per query head)


def log(msg):
    print(msg, flush=True)


def _case(name, n_layer, n_kvh, group, dtype, layout, max_len, lengths, seed):
    w = W.scaled(W.WORKLOADS["gqa8b_32k_bf16"], name=name, n_seq=len(lengths), n_layer=n_layer, n_kvh=n_kvh,
                 group=group, dtype=dtype, layout=layout, max_len=max_len)
    hp = W.make_params(w, lengths=lengths)
    dw = SD.build(w, hp=hp)
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((w.n_seq, w.n_layer, w.n_kvh * group, 128)).astype(np.float32)
    qpos = np.array([L + 3 for L in lengths], np.int64)
    return w, hp, dw, q, qpos


def _split_need(kv, q, qpos, w, layout, key_space):
    args, _out, _d = tri._attention_args(kv, q, qpos, w.base, w.group, None, 0, None, layout, key_space,
                                         torch.empty(q.shape, dtype=torch.float32, device="cuda"), False)
    need = ctypes.c_size_t(0)
    _abi.check(_abi.lib().tri_decode_attention(*args, None, ctypes.byref(need), None))
    return need.value


def _oracle_check(w, hp, q, qpos, out, lengths, layout, key_space):
    worst = 0.0
    g = w.group
    for s in range(w.n_seq):
        L = lengths[s]
        for l in range(w.n_layer):
            for h in range(w.n_kvh):
                unit = W.unit_index(w, s, l, h)
                k = oracle.decode_stored(synth.rows(w.seed, synth.TAG_K, unit, L, hp.mu_k[l, h], hp.sigma, w.sink,
                                                    w.dtype), w.dtype)
                v = oracle.decode_stored(synth.rows(w.seed, synth.TAG_V, unit, L, np.zeros(128, np.float32),
                                                    np.ones(128, np.float32), False, w.dtype), w.dtype)
                want = oracle.decode_attention(q[s, l, h * g:(h + 1) * g], k, v, base=w.base, key_pos=np.arange(L),
                                               query_pos=int(qpos[s]), layout=layout, key_space=key_space)
                scale = max(float(np.abs(v).max()), 1e-30) if L else 1.0
                err = float(np.abs(out[s, l, h * g:(h + 1) * g] - want).max()) / scale
                worst = max(worst, err)
    assert worst <= ATT_TOL, f"attention error {worst:.3e} of max |v|"
    return worst


def test_noalloc_equals_the_workspace_entry_point_on_consecutive_calls():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    cases = [
        # 4 unit passes of 4000 slots: split 16 ways
        dict(name="noalloc_a", n_layer=2, n_kvh=2, group=4, dtype="bf16", layout="half", key_space="pre",
             max_len=4000, lengths=[4000], seed=71),
        # smaller: 2 units, 2 passes each (G = 7), 700 slots (split 4 ways), float32 interleaved,
        # post-RoPE keys
        dict(name="noalloc_b", n_layer=1, n_kvh=2, group=7, dtype="f32", layout="interleaved", key_space="post",
             max_len=700, lengths=[700], seed=72),
        # not split at all (many short units): the scratch is not touched
        dict(name="noalloc_c", n_layer=16, n_kvh=20, group=2, dtype="bf16", layout="half", key_space="pre",
             max_len=96, lengths=[96], seed=73),
    ]
    runs = []
    for c in cases:
        w, hp, dw, q, qpos = _case(c["name"], c["n_layer"], c["n_kvh"], c["group"], c["dtype"], c["layout"],
                                   c["max_len"], c["lengths"], c["seed"])
        kv = dw.kv()
        qd, qp = torch.from_numpy(q).cuda(), torch.from_numpy(qpos).cuda()
        need = _split_need(kv, qd, qp, w, c["layout"], c["key_space"])
        log(f"no-alloc attention {c['name']}: {w.n_layer}x{w.n_kvh} units G={w.group} {w.dtype} {c['layout']} "
            f"{c['key_space']}-RoPE, {c['lengths'][0]} slots, split workspace {need} bytes")
        out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
        tri.tri_decode_attention_noalloc(kv, qd, qp, rope_base=w.base, group=w.group, out=out,
                                         rope_layout=c["layout"], key_space=c["key_space"])
        runs.append((c, w, hp, dw, kv, q, qpos, qd, qp, need, out))
    torch.cuda.synchronize()
    # the first two calls use the scratch, the second on a smaller input and a smaller part of it
    assert runs[0][9] > 0 and runs[1][9] > 0 and runs[2][9] == 0
    assert runs[1][9] < runs[0][9]
    assert runs[1][1].n_units * runs[1][1].max_len < runs[0][1].n_units * runs[0][1].max_len
    for c, w, hp, dw, kv, q, qpos, qd, qp, need, out in runs:
        ref = tri.tri_decode_attention(kv, qd, qp, rope_base=w.base, group=w.group, rope_layout=c["layout"],
                                       key_space=c["key_space"], workspace="auto")
        torch.cuda.synchronize()
        got, ref = out.cpu().numpy(), ref.cpu().numpy()
        assert np.array_equal(got, ref), f"{c['name']}: differs from tri_decode_attention with a workspace"
        err = _oracle_check(w, hp, q, qpos, got, c["lengths"], c["layout"], c["key_space"])
        log(f"  {c['name']}: equal to the workspace entry point; oracle error / max|v| = {err:.3e}")
