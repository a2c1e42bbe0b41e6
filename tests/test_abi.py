"""C-ABI contract checks that need no GPU.

The library must load, export every function declared in include/tri.h, and reject bad
arguments before it makes any HIP call (the fake device pointers used here are never
dereferenced: every call below fails validation or is a workspace-size query).
"""

import ctypes
import os
import re
import subprocess

import pytest

from kv_cache_compression_tri_amd import _abi
from kv_cache_compression_tri_amd.synth import device as synth_device

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tri.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_abi.LIB_PATH), reason="libtri.so not built")

FAKE = ctypes.c_void_p(0x10000)


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(tri_\w+)\s*\(", text, flags=re.M))


def test_header_declares_the_binding_names():
    assert declared_functions() == set(_abi.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(_abi.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _abi.LIB_PATH], capture_output=True, text=True).stdout
    defined = {line.split()[-1] for line in out.splitlines() if line.strip()}
    assert declared_functions() <= defined


def test_version_matches_header():
    m = re.search(r"#define TRI_VERSION (\d+)", open(HEADER).read())
    assert _abi.lib().tri_version() == int(m.group(1))


def _kv(**over):
    d = _abi.TriKV()
    d.layout, d.dtype, d.n_seq, d.n_layer, d.n_kvh, d.head_dim = _abi.TRI_DENSE, _abi.TRI_BF16, 1, 2, 2, 128
    d.max_len = 4096
    d.seq_len = FAKE.value
    d.k = FAKE.value
    d.v = FAKE.value
    d.page, d.max_pages, d.block_table, d.pos = 16, 256, FAKE.value, None
    for k, v in over.items():
        setattr(d, k, v)
    return d


def _cfg(**over):
    offs = (ctypes.c_int32 * 3)(1, 2, 4)
    c = _abi.TriScoreCfg()
    c.rope_base, c.rope_layout, c.n_offsets, c.group, c.reduce = 1e6, 0, 3, 4, 0
    c.offsets = ctypes.cast(offs, ctypes.POINTER(ctypes.c_int32))
    for k, v in over.items():
        setattr(c, k, v)
    return c, offs


def _score(cfg=None, kv=None, center=FAKE, scores=FAKE, ws_query=False, mean_abs=FAKE):
    L = _abi.lib()
    size = ctypes.c_size_t(123)
    rc = L.tri_score_keys(None if cfg is None else ctypes.byref(cfg), center, mean_abs,
                          None if kv is None else ctypes.byref(kv), None, scores, None,
                          ctypes.byref(size) if ws_query else None, None)
    return rc, size.value


def test_score_keys_validation():
    c, _o = _cfg()
    assert _score(None, _kv())[0] == _abi.TRI_EINVAL
    assert _score(c, None)[0] == _abi.TRI_EINVAL
    assert _score(c, _kv(head_dim=64))[0] == _abi.TRI_ENOTSUP
    assert _score(c, _kv(head_dim=127))[0] == _abi.TRI_EINVAL
    assert _score(c, _kv(dtype=7))[0] == _abi.TRI_EINVAL
    assert _score(c, _kv(k_scale=FAKE.value))[0] == _abi.TRI_EINVAL          # scale needs 8-bit keys
    cm, _om = _cfg(form=_abi.TRI_SCORE_MULTIPLICATIVE)
    cbad, _ob = _cfg(form=2)
    assert _score(cbad, _kv())[0] == _abi.TRI_EINVAL
    assert _score(cm, _kv(), ws_query=True, mean_abs=None) == (_abi.TRI_OK, 0)    # not read by that form
    assert _score(c, _kv(), mean_abs=None)[0] == _abi.TRI_EINVAL
    assert _score(c, _kv(dtype=_abi.TRI_FP8_E4M3), ws_query=True) == (_abi.TRI_OK, 0)
    assert _score(c, _kv(dtype=_abi.TRI_FP8_E4M3, k_scale=FAKE.value), ws_query=True) == (_abi.TRI_OK, 0)
    assert _score(c, _kv(dtype=_abi.TRI_INT8, k_scale=FAKE.value), ws_query=True) == (_abi.TRI_OK, 0)
    assert _score(c, _kv(dtype=_abi.TRI_INT8 + 1))[0] == _abi.TRI_EINVAL
    assert _score(c, _kv(layout=5))[0] == _abi.TRI_EINVAL
    assert _score(c, _kv(n_layer=0))[0] == _abi.TRI_EINVAL
    assert _score(c, _kv(seq_len=None))[0] == _abi.TRI_EINVAL
    assert _score(c, _kv(k=None))[0] == _abi.TRI_EINVAL
    assert _score(c, _kv(max_len=0))[0] == _abi.TRI_EINVAL
    assert _score(c, _kv(max_len=(1 << 20) + 1))[0] == _abi.TRI_ENOTSUP
    assert _score(c, _kv(layout=_abi.TRI_PAGED, page=32))[0] == _abi.TRI_ENOTSUP
    assert _score(c, _kv(layout=_abi.TRI_PAGED, block_table=None))[0] == _abi.TRI_EINVAL
    assert _score(c, _kv(), center=None)[0] == _abi.TRI_EINVAL
    assert _score(c, _kv(), scores=None)[0] == _abi.TRI_EINVAL
    for over, code in [(dict(group=0), _abi.TRI_EINVAL), (dict(group=9), _abi.TRI_ENOTSUP),
                       (dict(n_offsets=0), _abi.TRI_EINVAL), (dict(rope_base=0.0), _abi.TRI_EINVAL),
                       (dict(rope_base=float("nan")), _abi.TRI_EINVAL), (dict(reduce=3), _abi.TRI_EINVAL),
                       (dict(rope_layout=2), _abi.TRI_EINVAL), (dict(key_space=2), _abi.TRI_EINVAL),
                       (dict(key_space=-1), _abi.TRI_EINVAL)]:
        cc, _k = _cfg(**over)
        assert _score(cc, _kv())[0] == code, over
    many = (ctypes.c_int32 * 65)(*range(65))
    cc, _k = _cfg(n_offsets=65, offsets=ctypes.cast(many, ctypes.POINTER(ctypes.c_int32)))
    assert _score(cc, _kv())[0] == _abi.TRI_ENOTSUP
    neg = (ctypes.c_int32 * 2)(1, -3)
    cc, _k = _cfg(n_offsets=2, offsets=ctypes.cast(neg, ctypes.POINTER(ctypes.c_int32)))
    assert _score(cc, _kv())[0] == _abi.TRI_EINVAL


def test_score_keys_position_contract():
    # tri.h, tri_kv.pos: scoring reads explicit key positions for pre-RoPE keys in the additive
    # form, refuses them (TRI_ENOTSUP) in the multiplicative form, and does not need them for
    # keys cached after RoPE (either form).  The workspace query validates without launching.
    pre_add, _a = _cfg()
    pre_mul, _b = _cfg(form=_abi.TRI_SCORE_MULTIPLICATIVE)
    post_add, _c = _cfg(key_space=_abi.TRI_KEYS_POST_ROPE)
    post_mul, _d = _cfg(key_space=_abi.TRI_KEYS_POST_ROPE, form=_abi.TRI_SCORE_MULTIPLICATIVE)
    with_pos = dict(pos=FAKE.value)
    assert _score(pre_add, _kv(**with_pos), ws_query=True) == (_abi.TRI_OK, 0)
    assert _score(pre_mul, _kv(**with_pos), ws_query=True)[0] == _abi.TRI_ENOTSUP
    assert _score(pre_mul, _kv(**with_pos))[0] == _abi.TRI_ENOTSUP
    assert "multiplicative" in _abi.lib().tri_last_error().decode()
    assert _score(post_add, _kv(**with_pos), ws_query=True) == (_abi.TRI_OK, 0)
    assert _score(post_mul, _kv(**with_pos), ws_query=True) == (_abi.TRI_OK, 0)
    for dt in (_abi.TRI_F32, _abi.TRI_FP8_E4M3, _abi.TRI_INT8):
        assert _score(pre_add, _kv(dtype=dt, **with_pos), ws_query=True) == (_abi.TRI_OK, 0)
        assert _score(pre_add, _kv(dtype=dt, layout=_abi.TRI_PAGED, **with_pos), ws_query=True) == (_abi.TRI_OK, 0)


def test_score_keys_workspace_query_launches_nothing():
    c, _o = _cfg()
    rc, size = _score(c, _kv(), ws_query=True)
    assert rc == _abi.TRI_OK and size == 0
    rc, size = _score(c, _kv(layout=_abi.TRI_PAGED), ws_query=True)
    assert rc == _abi.TRI_OK and size == 0


def test_last_error_text():
    c, _o = _cfg(group=9)
    assert _score(c, _kv())[0] == _abi.TRI_ENOTSUP
    assert b"group" in _abi.lib().tri_last_error()


def test_select_validation():
    L = _abi.lib()
    size = ctypes.c_size_t(7)

    def sel(kv=None, budget=16, window=4, kept=FAKE, ws=False):
        return L.tri_select_topb(FAKE, ctypes.byref(kv or _kv()), budget, window, kept, FAKE, None,
                                 ctypes.byref(size) if ws else None, None)
    assert sel(budget=0) == _abi.TRI_EINVAL
    assert sel(window=-1) == _abi.TRI_EINVAL
    assert sel(kept=None) == _abi.TRI_EINVAL
    assert sel(kv=_kv(head_dim=96)) == _abi.TRI_ENOTSUP
    assert sel(ws=True) == _abi.TRI_OK and size.value == 0


def test_compact_validation():
    L = _abi.lib()

    def comp(kv, k_out=FAKE, v_out=FAKE, freed=None, n_freed=None, budget=8):
        return L.tri_compact_kv(ctypes.byref(kv), FAKE, FAKE, budget, k_out, v_out, None, freed, n_freed,
                                None, None)
    assert comp(_kv(), k_out=None) == _abi.TRI_EINVAL
    assert comp(_kv(), v_out=None) == _abi.TRI_EINVAL
    assert comp(_kv(v=None)) == _abi.TRI_EINVAL
    assert comp(_kv(), freed=FAKE, n_freed=FAKE) == _abi.TRI_EINVAL
    assert comp(_kv(), budget=0) == _abi.TRI_EINVAL
    paged = _kv(layout=_abi.TRI_PAGED)
    assert comp(paged) == _abi.TRI_ENOTSUP
    assert comp(paged, k_out=None, v_out=None, freed=FAKE) == _abi.TRI_EINVAL
    assert L.tri_compact_kv(ctypes.byref(paged), None, FAKE, 8, None, None, None, None, None, None,
                            None) == _abi.TRI_EINVAL
    # the dense grid is units x ceil(budget / rows per workgroup) workgroups: 2^20 units with a
    # budget of 2^20 slots exceed 2^31 - 1 and are refused before any launch
    assert comp(_kv(n_layer=1 << 12, n_kvh=1 << 8), budget=1 << 20) == _abi.TRI_ENOTSUP
    assert b"grid" in L.tri_last_error()


def test_calibrate_validation():
    L = _abi.lib()
    size = ctypes.c_size_t(5)

    def cal(n=10, dtype=0, head_dim=128, layout=0, q=FAKE, ws=False):
        return L.tri_calibrate_stats(q, dtype, n, 2, 4, head_dim, layout, FAKE, FAKE, None,
                                     ctypes.byref(size) if ws else None, None)
    assert cal(n=0) == _abi.TRI_EINVAL
    assert cal(dtype=4) == _abi.TRI_EINVAL
    assert cal(dtype=_abi.TRI_FP8_E4M3) == _abi.TRI_ENOTSUP                 # queries are f32 / bf16
    assert cal(dtype=_abi.TRI_INT8) == _abi.TRI_ENOTSUP
    assert cal(layout=9) == _abi.TRI_EINVAL
    assert cal(head_dim=96) == _abi.TRI_ENOTSUP
    assert cal(q=None) == _abi.TRI_EINVAL
    assert cal(ws=True) == _abi.TRI_OK and size.value == 0


def test_synth_library_exports_and_rejects_bad_arguments():
    L = synth_device.lib()
    for name in synth_device.SYNTH_EXPORTS:
        assert hasattr(L, name)
    assert L.tri_synth_fill_dense(None, 1, 1, 16, 1, FAKE, FAKE, 0, 0, 0, None, None) == -1
    assert L.tri_synth_fill_dense(FAKE, 1, 1, (1 << 20) + 1, 1, FAKE, FAKE, 0, 0, 0, None, None) == -1
    assert L.tri_synth_fill_dense(FAKE, 4, 1, 16, 1, FAKE, FAKE, 0, 0, 0, None, None) == -1    # dtype
    assert L.tri_synth_fill_paged(FAKE, 1, 1, 1, 1, 16, 0, FAKE, FAKE, FAKE, FAKE, 0, 0, 0, None, None) == -1


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(_abi, "_LIB", None)
    with pytest.raises(RuntimeError, match="missing"):
        _abi.lib(os.path.join(ROOT, "no_such_dir", "libtri.so"))


def test_header_is_c99_and_struct_layouts_match_the_binding(tmp_path):
    """include/tri.h compiles as strict C99, a C program links against libtri.so and calls it,
    and the struct layouts the C compiler sees are the ones the ctypes binding uses."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = tmp_path / "abi_check.c"
    src.write_text(r'''
#include <stddef.h>
#include <stdio.h>
#include "tri.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu\n", sizeof(tri_kv), offsetof(tri_kv, max_len), offsetof(tri_kv, block_table),
         offsetof(tri_kv, pos), offsetof(tri_kv, k_scale), sizeof(tri_score_cfg));
  printf("%zu %zu %zu %zu\n", offsetof(tri_score_cfg, offsets), offsetof(tri_score_cfg, group),
         offsetof(tri_score_cfg, key_space), offsetof(tri_score_cfg, form));
  printf("%d %d %d\n", tri_version(), tri_score_keys(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL),
         TRI_VERSION);
  printf("%d %d\n", tri_score_select(NULL, NULL, NULL, NULL, NULL, 1, 0, NULL, NULL, NULL, NULL, NULL, NULL),
         tri_select_topb(NULL, NULL, 1, 0, NULL, NULL, NULL, NULL, NULL));
  return 0;
}
''')
    lib_dir = os.path.dirname(_abi.LIB_PATH)
    exe = tmp_path / "abi_check"
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", f"-I{os.path.join(ROOT, 'include')}",
           str(src), "-o", str(exe), f"-L{lib_dir}", "-ltri", f"-Wl,-rpath,{lib_dir}",
           "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    lines = [list(map(int, ln.split())) for ln in out.stdout.strip().splitlines()]
    K, C = _abi.TriKV, _abi.TriScoreCfg
    assert lines[0] == [ctypes.sizeof(K), K.max_len.offset, K.block_table.offset, K.pos.offset, K.k_scale.offset,
                        ctypes.sizeof(C)]
    assert lines[1] == [C.offsets.offset, C.group.offset, C.key_space.offset, C.form.offset]
    assert lines[2][0] == lines[2][2] and lines[2][1] == _abi.TRI_EINVAL
    assert lines[3] == [_abi.TRI_EINVAL, _abi.TRI_EINVAL]


def test_decode_attention_validation():
    L = _abi.lib()
    out = FAKE

    def att(kv=None, layer0=0, n_layers=2, q=FAKE, qpos=FAKE, pos=None, stride=0, base=1e6, layout=0, ks=0,
            group=4):
        kv = _kv() if kv is None else kv
        return L.tri_decode_attention(ctypes.byref(kv), layer0, n_layers, q, qpos, pos, stride, base, layout, ks,
                                      group, out, None, None, None)
    assert att(q=None) == _abi.TRI_EINVAL
    assert att(qpos=None) == _abi.TRI_EINVAL
    assert att(kv=_kv(v=None)) == _abi.TRI_EINVAL
    assert att(kv=_kv(dtype=_abi.TRI_FP8_E4M3)) == _abi.TRI_ENOTSUP
    assert att(layer0=1, n_layers=2) == _abi.TRI_EINVAL
    assert att(n_layers=0) == _abi.TRI_EINVAL
    assert att(group=9) == _abi.TRI_ENOTSUP
    assert att(group=0) == _abi.TRI_EINVAL
    assert att(base=0.0) == _abi.TRI_EINVAL
    assert att(layout=2) == _abi.TRI_EINVAL
    assert att(ks=5) == _abi.TRI_EINVAL
    assert att(pos=FAKE, stride=100) == _abi.TRI_EINVAL        # stride below the 4096 slots
    assert "pos_stride" in L.tri_last_error().decode()


def test_decode_attention_workspace():
    """The optional workspace: size query, too small, misaligned; no launch in any case."""
    L = _abi.lib()

    def att(kv, group, ws, nbytes):
        return L.tri_decode_attention(ctypes.byref(kv), 0, kv.n_layer, FAKE, FAKE, None, 0, 1e6, 0, 0, group,
                                      FAKE, ws, nbytes, None)
    # 1 x 2 x 2 units, 4096 slots: 4 (sequence, layer, head) groups of <= 4 query heads are far
    # from 4 workgroups per CU at any split count, so they take the most splits (16); per split
    # and head 2 floats of (max, sum), padded to 256 bytes, and 128 floats of value sums
    n = ctypes.c_size_t(0)
    assert att(_kv(), 4, None, ctypes.byref(n)) == _abi.TRI_OK
    assert n.value == 4 * 16 * 4 * 2 * 4 + 4 * 16 * 4 * 128 * 4
    assert att(_kv(), 8, None, ctypes.byref(n)) == _abi.TRI_OK      # 8 heads: two passes
    assert n.value == 8 * 16 * 4 * 2 * 4 + 8 * 16 * 4 * 128 * 4
    assert att(_kv(max_len=512), 4, None, ctypes.byref(n)) == _abi.TRI_OK   # 512 slots: 4 splits of 128
    assert n.value == 4 * 4 * 4 * 2 * 4 + 4 * 4 * 4 * 128 * 4
    assert att(_kv(n_seq=128), 4, None, ctypes.byref(n)) == _abi.TRI_OK    # 512 groups: 2 splits (1024)
    assert n.value == 512 * 2 * 4 * 2 * 4 + 512 * 2 * 4 * 128 * 4
    assert att(_kv(n_seq=256), 4, None, ctypes.byref(n)) == _abi.TRI_OK    # 1024 groups: not split
    assert n.value == 0
    small = ctypes.c_size_t(1000)
    assert att(_kv(), 4, FAKE, ctypes.byref(small)) == _abi.TRI_EWORKSPACE
    big = ctypes.c_size_t(1 << 20)
    assert att(_kv(), 4, ctypes.c_void_p(FAKE.value + 8), ctypes.byref(big)) == _abi.TRI_EINVAL
    assert "aligned" in L.tri_last_error().decode()


def test_decode_attention_noalloc_validation():
    # the no-allocation attention validates like tri_decode_attention (no launch in any case)
    L = _abi.lib()

    def att(kv=None, group=4, n_layers=2, base=1e6, ks=0):
        kv = kv or _kv()
        return L.tri_decode_attention_noalloc(ctypes.byref(kv), 0, n_layers, FAKE, FAKE, None, 0, base, 0, ks,
                                              group, FAKE, None)
    assert att(kv=_kv(dtype=_abi.TRI_FP8_E4M3)) == _abi.TRI_ENOTSUP
    assert att(group=9) == _abi.TRI_ENOTSUP
    assert att(group=0) == _abi.TRI_EINVAL
    assert att(n_layers=3) == _abi.TRI_EINVAL
    assert att(base=0.0) == _abi.TRI_EINVAL
    assert att(ks=2) == _abi.TRI_EINVAL
    assert att(kv=_kv(v=None)) == _abi.TRI_EINVAL
    # The split rule stops at 4 workgroups per CU (1024 groups), so the partial states of any
    # shape stay under 2048 groups x 4 heads x 520 bytes and always fit the 8 MiB static
    # scratch (the refusal is a guard): sweep the group count over the range where the largest
    # states occur, for one and two passes, through the workspace query (no launch).
    need = ctypes.c_size_t(0)
    worst = 0
    for group in (4, 8):
        for n_layer in range(1, 1101):
            kv = _kv(n_layer=n_layer, n_kvh=1, max_len=1 << 16)
            assert L.tri_decode_attention(ctypes.byref(kv), 0, n_layer, FAKE, FAKE, None, 0, 1e6, 0, 0, group,
                                          FAKE, None, ctypes.byref(need), None) == _abi.TRI_OK
            worst = max(worst, need.value)
    assert 4_000_000 < worst <= 2048 * 4 * 520 + 256 < 8 << 20


def test_score_select_validation():
    # tri.h, tri_score_select: dense or paged float32 / bfloat16 caches of pre-RoPE keys at their
    # slots, additive form, at most 32768 slots; everything else is refused before any launch.  The
    # workspace query validates without launching and needs 0 bytes.
    L = _abi.lib()

    def call(cfg_over=None, kv=None, budget=64, window=8, kept=FAKE, mean_abs=FAKE, scores=None, query=True):
        cfg, _offs = _cfg(**(cfg_over or {}))
        kv = kv or _kv()
        size = ctypes.c_size_t(123)
        rc = L.tri_score_select(ctypes.byref(cfg), FAKE, mean_abs, ctypes.byref(kv), None, budget, window, scores,
                                kept, FAKE, None, ctypes.byref(size) if query else None, None)
        return rc, size.value

    assert call() == (_abi.TRI_OK, 0)
    assert call(kv=_kv(dtype=_abi.TRI_F32)) == (_abi.TRI_OK, 0)
    assert call(scores=FAKE) == (_abi.TRI_OK, 0)
    assert call(kv=_kv(max_len=32768)) == (_abi.TRI_OK, 0)
    assert call(kv=_kv(max_len=32769))[0] == _abi.TRI_ENOTSUP
    assert "32768" in L.tri_last_error().decode()
    assert call(kv=_kv(layout=_abi.TRI_PAGED)) == (_abi.TRI_OK, 0)
    assert call(kv=_kv(layout=_abi.TRI_PAGED, max_pages=2048)) == (_abi.TRI_OK, 0)
    assert call(kv=_kv(layout=_abi.TRI_PAGED, max_pages=2049))[0] == _abi.TRI_ENOTSUP
    for dt in (_abi.TRI_FP8_E4M3, _abi.TRI_INT8):
        assert call(kv=_kv(dtype=dt))[0] == _abi.TRI_ENOTSUP
    assert call(cfg_over=dict(key_space=_abi.TRI_KEYS_POST_ROPE))[0] == _abi.TRI_ENOTSUP
    assert call(cfg_over=dict(form=_abi.TRI_SCORE_MULTIPLICATIVE))[0] == _abi.TRI_ENOTSUP
    assert call(kv=_kv(pos=FAKE.value))[0] == _abi.TRI_ENOTSUP
    assert call(cfg_over=dict(group=9))[0] == _abi.TRI_ENOTSUP
    assert call(budget=0)[0] == _abi.TRI_EINVAL
    assert call(window=-1)[0] == _abi.TRI_EINVAL
    assert call(kept=None)[0] == _abi.TRI_EINVAL
    assert call(mean_abs=None)[0] == _abi.TRI_EINVAL
    assert call(query=False, kv=_kv(dtype=_abi.TRI_INT8))[0] == _abi.TRI_ENOTSUP


def test_select_workspace_query():
    # tri.h, tri_select_topb: the optional workspace lets units of more than 32768 slots be
    # selected in two stages; its size is units x runs x (budget - min(window, budget)) x 8
    # bytes while runs x that <= 32768, else 0 (and 0 for shorter units).
    L = _abi.lib()

    def need(kv, budget, window):
        size = ctypes.c_size_t(123)
        rc = L.tri_select_topb(FAKE, ctypes.byref(kv), budget, window, FAKE, FAKE, None, ctypes.byref(size), None)
        assert rc == _abi.TRI_OK
        return size.value

    units = 1 * 2 * 2
    assert need(_kv(max_len=4096), 2048, 128) == 0
    assert need(_kv(max_len=32768), 2048, 128) == 0
    assert need(_kv(max_len=131072), 4096, 256) == units * 4 * 3840 * 8
    assert need(_kv(max_len=32769), 2048, 128) == units * 2 * 1920 * 8
    assert need(_kv(max_len=131072), 8200, 8) == units * 4 * 8192 * 8
    assert need(_kv(max_len=131072), 8201, 8) == 0                  # 4 runs x 8193 > 32768
    assert need(_kv(max_len=131072), 2048, 2048) == 0               # the window is the budget
    assert need(_kv(layout=_abi.TRI_PAGED, max_pages=4096), 1024, 128) == units * 2 * 896 * 8
    # a workspace smaller than needed is refused
    size = ctypes.c_size_t(100)
    assert L.tri_select_topb(FAKE, ctypes.byref(_kv(max_len=131072)), 4096, 256, FAKE, FAKE, FAKE,
                             ctypes.byref(size), None) == _abi.TRI_EWORKSPACE
