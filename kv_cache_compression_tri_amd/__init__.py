"""TriAttention KV-cache compression pass for AMD Instinct MI355X (gfx950).

Thin Python binding of libtri.so with the same entry-point names as include/tri.h.  It only
marshals arguments (torch tensors -> device pointers, the current HIP stream, output
allocation); every step of the pass runs in the library's HIP kernels.  If the library is
not built, every call raises.

    kv = KVCache.dense(k, v, seq_len)                       # or KVCache.paged(...)
    scores = tri_score_keys(kv, center, mean_abs, rope_base=1e6, offsets=[1, 2, 4], group=4)
    kept, kept_n = tri_select_topb(scores, kv, budget=2048, window=128)
    out = tri_compact_kv(kv, kept, kept_n, budget=2048)
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional, Sequence

from . import _abi
from ._abi import TriError  # noqa: F401

__all__ = [
    "KVCache",
    "TriError",
    "tri_calibrate_stats",
    "save_stats",
    "load_stats",
    "tri_score_keys",
    "tri_select_topb",
    "select_workspace",
    "tri_score_select",
    "tri_compact_kv",
    "tri_decode_attention",
    "tri_decode_attention_noalloc",
    "tri_version",
    "compress",
]

_LAYOUTS = {"half": _abi.TRI_ROPE_HALF, "interleaved": _abi.TRI_ROPE_INTERLEAVED}
_REDUCE = {"max": _abi.TRI_REDUCE_MAX, "mean": _abi.TRI_REDUCE_MEAN}


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return _abi.TRI_BF16
    if t.dtype == torch.float32:
        return _abi.TRI_F32
    if t.dtype == torch.float8_e4m3fn:
        return _abi.TRI_FP8_E4M3
    if t.dtype == torch.int8:
        return _abi.TRI_INT8
    raise TypeError(f"unsupported dtype {t.dtype} (float32, bfloat16, float8_e4m3fn or int8)")


def _dev(t, name, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _shape(t, name, shape):
    """Require an exact shape: the kernels index these buffers with the descriptor's sizes."""
    if t is not None and tuple(int(x) for x in t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


@dataclass
class KVCache:
    """A pre-RoPE KV cache in device memory (see tri_kv in include/tri.h).

    dense: k, v [n_seq, n_layer, n_kvh, max_len, head_dim]
    paged: k, v pools [n_pages, n_layer, n_kvh, page, head_dim] with block_table
           [n_seq, max_pages] (int32) mapping slot j of sequence s to page
           block_table[s, j // page], row j % page
    seq_len: int32 [n_seq] on the device; pos: optional int32 RoPE positions
    k_scale: 8-bit caches only (torch.float8_e4m3fn = OCP E4M3, or torch.int8), optional
             float32 [n_layer, n_kvh]: key = decoded code * k_scale[l, h]
    """

    k: object
    v: object
    seq_len: object
    layout: str = "dense"
    block_table: object = None
    pos: object = None
    k_scale: object = None

    @classmethod
    def dense(cls, k, v, seq_len, pos=None, k_scale=None):
        return cls(k, v, seq_len, "dense", None, pos, k_scale)

    @classmethod
    def paged(cls, k_pool, v_pool, block_table, seq_len, pos=None, k_scale=None):
        return cls(k_pool, v_pool, seq_len, "paged", block_table, pos, k_scale)

    @property
    def n_seq(self) -> int:
        return int(self.seq_len.shape[0])

    @property
    def slots(self) -> int:
        if self.layout == "dense":
            return int(self.k.shape[3])
        return int(self.block_table.shape[1]) * int(self.k.shape[3])

    def descriptor(self) -> _abi.TriKV:
        torch = _torch()
        _dev(self.k, "k")
        _dev(self.v, "v")
        _dev(self.seq_len, "seq_len", torch.int32)
        _dev(self.pos, "pos", torch.int32)
        if self.v is not None and (self.v.shape != self.k.shape or self.v.dtype != self.k.dtype):
            raise ValueError("v must match k in shape and dtype")
        d = _abi.TriKV()
        d.dtype = _dtype_code(self.k)
        d.head_dim = int(self.k.shape[-1])
        d.n_layer = int(self.k.shape[1])
        d.n_kvh = int(self.k.shape[2])
        d.n_seq = self.n_seq
        d.seq_len = self.seq_len.data_ptr()
        d.k = self.k.data_ptr()
        d.v = None if self.v is None else self.v.data_ptr()
        d.pos = None if self.pos is None else self.pos.data_ptr()
        if self.k_scale is not None:
            if d.dtype not in (_abi.TRI_FP8_E4M3, _abi.TRI_INT8):
                raise ValueError("k_scale is only valid with 8-bit (float8_e4m3fn or int8) keys")
            _dev(self.k_scale, "k_scale", torch.float32)
            _shape(self.k_scale, "k_scale", (d.n_layer, d.n_kvh))
            d.k_scale = self.k_scale.data_ptr()
        if self.layout == "dense":
            if self.k.dim() != 5 or int(self.k.shape[0]) != self.n_seq:
                raise ValueError("dense k must be [n_seq, n_layer, n_kvh, max_len, head_dim]")
            d.layout = _abi.TRI_DENSE
            d.max_len = int(self.k.shape[3])
        elif self.layout == "paged":
            _dev(self.block_table, "block_table", torch.int32)
            if self.k.dim() != 5 or self.block_table.dim() != 2 or int(self.block_table.shape[0]) != self.n_seq:
                raise ValueError("paged k must be [n_pages, n_layer, n_kvh, page, head_dim] with "
                                 "block_table [n_seq, max_pages]")
            d.layout = _abi.TRI_PAGED
            d.page = int(self.k.shape[3])
            d.max_pages = int(self.block_table.shape[1])
            d.block_table = self.block_table.data_ptr()
        else:
            raise ValueError(f"unknown layout {self.layout!r}")
        if self.pos is not None and self.pos.numel() != self.n_seq * d.n_layer * d.n_kvh * self.slots:
            raise ValueError("pos must be [n_seq, n_layer, n_kvh, slots]")
        return d


def tri_version() -> int:
    return _abi.lib().tri_version()


def tri_calibrate_stats(q, rope_layout: str = "half", center=None, mean_abs=None, stream=None):
    """Query statistics from pre-RoPE samples q [n, n_layer, n_qh, head_dim].

    Returns (center [n_layer, n_qh, F, 2] float32, mean_abs [n_layer, n_qh, F] float32).
    """
    torch = _torch()
    L = _abi.lib()
    _dev(q, "q")
    if q.dim() != 4:
        raise ValueError("q must be [n, n_layer, n_qh, head_dim]")
    n, n_layer, n_qh, d = (int(x) for x in q.shape)
    if center is None:
        center = torch.empty((n_layer, n_qh, d // 2, 2), dtype=torch.float32, device=q.device)
    if mean_abs is None:
        mean_abs = torch.empty((n_layer, n_qh, d // 2), dtype=torch.float32, device=q.device)
    _dev(center, "center", torch.float32)
    _dev(mean_abs, "mean_abs", torch.float32)
    _shape(center, "center", (n_layer, n_qh, d // 2, 2))
    _shape(mean_abs, "mean_abs", (n_layer, n_qh, d // 2))
    _abi.check(L.tri_calibrate_stats(_ptr(q), _dtype_code(q), n, n_layer, n_qh, d, _LAYOUTS[rope_layout],
                                     _ptr(center), _ptr(mean_abs), None, None, _stream(stream)))
    return center, mean_abs


def save_stats(path, center, mean_abs, *, rope_base: float, rope_layout: str = "half"):
    """Write calibration statistics to an .npz file (arrays and their RoPE settings only; the
    statistics belong to one model and its RoPE base and pair layout: "TriAttention:
    trigonometric KV cache compression for long reasoning", section "Calibration statistics are
    tied to a specific model")."""
    import numpy as np
    if rope_layout not in _LAYOUTS:
        raise ValueError(f"unknown rope layout {rope_layout!r}")
    c = center.detach().float().cpu().numpy()
    m = mean_abs.detach().float().cpu().numpy()
    if c.ndim != 4 or c.shape[-1] != 2 or m.shape != c.shape[:3]:
        raise ValueError("center must be [n_layer, n_qh, F, 2] and mean_abs [n_layer, n_qh, F]")
    np.savez(path, center=c, mean_abs=m, rope_base=np.float64(rope_base), head_dim=np.int64(2 * c.shape[2]),
             rope_layout=np.str_(rope_layout))


def load_stats(path, *, device="cuda", rope_base=None, rope_layout=None, n_layer=None, n_qh=None):
    """Read statistics written by save_stats: (center, mean_abs, rope_base, rope_layout), the
    arrays as float32 tensors on `device`.  Any of rope_base, rope_layout, n_layer, n_qh given
    must match the file (ValueError otherwise): statistics of another model or RoPE setting
    would pick the wrong keys without any other error."""
    import numpy as np
    torch = _torch()
    with np.load(path, allow_pickle=False) as f:
        c, m = f["center"], f["mean_abs"]
        base, layout, hd = float(f["rope_base"]), str(f["rope_layout"]), int(f["head_dim"])
    if c.ndim != 4 or c.shape[-1] != 2 or m.shape != c.shape[:3] or hd != 2 * c.shape[2]:
        raise ValueError(f"{path}: malformed statistics (center {c.shape}, mean_abs {m.shape}, head_dim {hd})")
    for name, want, got in (("rope_base", rope_base, base), ("rope_layout", rope_layout, layout),
                            ("n_layer", n_layer, c.shape[0]), ("n_qh", n_qh, c.shape[1])):
        if want is not None and want != got:
            raise ValueError(f"{path}: statistics have {name} {got!r}, expected {want!r}")
    return (torch.from_numpy(np.ascontiguousarray(c, np.float32)).to(device),
            torch.from_numpy(np.ascontiguousarray(m, np.float32)).to(device), base, layout)


_KEY_SPACES = {"pre": _abi.TRI_KEYS_PRE_ROPE, "post": _abi.TRI_KEYS_POST_ROPE}
_FORMS = {"additive": _abi.TRI_SCORE_ADDITIVE, "multiplicative": _abi.TRI_SCORE_MULTIPLICATIVE}


def _score_cfg(rope_base, offsets, group, reduce, rope_layout, key_space="pre", form="additive"):
    offs = (ctypes.c_int32 * len(offsets))(*[int(o) for o in offsets])
    cfg = _abi.TriScoreCfg()
    cfg.rope_base = float(rope_base)
    cfg.rope_layout = _LAYOUTS[rope_layout]
    cfg.n_offsets = len(offsets)
    cfg.offsets = ctypes.cast(offs, ctypes.POINTER(ctypes.c_int32))
    cfg.group = int(group)
    cfg.reduce = _REDUCE[reduce]
    cfg.key_space = _KEY_SPACES[key_space]
    cfg.form = _FORMS[form]
    return cfg, offs


def tri_score_keys(kv: KVCache, center, mean_abs, *, rope_base: float, offsets: Sequence[int],
                   group: int, reduce: str = "max", rope_layout: str = "half", query_pos=None,
                   scores=None, stream=None, key_space: str = "pre", form: str = "additive"):
    """Score every cached key; returns float32 scores [n_seq, n_layer, n_kvh, slots].

    key_space "post": the cache holds keys already rotated by RoPE at their slot index.
    form "multiplicative": phase-only series times ||centre|| ||key|| (mean_abs may be None)."""
    torch = _torch()
    L = _abi.lib()
    desc = kv.descriptor()
    _dev(center, "center", torch.float32)
    if mean_abs is not None or form != "multiplicative":
        _dev(mean_abs, "mean_abs", torch.float32)
    _dev(query_pos, "query_pos", torch.int64)
    if scores is None:
        scores = torch.empty((kv.n_seq, desc.n_layer, desc.n_kvh, kv.slots), dtype=torch.float32,
                             device=kv.k.device)
    _dev(scores, "scores", torch.float32)
    n_qh = desc.n_kvh * int(group)
    _shape(center, "center", (desc.n_layer, n_qh, desc.head_dim // 2, 2))
    _shape(mean_abs, "mean_abs", (desc.n_layer, n_qh, desc.head_dim // 2))
    _shape(query_pos, "query_pos", (kv.n_seq,))
    _shape(scores, "scores", (kv.n_seq, desc.n_layer, desc.n_kvh, kv.slots))
    if mean_abs is None and form != "multiplicative":
        raise ValueError("mean_abs is required for the additive form")
    cfg, _keep = _score_cfg(rope_base, offsets, group, reduce, rope_layout, key_space, form)
    _abi.check(L.tri_score_keys(ctypes.byref(cfg), _ptr(center), _ptr(mean_abs), ctypes.byref(desc),
                                _ptr(query_pos), _ptr(scores), None, None, _stream(stream)))
    return scores


def select_workspace(scores, kv: KVCache, budget: int, window: int, kept, kept_n):
    """The workspace tri_select_topb can use for these buffers (a device uint8 tensor), or None
    when it needs none: allocate once and pass it to every call of a loop."""
    torch = _torch()
    L = _abi.lib()
    desc = kv.descriptor()
    need = ctypes.c_size_t(0)
    _abi.check(L.tri_select_topb(_ptr(scores), ctypes.byref(desc), int(budget), int(window), _ptr(kept),
                                 _ptr(kept_n), None, ctypes.byref(need), None))
    return torch.empty((need.value,), dtype=torch.uint8, device=scores.device) if need.value else None


def tri_select_topb(scores, kv: KVCache, budget: int, window: int, kept=None, kept_n=None, stream=None,
                    workspace="auto"):
    """Top-B per unit; returns (kept int32 [n_seq, n_layer, n_kvh, budget], kept_n int32 [n_seq]).

    workspace: "auto" (allocated here when units longer than 32768 slots can be selected in two
    stages over many workgroups), None (one workgroup per unit), or a device uint8 tensor."""
    torch = _torch()
    L = _abi.lib()
    desc = kv.descriptor()
    _dev(scores, "scores", torch.float32)
    if kept is None:
        kept = torch.empty((kv.n_seq, desc.n_layer, desc.n_kvh, budget), dtype=torch.int32, device=scores.device)
    if kept_n is None:
        kept_n = torch.empty((kv.n_seq,), dtype=torch.int32, device=scores.device)
    _dev(kept, "kept", torch.int32)
    _dev(kept_n, "kept_n", torch.int32)
    _shape(scores, "scores", (kv.n_seq, desc.n_layer, desc.n_kvh, kv.slots))
    _shape(kept, "kept", (kv.n_seq, desc.n_layer, desc.n_kvh, int(budget)))
    _shape(kept_n, "kept_n", (kv.n_seq,))
    ws, nbytes, cap = None, None, ctypes.c_size_t(0)
    if workspace is not None:
        need = ctypes.c_size_t(0)
        _abi.check(L.tri_select_topb(_ptr(scores), ctypes.byref(desc), int(budget), int(window), _ptr(kept),
                                     _ptr(kept_n), None, ctypes.byref(need), _stream(stream)))
        if isinstance(workspace, str):
            if workspace != "auto":
                raise ValueError("workspace must be 'auto', None or a device uint8 tensor")
            workspace = (torch.empty((need.value,), dtype=torch.uint8, device=scores.device) if need.value else None)
        if workspace is not None:
            _dev(workspace, "workspace", torch.uint8)
            cap.value = workspace.numel()
            ws, nbytes = _ptr(workspace), ctypes.byref(cap)
    _abi.check(L.tri_select_topb(_ptr(scores), ctypes.byref(desc), int(budget), int(window), _ptr(kept),
                                 _ptr(kept_n), ws, nbytes, _stream(stream)))
    return kept, kept_n


def tri_score_select(kv: KVCache, center, mean_abs, budget: int, window: int, *, rope_base: float,
                     offsets: Sequence[int], group: int, reduce: str = "max", rope_layout: str = "half",
                     query_pos=None, scores=None, kept=None, kept_n=None, stream=None):
    """Scoring and top-B selection in one launch (dense or paged float32 / bfloat16 pre-RoPE caches
    of at most 32768 slots, additive form); returns (kept, kept_n) as tri_select_topb does.  scores,
    if given, also receives the scores (as from tri_score_keys); None writes none."""
    torch = _torch()
    L = _abi.lib()
    desc = kv.descriptor()
    _dev(center, "center", torch.float32)
    _dev(mean_abs, "mean_abs", torch.float32)
    _dev(query_pos, "query_pos", torch.int64)
    _dev(scores, "scores", torch.float32)
    if kept is None:
        kept = torch.empty((kv.n_seq, desc.n_layer, desc.n_kvh, budget), dtype=torch.int32, device=kv.k.device)
    if kept_n is None:
        kept_n = torch.empty((kv.n_seq,), dtype=torch.int32, device=kv.k.device)
    _dev(kept, "kept", torch.int32)
    _dev(kept_n, "kept_n", torch.int32)
    n_qh = desc.n_kvh * int(group)
    _shape(center, "center", (desc.n_layer, n_qh, desc.head_dim // 2, 2))
    _shape(mean_abs, "mean_abs", (desc.n_layer, n_qh, desc.head_dim // 2))
    _shape(query_pos, "query_pos", (kv.n_seq,))
    _shape(scores, "scores", (kv.n_seq, desc.n_layer, desc.n_kvh, kv.slots))
    _shape(kept, "kept", (kv.n_seq, desc.n_layer, desc.n_kvh, int(budget)))
    _shape(kept_n, "kept_n", (kv.n_seq,))
    if mean_abs is None:
        raise ValueError("mean_abs is required (additive form)")
    cfg, _keep = _score_cfg(rope_base, offsets, group, reduce, rope_layout)
    _abi.check(L.tri_score_select(ctypes.byref(cfg), _ptr(center), _ptr(mean_abs), ctypes.byref(desc),
                                  _ptr(query_pos), int(budget), int(window), _ptr(scores), _ptr(kept),
                                  _ptr(kept_n), None, None, _stream(stream)))
    return kept, kept_n


def tri_compact_kv(kv: KVCache, kept, kept_n, budget: int, k_out=None, v_out=None, pos_out=None,
                   freed=None, n_freed=None, new_len=None, want_pos=True, want_freed=True, stream=None):
    """Forward-pack the survivors.  Returns a dict with the outputs that were written.

    dense: k_out / v_out [n_seq, n_layer, n_kvh, budget, d] (allocated if not given)
    paged: in place; freed [n_seq, max_pages] and n_freed [n_seq] list the emptied pages
    """
    torch = _torch()
    L = _abi.lib()
    desc = kv.descriptor()
    dev = kv.k.device
    _dev(kept, "kept", torch.int32)
    _dev(kept_n, "kept_n", torch.int32)
    shape_u = (kv.n_seq, desc.n_layer, desc.n_kvh)
    if kv.layout == "dense":
        if k_out is None:
            k_out = torch.empty(shape_u + (budget, desc.head_dim), dtype=kv.k.dtype, device=dev)
        if kv.v is not None and v_out is None:
            v_out = torch.empty_like(k_out)
    elif want_freed:
        if freed is None:
            freed = torch.empty((kv.n_seq, desc.max_pages), dtype=torch.int32, device=dev)
        if n_freed is None:
            n_freed = torch.empty((kv.n_seq,), dtype=torch.int32, device=dev)
    if want_pos and pos_out is None:
        pos_out = torch.empty(shape_u + (budget,), dtype=torch.int32, device=dev)
    if new_len is None:
        new_len = torch.empty((kv.n_seq,), dtype=torch.int32, device=dev)
    for t, name in ((k_out, "k_out"), (v_out, "v_out")):
        _dev(t, name, kv.k.dtype)
    for t, name in ((pos_out, "pos_out"), (freed, "freed"), (n_freed, "n_freed"), (new_len, "new_len")):
        _dev(t, name, torch.int32)
    _shape(kept, "kept", shape_u + (int(budget),))
    _shape(kept_n, "kept_n", (kv.n_seq,))
    _shape(k_out, "k_out", shape_u + (int(budget), desc.head_dim))
    _shape(v_out, "v_out", shape_u + (int(budget), desc.head_dim))
    _shape(pos_out, "pos_out", shape_u + (int(budget),))
    if kv.layout == "paged":
        _shape(freed, "freed", (kv.n_seq, desc.max_pages))
    _shape(n_freed, "n_freed", (kv.n_seq,))
    _shape(new_len, "new_len", (kv.n_seq,))
    _abi.check(L.tri_compact_kv(ctypes.byref(desc), _ptr(kept), _ptr(kept_n), int(budget), _ptr(k_out),
                                _ptr(v_out), _ptr(pos_out), _ptr(freed), _ptr(n_freed), _ptr(new_len),
                                _stream(stream)))
    return {"k_out": k_out, "v_out": v_out, "pos_out": pos_out, "freed": freed, "n_freed": n_freed,
            "new_len": new_len}


def _attention_args(kv: KVCache, q, query_pos, rope_base, group, pos, layer0, n_layers, rope_layout, key_space,
                    out, allocate_out):
    """Checked arguments of the attention entry points, up to and including out."""
    torch = _torch()
    desc = kv.descriptor()
    n_layers = desc.n_layer - layer0 if n_layers is None else int(n_layers)
    shape_q = (kv.n_seq, n_layers, desc.n_kvh * int(group), desc.head_dim)
    _dev(q, "q", torch.float32)
    _shape(q, "q", shape_q)
    _dev(query_pos, "query_pos", torch.int64)
    _shape(query_pos, "query_pos", (kv.n_seq,))
    pos_stride = 0
    if pos is not None:
        _dev(pos, "pos", torch.int32)
        if pos.dim() != 4 or tuple(pos.shape[:3]) != (kv.n_seq, desc.n_layer, desc.n_kvh):
            raise ValueError("pos must be [n_seq, n_layer, n_kvh, stride]")
        pos_stride = int(pos.shape[3])
    if out is None:
        if not allocate_out:
            raise ValueError("out is required")
        out = torch.empty(shape_q, dtype=torch.float32, device=q.device)
    _dev(out, "out", torch.float32)
    _shape(out, "out", shape_q)
    args = (ctypes.byref(desc), int(layer0), n_layers, _ptr(q), _ptr(query_pos), _ptr(pos), pos_stride,
            float(rope_base), _LAYOUTS[rope_layout], _KEY_SPACES[key_space], int(group), _ptr(out))
    return args, out, desc


def tri_decode_attention(kv: KVCache, q, query_pos, *, rope_base: float, group: int, pos=None, layer0: int = 0,
                         n_layers=None, rope_layout: str = "half", key_space: str = "pre", out=None, stream=None,
                         workspace="auto"):
    """Attention of the newest token over a (compressed) cache: keys rotated by RoPE at their
    positions (pos, e.g. the compaction's pos_out [n_seq, n_layer, n_kvh, budget]; None = slot
    index), softmax over kv.seq_len keys.  q: float32 [n_seq, n_layers, n_kvh * group, d]
    pre-RoPE queries at query_pos (int64 [n_seq]).  Returns float32 out of q's shape.
    workspace: "auto" (allocated here when the shape is split over several workgroups per
    unit), None (one workgroup per unit, no workspace), or a device uint8 tensor."""
    torch = _torch()
    L = _abi.lib()
    args, out, _desc = _attention_args(kv, q, query_pos, rope_base, group, pos, layer0, n_layers, rope_layout,
                                       key_space, out, True)
    ws, nbytes, cap = None, None, ctypes.c_size_t(0)
    if workspace is not None:
        need = ctypes.c_size_t(0)
        _abi.check(L.tri_decode_attention(*args, None, ctypes.byref(need), _stream(stream)))
        if isinstance(workspace, str):
            if workspace != "auto":
                raise ValueError("workspace must be 'auto', None or a device uint8 tensor")
            workspace = (torch.empty((need.value,), dtype=torch.uint8, device=q.device) if need.value else None)
        if workspace is not None:
            _dev(workspace, "workspace", torch.uint8)
            cap.value = workspace.numel()
            ws, nbytes = _ptr(workspace), ctypes.byref(cap)
    _abi.check(L.tri_decode_attention(*args, ws, nbytes, _stream(stream)))
    return out


def tri_decode_attention_noalloc(kv: KVCache, q, query_pos, *, rope_base: float, group: int, out, pos=None,
                                 layer0: int = 0, n_layers=None, rope_layout: str = "half", key_space: str = "pre",
                                 stream=None):
    """tri_decode_attention that allocates nothing: split shapes keep their partial results in
    the library's static per-GPU scratch (8 MiB; the split rule keeps every need under 4.3 MB,
    and a larger one would raise TriError TRI_EWORKSPACE).
    out must be given.  Calls that overlap on one GPU race on the scratch."""
    args, out, _desc = _attention_args(kv, q, query_pos, rope_base, group, pos, layer0, n_layers, rope_layout,
                                       key_space, out, False)
    _abi.check(_abi.lib().tri_decode_attention_noalloc(*args, _stream(stream)))
    return out


def compress(kv: KVCache, center, mean_abs, *, rope_base, offsets, group, budget, window,
             reduce="max", rope_layout="half", query_pos=None, stream=None, key_space="pre",
             form="additive"):
    """Score, select and compact in one call (convenience; not part of the C ABI)."""
    scores = tri_score_keys(kv, center, mean_abs, rope_base=rope_base, offsets=offsets, group=group,
                            reduce=reduce, rope_layout=rope_layout, query_pos=query_pos, stream=stream,
                            key_space=key_space, form=form)
    kept, kept_n = tri_select_topb(scores, kv, budget, window, stream=stream)
    out = tri_compact_kv(kv, kept, kept_n, budget, stream=stream)
    out.update(scores=scores, kept=kept, kept_n=kept_n)
    return out
