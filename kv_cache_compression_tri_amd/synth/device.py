"""Device-resident synthetic caches built with libtri_synth.so (test / benchmark infra)."""

from __future__ import annotations

import ctypes
import os
from ctypes import c_int32, c_int64, c_uint32, c_uint64, c_void_p
from dataclasses import dataclass

import numpy as np

from . import TAG_K, TAG_V
from .workloads import HostParams, Workload, make_params

PKG_DIR = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SYNTH_LIB = os.path.join(PKG_DIR, "lib", "libtri_synth.so")
SYNTH_EXPORTS = ("tri_synth_fill_dense", "tri_synth_fill_paged")

_LIB = None


def lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(SYNTH_LIB):
            raise RuntimeError(f"{SYNTH_LIB} is missing: build with python -m kv_cache_compression_tri_amd.build")
        L = ctypes.CDLL(SYNTH_LIB)
        L.tri_synth_fill_dense.argtypes = [c_void_p, c_int32, c_int64, c_int64, c_int32, c_void_p, c_void_p,
                                           c_int32, c_uint64, c_uint32, c_void_p, c_void_p]
        L.tri_synth_fill_paged.argtypes = [c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                           c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_uint64, c_uint32,
                                           c_void_p, c_void_p]
        L.tri_synth_fill_dense.restype = ctypes.c_int
        L.tri_synth_fill_paged.restype = ctypes.c_int
        _LIB = L
    return _LIB


def _stream():
    import torch
    return c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


@dataclass
class DeviceWorkload:
    w: Workload
    hp: HostParams
    k: object
    v: object
    seq_len: object
    block_table: object
    center: object
    mean_abs: object
    k_scale: object = None     # device [n_layer, n_kvh] float32 for 8-bit caches

    def kv(self):
        from .. import KVCache
        if self.w.paged:
            return KVCache.paged(self.k, self.v, self.block_table, self.seq_len, k_scale=self.k_scale)
        return KVCache.dense(self.k, self.v, self.seq_len, k_scale=self.k_scale)


def fill(w: Workload, hp: HostParams, k, v, seq_len, block_table):
    """(Re)generate K (and V) in place from the workload's seed."""
    import torch
    dev = k.device
    dtype_code = {"f32": 0, "bf16": 1, "fp8": 2, "int8": 3}[w.dtype]
    mu_k = torch.from_numpy(np.ascontiguousarray(hp.mu_k.reshape(-1, w.head_dim))).to(dev)
    sig_k = torch.from_numpy(hp.sigma).to(dev)
    mu_v = torch.zeros_like(mu_k)
    sig_v = torch.ones_like(sig_k)
    inv_k = torch.from_numpy((1.0 / hp.k_scale).astype(np.float32).reshape(-1)).to(dev)
    st = _stream()
    L = lib()
    jobs = [(k, mu_k, sig_k, int(w.sink), TAG_K, inv_k)]
    if v is not None:
        jobs.append((v, mu_v, sig_v, 0, TAG_V, None))
    for t, mu, sig, sink, tag, inv in jobs:
        inv_p = c_void_p(inv.data_ptr()) if inv is not None else None
        if w.paged:
            rc = L.tri_synth_fill_paged(c_void_p(t.data_ptr()), dtype_code, w.n_seq, w.n_layer, w.n_kvh, w.page,
                                        w.max_pages, c_void_p(block_table.data_ptr()), c_void_p(seq_len.data_ptr()),
                                        c_void_p(mu.data_ptr()), c_void_p(sig.data_ptr()), sink, w.seed, tag, inv_p,
                                        st)
        else:
            rc = L.tri_synth_fill_dense(c_void_p(t.data_ptr()), dtype_code, w.n_units, w.max_len,
                                        w.n_layer * w.n_kvh, c_void_p(mu.data_ptr()), c_void_p(sig.data_ptr()),
                                        sink, w.seed, tag, inv_p, st)
        _check(rc, "synthetic fill")
    # keep the parameter tensors alive until the fills have run
    torch.cuda.current_stream().synchronize()


def build(w: Workload, device="cuda", hp: HostParams = None) -> DeviceWorkload:
    """Allocate and generate the workload's cache and statistics on the device."""
    import torch
    hp = hp or make_params(w)
    tdtype = {"bf16": torch.bfloat16, "f32": torch.float32, "fp8": torch.float8_e4m3fn, "int8": torch.int8}[w.dtype]
    seq_len = torch.from_numpy(hp.lengths).to(device)
    if w.paged:
        shape = (hp.n_pages, w.n_layer, w.n_kvh, w.page, w.head_dim)
        block_table = torch.from_numpy(hp.block_table).to(device)
    else:
        shape = (w.n_seq, w.n_layer, w.n_kvh, w.max_len, w.head_dim)
        block_table = None
    k = torch.empty(shape, dtype=tdtype, device=device)
    v = torch.empty(shape, dtype=tdtype, device=device) if w.with_values else None
    fill(w, hp, k, v, seq_len, block_table)
    center = torch.from_numpy(hp.center).to(device)
    mean_abs = torch.from_numpy(hp.mean_abs).to(device)
    k_scale = torch.from_numpy(hp.k_scale).to(device) if w.dtype in ("fp8", "int8") else None
    return DeviceWorkload(w, hp, k, v, seq_len, block_table, center, mean_abs, k_scale)
