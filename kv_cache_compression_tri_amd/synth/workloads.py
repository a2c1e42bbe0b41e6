"""The synthetic workloads of the compression pass and their host-side parameters.

A workload fixes the cache shapes, the RoPE base, the future offsets, the budget and the
window, and the seed from which every input is drawn.  Host parameters (key centres,
calibrated query statistics, the low-concentration head mask, paged lengths and page
ids) come from ``numpy.random.default_rng(seed)`` in a fixed draw order; bulk key/value
noise comes from the counter-based generator in ``synth`` (host or device).

The shapes follow the pages' deployment scale: 32K-token reasoning with a budget near a
tenth of the context ("TriAttention: How a Geometric Trick Cuts LLM Memory Use by 10x
Without Losing Accuracy", section "What the Numbers Look Like"), 8B-class GQA models
("TriAttention: trigonometric KV cache compression for long reasoning", section
"Calibration statistics are tied to a specific model"), compression every ~128 decode
steps and 16-token paged blocks (dev.to article, section "Solving the Memory
Fragmentation Problem").  No dataset is involved.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np


def geometric_offsets(m: int):
    """D = {1, 2, 4, ..., 2^m}."""
    return tuple(1 << i for i in range(m + 1))


@dataclass(frozen=True)
class Workload:
    name: str
    n_seq: int
    n_layer: int
    n_kvh: int
    group: int
    max_len: int
    dtype: str                 # "f32" | "bf16" | "fp8" | "int8" (8-bit codes times a per-head scale)
    base: float
    offsets: tuple
    budget: int
    window: int
    reduce: str                # "max" | "mean"
    seed: int
    paged: bool = False
    with_values: bool = True
    sigma_low: float = 0.3     # key noise sigma for bands f < F/2
    sigma_high: float = 0.3    # key noise sigma for bands f >= F/2
    sink: bool = True          # row 0 of every unit scaled by 20
    low_r_frac: float = 0.1    # fraction of (layer, KV head) groups with R ~= 0.3
    len_range: tuple = None    # paged: inclusive (lo, hi) of the uniform lengths
    head_dim: int = 128
    layout: str = "half"
    page: int = 16

    @property
    def n_qh(self) -> int:
        return self.n_kvh * self.group

    @property
    def n_units(self) -> int:
        return self.n_seq * self.n_layer * self.n_kvh

    @property
    def max_pages(self) -> int:
        return -(-self.max_len // self.page)


WORKLOADS = {
    # one KV head, 2048 float32 keys, one query head, base 1e4, D = {1..1024}, B 256, W 64
    "single_head_2k_f32": Workload(
        "single_head_2k_f32", n_seq=1, n_layer=1, n_kvh=1, group=1, max_len=2048,
        dtype="f32", base=1e4, offsets=geometric_offsets(10), budget=256, window=64,
        reduce="max", seed=0, with_values=False, sink=False, low_r_frac=0.0),
    # 8B-class GQA decode step at 32K: 36 layers x 8 KV heads x 4 query heads, bf16
    "gqa8b_32k_bf16": Workload(
        "gqa8b_32k_bf16", n_seq=1, n_layer=36, n_kvh=8, group=4, max_len=32768,
        dtype="bf16", base=1e6, offsets=geometric_offsets(12), budget=2048, window=128,
        reduce="max", seed=1),
    # the same model at batch 16 x 16K, mean over the group, B 1024
    "gqa8b_batch16_16k_bf16": Workload(
        "gqa8b_batch16_16k_bf16", n_seq=16, n_layer=36, n_kvh=8, group=4, max_len=16384,
        dtype="bf16", base=1e6, offsets=geometric_offsets(12), budget=1024, window=128,
        reduce="mean", seed=2),
    # long context: 1 x 131072 tokens, 28 layers x 4 KV heads x 7 query heads
    "long_128k_bf16": Workload(
        "long_128k_bf16", n_seq=1, n_layer=28, n_kvh=4, group=7, max_len=131072,
        dtype="bf16", base=1e6, offsets=geometric_offsets(14), budget=4096, window=256,
        reduce="max", seed=3, sigma_low=0.1, sigma_high=1.0),
    # 64 ragged sequences (4096..32768 tokens) in 16-token pages of a shared pool
    "paged_ragged64_bf16": Workload(
        "paged_ragged64_bf16", n_seq=64, n_layer=36, n_kvh=8, group=4, max_len=32768,
        dtype="bf16", base=1e6, offsets=geometric_offsets(12), budget=1024, window=128,
        reduce="max", seed=4, paged=True, len_range=(4096, 32768)),
    # the 32K GQA step on an fp8 (OCP E4M3) cache with per-(layer, KV head) key scales
    "gqa8b_32k_fp8": Workload(
        "gqa8b_32k_fp8", n_seq=1, n_layer=36, n_kvh=8, group=4, max_len=32768,
        dtype="fp8", base=1e6, offsets=geometric_offsets(12), budget=2048, window=128,
        reduce="max", seed=5),
    # the 32K GQA step on an int8 cache with per-(layer, KV head) key scales
    "gqa8b_32k_int8": Workload(
        "gqa8b_32k_int8", n_seq=1, n_layer=36, n_kvh=8, group=4, max_len=32768,
        dtype="int8", base=1e6, offsets=geometric_offsets(12), budget=2048, window=128,
        reduce="max", seed=6),
}

BENCH_WORKLOAD = "gqa8b_32k_bf16"
# the five stated workloads (the 8-bit ones are the 32K pass on a quantised cache)
STATED_WORKLOADS = ("single_head_2k_f32", "gqa8b_32k_bf16", "gqa8b_batch16_16k_bf16", "long_128k_bf16",
                    "paged_ragged64_bf16")


def scaled(w: Workload, **changes) -> Workload:
    """A copy of a workload with some fields changed (smaller parity cases)."""
    return replace(w, **changes)


@dataclass
class HostParams:
    mu_k: np.ndarray          # [n_layer, n_kvh, d] float32 key centres
    center: np.ndarray        # [n_layer, n_qh, F, 2] float32 E[q_f] (re, im)
    mean_abs: np.ndarray      # [n_layer, n_qh, F] float32 E|q_f|
    low_r: np.ndarray         # [n_layer, n_kvh] bool
    sigma: np.ndarray         # [d] float32 per-element key noise
    lengths: np.ndarray       # [n_seq] int32
    block_table: np.ndarray = field(default=None)   # [n_seq, max_pages] int32 (paged)
    n_pages: int = 0
    k_scale: np.ndarray = field(default=None)       # [n_layer, n_kvh] float32 (8-bit keys)


def key_scales(w) -> np.ndarray:
    """Per-(layer, KV head) key scales of an 8-bit cache: powers of two in a checkerboard,
    so that encoding x / scale is exact before rounding (fp8: 1 and 1/2; int8: 1/16 and 1/8,
    which puts typical keys at codes of a few tens); 1 otherwise."""
    if w.dtype not in ("fp8", "int8"):
        return np.ones((w.n_layer, w.n_kvh), dtype=np.float32)
    lh = np.add.outer(np.arange(w.n_layer), np.arange(w.n_kvh))
    hi, lo = (1.0, 0.5) if w.dtype == "fp8" else (1.0 / 16, 1.0 / 8)
    return np.where(lh % 2 == 0, hi, lo).astype(np.float32)


def make_params(w: Workload, lengths=None) -> HostParams:
    """Host parameters of a workload.  ``lengths`` (optional) overrides the sequence lengths
    (each <= max_len); the rest of the draws are unchanged."""
    rng = np.random.default_rng(w.seed)
    d, F = w.head_dim, w.head_dim // 2
    mu_k = rng.standard_normal((w.n_layer, w.n_kvh, d)).astype(np.float32)
    mu_q = rng.standard_normal((w.n_layer, w.n_qh, d)).astype(np.float32)
    n_groups = w.n_layer * w.n_kvh
    n_low = int(round(w.low_r_frac * n_groups))
    low = np.zeros(n_groups, dtype=bool)
    low[rng.permutation(n_groups)[:n_low]] = True
    low = low.reshape(w.n_layer, w.n_kvh)

    if w.layout == "half":
        re, im = mu_q[..., :F], mu_q[..., F:]
    else:
        re, im = mu_q[..., 0::2], mu_q[..., 1::2]
    center = np.stack([re, im], axis=-1).astype(np.float32)
    mag = np.hypot(center[..., 0].astype(np.float64), center[..., 1].astype(np.float64))
    # E|q_f| = 1.1 |E q_f| (R ~= 0.91) on concentrated groups, |E q_f| / 0.3 on the rest
    factor = np.where(np.repeat(low, w.group, axis=1), 1.0 / 0.3, 1.1)
    mean_abs = (mag * factor[..., None]).astype(np.float32)

    sigma = np.empty(d, dtype=np.float32)
    band = np.arange(F)
    s_band = np.where(band < F // 2, w.sigma_low, w.sigma_high).astype(np.float32)
    if w.layout == "half":
        sigma[:F], sigma[F:] = s_band, s_band
    else:
        sigma[0::2], sigma[1::2] = s_band, s_band

    if w.paged:
        lo, hi = w.len_range
        drawn = rng.integers(lo, hi, size=w.n_seq, endpoint=True).astype(np.int32)
        lengths = drawn if lengths is None else np.asarray(lengths, dtype=np.int32)
        pages_per = -(-lengths.astype(np.int64) // w.page)
        n_pages = int(pages_per.sum())
        perm = rng.permutation(n_pages).astype(np.int32)
        bt = np.full((w.n_seq, w.max_pages), -1, dtype=np.int32)
        off = 0
        for s in range(w.n_seq):
            bt[s, : pages_per[s]] = perm[off: off + pages_per[s]]
            off += pages_per[s]
        return HostParams(mu_k, center, mean_abs, low, sigma, lengths, bt, n_pages, key_scales(w))
    if lengths is None:
        lengths = np.full(w.n_seq, w.max_len, dtype=np.int32)
    lengths = np.asarray(lengths, dtype=np.int32)
    if lengths.shape != (w.n_seq,) or lengths.min() < 0 or lengths.max() > w.max_len:
        raise ValueError("lengths must be n_seq values in [0, max_len]")
    return HostParams(mu_k, center, mean_abs, low, sigma, lengths, k_scale=key_scales(w))


def unit_index(w: Workload, s: int, layer: int, kv_head: int) -> int:
    return (s * w.n_layer + layer) * w.n_kvh + kv_head


def unit_coords(w: Workload, u: int):
    kv_head = u % w.n_kvh
    layer = (u // w.n_kvh) % w.n_layer
    s = u // (w.n_kvh * w.n_layer)
    return s, layer, kv_head
