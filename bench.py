#!/usr/bin/env python3
"""Throughput of the TriAttention KV-cache compression pass on one MI355X.

One step = one pass of the whole hot path over the resident synthetic cache:
tri_score_keys -> tri_select_topb -> tri_compact_kv, for every (layer, KV head).  The
default workload is the 32K-context GQA pass (36 layers x 8 KV heads x 32768 keys, bf16,
4 query heads per KV head, B = 2048, window 128, dense out-of-place compaction);
--workload picks another one (the paged workload compacts in place, so its pools are
regenerated before every step, outside the timed region, and each step is timed on its
own; the single-head float32 workload has no values and is scored and selected only).
Inputs are generated on the device before timing; the timed region is bracketed by
torch.cuda.synchronize().  Inside it the steps run back to back, with HIP events only
around the score kernel; the selection / compaction split comes from a short breakdown
loop after the timed region.

Prints one JSON line with the metric (keys scored+selected+compacted per second), the
roofline of the dominant kernel (scoring: algorithmic bytes = one key row per key read,
256 B for bf16, 128 B for fp8 and int8, 512 B for float32, over its average HIP-event
duration) and the CPU oracle timed on a bounded sample of units.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import multiprocessing as mp
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
# non-packed fp32 vector issue of MI355X: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz (lane operations / s)
PEAK_VALU_TLANEOPS = 256 * 4 * 16 * 2.4e9 / 1e12


def score_lane_ops_per_key(group_eff: int, key_space: str, form: str) -> int:
    """Vector lane operations the score needs per key, counting only the arithmetic of the
    method (per band: rotation by the phase table 4 (pre-RoPE keys only), |k_f|^2 and its
    square root 3, and per effective head 3 multiply-adds (multiplicative form: |k_f|^2 2,
    reciprocal square root 1, unit scaling 2, and 2 per head)); unpacking, reductions and
    addressing are overhead."""
    rot = 4 if key_space == "pre" else 0
    if form == "multiplicative":
        return 64 * (rot + 5 + 2 * group_eff)
    return 64 * (rot + 3 + 3 * group_eff)
METRIC = "Gkeys/s scored+selected+compacted at 32K ctx; % of HBM roofline"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "score_kernel_traffic.json")
# the scoring kernels' sources (the matrix-core kernel includes the vector kernel's header); the
# recorded traffic holds for the digest of both
SCORE_SRCS = [os.path.join(ROOT, "kv_cache_compression_tri_amd", "csrc", f) for f in ("score_kernel.h", "score_mx.h")]


def fused_applies(w, key_space: str = "pre", form: str = "additive", positions: bool = False) -> bool:
    """tri_score_select takes float32/bf16 caches of pre-RoPE keys at their slots, additive form,
    at most 32768 slots per unit."""
    slots = w.max_pages * 16 if w.paged else w.max_len
    return (w.dtype in ("f32", "bf16") and key_space == "pre" and form == "additive" and not positions
            and slots <= 32768)


def use_fused(mode: str, w, n_cu: int, key_space="pre", form="additive", positions=False) -> bool:
    """Whether a pass scores and selects in one launch.  auto: where the fused launch measured
    faster than the two launches.  It saves writing the scores and reading them back, which costs
    most when scoring is bound by the key stream (one effective head: the mean reduction or
    G = 1), and a workgroup per unit only balances when every CU gets many units (at the 32K
    pass, 288 units on 256 CUs, 32 CUs score two whole units) or when the units are so few and
    short that the two-launch path gives each at most one workgroup too (the 2K single-head
    pass: one launch less and a smaller phase table)."""
    ok = fused_applies(w, key_space, form, positions)
    if mode == "on":
        if not ok:
            raise SystemExit(f"--fused on: {w.name} is not a case tri_score_select takes")
        return True
    if mode == "off" or not ok:
        return False
    g_eff = 1 if w.reduce == "mean" else w.group
    if g_eff == 1 and w.n_units >= 8 * n_cu:         # many units per CU, bound by the key stream
        return True
    # few short units: the persistent scoring grid would give no unit more than one workgroup
    # either (one per 256 8-key steps, at most one per CU), and every unit gets its own CU
    slots = w.max_pages * 16 if w.paged else w.max_len
    grid = min(n_cu, -(-w.n_units * (-(-slots // 8)) // (32 * 8)))
    return grid <= w.n_units <= n_cu


def score_kernel_used(w, key_space: str, form: str, positions: bool) -> str:
    """The scoring kernel the library launches for this pass: the additive form with the max over
    the group takes the matrix-core kernel for bfloat16 keys at 4..8 heads (before RoPE at
    consecutive positions, or cached after RoPE, whose positions are not read) and for 8-bit keys
    cached after RoPE at 2..8 heads."""
    if form == "additive" and w.reduce == "max":
        if w.dtype == "bf16" and (key_space == "post" or not positions) and 4 <= w.group <= 8:
            return "score_mx_kernel"
        if w.dtype in ("fp8", "int8") and key_space == "post" and 2 <= w.group <= 8:
            return "score_mx_kernel"
    return "score_kernel"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # Defaults: 250 ms of untimed pre-roll passes (--preroll-ms), 10 warmup passes, then 200
    # timed passes (about 0.12 s on the 32K pass).
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--preroll-ms", type=float, default=250.0,
                    help="untimed passes for this long (wall ms) before the warmup passes (0 = none)")
    ap.add_argument("--workload", default=None, help="workload name (default: the 32K GQA pass)")
    ap.add_argument("--form", choices=("additive", "multiplicative"), default="additive",
                    help="score form: additive (default) or the phase-only series times the norms")
    ap.add_argument("--positions", action="store_true",
                    help="give the cache explicit key positions (slot index), scored without the phase table")
    ap.add_argument("--consumer", action="store_true",
                    help="time attention of a new token over the compressed cache (the default; kept for scripts)")
    ap.add_argument("--no-consumer", action="store_true",
                    help="skip timing attention over the compressed cache after each workload's timed passes")
    ap.add_argument("--key-space", choices=("pre", "post"), default="pre",
                    help="score the cache as pre-RoPE keys (default) or as keys already rotated by RoPE")
    ap.add_argument("--cpu-units", type=int, default=0,
                    help="units for the oracle baseline (0 = two per host core, capped at 32)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="time only the headline workload (skip the other stated workloads)")
    ap.add_argument("--fused", choices=("auto", "on", "off"), default="auto",
                    help="score and select in one launch (tri_score_select; f32/bf16 pre-RoPE caches of at most "
                         "32768 slots, additive form) instead of two, its time reported as score_ms: on, off, or "
                         "auto (default: where it measured faster, one effective head and at least 8 units per CU)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB mebibytes (calibrates HBM counters)")
    return ap.parse_args()


def copy_bandwidth(mib, reps=5):
    """Plain device-to-device copy of `mib` MiB; returns (bytes moved per copy, GB/s)."""
    import torch
    n = mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    return 2 * n, 2 * n / dt / 1e9


# ---------------------------------------------------------------------------------------
# CPU oracle baseline (bounded sample)
# ---------------------------------------------------------------------------------------

def _oracle_unit(job):
    """Score + select + compact one unit with the float64 oracle; returns seconds spent."""
    import numpy as np
    import oracle
    name, key_space, form, s, l, h = job
    from kv_cache_compression_tri_amd import synth
    from kv_cache_compression_tri_amd.synth import workloads as W
    w = W.WORKLOADS[name]
    hp = W.make_params(w)
    unit = W.unit_index(w, s, l, h)
    L = int(hp.lengths[s])
    scale = float(hp.k_scale[l, h])
    keys_raw = synth.rows(w.seed, synth.TAG_K, unit, L, hp.mu_k[l, h], hp.sigma, w.sink, w.dtype,
                          scale=scale)
    keys = oracle.decode_stored(keys_raw, w.dtype, scale)
    vals = synth.rows(w.seed, synth.TAG_V, unit, L, np.zeros(128, np.float32), np.ones(128, np.float32),
                      False, w.dtype)
    center, mean_abs = oracle.unit_heads(hp.center, hp.mean_abs, l, h, w.group)
    t0 = time.perf_counter()
    sc = oracle.score_keys(keys, center, mean_abs, base=w.base, offsets=w.offsets, layout=w.layout,
                           reduce=w.reduce, key_space=key_space, form=form)
    kept = oracle.select_top_b(sc, L, w.budget, w.window)
    if w.with_values:
        oracle.compact_dense(keys_raw, vals, kept)
    return time.perf_counter() - t0, L


def host_cpu():
    """What the host says about its CPU: model string, family / model / stepping, core counts."""
    info = {"model": platform.processor() or platform.machine(), "logical_cpus": os.cpu_count()}
    try:
        info["affinity_cpus"] = len(os.sched_getaffinity(0))
    except AttributeError:
        info["affinity_cpus"] = os.cpu_count()
    fields = {}
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if ":" not in line:
                    if fields:
                        break                     # first processor block only
                    continue
                k, v = (x.strip() for x in line.split(":", 1))
                fields.setdefault(k, v)
    except OSError:
        pass
    if fields.get("model name"):
        info["model"] = fields["model name"]
    for k in ("vendor_id", "cpu family", "model", "stepping", "cpu MHz", "cache size", "cpu cores", "siblings"):
        if k in fields:
            info["cpuinfo_" + k.replace(" ", "_")] = fields[k]
    return info


# Worker processes of the oracle baseline: the host cores this GPU's share of the box gives
# (16 per GPU); the host may show more.
ORACLE_WORKERS_MAX = 16


def cpu_baseline(name, n_units, key_space="pre", form="additive"):
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    from kv_cache_compression_tri_amd.synth import workloads as W
    import numpy as np
    w = W.WORKLOADS[name]
    host = host_cpu()
    cores = max(1, min(host["affinity_cpus"] or 1, ORACLE_WORKERS_MAX))
    if n_units <= 0:
        n_units = min(32, 2 * cores)
    rng = np.random.default_rng(2024)
    picks = rng.choice(w.n_units, size=min(n_units, w.n_units), replace=False)
    jobs = [(name, key_space, form) + tuple(int(x) for x in W.unit_coords(w, int(u))) for u in picks]
    workers = min(cores, len(jobs))
    ctx = mp.get_context("spawn")
    t0 = time.perf_counter()
    with ctx.Pool(workers, initializer=_pool_init) as pool:
        res = pool.map(_oracle_unit, jobs)
    wall = time.perf_counter() - t0
    busy = sum(r[0] for r in res)
    keys = sum(r[1] for r in res)
    # rate over the oracle's own work, run on `workers` cores in parallel
    rate = keys / (busy / workers) / 1e9
    hp = W.make_params(w)
    pass_keys = int(np.sum(np.minimum(hp.lengths, w.max_len))) * w.n_layer * w.n_kvh
    return {
        "value": rate,
        "unit": "Gkeys/s",
        "cores": workers,
        "kind": "oracle",
        "per_core_value": keys / busy / 1e9,
        "full_pass_s": pass_keys / (rate * 1e9),
        "host": host,
        "sample": (f"{len(jobs)} random units of {name} ({keys} keys; score+select+compact per unit, "
                   f"float64 numpy, one single-threaded process per core on {workers} of the host's "
                   f"{host['logical_cpus']} logical CPUs ({host['affinity_cpus']} in this process's "
                   f"affinity; 16 per GPU is this GPU's share); wall {wall:.1f} s, oracle time {busy:.1f} "
                   f"core-s) on {host['model']}; full_pass_s extrapolates to all {pass_keys} keys at this rate"),
    }


def _pool_init():
    os.environ["OMP_NUM_THREADS"] = "1"


# ---------------------------------------------------------------------------------------
# traffic counters recorded for the current scoring kernel
# ---------------------------------------------------------------------------------------

def recorded_traffic(name):
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
        h = hashlib.sha256()
        for src in SCORE_SRCS:
            with open(src, "rb") as fh:
                h.update(fh.read())
        digest = h.hexdigest()
    except (OSError, ValueError):
        return None
    entry = rec.get(name)
    if not entry or entry.get("score_sources_sha256") != digest:
        return None
    return entry.get("bytes_per_launch")


# ---------------------------------------------------------------------------------------

def consumer(args, w, dw, kv, kept_n, new_len, k_out, v_out, pos_out, reps=20):
    """Attention of a new token of every sequence over the cache the last pass compressed
    (RoPE at the kept keys' positions).  Bytes: every kept key and value row read once."""
    import numpy as np
    import torch
    import kv_cache_compression_tri_amd as tri
    torch.cuda.synchronize()
    if w.paged:
        # the pools were packed in place; positions of the packed slots at the cache's stride
        pos = torch.zeros((w.n_seq, w.n_layer, w.n_kvh, kv.slots), dtype=torch.int32, device=dw.k.device)
        pos[..., :w.budget] = pos_out
        cache = tri.KVCache.paged(dw.k, dw.v, dw.block_table, new_len, pos=pos)
    else:
        pos = pos_out
        cache = tri.KVCache.dense(k_out, v_out, new_len)
    rng = np.random.default_rng(7)
    q = torch.from_numpy(rng.standard_normal((w.n_seq, w.n_layer, w.n_qh, w.head_dim)).astype(np.float32)).cuda()
    qpos = dw.seq_len.to(torch.int64)
    out = torch.empty_like(q)
    # the entry point without allocation: the same kernels and split as with a workspace, and
    # one library call per attention (no workspace query or allocation on the host)
    run = lambda: tri.tri_decode_attention_noalloc(cache, q, qpos, rope_base=w.base, group=w.group, pos=pos,
                                                   rope_layout=w.layout, key_space=args.key_space, out=out)
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    rows = int(new_len.sum().item()) * w.n_layer * w.n_kvh
    elt = {"f32": 4, "bf16": 2}[w.dtype]
    nbytes = rows * w.head_dim * elt * 2
    return {"kernel": "decode_attention_kernel", "ms": ms, "keys": rows, "bytes": nbytes,
            "GBps": nbytes / (ms * 1e-3) / 1e9, "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}


def measure(args, name, steps, warmup, key_space="pre", form="additive", positions=False, with_consumer=False,
            preroll_ms=0.0, fused=False):
    """Build workload `name` in HBM, run untimed passes for preroll_ms of wall time, then
    `warmup` untimed passes, then time exactly `steps` passes; returns the measurements (the
    workload is freed before returning)."""
    import torch
    import kv_cache_compression_tri_amd as tri
    from kv_cache_compression_tri_amd.synth import device as SD
    from kv_cache_compression_tri_amd.synth import workloads as W

    w = W.WORKLOADS[name]
    dw = SD.build(w)
    kv = dw.kv()
    if positions:   # explicit positions (equal to the slot index, so the scores are unchanged)
        n_slots = kv.slots
        kv.pos = torch.arange(n_slots, dtype=torch.int32, device=dw.k.device).expand(
            w.n_seq, w.n_layer, w.n_kvh, n_slots).contiguous()
    dev = dw.k.device
    lengths = [int(x) for x in dw.hp.lengths]
    keys_per_step = sum(lengths) * w.n_layer * w.n_kvh
    slots = kv.slots
    compacts = w.with_values          # the single-head f32 case is scoring + selection only
    scores = torch.empty((w.n_seq, w.n_layer, w.n_kvh, slots), dtype=torch.float32, device=dev)
    kept = torch.empty((w.n_seq, w.n_layer, w.n_kvh, w.budget), dtype=torch.int32, device=dev)
    kept_n = torch.empty((w.n_seq,), dtype=torch.int32, device=dev)
    pos_out = torch.empty((w.n_seq, w.n_layer, w.n_kvh, w.budget), dtype=torch.int32, device=dev)
    new_len = torch.empty((w.n_seq,), dtype=torch.int32, device=dev)
    if w.paged:                       # in place: freed page list instead of output tensors
        k_out = v_out = None
        freed = torch.empty((w.n_seq, w.max_pages), dtype=torch.int32, device=dev)
        n_freed = torch.empty((w.n_seq,), dtype=torch.int32, device=dev)
    else:
        k_out = torch.empty((w.n_seq, w.n_layer, w.n_kvh, w.budget, w.head_dim), dtype=dw.k.dtype, device=dev)
        v_out = torch.empty_like(k_out) if dw.v is not None else None
        freed = n_freed = None

    # the selection's workspace (units longer than 32768 slots: two-stage selection), allocated once
    sel_ws = tri.select_workspace(scores, kv, w.budget, w.window, kept, kept_n)

    def step(ev=None):
        # ev: events recorded before the score kernel and after it (the timed loop), plus after
        # the selection and after the compaction (the breakdown loop); None entries are skipped
        if ev is not None and ev[0] is not None:
            ev[0].record()
        if fused:   # one launch scores and selects (its time is counted as the score kernel's)
            tri.tri_score_select(kv, dw.center, dw.mean_abs, w.budget, w.window, rope_base=w.base,
                                 offsets=w.offsets, group=w.group, reduce=w.reduce, rope_layout=w.layout,
                                 kept=kept, kept_n=kept_n)
        else:
            tri.tri_score_keys(kv, dw.center, dw.mean_abs, rope_base=w.base, offsets=w.offsets, group=w.group,
                               reduce=w.reduce, rope_layout=w.layout, scores=scores, key_space=key_space,
                               form=form)
        if ev is not None and ev[1] is not None:
            ev[1].record()
        if not fused:
            tri.tri_select_topb(scores, kv, w.budget, w.window, kept=kept, kept_n=kept_n, workspace=sel_ws)
        if ev is not None and ev[2] is not None:
            ev[2].record()
        if compacts:
            tri.tri_compact_kv(kv, kept, kept_n, w.budget, k_out=k_out, v_out=v_out, pos_out=pos_out,
                               freed=freed, n_freed=n_freed, new_len=new_len)
        if ev is not None and ev[3] is not None:
            ev[3].record()

    def regenerate():
        # in-place (paged) compaction rewrites the pools: restore them outside the timed region
        if w.paged:
            SD.fill(w, dw.hp, dw.k, dw.v, dw.seq_len, dw.block_table)

    preroll = {"ms": 0.0, "passes": 0}
    if preroll_ms > 0:
        # Untimed clock pre-roll: under sustained load the GPU's clock first dips (the score
        # kernel runs ~495 us for the first passes, ~575 us around passes 5-10, and settles near
        # 470-480 us after ~40 passes of the 32K pass); passes run back to back until preroll_ms
        # of wall time has passed, so that the timed passes see the steady state of a serving loop.
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < preroll_ms:
            for _ in range(8):
                regenerate()
                step()
                preroll["passes"] += 1
            torch.cuda.synchronize()
        preroll["ms"] = (time.perf_counter() - t0) * 1e3
    for _ in range(warmup):
        regenerate()
        step()
    torch.cuda.synchronize()
    # Timed loop: the steps run back to back; the only events inside it bracket the score
    # kernel (its average launch duration for the roofline) and the whole loop.
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] + [None, None] for _ in range(steps)]
    loop_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    if w.paged:
        ms_total = 0.0
        for i in range(steps):
            regenerate()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            step(events[i])
            torch.cuda.synchronize()
            ms_total += (time.perf_counter() - t0) * 1e3
        ms = ms_total / steps
        loop_event_ms = None
    else:
        t0 = time.perf_counter()
        loop_ev[0].record()
        for i in range(steps):
            step(events[i])
        loop_ev[1].record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms = (t1 - t0) * 1e3 / steps
        loop_event_ms = loop_ev[0].elapsed_time(loop_ev[1]) / steps
    score_ms = sum(e[0].elapsed_time(e[1]) for e in events) / steps

    # Breakdown loop (after the timed region, not part of the value): events between all
    # three kernels of each step, for the selection and compaction times.
    n_bd = min(steps, 10)
    bd = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_bd)]
    for i in range(n_bd):
        regenerate()
        step(bd[i])
    torch.cuda.synchronize()
    step_ms = sorted(e[0].elapsed_time(e[3]) for e in bd)           # per-step GPU time (events)
    select_ms = sum(e[1].elapsed_time(e[2]) for e in bd) / n_bd
    compact_ms = sum(e[2].elapsed_time(e[3]) for e in bd) / n_bd
    elt = {"f32": 4, "bf16": 2, "fp8": 1, "int8": 1}[w.dtype]
    score_bytes = keys_per_step * w.head_dim * elt                       # every key read once
    kept_rows = w.n_layer * w.n_kvh * sum(min(w.budget, L) for L in lengths)
    compact_bytes = kept_rows * w.head_dim * elt * 2 * 2 if compacts else 0   # K and V, read + write
    pass_bytes = score_bytes + compact_bytes
    cons = None
    if with_consumer and compacts and w.dtype in ("f32", "bf16"):
        cons = consumer(args, w, dw, kv, kept_n, new_len, k_out, v_out, pos_out)
    del dw, kv, scores, kept, kept_n, k_out, v_out, pos_out, new_len, freed, n_freed
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {
        "w": w, "name": name, "steps": steps, "warmup": warmup, "ms": ms, "loop_event_ms": loop_event_ms,
        "score_ms": score_ms, "select_ms": select_ms, "compact_ms": compact_ms, "step_ms": step_ms, "n_bd": n_bd,
        "keys_per_step": keys_per_step, "score_bytes": score_bytes, "pass_bytes": pass_bytes,
        "compacts": compacts, "consumer": cons, "preroll": preroll,
    }


def config_entry(m, fused=False):
    """Summary of one workload's measurement for the `configs` object."""
    w = m["w"]
    ms = m["ms"]
    return {
        "value": m["keys_per_step"] / (ms * 1e-3) / 1e9, "unit": "Gkeys/s", "ms_per_step": ms,
        "steps": m["steps"], "warmup": m["warmup"], "clock_preroll_ms": round(m["preroll"]["ms"], 1),
        "pass_hbm_frac": m["pass_bytes"] / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "score_kernel_hbm_frac": m["score_bytes"] / (m["score_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "score_ms": m["score_ms"], "select_ms": m["select_ms"], "compact_ms": m["compact_ms"],
        "score_kernel": "score_select_kernel" if fused else score_kernel_used(w, "pre", "additive", False),
        "fused_score_select": fused,
        "keys_per_step": m["keys_per_step"], "algorithmic_bytes": m["pass_bytes"],
        "shape": {"n_seq": w.n_seq, "n_layer": w.n_layer, "n_kv_heads": w.n_kvh, "group": w.group,
                  "context": w.max_len, "kv_dtype": w.dtype, "budget": w.budget, "window": w.window,
                  "reduce": w.reduce, "layout": "paged" if w.paged else "dense"},
        **({"consumer": m["consumer"]} if m["consumer"] is not None else {}),
    }


# The pages' end-to-end figures at 32K-token generation: context only, never a target (they
# need trained models and a serving stack; the pages do not state their hardware).
PAGES_CONTEXT = {
    "decode_throughput_vs_full_attention": 2.5,
    "kv_memory_reduction": 10.7,
    "setting": "32K-token generation, KV budget 3072, AIME25; hardware not stated on the pages "
               "(a 24 GB RTX 4090 deployment is described); not comparable with this pass",
}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(units are independent, so N GPUs would each run this pass on their share)",
              file=sys.stderr)
        return 2
    import torch
    if args.copy_probe:
        moved, gbs = copy_bandwidth(args.copy_probe)
        print(json.dumps({"copy_probe_bytes_read": moved // 2, "copy_probe_bytes_written": moved // 2,
                          "copy_GBps": gbs}), flush=True)
        return 0
    from kv_cache_compression_tri_amd.synth import workloads as W

    name = args.workload or W.BENCH_WORKLOAD
    if name not in W.WORKLOADS:
        print(f"unknown workload {name!r}; choose from {sorted(W.WORKLOADS)}", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    fused = use_fused(args.fused, W.WORKLOADS[name], n_cu, args.key_space, args.form, args.positions)
    m = measure(args, name, args.steps, args.warmup, args.key_space, args.form, args.positions, not args.no_consumer,
                args.preroll_ms, fused=fused)
    w = m["w"]
    ms, score_ms = m["ms"], m["score_ms"]
    keys_per_step, score_bytes, pass_bytes = m["keys_per_step"], m["score_bytes"], m["pass_bytes"]
    step_ms = m["step_ms"]
    achieved = score_bytes / (score_ms * 1e-3) / 1e9
    lane_ops = score_lane_ops_per_key(1 if w.reduce == "mean" else w.group, args.key_space, args.form)
    alu_achieved = lane_ops * keys_per_step / (score_ms * 1e-3) / 1e12
    value = keys_per_step / (ms * 1e-3) / 1e9
    traffic = recorded_traffic(name) if (args.key_space == "pre" and args.form == "additive"
                                         and not args.positions) else None
    kernel = "score_select_kernel" if fused else score_kernel_used(w, args.key_space, args.form, args.positions)
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "Gkeys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "clock_preroll": {"ms": m["preroll"]["ms"], "passes": m["preroll"]["passes"], "timed": False,
                          "why": "untimed passes before the warmup so that the timed passes run at the "
                                 "steady clock of sustained load (the clock dips over the first ~25 ms)"},
        "config": {
            "workload": name,
            "n_seq": w.n_seq, "n_layer": w.n_layer, "n_kv_heads": w.n_kvh, "group": w.group,
            "context": w.max_len, "head_dim": w.head_dim, "kv_dtype": w.dtype, "budget": w.budget,
            "window": w.window, "offsets": len(w.offsets), "reduce": w.reduce,
            "layout": "paged" if w.paged else "dense", "compaction": m["compacts"], "key_space": args.key_space,
            "form": args.form, "explicit_positions": bool(args.positions), "fused_score_select": fused,
            "keys_per_step": keys_per_step, "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": kernel,
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": score_bytes,
            "avg_launch_ms": score_ms,
        },
        "alu": {
            "bound": "alu",
            "kernel": kernel,
            # on the matrix-core kernel the head contraction runs on the bf16 matrix cores, so this
            # vector-ALU figure then counts work the VALUs do not do
            "head_contraction": "mfma_bf16" if kernel == "score_mx_kernel" else "valu",
            "lane_ops_per_key": lane_ops,
            "achieved": alu_achieved,
            "peak": PEAK_VALU_TLANEOPS,
            "unit": "Tlane-op/s",
            "frac": alu_achieved / PEAK_VALU_TLANEOPS,
        },
        "pass": {
            "algorithmic_bytes": pass_bytes,
            "hbm_frac": pass_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "score_ms": score_ms, "select_ms": m["select_ms"], "compact_ms": m["compact_ms"],
            "loop_event_ms_per_step": m["loop_event_ms"],
            "breakdown_steps": m["n_bd"],
            "step_event_ms": {"median": step_ms[len(step_ms) // 2], "min": step_ms[0],
                              "p90": step_ms[min(len(step_ms) - 1, int(0.9 * len(step_ms)))]},
            "algorithmic_GBps": pass_bytes / (ms * 1e-3) / 1e9,
        },
    }
    if m["consumer"] is not None:
        line["consumer"] = m["consumer"]
    # The other stated workloads, each timed in this run after the headline (same protocol: the
    # untimed clock pre-roll and warmup passes, then exactly the given number of timed passes;
    # the paged pools are refilled before every pass, outside the timed region).  Their pass
    # counts are capped so that the default run stays within a few minutes.
    if not args.workload and not args.no_configs and args.key_space == "pre" and args.form == "additive" \
            and not args.positions and args.fused != "on":
        configs = {}
        for other in W.STATED_WORKLOADS:
            if other == name:
                continue
            paged = W.WORKLOADS[other].paged
            k = min(args.steps, 20 if paged else 200)
            wu = min(args.warmup, 5 if paged else 50)
            fo = use_fused(args.fused, W.WORKLOADS[other], n_cu)
            configs[other] = config_entry(measure(args, other, max(k, 1), wu, with_consumer=not args.no_consumer,
                                                  preroll_ms=args.preroll_ms, fused=fo), fo)
        line["configs"] = configs
    _, copy_gbs = copy_bandwidth(1024)
    line["pass"]["copy_GBps"] = copy_gbs
    line["pass"]["frac_of_copy"] = pass_bytes / (ms * 1e-3) / 1e9 / copy_gbs
    line["context_from_pages"] = PAGES_CONTEXT
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(name, args.cpu_units, args.key_space, args.form)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
