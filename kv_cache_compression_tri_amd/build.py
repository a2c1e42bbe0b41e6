"""Build libtri.so (the compression pass) and libtri_synth.so (input generator) for gfx950.

Sources are compiled in-tree with hipcc into kv_cache_compression_tri_amd/lib/.  Packed
FP32 instructions are disabled on the device side (the host pass warns that it does not
know the feature; that is harmless).
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_DIR = os.path.join(PKG, "lib")
BUILD_DIR = os.path.join(PKG, "_build")
ARCH = os.environ.get("TRI_OFFLOAD_ARCH", "gfx950")

LIBS = {
    "libtri.so": {
        "dir": os.path.join(PKG, "csrc"),
        "sources": ["api.hip", "score.hip", "score_post.hip", "score_8bit.hip", "score_post_8bit.hip",
                    "score_mult.hip", "score_post_mult.hip", "score_mult_8bit.hip", "score_post_mult_8bit.hip",
                    "score_pos.hip", "score_pos_8bit.hip", "score_mx.hip", "score_mx_paged.hip", "score_mx_post.hip", "score_mx_post_paged.hip", "score_mx_post_8bit.hip", "score_select.hip", "score_select_f32.hip",
                    "score_select_paged.hip", "score_select_f32_paged.hip",
                    "select.hip", "compact.hip", "calib.hip", "decode.hip"],
        "includes": [os.path.join(ROOT, "include"), os.path.join(PKG, "csrc")],
    },
    "libtri_synth.so": {
        "dir": os.path.join(PKG, "synth", "csrc"),
        "sources": ["synth.hip"],
        "includes": [],
        "flags": ["-ffp-contract=off"],   # the generator's float32 ops round one by one
    },
}

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False, jobs: int = 8, extra_flags=()) -> dict:
    """Compile every HIP source and link both libraries.  Returns {lib: path}."""
    hipcc = _hipcc()
    os.makedirs(LIB_DIR, exist_ok=True)
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs_list = []
    for lib, spec in LIBS.items():
        for src in spec["sources"]:
            obj = os.path.join(BUILD_DIR, f"{lib[:-3]}_{src}.o")
            cmd = [hipcc, *FLAGS, *spec.get("flags", []), *extra_flags, *[f"-I{d}" for d in spec["includes"]],
                   "-c", os.path.join(spec["dir"], src), "-o", obj]
            jobs_list.append((lib, obj, cmd))
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        list(ex.map(lambda j: _run(j[2], verbose), jobs_list))
    out = {}
    for lib in LIBS:
        objs = [o for (lb, o, _) in jobs_list if lb == lib]
        target = os.path.join(LIB_DIR, lib)
        tmp = target + ".tmp"
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp, *objs],
             verbose)
        os.replace(tmp, target)
        out[lib] = target
    return out


if __name__ == "__main__":
    paths = build(verbose="-v" in sys.argv)
    for k, v in paths.items():
        print(k, "->", v)
