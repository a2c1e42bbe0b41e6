"""Summarize a rocprofv3 kernel-trace database of one bench.py run as markdown: per-kernel
statistics, with the pass kernels (scoring, selection, compaction) and the attention calls over
the compressed cache attributed to the workload whose scoring kernel ran last (bench.py times
one workload after another).

    python -m kv_cache_compression_tri_amd.profsum RESULTS_DB TITLE "COMMAND" [NOTE]
"""

import sqlite3
import statistics
import sys

# scoring-kernel names of the stated workloads, as bench.py launches them by default
PHASES = {
    "tri::score_mx_kernel<4, false, false, false, 1>": "gqa8b_32k_bf16",
    "tri::score_kernel<1, 0, false, false, false, false, false>": "single_head_2k_f32",
    "tri::score_select_kernel<1, 0, false, false>": "single_head_2k_f32",
    "tri::score_select_kernel<1, 1, false, false>": "gqa8b_batch16_16k_bf16",
    "tri::score_mx_kernel<7, false, false, false, 1>": "long_128k_bf16",
    "tri::score_mx_kernel<4, false, true, false, 1>": "paged_ragged64_bf16",
}
PASS_PREFIXES = ("tri::score", "tri::select", "tri::compact", "tri::decode")   # decode: the consumer calls


def short(name: str) -> str:
    s = name.replace("void ", "").replace("(anonymous namespace)::", "").split("(")[0]
    return s.split("<")[0] if s.startswith("at::native::") else s


def main(argv):
    db_path, title, cmd = argv[1], argv[2], argv[3]
    note = argv[4] if len(argv) > 4 else ""
    rows = list(sqlite3.connect(db_path).execute("select name, start, end from kernels order by start"))
    by = {}
    phase = None
    for n, s, e in rows:
        k = short(n)
        if k in PHASES:
            phase = PHASES[k]
        key = (phase if k.startswith(PASS_PREFIXES) else "-", k)
        by.setdefault(key, []).append((e - s) / 1e3)
    out = [f"# {title}\n", f"Command (run from /tmp with TMPDIR=/tmp; R = repository root):\n\n    {cmd}\n"]
    if note:
        out.append(note + "\n")
    out.append("| workload | kernel | dispatches | average us | median us | min us | max us |")
    out.append("|---|---|---|---|---|---|---|")
    order = list(PHASES.values()) + [None, "-"]
    for (ph, k), v in sorted(by.items(), key=lambda kv: (order.index(kv[0][0]), -sum(kv[1]))):
        out.append(f"| {ph or '-'} | `{k}` | {len(v)} | {statistics.mean(v):.1f} | {statistics.median(v):.1f} | "
                   f"{min(v):.1f} | {max(v):.1f} |")
    print("\n".join(out))


if __name__ == "__main__":
    main(sys.argv)
