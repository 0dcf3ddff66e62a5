"""Summaries of rocprofv3 output for the profiles/ folder.

    python -m expert_cache_host_amd.profiling stats <rocprof dir> <title> <command...>
    python -m expert_cache_host_amd.profiling pmc <rocprof dir> <counter> <title> <command...>
    python -m expert_cache_host_amd.profiling traffic <out.json> <copy fetch dir> <copy write dir> \
        <workload>=<fetch dir>,<write dir> [...]

`stats` reads the *_kernel_stats.csv of a `rocprofv3 --kernel-trace --stats
--output-format csv` run; `pmc` reads the *_counter_collection.csv of a
`rocprofv3 --pmc <counter> --output-format csv` run and averages the counter
per dispatch and kernel.  Both print markdown with the command that produced
the data.
"""
from __future__ import annotations

import csv
import glob
import os
import sys
from collections import defaultdict


def _find(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {d}")
    return hits[0]


def short(name: str, n: int = 90) -> str:
    return name if len(name) <= n else name[:n - 3] + "..."


def stats_md(d: str, title: str, command: str) -> str:
    rows = list(csv.DictReader(open(_find(d, "kernel_stats.csv"))))
    out = [f"# {title}", "", "Command:", "", "```", command, "```", "",
           "| kernel | calls | avg us | total ms | % |", "|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['TotalDurationNs']) / 1e6:.2f} | {float(r['Percentage']):.2f} |")
    return "\n".join(out) + "\n"


def pmc_table(d: str, counter: str):
    f = _find(d, "counter_collection.csv")
    acc = defaultdict(lambda: [0.0, 0])
    for r in csv.DictReader(open(f)):
        if r.get("Counter_Name") != counter:
            continue
        k = r["Kernel_Name"]
        acc[k][0] += float(r["Counter_Value"])
        acc[k][1] += 1
    return {k: (v[0] / v[1], v[1]) for k, v in acc.items()}


def pmc_md(d: str, counter: str, title: str, command: str) -> str:
    t = pmc_table(d, counter)
    out = [f"# {title}", "", "Command:", "", "```", command, "```", "",
           f"| kernel | dispatches | mean {counter} per dispatch (KiB) |", "|---|---|---|"]
    for k, (v, n) in sorted(t.items(), key=lambda kv: -kv[1][0] * kv[1][1]):
        out.append(f"| `{short(k)}` | {n} | {v:.1f} |")
    return "\n".join(out) + "\n"


# kernel classes of the library, as the benchmark names them, and their symbols
CLASSES = {"gateup": "q4_gateup_kernel", "down": "q4_down_kernel", "fill": "pull_kernel",
           "router": "router_kernel", "topk": "topk_", "combine": "combine_kernel",
           "mfma": "q4_mfma_kernel"}
COPY_BYTES = 256 << 20  # bytes read and written by each calibration copy


def _class_means(tab):
    out = {}
    for cls, sym in CLASSES.items():
        tot, n = 0.0, 0
        for k, (v, cnt) in tab.items():
            if sym in k:
                tot += v * cnt
                n += cnt
        if n:
            out[cls] = (tot / n, n)
    return out


def traffic_json(out_path, copy_fetch, copy_write, pairs):
    """Writes the calibrated per-dispatch FETCH/WRITE means the benchmark reads."""
    import hashlib
    import json
    cf = pmc_table(copy_fetch, "FETCH_SIZE")
    cw = pmc_table(copy_write, "WRITE_SIZE")
    ck = [k for k in cf if "copyBuffer" in k][0]
    fetch_scale = COPY_BYTES / (cf[ck][0] * 1024.0)
    write_scale = COPY_BYTES / (cw[ck][0] * 1024.0)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    src = os.path.join(root, "expert_cache_host_amd", "csrc", "kernels.hip")
    data = {"fetch_scale": fetch_scale, "write_scale": write_scale,
            "calibration": f"{ck}: 256 MiB copy reads FETCH_SIZE {cf[ck][0]:.1f} KiB, "
                           f"WRITE_SIZE {cw[ck][0]:.1f} KiB per dispatch",
            "kernel_source_sha256_16": hashlib.sha256(open(src, "rb").read()).hexdigest()[:16],
            "workloads": {}}
    for wl, (fd, wd) in pairs.items():
        f = _class_means(pmc_table(fd, "FETCH_SIZE"))
        w = _class_means(pmc_table(wd, "WRITE_SIZE"))
        data["workloads"][wl] = {c: {"fetch_KiB": f[c][0], "write_KiB": w.get(c, (0.0, 0))[0],
                                     "dispatches": f[c][1]} for c in f}
    with open(out_path, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
        fh.write("\n")
    return data


def main(argv):
    if len(argv) >= 4 and argv[0] == "stats":
        print(stats_md(argv[1], argv[2], " ".join(argv[3:])), end="")
    elif len(argv) >= 5 and argv[0] == "pmc":
        print(pmc_md(argv[1], argv[2], argv[3], " ".join(argv[4:])), end="")
    elif len(argv) >= 5 and argv[0] == "traffic":
        pairs = {}
        for a in argv[4:]:
            wl, dirs = a.split("=", 1)
            fd, wd = dirs.split(",", 1)
            pairs[wl] = (fd, wd)
        traffic_json(argv[1], argv[2], argv[3], pairs)
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
