"""Summaries of rocprofv3 output for the profiles/ folder.

    python -m expert_cache_host_amd.profiling stats <rocprof dir> <title> <command...>
    python -m expert_cache_host_amd.profiling pmc <rocprof dir> <counter> <title> <command...>
    python -m expert_cache_host_amd.profiling traffic <out.json> <copy fetch dir> <copy write dir> \
        <workload>=<fetch dir>,<write dir> [...]

    python -m expert_cache_host_amd.profiling copies <rocprof dir> <record bytes> <title> <command...>
    python -m expert_cache_host_amd.profiling mfma <rocprof dir> <title> <command...>
    python -m expert_cache_host_amd.profiling timeline <rocprof dir> <first kernel> <count>
    python -m expert_cache_host_amd.profiling markers <rocprof dir> <title> <command...>
    python -m expert_cache_host_amd.profiling pulls <rocprof dir> <record bytes> <workgroups per record>

`stats` reads the *_kernel_stats.csv of a `rocprofv3 --kernel-trace --stats
--output-format csv` run; `pmc` reads the *_counter_collection.csv of a
`rocprofv3 --pmc <counter> --output-format csv` run and averages the counter
per dispatch and kernel.  `copies` reads the *_memory_copy_trace.csv of a
`--memory-copy-trace` run: every host-to-device copy that starts after the
first expert kernel is a slot fill of one record, and the link rate is the
bytes over the time at least one such copy is in flight.  `mfma` reads a
`--pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_BUSY_CYCLES
GRBM_GUI_ACTIVE` run.  All print markdown with the command that produced the
data.
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
    hits = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if hits:
        out += ["", by_shape_md(d)]
    return "\n".join(out) + "\n"


def by_shape(d: str, marker: str = "moe::q4_"):
    """Dispatches of the expert kernels grouped by kernel and row tiles per
    launch (grid x in workgroups): one kernel serves several layer shapes, and
    the row tiles tell them apart.  {(kernel, tiles): (dispatches, mean us)}."""
    acc = defaultdict(lambda: [0, 0])
    for r in csv.DictReader(open(_find(d, "kernel_trace.csv"))):
        if marker not in r["Kernel_Name"]:
            continue
        tiles = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
        k = (r["Kernel_Name"].split("(")[0].replace("void ", ""), tiles)
        acc[k][0] += 1
        acc[k][1] += int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    return {k: (n, t / n / 1e3) for k, (n, t) in acc.items()}


def by_shape_md(d: str) -> str:
    out = ["Expert kernels by launch shape (row tiles = workgroups along x; from the kernel trace):",
           "", "| kernel | row tiles | dispatches | avg us |", "|---|---|---|---|"]
    for (k, tiles), (n, us) in sorted(by_shape(d).items(), key=lambda kv: (kv[0][0], -kv[0][1])):
        out.append(f"| `{k}` | {tiles} | {n} | {us:.2f} |")
    return "\n".join(out)


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


def copies_md(d: str, record_bytes: int, title: str, command: str) -> str:
    kt = list(csv.DictReader(open(_find(d, "kernel_trace.csv"))))
    first = min(int(r["Start_Timestamp"]) for r in kt if "q4_" in r["Kernel_Name"])
    rows = [r for r in csv.DictReader(open(_find(d, "memory_copy_trace.csv")))
            if r["Direction"] == "MEMORY_COPY_HOST_TO_DEVICE" and int(r["Start_Timestamp"]) >= first]
    iv = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows)
    busy, cur_s, cur_e = 0, None, None
    for a, b in iv:
        if cur_e is None or a > cur_e:
            if cur_e is not None:
                busy += cur_e - cur_s
            cur_s, cur_e = a, b
        else:
            cur_e = max(cur_e, b)
    if cur_e is not None:
        busy += cur_e - cur_s
    n = len(iv)
    per = [b - a for a, b in iv]
    mean_us = sum(per) / n / 1e3 if n else 0.0
    out = [f"# {title}", "", "Command:", "", "```", command, "```", "",
           "Host-to-device slot fills on the copy engines (one record each, "
           f"{record_bytes:,} bytes), after the first expert kernel:", "",
           "| fills | mean copy (us) | per-copy GB/s | link busy (ms) | link GB/s while busy |",
           "|---|---|---|---|---|"]
    if n:
        out.append(f"| {n} | {mean_us:.1f} | {record_bytes / (mean_us * 1e3):.1f} | {busy / 1e6:.1f} | "
                   f"{n * record_bytes / busy:.1f} |")
    return "\n".join(out) + "\n"


def timeline_md(d: str, anchor: str, count: int) -> str:
    """One call's kernels: `count` dispatches from the first `anchor` kernel at or
    after the middle of the trace, with start and end relative to the first."""
    rows = sorted(csv.DictReader(open(_find(d, "kernel_trace.csv"))),
                  key=lambda r: int(r["Start_Timestamp"]))
    i = next(j for j in range(len(rows) // 2, len(rows)) if anchor in rows[j]["Kernel_Name"])
    t0 = int(rows[i]["Start_Timestamp"])
    out = ["| kernel | workgroups | start us | end us |", "|---|---|---|---|"]
    for r in rows[i:i + count]:
        name = r["Kernel_Name"].split("(")[0].replace("void ", "")
        wg = 1
        for a in "XYZ":
            wg *= max(1, int(r["Grid_Size_" + a]) // max(1, int(r["Workgroup_Size_" + a])))
        out.append(f"| `{name}` | {wg} | {(int(r['Start_Timestamp']) - t0) / 1e3:.1f} | "
                   f"{(int(r['End_Timestamp']) - t0) / 1e3:.1f} |")
    return "\n".join(out) + "\n"


def pulls_md(d: str, record_bytes: int, wg_per_record: int) -> str:
    """Pull-kernel launches grouped by the records they carry (grid size / workgroups per record)."""
    import statistics
    by = defaultdict(list)
    for r in csv.DictReader(open(_find(d, "kernel_trace.csv"))):
        if "pull_kernel" not in r["Kernel_Name"]:
            continue
        n = int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"]) // wg_per_record
        by[n].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = ["| records per launch | launches | median us | us per record | GB/s (median) |",
           "|---|---|---|---|---|"]
    for n in sorted(by):
        med = statistics.median(by[n])
        out.append(f"| {n} | {len(by[n])} | {med:.1f} | {med / n:.1f} | {n * record_bytes / med / 1e3:.1f} |")
    return "\n".join(out) + "\n"


def markers_md(d: str, title: str, command: str) -> str:
    """Host-side ranges of a `--marker-trace` run: count, median, mean, p90 (us)."""
    import statistics
    by = defaultdict(list)
    for r in csv.DictReader(open(_find(d, "marker_api_trace.csv"))):
        by[r["Function"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = [f"# {title}", "", "Command:", "", "```", command, "```", "",
           "Host time of the library's named ranges (one per call, or per fill enqueue):", "",
           "| range | count | median us | mean us | p90 us |", "|---|---|---|---|---|"]
    for name in sorted(by, key=lambda k: -statistics.mean(by[k])):
        v = sorted(by[name])
        out.append(f"| `{name}` | {len(v)} | {statistics.median(v):.1f} | {statistics.mean(v):.1f} | "
                   f"{v[int(0.9 * (len(v) - 1))]:.1f} |")
    return "\n".join(out) + "\n"


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_BUSY_CYCLES",
                 "GRBM_GUI_ACTIVE")
XCDS, SIMDS = 8, 1024  # MI355X: 8 accelerator dies, 256 CUs x 4 SIMDs


def mfma_md(d: str, title: str, command: str) -> str:
    f = _find(d, "counter_collection.csv")
    acc = defaultdict(lambda: defaultdict(float))
    n = defaultdict(int)
    dur = defaultdict(float)
    for r in csv.DictReader(open(f)):
        k = r["Kernel_Name"]
        acc[k][r["Counter_Name"]] += float(r["Counter_Value"])
        if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
            n[k] += 1
            dur[k] += (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    out = [f"# {title}", "", "Command:", "", "```", command, "```", "",
           "GRBM_GUI_ACTIVE is summed over the 8 dies, so one die's active cycles are the sum / 8; "
           "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (die cycles x 1024 SIMDs); matrix flops = "
           "SQ_INSTS_VALU_MFMA_MOPS_F16 x 512 (they count the hi/lo split and padded token rows).", "",
           "| kernel | dispatches | mean us | MFMA busy % | matrix TFLOP/s |", "|---|---|---|---|---|"]
    for k in sorted(acc, key=lambda q: -dur[q]):
        c = acc[k]
        if not c.get("SQ_INSTS_VALU_MFMA_MOPS_F16"):
            continue
        busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (c["GRBM_GUI_ACTIVE"] / XCDS * SIMDS) * 100
        tf = c["SQ_INSTS_VALU_MFMA_MOPS_F16"] * 512 / (dur[k] * 1e-6) / 1e12
        out.append(f"| `{short(k)}` | {n[k]} | {dur[k] / n[k]:.1f} | {busy:.1f} | {tf:.0f} |")
    return "\n".join(out) + "\n"


# kernel classes of the library, as the benchmark names them, and their symbols
CLASSES = {"gateup": "q4_gateup_kernel", "down": "q4_down_kernel", "fill": "pull_kernel",
           "router": "router_", "topk": "topk_", "combine": "combine_kernel",
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
    elif len(argv) >= 5 and argv[0] == "copies":
        print(copies_md(argv[1], int(argv[2]), argv[3], " ".join(argv[4:])), end="")
    elif len(argv) == 4 and argv[0] == "pulls":
        print(pulls_md(argv[1], int(argv[2]), int(argv[3])), end="")
    elif len(argv) >= 4 and argv[0] == "markers":
        print(markers_md(argv[1], argv[2], " ".join(argv[3:])), end="")
    elif len(argv) == 4 and argv[0] == "timeline":
        print(timeline_md(argv[1], argv[2], int(argv[3])), end="")
    elif len(argv) >= 4 and argv[0] == "mfma":
        print(mfma_md(argv[1], argv[2], " ".join(argv[3:])), end="")
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
