"""The rocprofv3 summary tool (expert_cache_host_amd/profiling.py) on small
hand-made traces with known answers: pull launches grouped by records carried,
one call's timeline with workgroup counts, expert kernels split by launch
shape, ROCTx range statistics, and the calibrated traffic file the benchmark
reads."""
import csv
import json
import os

from expert_cache_host_amd import profiling as P

KT_FIELDS = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Grid_Size_Y",
             "Grid_Size_Z", "Workgroup_Size_X", "Workgroup_Size_Y", "Workgroup_Size_Z"]


def _write(path, fields, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _kernel(name, t0, t1, groups, wg=256):
    return {"Kernel_Name": name, "Start_Timestamp": t0, "End_Timestamp": t1,
            "Grid_Size_X": groups * wg, "Grid_Size_Y": 1, "Grid_Size_Z": 1,
            "Workgroup_Size_X": wg, "Workgroup_Size_Y": 1, "Workgroup_Size_Z": 1}


def test_pulls_group_launches_by_records(tmp_path):
    rec = 3_346_432
    rows = [_kernel("moe::pull_kernel(moe::PullList)", 0, 60_000, 32),
            _kernel("moe::pull_kernel(moe::PullList)", 100_000, 162_000, 32),
            _kernel("moe::pull_kernel(moe::PullList)", 200_000, 320_000, 64),
            _kernel("void moe::q4_down_kernel<8>(moe::GemvArgs)", 400_000, 405_000, 88)]
    _write(str(tmp_path / "t" / "run_kernel_trace.csv"), KT_FIELDS, rows)
    md = P.pulls_md(str(tmp_path), rec, 32)
    lines = [l for l in md.splitlines() if l.startswith("| 1 ") or l.startswith("| 2 ")]
    one = [c.strip() for c in lines[0].split("|")[1:-1]]
    two = [c.strip() for c in lines[1].split("|")[1:-1]]
    assert one[:4] == ["1", "2", "61.0", "61.0"]      # median of 60 and 62 us
    assert float(one[4]) == round(rec / 61.0 / 1e3, 1)
    assert two[:4] == ["2", "1", "120.0", "60.0"]
    assert float(two[4]) == round(2 * rec / 120.0 / 1e3, 1)


def test_timeline_starts_at_anchor_with_workgroups(tmp_path):
    rows = [_kernel("moe::router_decode_kernel<1>(float)", 0, 5_000, 128),
            _kernel("moe::topk_decode_kernel(float)", 5_000, 11_000, 1, wg=64),
            _kernel("moe::router_decode_kernel<1>(float)", 20_000, 24_500, 128),
            _kernel("moe::topk_decode_kernel(float)", 24_500, 30_000, 1, wg=64)]
    _write(str(tmp_path / "t" / "run_kernel_trace.csv"), KT_FIELDS, rows)
    md = P.timeline_md(str(tmp_path), "router_", 2)
    body = [l for l in md.splitlines() if l.startswith("| `")]
    # the first anchor at or after the middle of the trace: the second router
    assert body[0] == "| `moe::router_decode_kernel<1>` | 128 | 0.0 | 4.5 |"
    assert body[1] == "| `moe::topk_decode_kernel` | 1 | 4.5 | 10.0 |"


def test_markers_statistics(tmp_path):
    fields = ["Function", "Start_Timestamp", "End_Timestamp"]
    rows = [{"Function": "moe.plan", "Start_Timestamp": 0, "End_Timestamp": d}
            for d in (1000, 2000, 3000, 10000)]
    _write(str(tmp_path / "m" / "run_marker_api_trace.csv"), fields, rows)
    md = P.markers_md(str(tmp_path), "t", "cmd")
    row = [l for l in md.splitlines() if l.startswith("| `moe.plan`")][0]
    cells = [c.strip() for c in row.split("|")[1:-1]]
    assert cells == ["`moe.plan`", "4", "2.5", "4.0", "3.0"]  # median, mean, p90 (us)


def test_traffic_json_scales_by_the_copy(tmp_path):
    fields = ["Kernel_Name", "Counter_Name", "Counter_Value", "Dispatch_Id"]
    copy = "__amd_rocclr_copyBuffer"
    n = P.COPY_BYTES
    _write(str(tmp_path / "cf" / "run_counter_collection.csv"), fields,
           [{"Kernel_Name": copy, "Counter_Name": "FETCH_SIZE", "Counter_Value": n / 2048,
             "Dispatch_Id": 1}])
    _write(str(tmp_path / "cw" / "run_counter_collection.csv"), fields,
           [{"Kernel_Name": copy, "Counter_Name": "WRITE_SIZE", "Counter_Value": n / 1024,
             "Dispatch_Id": 1}])
    _write(str(tmp_path / "wf" / "run_counter_collection.csv"), fields,
           [{"Kernel_Name": "void moe::q4_gateup_kernel<8>(x)", "Counter_Name": "FETCH_SIZE",
             "Counter_Value": v, "Dispatch_Id": i} for i, v in ((1, 100.0), (2, 300.0))])
    _write(str(tmp_path / "ww" / "run_counter_collection.csv"), fields,
           [{"Kernel_Name": "void moe::q4_gateup_kernel<8>(x)", "Counter_Name": "WRITE_SIZE",
             "Counter_Value": v, "Dispatch_Id": i} for i, v in ((1, 10.0), (2, 30.0))])
    out = str(tmp_path / "traffic.json")
    d = P.traffic_json(out, str(tmp_path / "cf"), str(tmp_path / "cw"),
                       {"w/host": (str(tmp_path / "wf"), str(tmp_path / "ww"))})
    assert abs(d["fetch_scale"] - 2.0) < 1e-12 and abs(d["write_scale"] - 1.0) < 1e-12
    g = json.load(open(out))["workloads"]["w/host"]["gateup"]
    assert g["fetch_KiB"] == 200.0 and g["write_KiB"] == 20.0 and g["dispatches"] == 2


def test_expert_kernels_split_by_launch_shape(tmp_path):
    """One down kernel serving two layer shapes: 192 row tiles (d_model 6144)
    and 88 (2816) are reported apart, each with its own mean."""
    k = "void moe::q4_down_kernel<8, 4, 4, 1, 1, 4, 1>(moe::GemvArgs, moe::BucketTable)"
    rows = [_kernel(k, 0, 13_000, 192), _kernel(k, 50_000, 64_000, 192),
            _kernel(k, 100_000, 107_000, 88), _kernel(k, 200_000, 208_000, 88),
            _kernel(k, 300_000, 309_000, 88),
            _kernel("moe::combine_kernel(float)", 400_000, 407_000, 6)]
    _write(str(tmp_path / "t" / "run_kernel_trace.csv"), KT_FIELDS, rows)
    t = P.by_shape(str(tmp_path))
    name = "moe::q4_down_kernel<8, 4, 4, 1, 1, 4, 1>"
    assert t == {(name, 192): (2, 13.5), (name, 88): (3, 8.0)}
    md = P.by_shape_md(str(tmp_path))
    assert f"| `{name}` | 192 | 2 | 13.50 |" in md
    assert f"| `{name}` | 88 | 3 | 8.00 |" in md
