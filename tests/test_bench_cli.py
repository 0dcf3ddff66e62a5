"""The benchmark's contract pieces that need no GPU: a request for more than one
GPU ends with a message (this build measures one GPU), the CPU baseline's core
count is the process's CPU affinity, and every kernel name the line reports is
a kernel of the library's source (so that it matches rocprofv3's names)."""
import json
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"] and line["n_gpus_requested"] == 2


def test_cores_are_the_affinity():
    import bench
    assert bench.host_cores() == len(os.sched_getaffinity(0))


def test_reported_kernel_names_exist():
    import bench
    src = open(os.path.join(ROOT, "expert_cache_host_amd", "csrc", "kernels.hip")).read()
    kernels = set(re.findall(r"__global__\s+__launch_bounds__\([^)]*\)\s+void\s+(\w+)\s*\(", src))
    assert len(kernels) >= 10
    for name in set(bench.KERNEL_SYMBOL.values()) | set(bench.KERNEL_SYMBOL_GEMM.values()):
        base = name.split("<")[0]
        assert base in kernels, name
