"""Builds libmoecache.so in-tree: host C++ with g++, gfx950 kernels with hipcc;
also the streaming-read probe (expert_cache_host_amd/_build/readbw).

    python -m expert_cache_host_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmoecache.so")
BUILD = os.path.join(HERE, "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

# Packed fp32 instructions stay off; hipcc's host pass warns that it does not
# know the feature, which is harmless.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
CXX_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", "-ffp-contract=off"]


def _jobs():
    inc = ["-I", os.path.join(ROCM, "include"), "-D__HIP_PLATFORM_AMD__"]
    return [
        ([HIPCC] + HIP_FLAGS + ["-c", os.path.join(CSRC, "kernels.hip"), "-o",
                                os.path.join(BUILD, "kernels.o")]),
        (["g++"] + CXX_FLAGS + inc + ["-c", os.path.join(CSRC, "api.cpp"), "-o",
                                      os.path.join(BUILD, "api.o")]),
        (["g++"] + CXX_FLAGS + ["-c", os.path.join(CSRC, "planner.cpp"), "-o",
                                os.path.join(BUILD, "planner.o")]),
        (["g++"] + CXX_FLAGS + ["-c", os.path.join(CSRC, "host_expert.cpp"), "-o",
                                os.path.join(BUILD, "host_expert.o")]),
        (["g++"] + CXX_FLAGS + ["-c", os.path.join(CSRC, "workspace.cpp"), "-o",
                                os.path.join(BUILD, "workspace.o")]),
        (["g++"] + CXX_FLAGS + ["-c", os.path.join(CSRC, "host_routing.cpp"), "-o",
                                os.path.join(BUILD, "host_routing.o")]),
        # the streaming-read probe (a measurement aid, not part of the library)
        ([HIPCC] + HIP_FLAGS + [os.path.join(HERE, "probes", "readbw.hip"), "-o",
                                os.path.join(BUILD, "readbw")]),
    ]


def build(verbose: bool = False) -> str:
    """Compiles every source (always) and links the shared library."""
    os.makedirs(BUILD, exist_ok=True)
    procs = []
    for cmd in _jobs():
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for cmd, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        if p.returncode != 0:
            failed.append((cmd, text))
        elif verbose and text.strip():
            print(text, flush=True)
    if failed:
        msg = "\n".join(" ".join(c) + "\n" + t for c, t in failed)
        raise RuntimeError("libmoecache build failed:\n" + msg)
    objs = [os.path.join(BUILD, n) for n in ("kernels.o", "api.o", "planner.o", "host_expert.o",
                                             "workspace.o", "host_routing.o")]
    tmp = OUT + f".tmp{os.getpid()}"
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs + [
        "-L" + os.path.join(ROCM, "lib"), "-lrocprofiler-sdk-roctx", "-pthread"]
    if verbose:
        print(" ".join(link), flush=True)
    r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("libmoecache link failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
