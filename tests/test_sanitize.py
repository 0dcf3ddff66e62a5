"""The host-only runtime (slot planner, host-miss experts, thread pool, the
per-call device workspace layout, the host's expert selection) built
with g++ under AddressSanitizer and UndefinedBehaviorSanitizer and driven
through random calls (tests/sanitize/host_runtime_driver.cpp): no out-of-bounds
access, no use after free, no undefined behaviour, and the driver's own
invariant checks pass.  The thread pool and the host partial are also built
under ThreadSanitizer: no data race.  CPU only; the GPU code is not part of
these builds."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "expert_cache_host_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_host_runtime_under_sanitizers(tmp_path):
    exe = str(tmp_path / "driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           os.path.join(HERE, "sanitize", "host_runtime_driver.cpp"),
           os.path.join(CSRC, "planner.cpp"), os.path.join(CSRC, "host_expert.cpp"),
           os.path.join(CSRC, "workspace.cpp"), os.path.join(CSRC, "host_routing.cpp"),
           "-pthread", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.stdout[-2000:] +
                                                                     r.stderr[-4000:])


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_thread_pool_under_thread_sanitizer(tmp_path):
    exe = str(tmp_path / "driver_tsan")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=thread",
           os.path.join(HERE, "sanitize", "host_runtime_driver.cpp"),
           os.path.join(CSRC, "planner.cpp"), os.path.join(CSRC, "host_expert.cpp"),
           os.path.join(CSRC, "workspace.cpp"), os.path.join(CSRC, "host_routing.cpp"),
           "-pthread", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1:second_deadlock_stack=1")
    r = subprocess.run([exe, "threads"], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.stdout[-2000:] +
                                                                     r.stderr[-4000:])
    assert "ThreadSanitizer" not in r.stderr, r.stderr[-4000:]
