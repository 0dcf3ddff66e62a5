"""Failure handling forced from the host, on the GPU path (every kernel runs
normally; the conditions are made by host-side hooks):

* slot fills held back on their copy streams (a slow link) change nothing:
  outputs bit-identical to an undelayed cache, tables and logs as the oracle's;
* an allocation that fails inside moe_cache_create returns MOE_ENOMEM, and the
  device memory the attempt took is given back;
* an allocation that fails inside moe_layer_forward returns MOE_ENOMEM and the
  cache goes on working, call for call as the oracle."""

import numpy as np
import pytest

import synth
from layer_check import Runner, log

pytestmark = pytest.mark.gpu

ENOMEM = -2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import expert_cache_host_amd as m
    m.load_library()


def _lib():
    from expert_cache_host_amd.binding import load_library
    return load_library()


@pytest.mark.parametrize("mode,T,policy", [("host", 1, "lru"), ("host", 3, "lru"),
                                           ("stream", 64, "lru"), ("host", 1, "score")])
def test_delayed_fills_change_nothing(mode, T, policy):
    """Host mode publishes a call's fills at the layer's next call; staged
    stream calls wait for each stage's fills.  With every fill batch held 4 ms
    on its copy stream, both caches give the same bits (the score policy's
    admitted fills too)."""
    wl = synth.Workload("delay", 80, 2, 256, 512, 16, 4, 4, n_shared=1, router_sigma=0.12,
                        zipf_s=0.6, rho=0.6 if T < 64 else None, tokens=8 * T, batch=T)
    log(f"delayed fills mode={mode} T={T} policy={policy}")
    ref = Runner(wl, [0, 1], mode=mode, policy=policy)
    slow = Runner(wl, [0, 1], mode=mode, weights=ref.weights, policy=policy)
    assert _lib().moe_debug_fill_delay(slow.cache._h, 4000) == 0
    xs = [synth.gen_hidden(wl, l, 8) for l in (0, 1)]
    fills = 0
    for t in range(8):
        for li in (0, 1):
            a, _ = ref.call(li, xs[li][t])
            b, res = slow.call(li, xs[li][t])
            np.testing.assert_array_equal(a, b)
            fills += res.fills
    assert fills > 0
    ref.check_log()
    slow.check_log()
    ref.close()
    slow.close()


def _device_free():
    import torch
    torch.cuda.synchronize()
    return torch.cuda.mem_get_info()[0]


def _rss():
    with open("/proc/self/status") as f:
        for line in f:
            if line.startswith("VmRSS:"):
                return int(line.split()[1]) * 1024
    return 0


@pytest.mark.parametrize("mode", ["host", "stream"])
def test_create_allocation_failure_frees_everything(mode):
    """Every allocation of moe_cache_create in turn is made to fail: MOE_ENOMEM
    with a message, device memory back where it was (the slot arenas are ~0.7
    GB, so a leak would show), host memory not grown; past the last allocation
    the create succeeds."""
    import ctypes

    from expert_cache_host_amd.binding import Opts
    lib = _lib()
    wl = synth.Workload("oom", 81, 2, 6144, 2048, 16, 4, 16, n_shared=1, router_sigma=0.02,
                        rho=0.5, tokens=2, batch=1)
    weights = synth.gen_all_weights(wl)
    o = Opts()
    lib.moe_cache_default_opts(ctypes.byref(o))
    o.top_k, o.n_shared, o.miss_mode = 4, 1, 1 if mode == "host" else 0
    h = ctypes.c_void_p()
    # warm the runtime once, so that its own first-use allocations are not counted
    assert lib.moe_cache_create(2, 16, 16, 6144, 2048, weights.ctypes.data, ctypes.byref(o),
                                ctypes.byref(h)) == 0
    lib.moe_cache_destroy(h)
    free0, rss0 = _device_free(), _rss()
    nth, created = 0, False
    while not created:
        assert nth < 64
        assert lib.moe_debug_fail_alloc(nth) == 0
        rc = lib.moe_cache_create(2, 16, 16, 6144, 2048, weights.ctypes.data, ctypes.byref(o),
                                  ctypes.byref(h))
        msg = lib.moe_last_error()
        lib.moe_debug_fail_alloc(-1)
        if rc == 0:
            created = True
            lib.moe_cache_destroy(h)
        else:
            assert rc == ENOMEM, (nth, rc, msg)
            assert msg
            assert not h.value
        free1 = _device_free()
        assert abs(free1 - free0) <= (64 << 20), (nth, free0 - free1)
        assert _rss() - rss0 <= (256 << 20), (nth, _rss() - rss0)
        nth += 1
    log(f"create {mode}: {nth - 1} allocation points, each fails cleanly")
    assert nth >= 5


@pytest.mark.parametrize("mode", ["host", "stream"])
def test_forward_allocation_failure_keeps_the_cache(mode):
    """A call that must grow the workspace fails its allocation: MOE_ENOMEM, no
    state change (the oracle's tables stay in step), and the next calls work."""
    import torch
    lib = _lib()
    wl = synth.Workload("oomf", 82, 1, 256, 512, 16, 4, 6, n_shared=1, router_sigma=0.12,
                        zipf_s=0.6, rho=None, tokens=40, batch=20)
    r = Runner(wl, [0], mode=mode)
    x = synth.gen_hidden(wl, 0, 2)
    r.call(0, x[0][:1])
    w_r, b, w_d, b_d = r.routers[0]
    xd = torch.from_numpy(np.ascontiguousarray(x[1])).cuda()
    out = torch.empty_like(xd)
    assert lib.moe_debug_fail_alloc(0) == 0
    rc = lib.moe_layer_forward(r.cache._h, 0, xd.data_ptr(), xd.shape[0], w_d.data_ptr(),
                               b_d.data_ptr(), out.data_ptr(),
                               torch.cuda.current_stream().cuda_stream)
    msg = lib.moe_last_error()
    lib.moe_debug_fail_alloc(-1)
    assert rc == ENOMEM and msg
    assert r.cache.stats()["calls"] == 1
    r.call(0, x[1])
    r.call(0, x[0][:3])
    r.check_log()
    r.close()
