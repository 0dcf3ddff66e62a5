"""The allocation-free entry point against the ordinary one, through the C ABI.

Two caches built from the same bytes take the same calls, one through
moe_layer_forward and one through moe_layer_forward_noalloc (the library's fixed
per-device scratch).  Outputs must match each other bit for bit (same kernels,
same order) and the oracle within the layer's tolerance; routing, slot tables,
slot state and the replacement log must match the oracle exactly.  Each case
makes two calls in a row per layer, the second with fewer tokens, so the second
runs on scratch that still holds the first call's data.  Calls the scratch
cannot hold are refused with MOE_EINVAL and change nothing."""
import ctypes

import numpy as np
import pytest

import synth
from layer_check import Runner, check_close, log
from oracle.layer import moe_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import expert_cache_host_amd as m
    m.load_library()


CASES = {
    # name: workload, miss mode, tokens of the two calls
    "tiny_stream": (synth.Workload("na_tiny", 70, 1, 256, 512, 8, 2, 4, router_sigma=0.1,
                                   rho=0.8, tokens=8, batch=4), "stream", (4, 2)),
    "tiny_host": (synth.Workload("na_tiny", 70, 1, 256, 512, 8, 2, 4, router_sigma=0.1,
                                 rho=0.8, tokens=8, batch=4), "host", (3, 1)),
    "shared_stream": (synth.Workload("na_sh", 71, 2, 512, 256, 32, 8, 6, n_shared=1,
                                     router_sigma=0.1, zipf_s=0.8, rho=0.7, tokens=8, batch=4),
                      "stream", (4, 1)),
    # 4 tokens x (16 + 1 shared) = 68 pairs: the matrix-core path on scratch
    "matrix_core_host": (synth.Workload("na_mc", 72, 1, 128, 128, 64, 16, 16, n_shared=1,
                                        router_sigma=0.3, zipf_s=0.8, rho=0.5, tokens=8, batch=4),
                         "host", (4, 2)),
    "gemma_host": (synth.Workload("na_gemma", 73, 1, 2816, 704, 128, 8, 32,
                                  router_sigma=1.6 / np.sqrt(2816), zipf_s=1.1, rho=0.8,
                                  tokens=8, batch=2, weight_wid=2), "host", (2, 1)),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_noalloc_matches_ordinary_entry_point(case):
    import torch
    wl, mode, sizes = CASES[case]
    log(f"noalloc {case}: mode={mode} calls of {sizes} tokens")
    ref = Runner(wl, list(range(wl.layers)), mode=mode)
    na = Runner(wl, list(range(wl.layers)), mode=mode, weights=ref.weights)
    x = synth.gen_hidden(wl, 0, 2)
    for rep in range(2):  # two rounds, so each layer also sees a call after a smaller one
        for li in range(wl.layers):
            for ci, T in enumerate(sizes):
                xs = np.ascontiguousarray(x[ci][:T])
                out_ref, res_ref = ref.call(li, xs)
                w_r, b, w_d, b_d = na.routers[li]
                x_d = torch.from_numpy(xs).cuda()
                out = torch.full_like(x_d, float("nan"))
                na.cache.forward(li, x_d, w_d, b_d, out=out, noalloc=True)
                torch.cuda.synchronize()
                got = out.cpu().numpy()
                np.testing.assert_array_equal(got, out_ref)
                o = moe_layer(xs, w_r, b, na.layer_buf(li), wl.d_model, wl.d_ff, wl.n_experts,
                              wl.top_k, n_shared=wl.n_shared)
                check_close(got, o["out64"])
                idx, _ = na.cache.routing(li)
                assert np.array_equal(idx, o["idx"])
                res = na.sims[li].plan(o["idx"].ravel().tolist(), mode, -1, tokens=T)
                ns, nt = na.cache.last_call(li)
                assert (ns, nt) == (len(res.stage_views), T)
                for s in range(ns):
                    sv, hv = na.cache.views(li, s)
                    assert sv.tolist() == res.stage_views[s]
                    assert hv.tolist() == res.host_view
                ein, lu = na.cache.slot_state(li)
                assert ein.tolist() == na.sims[li].expert_in
                assert lu.tolist() == na.sims[li].last_use
    na.check_log()
    ref.check_log()
    a, b_ = ref.cache.stats(), na.cache.stats()
    for key in ("calls", "hits", "misses", "fills", "evictions", "host_selections", "stages"):
        assert a[key] == b_[key], key
    ref.close()
    na.close()


def test_noalloc_refuses_what_it_cannot_hold():
    """More than 4 tokens, a workspace past the 16 MiB scratch, or a cache with
    keep_debug: MOE_EINVAL with a message, and the cache unchanged (the next
    calls still match the oracle)."""
    import torch

    from expert_cache_host_amd.binding import load_library
    lib = load_library()
    wl = synth.Workload("na_ref", 74, 1, 256, 512, 8, 2, 4, router_sigma=0.1, rho=0.8,
                        tokens=8, batch=1)
    log("noalloc refusals")
    r = Runner(wl, [0], mode="stream")
    w_r, b, w_d, b_d = r.routers[0]
    x = synth.gen_hidden(wl, 0, 8)
    st = torch.cuda.current_stream().cuda_stream
    x5 = torch.zeros((5, wl.d_model), device="cuda")
    o5 = torch.empty_like(x5)
    rc = lib.moe_layer_forward_noalloc(r.cache._h, 0, x5.data_ptr(), 5, w_d.data_ptr(), None,
                                       o5.data_ptr(), st)
    assert rc == -1 and b"4" in lib.moe_last_error()
    assert r.cache.stats()["calls"] == 0
    for t in range(4):
        r.call(0, x[t])
    r.check_log()
    r.close()
    # 4 tokens x 64 experts x d_model 16384 floats of outputs alone exceed 16 MiB
    big = synth.Workload("na_big", 75, 1, 16384, 32, 64, 64, 64, router_sigma=0.01, rho=0.5,
                         tokens=4, batch=4)
    rb = Runner(big, [0], mode="stream")
    xb = torch.zeros((4, big.d_model), device="cuda")
    ob = torch.empty_like(xb)
    rc = lib.moe_layer_forward_noalloc(rb.cache._h, 0, xb.data_ptr(), 4, rb.routers[0][2].data_ptr(),
                                       None, ob.data_ptr(), st)
    assert rc == -1 and b"scratch" in lib.moe_last_error()
    assert rb.cache.stats()["calls"] == 0
    rb.close()
    rd = Runner(wl, [0], mode="stream", keep_debug=True)
    x1 = torch.zeros((1, wl.d_model), device="cuda")
    o1 = torch.empty_like(x1)
    rc = lib.moe_layer_forward_noalloc(rd.cache._h, 0, x1.data_ptr(), 1, rd.routers[0][2].data_ptr(),
                                       None, o1.data_ptr(), st)
    assert rc == -1 and b"keep_debug" in lib.moe_last_error()
    rd.close()
