"""GPU parity of the whole layer through the C ABI, call by call, against the
oracle: bit-exact top-k ids, slot tables, slot state and replacement log;
outputs within 2e-3 of the oracle's RMS."""
import numpy as np
import pytest

import synth
from layer_check import Runner, check_close, log
from oracle.routing import router_logits_fp32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import expert_cache_host_amd as m
    m.load_library()


@pytest.mark.parametrize("mode", ["stream", "host"])
@pytest.mark.parametrize("slots", [1, 2, 4, 8])
def test_tiny_all_calls(mode, slots):
    wl = synth.WORKLOADS["tiny"]
    log(f"tiny mode={mode} slots={slots}")
    r = Runner(wl, [0], slots=slots, mode=mode)
    x = synth.gen_hidden(wl, 0)
    for t in range(x.shape[0]):
        r.call(0, x[t])
    r.check_log()
    st = r.cache.stats()
    assert st["calls"] == 64 and st["selections"] == 128
    assert st["hits"] + st["misses"] == 128
    if slots == 8:
        assert st["hits"] == 128 and st["evictions"] == 0
    r.close()


def test_tiny_host_partials_sum():
    wl = synth.WORKLOADS["tiny"]
    log("tiny host partials")
    r = Runner(wl, [0], slots=2, mode="host", keep_debug=True)
    x = synth.gen_hidden(wl, 0)
    saw_host = False
    for t in range(24):
        out, res = r.call(0, x[t])
        g, h = r.cache.partials(0)
        np.testing.assert_array_equal(g + h, out)
        if res.misses:
            saw_host = True
            assert np.any(h != 0)
        else:
            assert np.all(h == 0)
    assert saw_host
    r.close()


@pytest.mark.parametrize("T", [2, 3, 4, 5, 17])
@pytest.mark.parametrize("mode", ["stream", "host"])
def test_multi_token_ragged(T, mode):
    wl = synth.Workload("rag", 11, 1, 256, 512, 16, 4, 6, n_shared=1, router_sigma=0.1,
                        zipf_s=0.5, rho=None, tokens=T * 6, batch=T)
    log(f"ragged T={T} mode={mode}")
    r = Runner(wl, [0], mode=mode)
    x = synth.gen_hidden(wl, 0)
    for c in range(x.shape[0]):
        r.call(0, x[c])
    r.check_log()
    r.close()


def test_staged_small_prefill():
    # 64 tokens x top-8 of 64 experts through 8 slots: several stages per call
    wl = synth.Workload("stg", 12, 1, 128, 256, 64, 8, 8, n_shared=1, router_sigma=0.14,
                        rho=None, tokens=192, batch=64)
    log("staged small prefill")
    r = Runner(wl, [0], mode="stream")
    x = synth.gen_hidden(wl, 0)
    for c in range(x.shape[0]):
        _, res = r.call(0, x[c])
        assert len(res.stage_views) > 1
    r.check_log()
    r.close()


@pytest.mark.parametrize("adopt", [0, 500, 1000])
def test_staged_small_prefill_preheat(adopt):
    """Prefill preheat: the staging pool, miss order and final slots of every
    staged call match the oracle, and so do the outputs; decode-sized calls in
    between follow the plain rule."""
    wl = synth.Workload("stg", 12, 1, 128, 256, 64, 8, 8, n_shared=1, router_sigma=0.14,
                        rho=None, tokens=192, batch=64)
    log(f"staged small prefill, preheat adopt={adopt}")
    r = Runner(wl, [0], mode="stream", adopt=adopt)
    x = synth.gen_hidden(wl, 0)
    for c in range(x.shape[0]):
        _, res = r.call(0, x[c])
        assert len(res.stage_views) > 1
        r.call(0, x[c][:2])
    r.check_log()
    r.close()


def test_prefill_ubatch_preheat_sampled():
    wl = synth.WORKLOADS["prefill"]
    log("prefill shape with preheat, 1 layer x 2 ubatches of 512, sampled tokens and columns")
    r = Runner(wl, [2], adopt=1000)
    x = synth.gen_hidden(wl, 2, 2)
    rng = np.random.default_rng(2)
    for u in range(2):
        toks = np.sort(rng.choice(512, 4, replace=False))
        cols = rng.choice(wl.d_model, 48, replace=False)
        _, res = r.call(0, x[u], tok_sample=toks, col_sample=cols)
        assert len(res.stage_views) >= 4
    r.check_log()
    r.close()


@pytest.mark.parametrize("T", [1, 3, 17])
def test_topk_exact_ties(T):
    """Exact logit ties through the whole layer: duplicated router rows give equal
    logits (the lower id must win), two zero rows tie at 0 and a negated row
    mirrors another; a bias of -100 keeps every other expert out, so the ties
    decide the selection.  The top-k ids must match the oracle bit for bit."""
    import torch
    wl = synth.Workload("ties", 13, 1, 256, 512, 32, 6, 6, router_sigma=0.1, rho=0.9,
                        tokens=24, batch=T)
    log(f"top-k exact ties, T={T}")
    r = Runner(wl, [0], mode="stream")
    w_r, b, _, _ = r.routers[0]
    w_r = w_r.copy()
    w_r[5] = w_r[2]      # ties between experts 2 and 5
    w_r[9] = w_r[4]      # and 4, 9, 30
    w_r[30] = w_r[4]
    w_r[11] = 0.0        # two logits of exactly 0
    w_r[12] = 0.0
    w_r[20] = -w_r[21]   # exact negation: z20 = -z21
    # only these nine compete
    b = np.full(wl.n_experts, -100.0, np.float32)
    b[[2, 4, 5, 9, 11, 12, 20, 21, 30]] = 0.0
    r.routers[0] = (w_r, b, torch.from_numpy(w_r).cuda(), torch.from_numpy(b).cuda())
    x = synth.gen_hidden(wl, 0, 8)
    for c in range(x.shape[0]):
        r.call(0, x[c])
    r.check_log()
    r.close()


def test_gemma_shape_two_layers():
    wl = synth.WORKLOADS["gemma"]
    log("gemma shape, 2 layers x 6 calls")
    r = Runner(wl, [0, 17])
    xs = [synth.gen_hidden(wl, l, 6) for l in (0, 17)]
    for t in range(6):
        for li in range(2):
            r.call(li, xs[li][t])
    r.check_log()
    r.close()


@pytest.mark.parametrize("b", [2, 4])
def test_qwen_shape_batches(b):
    wl = synth.qwen_batch(b)
    log(f"qwen shape b={b}")
    r = Runner(wl, [5])
    x = synth.gen_hidden(wl, 5, 6)
    for t in range(6):
        r.call(0, x[t])
    r.check_log()
    r.close()


def test_large_host_mode_sampled():
    wl = synth.WORKLOADS["large"]
    log("large shape, host mode, 1 layer x 4 calls, sampled columns")
    r = Runner(wl, [3], mode="host", keep_debug=True)
    x = synth.gen_hidden(wl, 3, 4)
    cols = np.random.default_rng(0).choice(wl.d_model, 96, replace=False)
    for t in range(4):
        out, _ = r.call(0, x[t], col_sample=cols)
        g, h = r.cache.partials(0)
        np.testing.assert_array_equal(g + h, out)
    r.check_log()
    r.close()


def test_prefill_ubatch_sampled():
    wl = synth.WORKLOADS["prefill"]
    log("prefill shape, 1 layer x 1 ubatch of 512, sampled tokens and columns")
    r = Runner(wl, [2])
    x = synth.gen_hidden(wl, 2, 1)[0]
    rng = np.random.default_rng(1)
    toks = np.sort(rng.choice(512, 6, replace=False))
    cols = rng.choice(wl.d_model, 64, replace=False)
    _, res = r.call(0, x, tok_sample=toks, col_sample=cols)
    assert len(res.stage_views) >= 4
    r.check_log()
    r.close()


@pytest.mark.parametrize("mode,budget", [("host", -1), ("host", 1), ("host", 0), ("stream", -1)])
def test_tiny_score_policy(mode, budget):
    """Decayed-score slots: every call's tables, scores and outputs against the oracle."""
    wl = synth.WORKLOADS["tiny"]
    log(f"tiny score policy mode={mode} budget={budget}")
    r = Runner(wl, [0], slots=3, mode=mode, max_fills=budget, policy="score")
    x = synth.gen_hidden(wl, 0)
    for t in range(x.shape[0]):
        r.call(0, x[t])
    r.check_log()
    st = r.cache.stats()
    if budget == 0:
        assert st["fills"] == 0
    r.close()


@pytest.mark.parametrize("T", [3, 4])
def test_multi_token_score_policy(T):
    wl = synth.Workload("rag", 11, 1, 256, 512, 16, 4, 6, n_shared=1, router_sigma=0.1,
                        zipf_s=0.5, rho=None, tokens=T * 6, batch=T)
    log(f"score policy T={T}")
    r = Runner(wl, [0], mode="host", max_fills=2, policy="score")
    x = synth.gen_hidden(wl, 0)
    for c in range(x.shape[0]):
        r.call(0, x[c])
    r.check_log()
    r.close()


def test_gemma_shape_score_policy_host():
    wl = synth.WORKLOADS["gemma"]
    log("gemma shape, score policy, host mode, one fill per call")
    r = Runner(wl, [0, 1], mode="host", max_fills=1, policy="score")
    xs = [synth.gen_hidden(wl, l, 24) for l in (0, 1)]
    for t in range(24):
        for li in range(2):
            r.call(li, xs[li][t], check_out=(t % 4 == 0))
    r.check_log()
    r.close()


@pytest.mark.parametrize("mode,policy", [("host", "score"), ("stream", "lru")])
def test_usage_profile_preload(mode, policy):
    """Lifetime counts read back; a preloaded profile re-seats the slots on the GPU
    exactly as the oracle does, and outputs stay exact."""
    wl = synth.WORKLOADS["gemma"]
    log(f"usage profile preload mode={mode} policy={policy}")
    r = Runner(wl, [0, 1], mode=mode, max_fills=1 if mode == "host" else -1, policy=policy)
    xs = [synth.gen_hidden(wl, l, 20) for l in (0, 1)]
    for t in range(8):
        for li in range(2):
            r.call(li, xs[li][t], check_out=(t % 4 == 0))
    u = r.cache.usage()
    assert u.tolist() == [sim.usage for sim in r.sims]
    rng = np.random.default_rng(5)
    counts = (u[:, ::-1] + rng.integers(0, 3, size=u.shape)).astype(np.uint32)
    r.cache.preload(counts)
    for li in range(2):
        r.sims[li].preload(counts[li].tolist())
        ein, _ = r.cache.slot_state(li)
        assert ein.tolist() == r.sims[li].expert_in
    for t in range(8, 20):
        for li in range(2):
            r.call(li, xs[li][t], check_out=(t % 3 == 0))
    r.check_log()
    r.close()


# Degenerate and maximum cases: every selection, one selection, the most experts
# the boundary takes, the smallest shapes it takes, the decode path's pair limit
# and one pair past it (the matrix-core path), slots for every expert.
EDGE = {
    # name: (d, f, E, k, S, shared, tokens per call)
    "k_eq_E": (256, 512, 8, 8, 4, 0, 1),
    "k_eq_E_slots_all": (256, 512, 8, 8, 8, 0, 1),
    "k_1": (256, 512, 8, 1, 2, 0, 1),
    "E_512": (64, 64, 512, 8, 32, 0, 1),
    "E_512_T4": (64, 64, 512, 8, 32, 1, 4),
    "min_shape": (64, 32, 16, 4, 4, 1, 3),
    "pairs_64": (128, 128, 64, 15, 16, 1, 4),
    "pairs_68": (128, 128, 64, 16, 16, 1, 4),
    "slots_eq_E": (128, 256, 16, 4, 16, 1, 2),
}


@pytest.mark.parametrize("mode", ["stream", "host"])
@pytest.mark.parametrize("case", sorted(EDGE))
def test_edge_shapes(case, mode):
    d, f, E, k, S, ns, T = EDGE[case]
    wl = synth.Workload("edge_" + case, 20 + sorted(EDGE).index(case), 1, d, f, E, k, S,
                        n_shared=ns, router_sigma=0.3, zipf_s=0.8, rho=0.5, tokens=10, batch=T)
    log(f"edge {case} mode={mode}: d={d} f={f} E={E} k={k} S={S} shared={ns} T={T}")
    r = Runner(wl, [0], mode=mode)
    x = synth.gen_hidden(wl, 0)
    for c in range(x.shape[0]):
        _, res = r.call(0, x[c])
        if S == E:
            assert res.fills == 0 and res.misses == 0 and set(res.host_view) == {-1}
    r.check_log()
    st = r.cache.stats()
    assert st["selections"] == 10 * T * k
    assert st["hits"] + st["misses"] == st["selections"]
    if S == E:
        assert st["hits"] == st["selections"] and st["evictions"] == 0
    r.close()


def test_decode_and_matrix_core_calls_alternate():
    """One cache takes decode calls and matrix-core calls of up to 4 tokens in
    any order (4 tokens x (16 + 1 shared) = 68 pairs exceed the decode path; 1-3
    tokens do not): the workspace follows the path, both miss modes."""
    wl = synth.Workload("alt", 31, 1, 128, 128, 64, 16, 16, n_shared=1, router_sigma=0.3,
                        zipf_s=0.8, rho=0.5, tokens=14, batch=1)
    x = synth.gen_hidden(wl, 0)[:, 0, :]
    for mode in ("stream", "host"):
        log(f"decode / matrix-core alternation mode={mode}")
        r = Runner(wl, [0], mode=mode)
        c = 0
        for T in (1, 4, 2, 4, 3, 1, 4):
            r.call(0, x[c:c + T])
            c += T % 3
        r.check_log()
        r.close()


def test_invalid_calls_leave_the_cache_unchanged():
    """Invalid arguments to a live cache return MOE_EINVAL with a message and
    change nothing: the next valid calls still match the oracle, table for table,
    and the replacement log has no entry from the rejected calls."""
    import ctypes

    import torch

    from expert_cache_host_amd.binding import load_library
    wl = synth.WORKLOADS["tiny"]
    log("invalid calls on a live cache")
    r = Runner(wl, [0], slots=2, mode="stream")
    x = synth.gen_hidden(wl, 0)
    r.call(0, x[0])
    lib = load_library()
    h = r.cache._h
    xd = torch.from_numpy(np.ascontiguousarray(x[1])).cuda()
    w = r.routers[0][2]
    out = torch.empty_like(xd)
    st = torch.cuda.current_stream().cuda_stream
    bad = [
        (1, xd.data_ptr(), 1, w.data_ptr(), out.data_ptr()),    # layer past the last
        (-1, xd.data_ptr(), 1, w.data_ptr(), out.data_ptr()),   # negative layer
        (0, xd.data_ptr(), 0, w.data_ptr(), out.data_ptr()),    # no tokens
        (0, None, 1, w.data_ptr(), out.data_ptr()),             # no x
        (0, xd.data_ptr(), 1, None, out.data_ptr()),            # no router
        (0, xd.data_ptr(), 1, w.data_ptr(), None),              # no output
    ]
    for layer, xp, T, wp, op in bad:
        rc = lib.moe_layer_forward(h, layer, xp, T, wp, None, op, st)
        assert rc == -1, (layer, T, rc)
        assert lib.moe_last_error()
    assert r.cache.stats()["calls"] == 1
    for t in range(1, 8):
        r.call(0, x[t])
    r.check_log()
    r.close()


# Router logits, bit for bit: (d_model, n_experts, top_k, tokens per call, Zipf s).
# Decode calls of 1-4 tokens take the one-workgroup-per-expert router unless the
# tokens' products exceed 64 KiB of LDS (6144 x 4 tokens); those and longer
# calls take the tiled router.  Both must give the oracle's fixed-order sums.
ROUTER = {
    "gemma_T1": (2816, 128, 8, 1, 1.1),
    "large_T1": (6144, 256, 8, 1, 1.2),
    "large_T4": (6144, 256, 8, 4, 1.2),
    "qwen_T2": (2048, 128, 8, 2, 1.0),
    "qwen_T3": (2048, 128, 8, 3, 1.0),
    "E512_T1": (256, 512, 8, 1, None),
    "d64_T4": (64, 16, 2, 4, None),
    "T17": (1024, 64, 4, 17, 1.0),
}


@pytest.mark.parametrize("case", sorted(ROUTER))
def test_router_logits_bit_exact(case):
    """The GPU's router logits (bias included) equal the oracle's fixed-order
    float32 sums bit for bit, on every call, for both router kernels."""
    d, E, k, T, zipf = ROUTER[case]
    wl = synth.Workload("router_" + case, 40 + sorted(ROUTER).index(case), 1, d, 64, E, k,
                        min(E, 16), router_sigma=1.6 / np.sqrt(d), zipf_s=zipf, rho=0.8,
                        tokens=4, batch=T)
    log(f"router logits {case}: d={d} E={E} T={T}")
    r = Runner(wl, [0], mode="stream", keep_debug=True)
    w_r, b, _, _ = r.routers[0]
    x = synth.gen_hidden(wl, 0, 3)
    for c in range(x.shape[0]):
        r.call(0, x[c])
        z = r.cache.logits(0)
        ref = router_logits_fp32(x[c], w_r, b)
        assert z.shape == ref.shape
        bad = np.argwhere(z.view(np.uint32) != ref.view(np.uint32))
        assert bad.size == 0, f"call {c}: {len(bad)} logits differ, first {bad[:4].tolist()}"
    r.check_log()
    r.close()


@pytest.mark.parametrize("d,T", [(6144, 1), (6144, 3), (2048, 4)])
def test_host_misses_read_x_copied_by_router_or_stream(d, T):
    """Host misses read a page-locked copy of x: written by the decode router
    when its products fit in LDS (6144 x 1, 2048 x 4 tokens), else copied on
    the stream (6144 x 3 and 4 tokens).  Outputs, tables and log against the
    oracle on every call."""
    wl = synth.Workload(f"hx_{d}_{T}", 50 + d // 1024 + T, 1, d, 64, 16, 2, 4,
                        router_sigma=1.6 / np.sqrt(d), zipf_s=1.0, rho=0.8, tokens=6, batch=T)
    log(f"host misses, x copy: d={d} T={T}")
    r = Runner(wl, [0], mode="host")
    x = synth.gen_hidden(wl, 0, 6)
    for c in range(x.shape[0]):
        r.call(0, x[c])
    r.check_log()
    r.close()


@pytest.mark.parametrize("mode", ["stream", "host"])
def test_calls_alternating_between_two_streams(mode):
    """Calls for two layers alternate between two streams and are enqueued back
    to back, with no synchronisation by the caller; the library orders them
    (the layers share its workspace).  Every output, collected at the end,
    matches the oracle, and so does each layer's replacement log."""
    import torch

    from oracle.layer import moe_layer
    from oracle.lru import LayerSlots
    wl = synth.Workload("twostreams", 33, 2, 256, 512, 16, 4, 6, n_shared=1, router_sigma=0.1,
                        rho=0.8, tokens=8, batch=1)
    log(f"two streams, {mode}")
    r = Runner(wl, [0, 1], mode=mode)
    xs = [synth.gen_hidden(wl, l, 8) for l in (0, 1)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    torch.cuda.synchronize()
    for t in range(8):
        for li in (0, 1):
            s = streams[(t + li) % 2]
            with torch.cuda.stream(s):
                x_d = torch.from_numpy(np.ascontiguousarray(xs[li][t])).cuda()
                w_d, b_d = r.routers[li][2], r.routers[li][3]
                outs.append((li, t, r.cache.forward(li, x_d, w_d, b_d), x_d))
    torch.cuda.synchronize()
    for li, t, out, _ in outs:
        w_r, b, _, _ = r.routers[li]
        ref = moe_layer(xs[li][t], w_r, b, r.layer_buf(li), wl.d_model, wl.d_ff, wl.n_experts,
                        wl.top_k, n_shared=wl.n_shared)
        check_close(out.cpu().numpy(), ref["out64"])
        r.sims[li].plan(ref["idx"].ravel().tolist(), mode, -1, tokens=1)
    r.check_log()
    r.close()


# ---------------------------------------------------------------- activation corners
# The decode GEMV encodes activations as 16-bit fixed point with one scale per
# 32-element block; the matrix-core GEMM splits them into binary16 hi/lo parts
# after a power-of-two row scale.  Inputs with one large channel, and inputs far
# from unit scale, must still meet the bar (tolerance unchanged).

def _with_outlier(x, factor, ch=701):
    x = np.array(x, copy=True)
    x[..., ch] *= factor
    return x


@pytest.mark.parametrize("T", [1, 4])
@pytest.mark.parametrize("outlier", [10, 100, 1000])
def test_decode_outlier_channel_gemma_shape(T, outlier):
    """Gemma-like expert shape, one hidden channel at 10x-1000x the rest, decode
    calls of 1 and 4 tokens (the one-workgroup-per-expert router prepares x)."""
    wl = synth.Workload("outlier", 60, 1, 2816, 704, 128, 8, 32, router_sigma=1.6 / np.sqrt(2816),
                        zipf_s=1.1, rho=0.8, tokens=4, batch=T, weight_wid=2)
    log(f"decode outlier channel x{outlier}, T={T}, Gemma-like shape")
    r = Runner(wl, [0], mode="host")
    x = synth.gen_hidden(wl, 0, 4)
    for c in range(x.shape[0]):
        r.call(0, _with_outlier(x[c], outlier))
    r.check_log()
    r.close()


@pytest.mark.parametrize("outlier", [100, 1000])
def test_decode_outlier_channel_tiled_router(outlier):
    """d_model 6144 at 4 tokens: the tokens' products exceed the decode router's
    LDS, so the tiled router prepares the block-scaled planes."""
    wl = synth.Workload("outlier6144", 61, 1, 6144, 256, 16, 4, 8, n_shared=1,
                        router_sigma=1.6 / np.sqrt(6144), zipf_s=1.0, rho=0.8, tokens=4, batch=4)
    log(f"decode outlier channel x{outlier}, T=4, d_model 6144 (tiled router)")
    r = Runner(wl, [0], mode="stream")
    x = synth.gen_hidden(wl, 0, 4)
    for c in range(x.shape[0]):
        r.call(0, _with_outlier(x[c], outlier, ch=4097))
    r.check_log()
    r.close()


@pytest.mark.parametrize("scale", [2.0 ** -20, 2.0 ** 20])
@pytest.mark.parametrize("mode", ["stream", "host"])
def test_matrix_core_extreme_scales(scale, mode):
    """17-token calls (matrix-core GEMM) on inputs scaled by 2^-20 and 2^20."""
    wl = synth.Workload("rag", 11, 1, 256, 512, 16, 4, 6, n_shared=1, router_sigma=0.1,
                        zipf_s=0.5, rho=None, tokens=17 * 4, batch=17)
    log(f"matrix-core path, T=17, inputs x {scale:g}, mode={mode}")
    r = Runner(wl, [0], mode=mode)
    x = synth.gen_hidden(wl, 0)
    for c in range(x.shape[0]):
        r.call(0, (x[c] * scale).astype(np.float32))
    r.check_log()
    r.close()


@pytest.mark.parametrize("d,f", [(1024, 3072), (3072, 1024), (1280, 2816)])
def test_matrix_core_scale_windows(d, f):
    """Matrix-core calls on rows of 32 and 96 blocks, where the scale windows of
    32 blocks number one and three (the large shape has six and two), and on
    rows of 40 and 88 blocks, which take per-chunk scales; a 40-token call has
    a pass of 8 tokens after one of 32."""
    wl = synth.Workload(f"win_{d}_{f}", 70 + d // 1024, 1, d, f, 16, 4, 6, n_shared=1,
                        router_sigma=0.4 / np.sqrt(d), zipf_s=0.5, rho=None, tokens=40 * 3,
                        batch=40)
    log(f"matrix-core scale windows d={d} f={f}, T=40")
    r = Runner(wl, [0], mode="stream")
    x = synth.gen_hidden(wl, 0)
    for c in range(x.shape[0]):
        _, res = r.call(0, x[c])
        assert len(res.stage_views) > 1
    r.check_log()
    r.close()


@pytest.mark.parametrize("scale", [2.0 ** -20, 1.0 / 3000.0])
def test_decode_extreme_scales(scale):
    """Decode calls on inputs far below unit scale (the block scales follow)."""
    wl = synth.Workload("outlier", 60, 1, 2816, 704, 128, 8, 32, router_sigma=1.6 / np.sqrt(2816),
                        zipf_s=1.1, rho=0.8, tokens=4, batch=1, weight_wid=2)
    log(f"decode, inputs x {scale:g}")
    r = Runner(wl, [0], mode="stream")
    x = synth.gen_hidden(wl, 0, 4)
    for c in range(x.shape[0]):
        r.call(0, (x[c] * scale).astype(np.float32))
    r.check_log()
    r.close()


def test_prefill_ubatch_small_scale_sampled():
    wl = synth.WORKLOADS["prefill"]
    log("prefill shape, 1 ubatch of 512 scaled by 2^-20, sampled tokens and columns")
    r = Runner(wl, [1])
    x = (synth.gen_hidden(wl, 1, 1)[0] * 2.0 ** -20).astype(np.float32)
    rng = np.random.default_rng(3)
    toks = np.sort(rng.choice(512, 6, replace=False))
    cols = rng.choice(wl.d_model, 96, replace=False)
    _, res = r.call(0, x, tok_sample=toks, col_sample=cols)
    assert len(res.stage_views) >= 4
    r.check_log()
    r.close()


def _prefill_check_tokens(idx, k):
    """32 tokens of a 512-token ubatch: one in every 32-token pass of the shared
    expert (whose bucket holds all 512 tokens), and 16 that sit in the second
    16-token tile of a routed expert's bucket (bucket position >= 16: pairs are
    bucketed in ascending (token, rank) order)."""
    T = idx.shape[0]
    toks = [32 * p + (7 * p) % 32 for p in range(T // 32)]
    counts = np.bincount(idx.ravel(), minlength=idx.max() + 1)
    second = []
    for e in np.argsort(-counts, kind="stable"):
        if counts[e] < 17 or len(second) >= 16:
            break
        members = np.nonzero((idx == e).any(axis=1))[0]
        for t in members[16:20]:
            if int(t) not in toks and int(t) not in second:
                second.append(int(t))
    assert len(second) >= 8, "no routed bucket with a second 16-token tile"
    return np.array(sorted(set(toks) | set(second[:16])))


def test_prefill_ubatch_all_columns():
    """One 512-token ubatch through 64 slots (4+ stages), all 6144 output
    columns of 32 tokens: every 32-token pass of the shared expert and the
    second 16-token tiles of the largest routed buckets."""
    from oracle.routing import topk
    wl = synth.WORKLOADS["prefill"]
    log("prefill shape, 1 ubatch of 512, all columns of 32 tokens")
    r = Runner(wl, [0])
    x = synth.gen_hidden(wl, 0, 1)[0]
    w_r, b, _, _ = r.routers[0]
    toks = _prefill_check_tokens(topk(router_logits_fp32(x, w_r, b), wl.top_k), wl.top_k)
    assert len(toks) >= 24
    log(f"  checking tokens {toks.tolist()}")
    _, res = r.call(0, x, tok_sample=toks)
    assert len(res.stage_views) >= 4
    r.check_log()
    r.close()


def test_gemma_shape_host_lru_two_layers():
    """The Gemma-like decode as benchmarked: host misses, LRU, two layers called
    token-major for 16 calls; every call's output against the oracle."""
    wl = synth.WORKLOADS["gemma"]
    log("gemma shape, host misses, LRU, 2 layers x 16 calls")
    r = Runner(wl, [3, 11], mode="host", keep_debug=True)
    xs = [synth.gen_hidden(wl, l, 16) for l in (3, 11)]
    saw_host = False
    for t in range(16):
        for li in range(2):
            out, res = r.call(li, xs[li][t])
            g, h = r.cache.partials(li)
            np.testing.assert_array_equal(g + h, out)
            saw_host |= res.misses > 0
    assert saw_host
    r.check_log()
    r.close()


def test_large_host_lru_all_columns():
    """The large-expert decode as benchmarked (host misses, LRU, shared expert):
    8 calls of one layer, every output column."""
    wl = synth.WORKLOADS["large"]
    log("large shape, host misses, LRU, 1 layer x 8 calls, all columns")
    r = Runner(wl, [5], mode="host")
    x = synth.gen_hidden(wl, 5, 8)
    for t in range(8):
        r.call(0, x[t])
    r.check_log()
    r.close()
