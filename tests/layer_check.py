"""Shared driver of the GPU parity tests: runs a workload through the library
call by call and checks each call against the oracle.

Checked bit for bit: top-k ids of every token, both lookup tables of every
stage, the slot state, the usage scores (score policy) and the whole
replacement log; and that the tables map every selected expert exactly once
(one stage's slot table or the host table).  Checked within tolerance
(max |out - oracle| <= 2e-3 * RMS(oracle) over the compared block of each call):
the layer output, on all of it or on a seeded sample of tokens and columns.
"""
from __future__ import annotations

import sys

import numpy as np

from oracle.layer import moe_layer
from oracle.lru import LayerSlots
from oracle.routing import router_logits_fp32, topk

TOL = 2e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class Runner:
    def __init__(self, wl, layers, slots=None, mode="stream", max_fills=-1, keep_debug=False,
                 host_threads=0, weights=None, policy="lru", adopt=-1):
        import torch
        import expert_cache_host_amd as m
        import synth
        self.torch = torch
        self.wl = wl
        self.layers = list(layers)
        self.S = slots if slots is not None else wl.slots
        self.mode = mode
        self.max_fills = max_fills
        nl = len(self.layers)
        if weights is None:
            weights = np.empty(nl * wl.layer_bytes, np.uint8)
            for i, l in enumerate(self.layers):
                synth.gen_experts(wl, l, out=weights[i * wl.layer_bytes:(i + 1) * wl.layer_bytes])
        self.weights = weights
        self.cache = m.MoECache(nl, wl.n_experts, self.S, wl.d_model, wl.d_ff, weights,
                                top_k=wl.top_k, miss_mode=mode, n_shared=wl.n_shared,
                                max_fills_per_call=max_fills, keep_debug=keep_debug,
                                host_threads=host_threads, policy=policy, adopt=adopt)
        self.policy = policy
        self.sims = [LayerSlots(wl.n_experts, self.S, policy, adopt) for _ in self.layers]
        self.routers = []
        for l in self.layers:
            w_r, b = synth.gen_router(wl, l)
            self.routers.append((w_r, b, torch.from_numpy(w_r).cuda(),
                                 torch.from_numpy(b).cuda() if b is not None else None))

    def layer_buf(self, li):
        return self.weights[li * self.wl.layer_bytes:(li + 1) * self.wl.layer_bytes]

    def call(self, li, x_np, check_out=True, tok_sample=None, col_sample=None):
        """Runs one call on layer index li and checks it; returns the GPU output."""
        torch = self.torch
        wl = self.wl
        w_r, b, w_r_d, b_d = self.routers[li]
        x_d = torch.from_numpy(np.ascontiguousarray(x_np)).cuda()
        out = self.cache.forward(li, x_d, w_r_d, b_d)
        torch.cuda.synchronize()
        out_np = out.cpu().numpy()
        # routing, bit for bit
        z = router_logits_fp32(x_np, w_r, b)
        idx_ref = topk(z, wl.top_k)
        idx_gpu, w_gpu = self.cache.routing(li)
        if not np.array_equal(idx_gpu, idx_ref):
            bad = np.argwhere(idx_gpu != idx_ref)[:5]
            raise AssertionError(f"top-k ids differ at {bad.tolist()}")
        # tables and slot state, bit for bit
        res = self.sims[li].plan(idx_ref.ravel().tolist(), self.mode, self.max_fills,
                                 tokens=x_np.shape[0])
        ns, nt = self.cache.last_call(li)
        assert nt == x_np.shape[0]
        assert ns == len(res.stage_views), (ns, len(res.stage_views))
        for s in range(ns):
            sv, hv = self.cache.views(li, s)
            assert sv.tolist() == res.stage_views[s], f"slot table differs in stage {s}"
            assert hv.tolist() == res.host_view, f"host table differs in stage {s}"
        # every selected expert is computed exactly once: mapped by exactly one of
        # the call's tables (one stage's slot table, or the host table).  Work
        # follows the selected pairs; the tables also place experts nobody
        # selected (in host mode they split all experts between slot and host).
        mapped = {e: 0 for e in set(idx_ref.ravel().tolist())}
        for s in range(ns):
            sv, hv = self.cache.views(li, s)
            for e in mapped:
                mapped[e] += int(sv[e] >= 0) + (int(hv[e] >= 0) if s == 0 else 0)
        for e, n in mapped.items():
            assert n == 1, (e, n)
        ein, lu = self.cache.slot_state(li)
        assert ein.tolist() == self.sims[li].expert_in
        assert lu.tolist() == self.sims[li].last_use
        if self.policy == "score":
            assert self.cache.scores(li).tolist() == self.sims[li].score
        if check_out:
            xs = x_np if tok_sample is None else x_np[tok_sample]
            ref = moe_layer(xs, w_r, b, self.layer_buf(li), wl.d_model, wl.d_ff, wl.n_experts,
                            wl.top_k, n_shared=wl.n_shared, out_cols=col_sample)
            got = out_np if tok_sample is None else out_np[tok_sample]
            if col_sample is not None:
                got = got[:, col_sample]
            check_close(got, ref["out64"])
        return out_np, res

    def check_log(self):
        for li in range(len(self.layers)):
            assert self.cache.evictions(li) == self.sims[li].log

    def close(self):
        self.cache.close()


def check_close(got, ref64):
    rms = float(np.sqrt(np.mean(ref64 ** 2)))
    err = float(np.max(np.abs(got.astype(np.float64) - ref64)))
    assert np.all(np.isfinite(got)), "non-finite output"
    assert err <= TOL * rms, f"max |err| {err:.3e} > {TOL} * rms {rms:.3e} (ratio {err / rms:.2e})"
    return err / rms
