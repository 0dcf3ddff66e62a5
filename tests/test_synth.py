"""The seeded input generators: determinism, shapes and the stated recipe."""
import numpy as np

import synth


def test_weights_deterministic_and_thread_independent():
    wl = synth.WORKLOADS["tiny"]
    a = synth.gen_experts(wl, 0, threads=1)
    b = synth.gen_experts(wl, 0, threads=5)
    assert a.size == wl.layer_bytes
    np.testing.assert_array_equal(a, b)
    # a sub-range equals the same slice of the full layer
    c = synth.gen_experts(wl, 0, 3, 5)
    np.testing.assert_array_equal(c, a[3 * wl.expert_bytes:5 * wl.expert_bytes])


def test_hidden_states_ar1():
    wl = synth.WORKLOADS["tiny"]
    x = synth.gen_hidden(wl, 0)
    assert x.shape == (64, 1, 256) and x.dtype == np.float32
    np.testing.assert_array_equal(x[:10], synth.gen_hidden(wl, 0, 10))
    # lag-1 correlation close to rho, variance close to 1/(1-rho^2)
    xx = x[:, 0, :].astype(np.float64)
    r = (xx[1:] * xx[:-1]).mean() / (xx * xx).mean()
    assert abs(r - 0.8) < 0.1
    assert abs(xx.var() - 1 / (1 - 0.64)) < 0.6


def test_router_recipe():
    wl = synth.WORKLOADS["gemma"]
    w, b = synth.gen_router(wl, 3)
    assert w.shape == (128, 2816) and b.shape == (128,)
    assert abs(w.std() - 1.6 / np.sqrt(2816)) < 0.002
    ranks = np.exp(-b.astype(np.float64) / 1.1)
    np.testing.assert_allclose(np.sort(ranks), np.arange(1, 129), rtol=1e-5)
    assert synth.gen_router(synth.WORKLOADS["prefill"], 0)[1] is None


def test_sizes():
    assert synth.WORKLOADS["gemma"].expert_bytes == 3_345_408
    assert synth.WORKLOADS["large"].expert_bytes == 21_233_664
    assert abs(synth.WORKLOADS["large"].total_bytes / 1e9 - 43.66) < 0.01
