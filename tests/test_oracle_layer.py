"""Pins of oracle/expert.py and oracle/layer.py: closed forms on hand-built Q4
experts, the brute-force all-expert mixture, and the dense k = E mixture."""
import numpy as np

import synth
from oracle.expert import expert_forward, silu
from oracle.layer import dense_mixture, expert_output, moe_layer
from oracle.q4 import expert_nbytes


def _const_matrix(rows, cols, scale_of_row, q=9):
    """Q4 bytes of a matrix whose row r is all scale_of_row(r) * (q - 8)."""
    out = []
    for r in range(rows):
        dbytes = np.float16(scale_of_row(r)).tobytes()
        blk = dbytes + bytes([(q & 15) | (q << 4)] * 16)
        out.append(np.frombuffer(blk * (cols // 32), dtype=np.uint8))
    return np.concatenate(out)


def test_silu_values():
    assert silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(silu(np.array([30.0]))[0], 30.0, rtol=1e-12)
    assert abs(silu(np.array([-40.0]))[0]) < 1e-15
    np.testing.assert_allclose(silu(np.array([1.0]))[0], 1.0 / (1.0 + np.exp(-1.0)), rtol=1e-15)


def test_expert_closed_form():
    # G rows r: value (r+1)/8 -> g_r = (r+1)/8 * sum(x); U rows: 1/4 -> u = sum(x)/4;
    # D rows i: value 1/2 -> y_i = sum_r h_r / 2.
    d, f = 64, 32
    gb = _const_matrix(f, d, lambda r: (r + 1) / 8.0)
    ub = _const_matrix(f, d, lambda r: 0.25)
    db = _const_matrix(d, f, lambda r: 0.5)
    buf = np.concatenate([gb, ub, db])
    assert buf.size == expert_nbytes(d, f)
    x = np.linspace(-1.0, 1.5, d)[None, :]
    s = x.sum()
    g = (np.arange(f) + 1) / 8.0 * s
    h = g / (1 + np.exp(-g)) * (s / 4.0)
    y = np.full(d, h.sum() / 2.0)
    got = expert_output(buf, 0, d, f, x)
    np.testing.assert_allclose(got[0], y, rtol=1e-13)
    got_cols = expert_output(buf, 0, d, f, x, out_cols=[3, 7])
    np.testing.assert_allclose(got_cols[0], y[[3, 7]], rtol=1e-13)


def test_expert_one_hot_picks_column():
    rng = np.random.default_rng(7)
    g = rng.standard_normal((32, 64))
    u = rng.standard_normal((32, 64))
    dm = rng.standard_normal((64, 32))
    for i in (0, 17, 63):
        x = np.zeros((1, 64))
        x[0, i] = 1.0
        h = silu(g[:, i]) * u[:, i]
        np.testing.assert_allclose(expert_forward(g, u, dm, x)[0], dm @ h, rtol=1e-13)


def _tiny_layer(n_shared=0, e=8, k=2):
    wl = synth.Workload("t", 99, 1, 64, 64, e, k, 2, n_shared=n_shared, router_sigma=0.3)
    buf = synth.gen_experts(wl, 0)
    w_r, _ = synth.gen_router(wl, 0)
    rng = np.random.default_rng(11)
    x = rng.standard_normal((6, 64)).astype(np.float32)
    b = rng.standard_normal(e).astype(np.float32) * 0.1
    return wl, buf, w_r, b, x


def test_sparse_equals_all_expert_mixture():
    wl, buf, w_r, b, x = _tiny_layer(n_shared=1)
    res = moe_layer(x, w_r, b, buf, 64, 64, 8, 2, n_shared=1)
    dense = dense_mixture(x, w_r, b, buf, 64, 64, 8, 2, n_shared=1)
    np.testing.assert_allclose(res["out64"], dense, rtol=1e-12, atol=1e-15)


def test_k_equals_e_is_softmax_mixture():
    wl, buf, w_r, b, x = _tiny_layer(e=6, k=6)
    res = moe_layer(x, w_r, b, buf, 64, 64, 6, 6)
    z = res["z"].astype(np.float64)
    p = np.exp(z - z.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    ref = np.zeros((x.shape[0], 64))
    for e in range(6):
        ref += p[:, e:e + 1] * expert_output(buf, e, 64, 64, x.astype(np.float64))
    np.testing.assert_allclose(res["out64"], ref, rtol=1e-12, atol=1e-15)


def test_shared_expert_adds_with_weight_one():
    wl, buf, w_r, b, x = _tiny_layer(n_shared=1)
    with_sh = moe_layer(x, w_r, b, buf, 64, 64, 8, 2, n_shared=1)["out64"]
    without = moe_layer(x, w_r, b, buf, 64, 64, 8, 2, n_shared=0)["out64"]
    sh = expert_output(buf, 8, 64, 64, x.astype(np.float64))
    np.testing.assert_allclose(with_sh - without, sh, rtol=1e-10, atol=1e-14)


def test_out_cols_sample_matches_full():
    wl, buf, w_r, b, x = _tiny_layer(n_shared=1)
    full = moe_layer(x, w_r, b, buf, 64, 64, 8, 2, n_shared=1)["out64"]
    cols = [0, 5, 63]
    part = moe_layer(x, w_r, b, buf, 64, 64, 8, 2, n_shared=1, out_cols=cols)["out64"]
    np.testing.assert_allclose(part, full[:, cols], rtol=1e-13, atol=1e-16)
