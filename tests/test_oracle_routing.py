"""Pins of oracle/routing.py: hand-worked order-sensitive logits, exact cases,
the recursive-summation error bound, brute-force top-k and closed-form gating."""
import itertools
import os

import numpy as np
import pytest

from oracle.routing import gate_weights, router_logits_fp32, topk

G = os.path.join(os.path.dirname(__file__), "golden")


def _lines(name):
    for line in open(os.path.join(G, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            yield [p.strip() for p in line.split("|")]


@pytest.mark.parametrize("row", list(_lines("router_order.txt")))
def test_router_order_golden(row):
    d = int(row[0])
    w = np.zeros((1, d), np.float32)
    for ent in row[1].split():
        i, v = ent.split(":")
        w[0, int(i)] = np.float32(float(v))
    x = np.ones((1, d), np.float32)
    b = np.array([float(row[2])], np.float32)
    z = router_logits_fp32(x, w, b)
    assert z.dtype == np.float32
    assert z.view(np.uint32)[0, 0] == int(row[3], 16)


def test_router_one_hot_is_exact():
    rng = np.random.default_rng(1)
    e, d = 5, 192
    w = rng.standard_normal((e, d)).astype(np.float32)
    b = rng.standard_normal(e).astype(np.float32)
    for i in (0, 63, 64, 191):
        x = np.zeros((1, d), np.float32)
        x[0, i] = 1.0
        z = router_logits_fp32(x, w, b)
        np.testing.assert_array_equal(z[0], (w[:, i] + b).astype(np.float32))


def test_router_integers_exact():
    # Small integers: every partial sum is exact, so any order gives the exact dot.
    rng = np.random.default_rng(2)
    x = rng.integers(-8, 9, (3, 256)).astype(np.float32)
    w = rng.integers(-8, 9, (7, 256)).astype(np.float32)
    b = rng.integers(-100, 100, 7).astype(np.float32)
    z = router_logits_fp32(x, w, b)
    exact = x.astype(np.int64) @ w.T.astype(np.int64) + b.astype(np.int64)
    np.testing.assert_array_equal(z, exact.astype(np.float32))


def test_router_error_bound():
    # |z32 - z64| <= (d/64 + 8) * 2^-24 * (sum |x w| + |b|): d/64 lane sums,
    # six tree levels, one product rounding, one bias add.
    rng = np.random.default_rng(3)
    for d in (64, 256, 2816, 6144):
        x = rng.standard_normal((4, d)).astype(np.float32)
        w = (rng.standard_normal((9, d)) * 0.05).astype(np.float32)
        b = rng.standard_normal(9).astype(np.float32)
        z = router_logits_fp32(x, w, b).astype(np.float64)
        x64, w64 = x.astype(np.float64), w.astype(np.float64)
        exact = x64 @ w64.T + b
        mag = np.abs(x64) @ np.abs(w64).T + np.abs(b)
        bound = (d / 64 + 8) * 2.0 ** -24 * mag
        assert np.all(np.abs(z - exact) <= bound)


@pytest.mark.parametrize("row", list(_lines("topk_ties.txt")))
def test_topk_ties_golden(row):
    z = np.array([[float(v) for v in row[0].split()]], np.float32)
    k = int(row[1])
    exp = [int(v) for v in row[2].split()]
    assert topk(z, k)[0].tolist() == exp


def test_topk_brute_force():
    rng = np.random.default_rng(4)
    for e, k in ((8, 2), (8, 3), (6, 6), (7, 1)):
        z = rng.standard_normal((20, e)).astype(np.float32)
        got = topk(z, k)
        for r in range(z.shape[0]):
            best = max(itertools.combinations(range(e), k),
                       key=lambda s: (sum(float(z[r, i]) for i in s), [-i for i in s]))
            assert sorted(got[r].tolist()) == sorted(best)
            vals = z[r, got[r]]
            assert np.all(np.diff(vals) <= 0)


def test_topk_all():
    z = np.array([[0.5, -1.0, 2.0, 0.0]], np.float32)
    assert topk(z, 4)[0].tolist() == [2, 0, 3, 1]
    with pytest.raises(ValueError):
        topk(np.array([[np.nan, 1.0]], np.float32), 1)


def test_gate_weights_closed_forms():
    rng = np.random.default_rng(5)
    z = rng.standard_normal((10, 16)).astype(np.float32)
    idx = topk(z, 4)
    w = gate_weights(z, idx, True)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert np.all(w[:, :-1] >= w[:, 1:])
    # k = 1 -> weight 1
    w1 = gate_weights(z, topk(z, 1), True)
    np.testing.assert_array_equal(w1, 1.0)
    # E = 2, k = 2, no renormalisation -> logistic of the logit difference
    z2 = np.array([[1.25, -0.5]], np.float32)
    w2 = gate_weights(z2, topk(z2, 2), False)
    np.testing.assert_allclose(w2[0, 0], 1.0 / (1.0 + np.exp(-1.75)), rtol=1e-15)
    np.testing.assert_allclose(w2[0, 1], 1.0 / (1.0 + np.exp(1.75)), rtol=1e-15)
    # without renormalisation the weights are softmax probabilities (sum < 1)
    w0 = gate_weights(z, idx, False)
    assert np.all(w0.sum(axis=1) < 1.0)
    np.testing.assert_allclose(w0 / w0.sum(axis=1, keepdims=True), w, rtol=1e-13)
