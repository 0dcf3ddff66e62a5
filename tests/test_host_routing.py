"""The host's expert selection on decode calls (moe_host_topk) against the
oracle's top-k and gating weights.  The host plans from this selection while the
GPU builds its buckets from its own; both must pick the same ids in the same
order from the same float32 logits, including exact ties (lower id first) and
-0 against +0."""
import numpy as np
import pytest

import expert_cache_host_amd as m
from oracle.routing import gate_weights, topk


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (4, 128, 8), (3, 256, 8), (2, 512, 64), (1, 16, 16),
                                   (4, 64, 1)])
@pytest.mark.parametrize("norm", [True, False])
def test_host_topk_matches_oracle(T, E, k, norm):
    rng = np.random.default_rng(T * 1000 + E + k)
    z = (rng.standard_normal((T, E)) * 2).astype(np.float32)
    idx, w = m.host_topk(z, k, norm)
    ref = topk(z, k)
    np.testing.assert_array_equal(idx, ref)
    w_ref = gate_weights(z, ref, norm)
    assert np.max(np.abs(w.astype(np.float64) - w_ref)) <= 2e-7 * max(1.0, np.max(w_ref))


def test_host_topk_exact_ties_and_signed_zero():
    z = np.array([[0.5, 1.0, 1.0, -0.0, 0.0, 1.0, 0.5, -1.0],
                  [0.0, -0.0, 0.0, -0.0, -2.0, -2.0, -3.0, 7.0]], np.float32)
    idx, _ = m.host_topk(z, 6)
    np.testing.assert_array_equal(idx, topk(z, 6))
    assert idx[0].tolist() == [1, 2, 5, 0, 6, 3]    # ties to the lower id; -0 == +0
    assert idx[1].tolist() == [7, 0, 1, 2, 3, 4]


def test_host_topk_rejects_bad_arguments():
    z = np.zeros((1, 8), np.float32)
    with pytest.raises(m.MoeError):
        m.host_topk(z, 9)
    with pytest.raises(m.MoeError):
        m.host_topk(z, 0)


def _key_order(zt):
    """The GPU top-k's order: float bits of z + 0 mapped to keys that order as
    the floats do (sign-magnitude to offset binary), larger key first, lower id
    on equal keys."""
    b = (zt.astype(np.float32) + np.float32(0.0)).view(np.uint32).astype(np.uint64)
    key = np.where(b & 0x80000000, (~b) & 0xFFFFFFFF, b | 0x80000000)
    return np.lexsort((np.arange(zt.size), -key.astype(np.int64)))


def test_host_topk_infinities():
    """Hand-worked: +inf twice (lower id first), then 3, 1, 0, -1, then -inf
    twice (the oracle refuses non-finite logits, so this is its own pin)."""
    z = np.array([[1.0, np.inf, -np.inf, 3.0, np.inf, -1.0, 0.0, -np.inf]], np.float32)
    idx, _ = m.host_topk(z, 8, False)
    np.testing.assert_array_equal(idx[0], [1, 4, 3, 0, 6, 5, 2, 7])
    np.testing.assert_array_equal(idx[0], _key_order(z[0]))


def test_host_topk_nan_follows_the_gpu_key_order():
    """Non-finite logits lie outside the method; a NaN still gets the GPU's
    key order (a positive NaN above +inf, a negative one below -inf), so host
    and GPU select the same ids, and the selection stays well defined."""
    pos_nan = np.array([0x7FC00000], np.uint32).view(np.float32)[0]
    neg_nan = np.array([0xFFC00000], np.uint32).view(np.float32)[0]
    z = np.array([[1.0, pos_nan, 2.0, neg_nan, -np.inf, np.inf, 0.5, -0.0]], np.float32)
    idx, _ = m.host_topk(z, 8, False)
    np.testing.assert_array_equal(idx[0], _key_order(z[0])[:8])
    assert idx[0][0] == 1 and idx[0][1] == 5 and idx[0][-1] == 3
