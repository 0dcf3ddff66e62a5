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
