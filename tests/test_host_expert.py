"""The library's host-core expert (the host-miss path) against the oracle's
fp64 expert on the same interchange bytes."""
import numpy as np
import pytest

import expert_cache_host_amd as m
import synth
from oracle.layer import expert_output


@pytest.mark.parametrize("d,f,T", [(256, 512, 1), (256, 512, 3), (2048, 768, 2), (128, 96, 5)])
def test_host_expert_matches_oracle(d, f, T):
    wl = synth.Workload("h", 77, 1, d, f, 2, 1, 1)
    buf = synth.gen_experts(wl, 0, 0, 1)
    rng = np.random.default_rng(d + f + T)
    x = rng.standard_normal((T, d)).astype(np.float32) * 1.5
    y = m.host_expert_forward(buf, d, f, x, threads=3)
    ref = expert_output(buf, 0, d, f, x.astype(np.float64))
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.max(np.abs(y - ref)) <= 1e-4 * rms
