"""The library's LRU planner (C++, via the C ABI, no GPU) against the oracle's
step-by-step simulator: views, hits, slot state and the replacement log must
agree bit for bit."""
import random

import numpy as np
import pytest

import expert_cache_host_amd as m
from oracle.lru import LayerSlots


def _compare(e_count, s_count, mode, max_fills, calls, seed, policy="lru", adopt=-1):
    rnd = random.Random(seed)
    lib_p = m.Planner(e_count, s_count, mode, max_fills, policy, adopt)
    sim = LayerSlots(e_count, s_count, policy, adopt)
    for _ in range(calls):
        t, k = rnd.choice([(1, 1), (1, 2), (1, 8), (2, 4), (4, 8), (3, 3)])
        k = min(k, e_count)
        hot = max(1, e_count // 4)
        idx = []
        for _t in range(t):
            pool = list(range(e_count))
            if rnd.random() < 0.7:
                pool = list(range(hot)) + rnd.sample(range(e_count), min(e_count, k))
                pool = sorted(set(pool))
            idx += rnd.sample(pool, k) if len(pool) >= k else rnd.sample(range(e_count), k)
        ns, hits, misses = lib_p.plan(idx, tokens=t)
        res = sim.plan(idx, mode, max_fills, tokens=t)
        assert (ns, hits, misses) == (len(res.stage_views), res.hits, res.misses)
        for s in range(ns):
            sv, hv = lib_p.views(s)
            assert sv.tolist() == res.stage_views[s]
            if mode == "host":
                assert hv.tolist() == res.host_view
            else:
                assert hv.tolist() == [-1] * e_count
        ein, lu = lib_p.slot_state()
        assert ein.tolist() == sim.expert_in
        assert lu.tolist() == sim.last_use
        # binary64 scores bit for bit (same operations in the same order)
        assert lib_p.scores().tolist() == sim.score
        assert lib_p.usage().tolist() == sim.usage
    assert lib_p.evictions() == sim.log


@pytest.mark.parametrize("mode", ["stream", "host"])
@pytest.mark.parametrize("e_count,s_count", [(8, 4), (8, 1), (16, 16), (128, 32), (256, 64), (20, 3)])
def test_planner_matches_oracle(mode, e_count, s_count):
    _compare(e_count, s_count, mode, -1, 150, seed=e_count * 31 + s_count)


@pytest.mark.parametrize("max_fills", [0, 1, 2])
def test_planner_budget_matches_oracle(max_fills):
    _compare(32, 6, "host", max_fills, 200, seed=max_fills)


def test_planner_staging_prefill_like():
    # 512 tokens x top-8 of 256 experts through 64 slots: many stages
    rng = np.random.default_rng(0)
    lib_p = m.Planner(256, 64, "stream")
    sim = LayerSlots(256, 64)
    for _ in range(3):
        idx = np.stack([rng.choice(256, 8, replace=False) for _ in range(512)]).ravel()
        ns, hits, misses = lib_p.plan(idx)
        res = sim.plan(idx.tolist(), "stream")
        assert ns == len(res.stage_views) >= 4
        for s in range(ns):
            assert lib_p.views(s)[0].tolist() == res.stage_views[s]
    assert lib_p.evictions() == sim.log


@pytest.mark.parametrize("mode", ["stream", "host"])
@pytest.mark.parametrize("e_count,s_count", [(8, 4), (8, 1), (16, 16), (128, 32), (256, 64), (20, 3)])
def test_score_planner_matches_oracle(mode, e_count, s_count):
    _compare(e_count, s_count, mode, -1, 150, seed=e_count * 17 + s_count, policy="score")


@pytest.mark.parametrize("max_fills", [0, 1, 2])
def test_score_planner_budget_matches_oracle(max_fills):
    _compare(32, 6, "host", max_fills, 200, seed=100 + max_fills, policy="score")


def test_planner_rejects_bad_policy_and_token_split():
    with pytest.raises(ValueError):
        m.Planner(8, 4, "host", -1, "fifo")
    p = m.Planner(8, 4, "host", -1, "score")
    with pytest.raises(m.MoeError):
        p.plan([0, 1, 2], tokens=2)


@pytest.mark.parametrize("policy", ["lru", "score"])
@pytest.mark.parametrize("mode", ["stream", "host"])
def test_planner_preload_matches_oracle(policy, mode):
    rnd = random.Random(31)
    e_count, s_count = 64, 8
    lib_p = m.Planner(e_count, s_count, mode, -1, policy)
    sim = LayerSlots(e_count, s_count, policy)
    for rnd_call in range(120):
        if rnd_call in (0, 50):
            counts = np.array([rnd.choice([0, 1, 3, 3, 7, 2 ** 32 - 1]) for _ in range(e_count)],
                              np.uint32)
            lib_p.preload(counts)
            sim.preload(counts.tolist())
        idx = rnd.sample(range(e_count), 4)
        ns, hits, misses = lib_p.plan(idx)
        res = sim.plan(idx, mode, -1)
        assert (ns, hits) == (len(res.stage_views), res.hits)
        assert lib_p.views(0)[0].tolist() == res.stage_views[0]
        ein, lu = lib_p.slot_state()
        assert ein.tolist() == sim.expert_in and lu.tolist() == sim.last_use
        assert lib_p.usage().tolist() == sim.usage
        assert lib_p.scores().tolist() == sim.score
    assert lib_p.evictions() == sim.log


# ---------------------------------------------------------------- prefill preheat
@pytest.mark.parametrize("adopt", [0, 1, 250, 500, 1000])
@pytest.mark.parametrize("e_count,s_count", [(8, 4), (8, 1), (20, 3), (128, 32), (256, 64)])
def test_preheat_planner_matches_oracle(adopt, e_count, s_count):
    _compare(e_count, s_count, "stream", -1, 120, seed=e_count * 7 + s_count + adopt,
             adopt=adopt)


@pytest.mark.parametrize("adopt", [250, 1000])
def test_preheat_planner_score_policy_matches_oracle(adopt):
    _compare(64, 8, "stream", -1, 150, seed=adopt, policy="score", adopt=adopt)


def test_preheat_host_mode_ignores_the_share():
    _compare(32, 6, "host", 2, 150, seed=3, adopt=1000)


@pytest.mark.parametrize("adopt", [125, 1000])
def test_preheat_planner_prefill_like(adopt):
    # 512 tokens x top-8 of 256 experts through 64 slots, Zipf-like popularity
    rng = np.random.default_rng(1)
    p = 1.0 / np.arange(1, 257) ** 0.8
    p /= p.sum()
    lib_p = m.Planner(256, 64, "stream", adopt=adopt)
    sim = LayerSlots(256, 64, "lru", adopt)
    for _ in range(4):
        idx = np.stack([rng.choice(256, 8, replace=False, p=p) for _ in range(512)]).ravel()
        ns, hits, misses = lib_p.plan(idx, tokens=512)
        res = sim.plan(idx.tolist(), "stream", -1, 512)
        assert ns == len(res.stage_views) and (hits, misses) == (res.hits, res.misses)
        for s in range(ns):
            assert lib_p.views(s)[0].tolist() == res.stage_views[s]
        assert lib_p.slot_state()[0].tolist() == sim.expert_in
    assert lib_p.evictions() == sim.log


def test_preheat_bad_share_rejected():
    with pytest.raises(m.MoeError):
        m.Planner(8, 4, adopt=1001)
    with pytest.raises(m.MoeError):
        m.Planner(8, 4, adopt=-2)
