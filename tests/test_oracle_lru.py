"""Pins of the LRU slot simulator (oracle/lru.py): hand-worked traces, the
textbook LRU list for k = 1, S = E, a full-scan victim check and invariants."""
import os
import random
from collections import OrderedDict

import pytest

from oracle.lru import DECAY, HOST, LRU, SCORE, STREAM, LayerSlots

G = os.path.join(os.path.dirname(__file__), "golden", "lru_traces.txt")


def _parse_traces():
    traces = {}
    for line in open(G):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        parts = [p.strip() for p in line.split("|")]
        name = parts[0]
        tr = traces.setdefault(name, {"calls": [], "views": [], "stages": None})
        if parts[1].startswith("E="):
            kv = dict(p.split("=") for p in parts[1].split())
            tr.update(E=int(kv["E"]), S=int(kv["S"]), mode=kv["mode"], fills=int(kv["fills"]),
                      policy=kv.get("policy", LRU), tokens=int(kv.get("tokens", "1")),
                      adopt=int(kv.get("adopt", "-1")))
        elif parts[1].startswith("call"):
            idx = [int(v) for v in parts[2].split()[1:]]
            hits = int(parts[3].split()[1])
            ev_txt = parts[4][len("evict"):].strip()
            evs = [] if ev_txt == "-" else [tuple(int(v) for v in t.strip("()").split(","))
                                            for t in ev_txt.split()]
            tr["calls"].append((idx, hits, evs))
        elif parts[1] == "views":
            sv = [int(v) for v in parts[2].split()[1:]]
            hv = [int(v) for v in parts[3].split()[1:]]
            tr["views"].append((sv, hv))
        elif parts[1] == "stages":
            # stage members of the call on the line above
            st = [[int(e) for e in s.split(":")[1].split(",")] for s in parts[2].split()]
            if tr["stages"] is None:
                tr["stages"] = {}
            tr["stages"][len(tr["calls"]) - 1] = st
        elif parts[1] == "preload":
            tr["preload"] = [int(v) for v in parts[2].split()]
        elif parts[1] == "final":
            tr["final"] = [int(v) for v in parts[2].split()[1:]]
    return traces


TRACES = _parse_traces()


@pytest.mark.parametrize("name", sorted(TRACES))
def test_golden_trace(name):
    tr = TRACES[name]
    sim = LayerSlots(tr["E"], tr["S"], tr["policy"], tr["adopt"])
    if "preload" in tr:
        sim.preload(tr["preload"])
    for c, (idx, hits, evs) in enumerate(tr["calls"]):
        res = sim.plan(idx, tr["mode"], tr["fills"], tr["tokens"])
        assert res.hits == hits
        assert res.evictions == evs
        if tr["views"]:
            sv, hv = tr["views"][c]
            assert res.stage_views[0] == sv
            assert res.host_view == hv
        if tr["stages"] is not None and c in tr["stages"]:
            assert res.stage_experts == tr["stages"][c]
        sim.check_invariants()
    assert sim.expert_in == tr["final"]


def test_k1_host_mode_is_textbook_lru():
    rnd = random.Random(5)
    for e_count, s_count in ((5, 2), (8, 3), (16, 7), (4, 4)):
        sim = LayerSlots(e_count, s_count)
        lru = OrderedDict((e, None) for e in range(s_count))  # first = least recent
        for _ in range(400):
            e = rnd.randrange(e_count) if rnd.random() < 0.6 else rnd.randrange(min(3, e_count))
            res = sim.plan([e], HOST)
            if e in lru:
                assert res.hits == 1 and res.evictions == []
                lru.move_to_end(e)
            else:
                old, _ = lru.popitem(last=False)
                lru[e] = None
                assert res.hits == 0
                assert [(r[3], r[4]) for r in res.evictions] == [(old, e)]
            assert set(sim.expert_in) == set(lru)


@pytest.mark.parametrize("mode", [STREAM, HOST])
def test_slots_equal_experts_all_hits(mode):
    rnd = random.Random(6)
    sim = LayerSlots(16, 16)
    for _ in range(100):
        idx = rnd.sample(range(16), 4) + rnd.sample(range(16), 4)
        res = sim.plan(idx, mode)
        assert res.misses == 0 and res.hits == 8 and res.evictions == []
    assert sim.stats["evictions"] == 0


def _full_scan_victim(sim):
    empty = [s for s in range(sim.S) if sim.expert_in[s] == -1]
    if empty:
        return empty[0]
    cands = sorted((sim.last_use[s], s) for s in range(sim.S) if sim.last_use[s] < sim.clock)
    return cands[0][1] if cands else None


@pytest.mark.parametrize("mode", [STREAM, HOST])
def test_invariants_random(mode):
    rnd = random.Random(7)
    for e_count, s_count, k, t in ((8, 4, 2, 1), (32, 5, 4, 3), (64, 8, 8, 4), (20, 2, 3, 6)):
        sim = LayerSlots(e_count, s_count)
        orig_victim = sim.victim
        sim.victim = lambda: (lambda v: (v, _assert_eq(v, _full_scan_victim(sim)))[0])(orig_victim())
        for _ in range(200):
            idx = []
            for _t in range(t):
                idx += rnd.sample(range(e_count), k)
            before_use = list(sim.last_use)
            res = sim.plan(idx, mode, max_fills=rnd.choice([-1, -1, 0, 1, 2]) if mode == HOST else -1)
            sim.check_invariants()
            assert res.hits + res.misses == len(idx)
            uniq = sorted(set(idx))
            if mode == STREAM:
                # every unique expert is computed in exactly one stage
                flat = [e for st in res.stage_experts for e in st]
                assert sorted(flat) == uniq
                for v, members in zip(res.stage_views, res.stage_experts):
                    assert sorted(e for e in range(e_count) if v[e] >= 0) == members
                # within a stage, no stage member's slot is evicted in that stage
                for (call, stage, slot, old, new) in res.evictions:
                    assert old not in res.stage_experts[stage]
            else:
                hits = [e for e in uniq if res.stage_views[0][e] >= 0]
                evicted = [r[3] for r in res.evictions]
                assert not set(hits) & set(evicted)
                for e in range(e_count):
                    assert (res.stage_views[0][e] >= 0) != (res.host_view[e] >= 0)
            del before_use


def _assert_eq(a, b):
    assert a == b
    return True


def test_stream_stage_count_closed_form():
    # cold selection of all E experts with S slots: ceil((E - S) / S) fill stages
    # after the stage of the S initial hits.
    for e_count, s_count in ((8, 2), (9, 2), (256, 64), (12, 5)):
        sim = LayerSlots(e_count, s_count)
        res = sim.plan(list(range(e_count)), STREAM)
        assert len(res.stage_views) == 1 + -(-(e_count - s_count) // s_count)
        assert res.hits == s_count and res.fills == e_count - s_count


class _MRU(LayerSlots):
    def victim(self):  # planted mistake: most recently used
        for s in range(self.S):
            if self.expert_in[s] == -1:
                return s
        c = [s for s in range(self.S) if self.last_use[s] < self.clock]
        return max(c, key=lambda s: (self.last_use[s], s)) if c else None


class _NoProtect(LayerSlots):
    def victim(self):  # planted mistake: protected slots may be evicted
        for s in range(self.S):
            if self.expert_in[s] == -1:
                return s
        return min(range(self.S), key=lambda s: (self.last_use[s], s))


class _HighTie(LayerSlots):
    def victim(self):  # planted mistake: ties on last_use go to the higher slot
        for s in range(self.S):
            if self.expert_in[s] == -1:
                return s
        c = [s for s in range(self.S) if self.last_use[s] < self.clock]
        return max(c, key=lambda s: (-self.last_use[s], s)) if c else None


def _trace_passes(cls, tr):
    sim = cls(tr["E"], tr["S"], tr["policy"], tr["adopt"])
    try:
        if "preload" in tr:
            sim.preload(tr["preload"])
        for c, (idx, hits, evs) in enumerate(tr["calls"]):
            res = sim.plan(idx, tr["mode"], tr["fills"], tr["tokens"])
            if res.hits != hits or res.evictions != evs:
                return False
            if tr["views"] and (res.stage_views[0], res.host_view) != tr["views"][c]:
                return False
            if tr["stages"] is not None and c in tr["stages"] and \
                    res.stage_experts != tr["stages"][c]:
                return False
    except Exception:
        return False
    return sim.expert_in == tr["final"]


@pytest.mark.parametrize("cls", [_MRU, _NoProtect, _HighTie])
def test_planted_victim_mistakes_fail_the_traces(cls):
    """Each plausible slip in the victim rule contradicts at least one hand-worked trace."""
    assert all(_trace_passes(LayerSlots, tr) for tr in TRACES.values())
    assert not all(_trace_passes(cls, tr) for tr in TRACES.values())


# ---------------------------------------------------------------- score policy

class _DecayPerCall(LayerSlots):
    def _update_scores(self, idx, tokens):  # planted mistake: one decay per call
        return super()._update_scores(idx, 1)


class _NoDecay(LayerSlots):
    def _update_scores(self, idx, tokens):  # planted mistake: plain use counts
        for e in idx:
            self.score[e] += 1.0


class _ScoreButLruVictim(LayerSlots):
    def _key(self, s):  # planted mistake: the score policy evicts by recency
        return (self.last_use[s], s)


@pytest.mark.parametrize("cls", [_DecayPerCall, _NoDecay, _ScoreButLruVictim])
def test_planted_score_mistakes_fail_the_traces(cls):
    score_traces = [tr for tr in TRACES.values() if tr["policy"] == SCORE]
    assert score_traces and all(_trace_passes(LayerSlots, tr) for tr in score_traces)
    assert not all(_trace_passes(cls, tr) for tr in score_traces)


def test_score_candidate_order_pinned():
    # trace G's first call has candidates 1 (0.9) and 2 (1.0): taking them in id
    # order would put expert 1 in the slot
    tr = TRACES["G"]
    sim = LayerSlots(tr["E"], tr["S"], SCORE)
    res = sim.plan(tr["calls"][0][0], HOST, -1, tr["tokens"])
    assert [r[4] for r in res.evictions] == [2]
    assert sim.score[2] > sim.score[1] > 0.0


def test_score_closed_forms():
    # n consecutive single-token uses: sum_{i<n} 0.9^i = (1 - 0.9^n) / 0.1;
    # one use followed by m calls without it: 0.9^m
    sim = LayerSlots(8, 2, SCORE)
    for n in range(1, 40):
        sim.plan([5], HOST)
        assert abs(sim.score[5] - (1.0 - DECAY ** n) / (1.0 - DECAY)) < 1e-12
    sim = LayerSlots(8, 2, SCORE)
    sim.plan([6], HOST)
    for m in range(1, 30):
        sim.plan([0], HOST)
        assert abs(sim.score[6] - DECAY ** m) < 1e-15
    # T tokens in one call decay T times
    sim = LayerSlots(8, 2, SCORE)
    sim.plan([3, 1, 1, 1], HOST, -1, tokens=4)
    assert abs(sim.score[3] - DECAY ** 3) < 1e-15
    assert abs(sim.score[1] - (1.0 + DECAY + DECAY ** 2)) < 1e-15


def test_score_admission_needs_a_strictly_higher_score():
    # "Missed experts that score higher than the weakest slot are promoted":
    # an equal score does not promote, the next representable one above does
    import math
    for cand, promoted in ((1.0, False), (math.nextafter(1.0, 2.0), True), (0.5, False)):
        sim = LayerSlots(3, 1, SCORE)          # slot 0 holds expert 0
        sim._update_scores = lambda idx, tokens, c=cand, s=sim: s.score.__setitem__(
            slice(None), [1.0, 0.0, c])
        res = sim.plan([2], HOST)
        assert (res.evictions == [(0, 0, 0, 0, 2)]) == promoted


def _full_scan_weakest(sim):
    empty = [s for s in range(sim.S) if sim.expert_in[s] == -1]
    if empty:
        return empty[0]
    cands = sorted((sim.score[sim.expert_in[s]], s) for s in range(sim.S)
                   if sim.last_use[s] < sim.clock)
    return cands[0][1] if cands else None


@pytest.mark.parametrize("mode", [STREAM, HOST])
def test_score_invariants_random(mode):
    rnd = random.Random(11)
    for e_count, s_count, k, t in ((8, 4, 2, 1), (32, 5, 4, 3), (64, 8, 8, 1), (20, 2, 3, 2)):
        sim = LayerSlots(e_count, s_count, SCORE)
        orig_victim = sim.victim
        sim.victim = lambda: (lambda v: (v, _assert_eq(v, _full_scan_weakest(sim)))[0])(orig_victim())
        for _ in range(200):
            idx = []
            for _t in range(t):
                idx += rnd.sample(range(min(e_count, 3 * k)) if rnd.random() < 0.6
                                  else range(e_count), k)
            budget = rnd.choice([-1, -1, 0, 1, 2]) if mode == HOST else -1
            scores_before = None
            res = sim.plan(idx, mode, budget, tokens=t)
            sim.check_invariants()
            assert res.hits + res.misses == len(idx)
            if mode == HOST:
                if budget >= 0:
                    assert len(res.evictions) <= budget
                hits = [e for e in sorted(set(idx)) if res.stage_views[0][e] >= 0]
                for (_c, _st, _slot, old, new) in res.evictions:
                    assert old not in hits
                    assert old == -1 or sim.score[new] > sim.score[old]
            else:
                flat = [e for st in res.stage_experts for e in st]
                assert sorted(flat) == sorted(set(idx))
            del scores_before


@pytest.mark.parametrize("mode", [STREAM, HOST])
def test_score_slots_equal_experts_all_hits(mode):
    rnd = random.Random(12)
    sim = LayerSlots(16, 16, SCORE)
    for _ in range(100):
        res = sim.plan(rnd.sample(range(16), 4), mode)
        assert res.misses == 0 and res.evictions == []


def test_score_budget_zero_never_fills():
    rnd = random.Random(13)
    sim = LayerSlots(32, 4, SCORE)
    for _ in range(200):
        assert sim.plan(rnd.sample(range(32), 4), HOST, 0).evictions == []
    assert sim.expert_in == [0, 1, 2, 3]


# ---------------------------------------------------------------- usage profile

class _MostUsedFirst(LayerSlots):
    def preload(self, counts):  # planted mistake: the most used expert in slot 0
        super().preload(counts)
        self.expert_in = list(reversed(self.expert_in))
        for s, e in enumerate(self.expert_in):
            self.slot_of[e] = s


def test_planted_preload_order_fails_trace():
    tr = TRACES["H"]
    assert _trace_passes(LayerSlots, tr)
    assert not _trace_passes(_MostUsedFirst, tr)


def test_preload_takes_the_top_slots_by_brute_force():
    rnd = random.Random(21)
    for e_count, s_count in ((8, 3), (32, 32), (64, 5), (128, 32)):
        counts = [rnd.choice([0, 1, 2, 5, 5, 40, 2 ** 32 - 1]) for _ in range(e_count)]
        sim = LayerSlots(e_count, s_count)
        sim.preload(counts)
        sim.check_invariants()
        # every kept expert is used at least as often as every dropped one, and
        # at an equal count the lower id is kept
        kept = set(sim.expert_in)
        for a in kept:
            for b in set(range(e_count)) - kept:
                assert counts[a] > counts[b] or (counts[a] == counts[b] and a < b)
        # slot order: non-decreasing rank of use from slot S-1 down to slot 0
        keys = [(-counts[e], e) for e in sim.expert_in]
        assert keys == sorted(keys, reverse=True)


def test_usage_counts_every_selection():
    rnd = random.Random(22)
    sim = LayerSlots(16, 4, SCORE)
    seen = [0] * 16
    for _ in range(300):
        t = rnd.choice([1, 2, 3])
        idx = []
        for _t in range(t):
            idx += rnd.sample(range(16), 3)
        for e in idx:
            seen[e] += 1
        sim.plan(idx, rnd.choice([STREAM, HOST]), -1, tokens=t)
    assert sim.usage == seen
    sim.preload([1] * 16)
    assert sim.usage == [c + 1 for c in seen]
    assert sim.score == [0.0] * 16


def test_preloaded_profile_serves_its_own_routing():
    # host mode with no fills: after preloading a sequence's own counts, a
    # selection hits exactly when its expert is among the S most used
    rnd = random.Random(23)
    e_count, s_count = 32, 8
    seq = [rnd.sample(list(range(6)) + rnd.sample(range(32), 4), 4) for _ in range(100)]
    counts = [0] * e_count
    for idx in seq:
        for e in idx:
            counts[e] += 1
    top = set(sorted(range(e_count), key=lambda e: (-counts[e], e))[:s_count])
    sim = LayerSlots(e_count, s_count)
    sim.preload(counts)
    hits = sum(sim.plan(idx, HOST, 0).hits for idx in seq)
    assert hits == sum(1 for idx in seq for e in idx if e in top)


# ---------------------------------------------------------------- prefill preheat
class _PreheatAscending(LayerSlots):
    def _preheat_pool(self, idx, uniq, pending):  # planted mistake: plain miss order
        pool, weak, order = super()._preheat_pool(idx, uniq, pending)
        return pool, weak, sorted(pending)


class _PreheatStrongPool(LayerSlots):
    def _preheat_pool(self, idx, uniq, pending):  # planted mistake: strongest slots pool
        pool, weak, order = super()._preheat_pool(idx, uniq, pending)
        others = sorted((s for s in range(self.S) if s not in pool), key=weak, reverse=True)
        cand = sorted(pool + others, key=weak, reverse=True)
        return cand[:len(pool)], weak, order


class _PreheatLruVictim(LayerSlots):
    def _pool_victim(self, pool, weakness):  # planted mistake: recency inside the pool
        c = [s for s in pool if self.expert_in[s] == -1 or self.last_use[s] < self.clock]
        return min(c, key=lambda s: (self.last_use[s], s)) if c else None


class _PreheatNoKeep(LayerSlots):
    def _pool_victim(self, pool, weakness):  # planted mistake: every slot stages
        return self.victim()


@pytest.mark.parametrize("cls", [_PreheatAscending, _PreheatStrongPool, _PreheatLruVictim,
                                 _PreheatNoKeep])
def test_planted_preheat_mistakes_fail_the_traces(cls):
    assert not all(_trace_passes(cls, tr) for tr in TRACES.values())


def _counts(idx):
    c = {}
    for e in idx:
        c[e] = c.get(e, 0) + 1
    return c


def _staged_call(rnd, e_count, k, t):
    idx = []
    for _ in range(t):
        idx += rnd.sample(range(e_count), k)
    return idx


@pytest.mark.parametrize("e_count,s_count,k,t", [(16, 4, 2, 9), (32, 6, 4, 12), (64, 8, 8, 16),
                                                 (12, 3, 3, 7)])
def test_preheat_full_share_ends_with_the_call_top_experts(e_count, s_count, k, t):
    """adopt = 1000: after a staged call the layer holds exactly the call's S
    top-ranked experts by (-count, id), each miss is filled once, and every stage
    view maps only its own experts."""
    rnd = random.Random(31)
    sim = LayerSlots(e_count, s_count, LRU, 1000)
    n_staged = 0
    for _ in range(120):
        idx = _staged_call(rnd, e_count, k, t)
        before = list(sim.slot_of)
        res = sim.plan(idx, STREAM, -1, t)
        sim.check_invariants()
        cnt = _counts(idx)
        uniq = sorted(cnt)
        hits = [e for e in uniq if before[e] >= 0]
        misses = [e for e in uniq if before[e] < 0]
        staged = len(misses) > s_count - len(hits)
        filled = [r[4] for r in res.evictions]
        assert sorted(filled) == misses  # each miss exactly once
        assert sorted(sum(res.stage_experts, [])) == uniq  # each selected expert in one stage
        if staged:
            n_staged += 1
            top = sorted(uniq, key=lambda e: (-cnt[e], e))[:s_count]
            assert sorted(sim.expert_in) == sorted(top)
    assert n_staged > 50


@pytest.mark.parametrize("adopt", [0, 100, 250, 500, 750])
def test_preheat_share_bounds_the_replaced_slots(adopt):
    """Slots outside the pool keep their experts: at most
    max(1, floor(adopt * S / 1000)) slots change in a staged call, and the pool
    ends holding the best-ranked misses."""
    rnd = random.Random(37 + adopt)
    e_count, s_count, k, t = 40, 8, 4, 10
    sim = LayerSlots(e_count, s_count, LRU, adopt)
    cap = max(1, adopt * s_count // 1000)
    for _ in range(100):
        idx = _staged_call(rnd, e_count, k, t)
        before_in = list(sim.expert_in)
        before = list(sim.slot_of)
        sim.plan(idx, STREAM, -1, t)
        cnt = _counts(idx)
        hits = [e for e in cnt if before[e] >= 0]
        misses = sorted(e for e in cnt if before[e] < 0)
        if len(misses) <= s_count - len(hits):
            continue
        changed = [s for s in range(s_count) if sim.expert_in[s] != before_in[s]]
        assert 1 <= len(changed) <= cap
        ranked = sorted(misses, key=lambda e: (-cnt[e], e))
        assert sorted(sim.expert_in[s] for s in changed) == sorted(ranked[:len(changed)])


def test_preheat_leaves_unstaged_calls_to_the_plain_rule():
    rnd = random.Random(41)
    plain = LayerSlots(24, 8, LRU, -1)
    pre = LayerSlots(24, 8, LRU, 1000)
    for _ in range(300):
        idx = rnd.sample(range(24), rnd.choice((1, 2, 3)))
        a = plain.plan(idx, STREAM)
        b = pre.plan(idx, STREAM)
        assert a.evictions == b.evictions and a.stage_views == b.stage_views
    assert plain.expert_in == pre.expert_in


def test_preheat_bad_share_rejected():
    with pytest.raises(ValueError):
        LayerSlots(8, 4, LRU, 1001)
    with pytest.raises(ValueError):
        LayerSlots(8, 4, LRU, -2)
