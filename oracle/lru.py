"""Per-layer slot table as a step-by-step LRU simulator (oracle side, plain ints).

What the pages fix:

* each layer owns a fixed number of GPU slots holding copies of experts; the
  routing yields two tables, expert -> GPU slot (-1 when not cached) and
  expert -> CPU id (-1 when cached) ("How it works", llama.cpp + MoE expert
  cache, step 2);
* replacement is least-recently-used, independently per layer; the experts of
  the current batch are planned together, those already needed by the batch
  are protected from eviction and duplicate ids load once; when one step needs
  more experts than there are slots, the routed computation runs in stages whose
  partial results are summed (longhaul.md, "Longhaul MoE loading");
* a slot leaves the table before its copy starts and is published after it
  ("Keeping the cache fresh", llama.cpp + MoE expert cache).

Readings taken where the pages are silent:

* start: slot s holds expert s (s < S), last_use = 0, clock = 0;
* per call: U = sorted unique selected ids; pre_view = the table at call start;
  a selection is a hit when pre_view[e] >= 0 (counted per selection);
* each stage: clock += 1; the stage's resident experts are protected
  (last_use = clock); pending misses are taken in ascending id; the victim is the
  lowest-index empty slot, else the slot with the smallest (last_use, index)
  among last_use < clock; evict, insert, last_use = clock, log
  (call, stage, slot, old expert, new expert); no victim -> the stage ends;
* stream mode: every miss is filled; stage views map the experts of that stage
  to their slot and every other expert to -1; the host table is all -1;
* host mode: one stage; fills capped by max_fills (-1 = no cap), in ascending
  id; the views are the full tables at call start (cached -> slot,
  uncached -> -1 / uncached -> own id, cached -> -1); fills are visible from the
  same layer's next call on.

The score policy follows "Keeping the cache fresh" (llama.cpp + MoE expert
cache): after each step the routing is read back and a usage score per expert
decays by 0.9 per token; missed experts scoring higher than the weakest slot
are promoted, within a budget of copies.  Readings:

* score[e] starts at 0.0 (binary64); per call, for each token t in order:
  every score is multiplied by 0.9, then each expert token t selected gains
  1.0 -- before any slot decision of the call;
* protection and the clock are those of the LRU rule (a stage's resident
  experts and the experts inserted in it are protected for that stage);
* the weakest slot is the lowest-index empty slot, else the unprotected slot
  with the smallest (score of its expert, slot index);
* host mode: the missed experts are candidates in order of (-score, id); a
  candidate is promoted into the weakest slot only when its score is strictly
  greater than that slot's (an empty slot always loses), up to max_fills
  promotions; the first candidate that does not beat the weakest slot ends the
  call's promotions (later candidates score no higher, and the weakest slot
  only rises);
* stream mode: every miss is still filled, stage by stage in ascending id, the
  victim being the weakest slot instead of the least recently used one.

Usage profile (llama.cpp fork with multi GPU acceleration, "Persistent hot
experts": the cache saves how often each expert was used and the next start
preloads each layer's most-used experts).  Readings:

* every selection of a call adds 1 to its expert's lifetime count (uint32);
* preload(counts): the layer's S most-used experts by (-count, id) take the
  slots, the least used of them in slot 0 and the most used in slot S-1, so
  that with equal last_use the least used is the first victim; every slot gets
  last_use = the current clock (unprotected from the next stage on), usage
  scores restart at 0, and the loaded counts are added to the lifetime counts.

Prefill preheat (llama.cpp fork with multi GPU acceleration, "Prefill
preheat": a prompt batch's experts are on the GPU anyway for its matmuls; the
cache keeps the batch's most-used ones, device to device, in place of cached
experts the batch used less; an adopt share bounds the share of a layer's
slots that one batch may replace).  Here the slots themselves are the staging
area of a call that needs more experts than fit, so the reading is a choice of
which slots stage and in what order.  Readings, for a stream-mode call whose
misses outnumber the slots that hold none of its hits (a staged call), when
adopt >= 0 (per mille; -1 = off, the plain rule above):

* cnt[e] = selections of e in the call; an expert ranks above another by
  (-cnt, id); F = the call's S top-ranked experts;
* weakness order of slots: empty slots first (by index), then occupied ones
  with the lowest-ranked expert first;
* the pool is the first P = min(#slots holding no expert of F,
  floor(adopt * S / 1000)) of the slots holding no expert of F, in weakness
  order; when P = 0 the pool is one slot, the weakest of those slots if any,
  else the weakest slot (the staging needs a slot);
* slots outside the pool are never victims in the call (they keep their
  experts; hits among them run in stage 0);
* stages as in the plain rule (stage 0 protects the hits), but misses are
  placed lowest-ranked first, and the victim is the first unprotected pool
  slot in weakness order;
* so the pool ends holding the top-ranked misses, and with
  P = #(slots without an F expert) the layer ends holding exactly F.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

STREAM = "stream"
HOST = "host"
LRU = "lru"
SCORE = "score"
DECAY = 0.9  # usage score factor per token


@dataclass
class PlanResult:
    call: int
    unique: List[int]
    hits: int
    misses: int
    stage_views: List[List[int]]          # one slot view per stage
    host_view: List[int]
    evictions: List[Tuple[int, int, int, int, int]] = field(default_factory=list)
    fills: int = 0
    stage_experts: List[List[int]] = field(default_factory=list)


class LayerSlots:
    """LRU slot state of one layer."""

    def __init__(self, n_experts: int, slots: int, policy: str = LRU, adopt: int = -1):
        if not 1 <= slots <= n_experts:
            raise ValueError("slots must be in [1, n_experts]")
        if policy not in (LRU, SCORE):
            raise ValueError("policy must be 'lru' or 'score'")
        if not -1 <= adopt <= 1000:
            raise ValueError("adopt must be -1 (off) or a share in per mille, 0..1000")
        self.E = n_experts
        self.S = slots
        self.policy = policy
        self.adopt = adopt
        self.score = [0.0] * n_experts
        self.usage = [0] * n_experts
        self.expert_in = list(range(slots))
        self.slot_of = [-1] * n_experts
        for s in range(slots):
            self.slot_of[s] = s
        self.last_use = [0] * slots
        self.clock = 0
        self.calls = 0
        self.log: List[Tuple[int, int, int, int, int]] = []
        self.stats = dict(calls=0, selections=0, hits=0, misses=0, unique=0, fills=0,
                          evictions=0, host_selections=0, stages=0)

    # -- victim choice -------------------------------------------------------
    def victim(self):
        """Lowest-index empty slot, else the unprotected slot with the smallest
        (last_use, index) under LRU or (score of its expert, index) under the
        score policy; None when every slot is protected."""
        for s in range(self.S):
            if self.expert_in[s] == -1:
                return s
        best = None
        for s in range(self.S):
            if self.last_use[s] < self.clock:
                if best is None or self._key(s) < self._key(best):
                    best = s
        return best

    def _key(self, s):
        if self.policy == SCORE:
            return (self.score[self.expert_in[s]], s)
        return (self.last_use[s], s)

    def _update_scores(self, idx, tokens):
        if tokens < 1 or len(idx) % tokens:
            raise ValueError("selections must split evenly over the tokens")
        k = len(idx) // tokens
        for t in range(tokens):
            for e in range(self.E):
                self.score[e] = self.score[e] * DECAY
            for e in idx[t * k:(t + 1) * k]:
                self.score[e] = self.score[e] + 1.0

    def _insert(self, call, stage, slot, e, log):
        old = self.expert_in[slot]
        if old >= 0:
            self.slot_of[old] = -1
            self.stats["evictions"] += 1
        self.expert_in[slot] = e
        self.slot_of[e] = slot
        self.last_use[slot] = self.clock
        rec = (call, stage, slot, old, e)
        self.log.append(rec)
        log.append(rec)
        self.stats["fills"] += 1

    # -- one call ------------------------------------------------------------
    def plan(self, idx, mode: str = STREAM, max_fills: int = -1, tokens: int = 1) -> PlanResult:
        idx = [int(e) for e in idx]
        for e in idx:
            if not 0 <= e < self.E:
                raise ValueError("expert id out of range")
        if self.policy == SCORE:
            self._update_scores(idx, tokens)
        for e in idx:
            self.usage[e] = (self.usage[e] + 1) & 0xFFFFFFFF
        call = self.calls
        self.calls += 1
        uniq = sorted(set(idx))
        pre_view = list(self.slot_of)
        hits = sum(1 for e in idx if pre_view[e] >= 0)
        misses = len(idx) - hits
        hit_experts = [e for e in uniq if pre_view[e] >= 0]
        pending = [e for e in uniq if pre_view[e] < 0]
        log: List[Tuple[int, int, int, int, int]] = []
        views: List[List[int]] = []
        stage_experts: List[List[int]] = []

        if mode == STREAM:
            pool = None
            weak = None
            if self.adopt >= 0 and len(pending) > self.S - len(hit_experts):
                pool, weak, pending = self._preheat_pool(idx, uniq, pending)
            stage = 0
            while stage == 0 or pending:
                self.clock += 1
                members = []
                if stage == 0:
                    for e in hit_experts:
                        self.last_use[self.slot_of[e]] = self.clock
                        members.append(e)
                placed = 0
                for e in pending:
                    v = self.victim() if pool is None else self._pool_victim(pool, weak)
                    if v is None:
                        break
                    self._insert(call, stage, v, e, log)
                    members.append(e)
                    placed += 1
                pending = pending[placed:]
                view = [-1] * self.E
                for e in members:
                    view[e] = self.slot_of[e]
                views.append(view)
                stage_experts.append(sorted(members))
                stage += 1
            host_view = [-1] * self.E
        elif mode == HOST:
            self.clock += 1
            for e in hit_experts:
                self.last_use[self.slot_of[e]] = self.clock
            placed = 0
            order = pending
            if self.policy == SCORE:
                order = sorted(pending, key=lambda e: (-self.score[e], e))
            for e in order:
                if max_fills >= 0 and placed >= max_fills:
                    break
                v = self.victim()
                if v is None:
                    break
                if self.policy == SCORE and self.expert_in[v] >= 0 and \
                        not self.score[e] > self.score[self.expert_in[v]]:
                    break
                self._insert(call, 0, v, e, log)
                placed += 1
            views.append(pre_view)
            stage_experts.append(hit_experts)
            host_view = [e if pre_view[e] < 0 else -1 for e in range(self.E)]
            self.stats["host_selections"] += misses
        else:
            raise ValueError("mode must be 'stream' or 'host'")

        st = self.stats
        st["calls"] += 1
        st["selections"] += len(idx)
        st["hits"] += hits
        st["misses"] += misses
        st["unique"] += len(uniq)
        st["stages"] += len(views)
        return PlanResult(call=call, unique=uniq, hits=hits, misses=misses, stage_views=views,
                          host_view=host_view, evictions=log, fills=len(log),
                          stage_experts=stage_experts)

    # -- prefill preheat ------------------------------------------------------
    def _preheat_pool(self, idx, uniq, pending):
        """Pool slots, weakness key and miss order of a staged call under the
        adopt share; see the module notes."""
        cnt = {}
        for e in idx:
            cnt[e] = cnt.get(e, 0) + 1

        def rank(e):
            return (-cnt.get(e, 0), e)

        def weakness(s):
            e = self.expert_in[s]
            if e < 0:
                return (0, s)
            r = rank(e)
            return (1, -r[0], -r[1])  # lowest-ranked expert first

        top = set(sorted(uniq, key=rank)[:self.S])
        others = sorted((s for s in range(self.S) if self.expert_in[s] not in top),
                        key=weakness)
        n = min(len(others), self.adopt * self.S // 1000)
        if n > 0:
            pool = others[:n]
        elif others:
            pool = others[:1]
        else:
            pool = [min(range(self.S), key=weakness)]
        order = sorted(pending, key=rank, reverse=True)
        return pool, weakness, order

    def _pool_victim(self, pool, weakness):
        """First unprotected pool slot in weakness order (empty slots first);
        None when every pool slot is protected."""
        best = None
        for s in pool:
            if self.expert_in[s] == -1 or self.last_use[s] < self.clock:
                if best is None or weakness(s) < weakness(best):
                    best = s
        return best

    def preload(self, counts):
        """Loads the S most-used experts by (-count, id); see the module notes."""
        counts = [int(c) for c in counts]
        if len(counts) != self.E or any(c < 0 or c > 0xFFFFFFFF for c in counts):
            raise ValueError("counts must be E uint32 values")
        ranked = sorted(range(self.E), key=lambda e: (-counts[e], e))[:self.S]
        self.expert_in = list(reversed(ranked))
        self.slot_of = [-1] * self.E
        for s, e in enumerate(self.expert_in):
            self.slot_of[e] = s
        self.last_use = [self.clock] * self.S
        self.score = [0.0] * self.E
        self.usage = [(u + c) & 0xFFFFFFFF for u, c in zip(self.usage, counts)]

    def check_invariants(self):
        for s, e in enumerate(self.expert_in):
            if e >= 0:
                assert self.slot_of[e] == s
        for e, s in enumerate(self.slot_of):
            if s >= 0:
                assert self.expert_in[s] == e
