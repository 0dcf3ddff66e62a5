#include "planner.hpp"

#include <algorithm>

namespace moe {

SlotPlanner::SlotPlanner(int32_t n_experts, int32_t slots, int32_t policy, int32_t adopt)
    : E_(n_experts), S_(slots), policy_(policy), adopt_(adopt), cnt_(n_experts, 0),
      score_(n_experts, 0.0), usage_(n_experts, 0),
      expert_in_(slots),
      slot_of_(n_experts, -1), last_use_(slots, 0), seen_(n_experts, 0) {
  for (int32_t s = 0; s < slots; ++s) {
    expert_in_[s] = s;
    slot_of_[s] = s;
  }
}

bool SlotPlanner::weaker(int32_t a, int32_t b) const {
  if (policy_ == kPolicyScore) {
    const double sa = score_[expert_in_[a]], sb = score_[expert_in_[b]];
    return sa < sb || (sa == sb && a < b);
  }
  return last_use_[a] < last_use_[b] || (last_use_[a] == last_use_[b] && a < b);
}

int32_t SlotPlanner::victim() const {
  for (int32_t s = 0; s < S_; ++s)
    if (expert_in_[s] < 0) return s;
  int32_t best = -1;
  for (int32_t s = 0; s < S_; ++s) {
    if (last_use_[s] >= clock_) continue;
    if (best < 0 || weaker(s, best)) best = s;
  }
  return best;
}

// Per token: every score times 0.9, then +1 for the token's experts (separate
// roundings; the build keeps floating-point contraction off).
void SlotPlanner::update_scores(const int32_t *idx, int32_t n_sel, int32_t tokens) {
  const int32_t k = n_sel / tokens;
  for (int32_t t = 0; t < tokens; ++t) {
    for (double &v : score_) v = v * kScoreDecay;
    for (int32_t j = 0; j < k; ++j) score_[idx[t * k + j]] = score_[idx[t * k + j]] + 1.0;
  }
}

void SlotPlanner::insert(int64_t call, int32_t stage, int32_t slot, int32_t e, CallPlan &out) {
  const int32_t old = expert_in_[slot];
  if (old >= 0) {
    slot_of_[old] = -1;
    out.evictions++;
  }
  expert_in_[slot] = e;
  slot_of_[e] = slot;
  last_use_[slot] = clock_;
  log_.push_back(EvictRecord{call, stage, slot, old, e});
  out.fills++;
}

bool SlotPlanner::ranks_above(int32_t a, int32_t b) const {
  return cnt_[a] > cnt_[b] || (cnt_[a] == cnt_[b] && a < b);
}

bool SlotPlanner::weaker_slot(int32_t a, int32_t b) const {
  const int32_t ea = expert_in_[a], eb = expert_in_[b];
  if (ea < 0 || eb < 0) return ea < 0 && (eb >= 0 || a < b);
  return ranks_above(eb, ea);  // the lower-ranked expert is the weaker slot
}

int32_t SlotPlanner::pool_victim(const std::vector<int32_t> &pool) const {
  int32_t best = -1;
  for (int32_t s : pool) {
    if (expert_in_[s] >= 0 && last_use_[s] >= clock_) continue;
    if (best < 0 || weaker_slot(s, best)) best = s;
  }
  return best;
}

void SlotPlanner::preheat_pool(const int32_t *idx, int32_t n_sel,
                               const std::vector<int32_t> &uniq, std::vector<int32_t> &pending,
                               std::vector<int32_t> &pool) {
  std::fill(cnt_.begin(), cnt_.end(), 0);
  for (int32_t i = 0; i < n_sel; ++i) cnt_[idx[i]]++;
  std::vector<int32_t> ranked = uniq;
  std::sort(ranked.begin(), ranked.end(),
            [&](int32_t a, int32_t b) { return ranks_above(a, b); });
  // mark F, the S top-ranked experts of the call
  const size_t n_top = std::min(ranked.size(), (size_t)S_);
  for (size_t i = 0; i < n_top; ++i) seen_[ranked[i]] = 1;
  std::vector<int32_t> others;
  for (int32_t s = 0; s < S_; ++s)
    if (expert_in_[s] < 0 || !seen_[expert_in_[s]]) others.push_back(s);
  for (size_t i = 0; i < n_top; ++i) seen_[ranked[i]] = 0;
  std::sort(others.begin(), others.end(),
            [&](int32_t a, int32_t b) { return weaker_slot(a, b); });
  const size_t share = (size_t)((int64_t)adopt_ * S_ / 1000);
  const size_t n = std::min(others.size(), share);
  pool.clear();
  if (n > 0) {
    pool.assign(others.begin(), others.begin() + n);
  } else if (!others.empty()) {
    pool.push_back(others[0]);
  } else {
    int32_t w = 0;
    for (int32_t s = 1; s < S_; ++s)
      if (weaker_slot(s, w)) w = s;
    pool.push_back(w);
  }
  // lowest-ranked misses first
  std::sort(pending.begin(), pending.end(),
            [&](int32_t a, int32_t b) { return ranks_above(b, a); });
}

void SlotPlanner::plan(const int32_t *idx, int32_t n_sel, int32_t tokens, int32_t mode,
                       int32_t max_fills, CallPlan &out) {
  if (policy_ == kPolicyScore) update_scores(idx, n_sel, tokens);
  for (int32_t i = 0; i < n_sel; ++i) usage_[idx[i]]++;
  out = CallPlan();
  out.call = calls_++;
  out.mode = mode;
  out.pre_view = slot_of_;
  // distinct ids in ascending order; hits counted per selection
  std::vector<int32_t> uniq;
  uniq.reserve(n_sel);
  for (int32_t i = 0; i < n_sel; ++i) {
    const int32_t e = idx[i];
    if (slot_of_[e] >= 0) out.hits++;
    if (!seen_[e]) {
      seen_[e] = 1;
      uniq.push_back(e);
    }
  }
  for (int32_t e : uniq) seen_[e] = 0;
  std::sort(uniq.begin(), uniq.end());
  out.misses = n_sel - out.hits;
  out.unique = (int32_t)uniq.size();

  std::vector<int32_t> hit_experts, pending;
  for (int32_t e : uniq) (slot_of_[e] >= 0 ? hit_experts : pending).push_back(e);

  if (mode == 0) {
    std::vector<int32_t> pool;  // empty: the plain rule
    if (adopt_ >= 0 && (int64_t)pending.size() > (int64_t)S_ - (int64_t)hit_experts.size())
      preheat_pool(idx, n_sel, uniq, pending, pool);
    size_t next = 0;
    int32_t stage = 0;
    while (stage == 0 || next < pending.size()) {
      clock_++;
      PlanStage st;
      if (stage == 0) {
        for (int32_t e : hit_experts) {
          last_use_[slot_of_[e]] = clock_;
          st.members.push_back(e);
        }
      }
      while (next < pending.size()) {
        const int32_t v = pool.empty() ? victim() : pool_victim(pool);
        if (v < 0) break;
        const int32_t e = pending[next++];
        insert(out.call, stage, v, e, out);
        st.members.push_back(e);
        st.fills.push_back(Fill{e, v});
      }
      std::sort(st.members.begin(), st.members.end());
      out.stages.push_back(std::move(st));
      stage++;
    }
  } else {
    clock_++;
    PlanStage st;
    for (int32_t e : hit_experts) {
      last_use_[slot_of_[e]] = clock_;
      st.members.push_back(e);
    }
    int32_t placed = 0;
    std::vector<int32_t> order = pending;
    if (policy_ == kPolicyScore)
      std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
        return score_[a] > score_[b] || (score_[a] == score_[b] && a < b);
      });
    for (int32_t e : order) {
      if (max_fills >= 0 && placed >= max_fills) break;
      const int32_t v = victim();
      if (v < 0) break;
      if (policy_ == kPolicyScore && expert_in_[v] >= 0 && !(score_[e] > score_[expert_in_[v]]))
        break;
      insert(out.call, 0, v, e, out);
      st.fills.push_back(Fill{e, v});
      placed++;
    }
    out.stages.push_back(std::move(st));
    out.host_experts = pending;
  }
}

void SlotPlanner::preload(const uint32_t *counts) {
  std::vector<int32_t> order(E_);
  for (int32_t e = 0; e < E_; ++e) order[e] = e;
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t b) { return counts[a] > counts[b]; });
  std::fill(slot_of_.begin(), slot_of_.end(), -1);
  for (int32_t s = 0; s < S_; ++s) {
    const int32_t e = order[S_ - 1 - s];
    expert_in_[s] = e;
    slot_of_[e] = s;
    last_use_[s] = clock_;
  }
  std::fill(score_.begin(), score_.end(), 0.0);
  for (int32_t e = 0; e < E_; ++e) usage_[e] += counts[e];
}

void SlotPlanner::stage_view(const CallPlan &p, int32_t s, int32_t *slot_view,
                             int32_t *host_view) const {
  if (p.mode == 0) {
    if (slot_view) {
      std::fill(slot_view, slot_view + E_, -1);
      // members of stage s keep the slot they were given; later stages may
      // reuse slots, so rebuild from the stage's own record
      const PlanStage &st = p.stages[s];
      for (int32_t e : st.members) slot_view[e] = -1;
      for (const Fill &f : st.fills) slot_view[f.expert] = f.slot;
      if (s == 0)
        for (int32_t e : st.members)
          if (p.pre_view[e] >= 0) slot_view[e] = p.pre_view[e];
    }
    if (host_view) std::fill(host_view, host_view + E_, -1);
  } else {
    for (int32_t e = 0; e < E_; ++e) {
      if (slot_view) slot_view[e] = p.pre_view[e];
      if (host_view) host_view[e] = p.pre_view[e] < 0 ? e : -1;
    }
  }
}

}  // namespace moe
