// Per-layer LRU slot planner (host only, no HIP calls).
//
// Rules (longhaul.md, "Longhaul MoE loading": fixed budget, least-recently-used
// replacement per layer, the batch's experts protected, duplicate ids loaded
// once, staged execution when one step needs more experts than slots;
// "How it works", llama.cpp + MoE expert cache, step 2: expert -> slot table
// with -1 when not cached and expert -> CPU id table with -1 when cached):
//
//   start: slot s holds expert s, last_use 0, clock 0.
//   per call: U = sorted distinct ids; a selection hits when its expert is
//   cached at call start.
//   per stage: clock += 1; resident experts of the stage get last_use = clock;
//   pending misses in ascending id take the lowest-index empty slot, else the
//   slot with the smallest (last_use, index) among last_use < clock; no such
//   slot ends the stage.
//   stream mode: every miss is filled, over as many stages as needed; a stage's
//   slot table maps that stage's experts only; the host table is all -1.
//   host mode: one stage; at most max_fills fills (-1 = no cap) in ascending id;
//   the tables are the full tables at call start.
//
// Score policy ("Keeping the cache fresh", llama.cpp + MoE expert cache: a
// decayed usage score per expert, x0.9 per token; missed experts scoring higher
// than the weakest slot are promoted, within a copy budget):
//   score[e] starts at 0 (binary64); per call, for each token in order, every
//   score is multiplied by 0.9 and each expert the token selected gains 1, before
//   any slot decision.  The victim is the lowest-index empty slot, else the
//   unprotected slot with the smallest (score of its expert, index).  Host mode
//   takes the misses in order of (-score, id) and promotes one only when its
//   score is strictly greater than the victim's, up to max_fills; the first
//   that is not ends the call's promotions.  Stream mode fills every miss.
//
// Usage profile ("Persistent hot experts", llama.cpp fork with multi GPU
// acceleration): every selection adds 1 to its expert's lifetime count
// (uint32).  preload(counts) puts the S most-used experts by (-count, id) in
// the slots, the least used of them in slot 0 and the most used in slot S-1,
// gives every slot last_use = clock, resets the scores and adds the counts to
// the lifetime counts.
//
// Prefill preheat ("Prefill preheat", llama.cpp fork with multi GPU
// acceleration: the cache keeps a prompt batch's most-used experts in place of
// cached experts the batch used less, within an adopt share of the slots).
// With adopt >= 0 (per mille; -1 = off), a stream-mode call whose misses
// outnumber the slots holding none of its hits is staged through a pool:
//   experts rank by (-count in the call, id); F = the S top-ranked; slot
//   weakness: empty first, then the lowest-ranked expert first; the pool is the
//   first min(#slots without an F expert, floor(adopt * S / 1000)) slots without
//   an F expert in weakness order, or one slot when that is 0 (the weakest
//   without an F expert, else the weakest); other slots are never victims in
//   the call; misses are placed lowest-ranked first into the first unprotected
//   pool slot in weakness order.
#pragma once
#include <cstdint>
#include <vector>

namespace moe {

struct EvictRecord {
  int64_t call;
  int32_t stage, slot, evicted, inserted;
};

struct Fill {
  int32_t expert, slot;
};

struct PlanStage {
  std::vector<int32_t> members;  // experts computed in this stage, ascending
  std::vector<Fill> fills;       // copies that must land before the stage runs
};

enum Policy : int32_t { kPolicyLru = 0, kPolicyScore = 1 };
constexpr double kScoreDecay = 0.9;

struct CallPlan {
  int64_t call = -1;
  int32_t hits = 0, misses = 0, unique = 0, fills = 0, evictions = 0;
  std::vector<PlanStage> stages;
  std::vector<int32_t> host_experts;  // host mode: experts computed on host cores
  std::vector<int32_t> pre_view;      // table at call start [E]
  int32_t mode = 0;
};

class SlotPlanner {
 public:
  SlotPlanner(int32_t n_experts, int32_t slots, int32_t policy = kPolicyLru,
              int32_t adopt = -1);

  // Plans one call on n_sel = tokens * k router ids (token-major).  mode: 0
  // stream, 1 host.
  void plan(const int32_t *idx, int32_t n_sel, int32_t tokens, int32_t mode, int32_t max_fills,
            CallPlan &out);

  // Slot table of stage s of `p` (stream: that stage's members; host: pre_view).
  void stage_view(const CallPlan &p, int32_t s, int32_t *slot_view, int32_t *host_view) const;

  int32_t n_experts() const { return E_; }
  int32_t slots() const { return S_; }
  const std::vector<int32_t> &expert_in() const { return expert_in_; }
  const std::vector<int32_t> &slot_of() const { return slot_of_; }
  const std::vector<uint64_t> &last_use() const { return last_use_; }
  const std::vector<double> &scores() const { return score_; }
  const std::vector<uint32_t> &usage() const { return usage_; }

  // Loads the usage profile counts[n_experts] (see above).
  void preload(const uint32_t *counts);
  int32_t policy() const { return policy_; }
  int32_t adopt() const { return adopt_; }
  void set_adopt(int32_t adopt) { adopt_ = adopt; }  // -1 off, else per mille 0..1000
  const std::vector<EvictRecord> &log() const { return log_; }
  uint64_t clock() const { return clock_; }

 private:
  int32_t victim() const;
  bool weaker(int32_t a, int32_t b) const;  // slot a before slot b as a victim
  void update_scores(const int32_t *idx, int32_t n_sel, int32_t tokens);
  void insert(int64_t call, int32_t stage, int32_t slot, int32_t e, CallPlan &out);
  // preheat: pool slots and miss order of a staged stream call
  void preheat_pool(const int32_t *idx, int32_t n_sel, const std::vector<int32_t> &uniq,
                    std::vector<int32_t> &pending, std::vector<int32_t> &pool);
  bool ranks_above(int32_t a, int32_t b) const;   // expert a before expert b
  bool weaker_slot(int32_t a, int32_t b) const;   // slot a before slot b (weakness)
  int32_t pool_victim(const std::vector<int32_t> &pool) const;

  int32_t E_, S_, policy_, adopt_;
  std::vector<int32_t> cnt_;  // selections per expert in the current call (preheat)
  std::vector<double> score_;
  std::vector<uint32_t> usage_;
  std::vector<int32_t> expert_in_, slot_of_;
  std::vector<uint64_t> last_use_;
  std::vector<uint8_t> seen_;
  uint64_t clock_ = 0;
  int64_t calls_ = 0;
  std::vector<EvictRecord> log_;
};

}  // namespace moe
