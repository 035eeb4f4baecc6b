// Host-side residency manager of the HBM expert slots (no HIP dependency).
//
// The pages fix the problem, not the policy: a per-layer budget of resident
// experts with the rest streamed ("Documentation" page, Signature: budget and
// policy arguments), a GPU cache of the most-used experts that adapts to the
// workload over an all-experts copy pinned in host RAM ("Strata, Explained",
// section 2), a learned cache that can be saved across restarts and a tunable
// adaptation rate (same page, section 8), and predictors that may reorder
// work but not change it (ro99/strata README, rules).  The rules below are the
// reading this library implements:
//   * each expert has last_use (forward number) and a frequency score
//     (unsigned, one use = kUnit); create fills slots 0..B-1 with experts
//     0..B-1 and, given a profile, sets the scores and rebalances (below);
//   * a forward needs the experts with at least one token, N ascending;
//     hits are those resident when it starts, misses the rest;
//   * N is run as hits (ascending) then misses by increasing key (the
//     coldest first, so the hottest misses stream last and are still
//     resident for the next forward; keys as below); if N fits in B
//     slots it is one wave; otherwise the floor(B/4) hits with the largest
//     keys stay pinned for the whole forward (a long prompt does not flush the
//     hot set) and the list runs in waves of W = floor(S/2) (1 if S < 2),
//     S = B - pinned, so the next wave's pages land while a wave computes;
//   * a miss takes the lowest free slot, else evicts, among residents outside
//     the current wave, the previous wave (multi-wave, S >= 2) and the pinned
//     set, the one with the smallest key: LRU (last_use, id), LFU and WARM
//     (score, last_use, id); each page records the wave of this forward that
//     last read its slot (after_wave), the only compute it has to wait for;
//   * then (WARM only) every score loses score >> decay_shift, and every
//     expert of N gains kUnit and gets last_use = forward number;
//   * with prefetch P > 0, non-residents by decreasing rank (the key without
//     the id; ties to the lower id) are paired with residents by increasing
//     key, and while fewer than P pairs are taken and the candidate outranks
//     the resident strictly, the candidate is paged into that slot;
//   * a profile load sets the scores, then the B experts with the largest
//     score (ties to the lower id) take the slots of the residents outside
//     that set, newcomers ascending by id into freed slots ascending;
//   * a hybrid forward (host cores compute what the GPU does not hold:
//     "Strata, Explained", section 2; the `hybrid` policy value of the
//     "Documentation" page) runs its hits from their slots and hands every
//     other needed expert to the host; it pages nothing for them, then updates
//     scores and prefetches like any forward, as one wave;
//   * a hybrid prefill with row limit R hands the needed experts that are not
//     resident and have at most R tokens to the host and runs the others as
//     above (hits, misses in waves); scores and prefetch cover every needed
//     expert; at least one wave is counted.
// None of this changes what a forward computes, only what it copies.
#pragma once
#include <stdint.h>

#include <vector>

namespace strata {

struct PlanEntry {
  int32_t expert;
  int32_t slot;
  bool paged;
  int32_t after_wave = -1;  // a page's slot was last read by this wave of the
                            // same forward (-1: by no wave of it)
};

class ResidencyManager {
 public:
  static constexpr int kLRU = 1;
  static constexpr int kLFU = 2;
  static constexpr int kWARM = 3;
  static constexpr uint64_t kUnit = uint64_t(1) << 16;
  static constexpr uint64_t kMaxScore = uint64_t(1) << 62;

  void init(int num_experts, int budget, int policy, int decay_shift, int prefetch, uint64_t expert_bytes);
  // `needed` must be ascending and unique.  Fills `waves` with the plan and
  // `ahead` with the pages to make once the forward's compute is done.  With
  // `host` (hybrid prefill), the needed experts that are not resident and have
  // at most host_rows tokens (rows[e]) go to `host` (ascending) instead of
  // being paged; the scores and the prefetch still cover every needed expert.
  void forward(const std::vector<int32_t>& needed, std::vector<std::vector<PlanEntry>>& waves,
               std::vector<PlanEntry>& ahead, const int32_t* rows = nullptr, int host_rows = 0,
               std::vector<int32_t>* host = nullptr);
  // Sets the scores (E values, each <= kMaxScore; checked by the caller) and
  // rebalances; `count` books the pages as prefetches (run time) or not
  // (create).  Fills `pages` with the copies to make.
  void load_profile(const uint64_t* scores, bool count, std::vector<PlanEntry>& pages);
  // Hybrid forward: `hits` gets the resident experts of `needed` (ascending,
  // unique) with their slots, `host` the others; `ahead` as in forward().
  void forward_hybrid(const std::vector<int32_t>& needed, std::vector<PlanEntry>& hits,
                      std::vector<int32_t>& host, std::vector<PlanEntry>& ahead);
  const std::vector<uint64_t>& scores() const { return score_; }

  int budget() const { return budget_; }
  int resident() const;
  int slot_of(int e) const { return expert_slot_[e]; }
  int expert_in(int slot) const { return slot_expert_[slot]; }

  uint64_t forwards = 0, hits = 0, misses = 0, evictions = 0, bytes_h2d = 0, waves = 0;
  uint64_t prefetched = 0, prefetch_hits = 0, host_experts = 0;

 private:
  void finish(const std::vector<int32_t>& needed, std::vector<PlanEntry>& ahead);
  bool rank_less(int a, int b) const;  // rank of a < rank of b (ids ignored)
  bool before(int a, int b) const;     // a is a better victim than b
  void page(int e, int slot, bool count, std::vector<PlanEntry>& pages);
  int num_experts_ = 0, budget_ = 0, policy_ = kLRU, decay_shift_ = 0, prefetch_ = 0;
  uint64_t expert_bytes_ = 0, n_ = 0;
  std::vector<int32_t> slot_expert_, expert_slot_;
  std::vector<uint64_t> last_use_, score_;
  std::vector<uint8_t> in_wave_, keep_, from_prefetch_;
  std::vector<int32_t> wave_of_;  // wave of the current forward that runs the expert, or -1
};

}  // namespace strata
