// Host-side residency manager of the HBM expert slots (no HIP dependency).
//
// The pages fix the problem, not the policy: a per-layer budget of resident
// experts with the rest streamed ("Documentation" page, Signature: budget and
// policy arguments), a GPU cache of the most-used experts that adapts to the
// workload over an all-experts copy pinned in host RAM ("Strata, Explained",
// section 2).  The rules below are the reading this library implements:
//   * create fills slots 0..B-1 with experts 0..B-1 (last_use 0, use_count 0);
//   * a forward needs the experts with at least one token, N ascending;
//     hits are those resident when it starts, misses the rest;
//   * N is run as hits (ascending) then misses (ascending), in waves of at most
//     B experts; a wave's compute finishes before any of its slots is reused;
//   * a miss takes the lowest free slot, else evicts the resident outside the
//     current wave with the smallest key: LRU (last_use, id), LFU (use_count,
//     last_use, id);
//   * then every expert of N gets last_use = forward number, use_count += 1.
// None of this changes what a forward computes, only what it copies.
#pragma once
#include <stdint.h>

#include <vector>

namespace strata {

struct PlanEntry {
  int32_t expert;
  int32_t slot;
  bool paged;
};

class ResidencyManager {
 public:
  static constexpr int kLRU = 1;
  static constexpr int kLFU = 2;

  void init(int num_experts, int budget, int policy, uint64_t expert_bytes);
  // `needed` must be ascending and unique.  Fills `waves` with the plan.
  void forward(const std::vector<int32_t>& needed, std::vector<std::vector<PlanEntry>>& waves);

  int budget() const { return budget_; }
  int resident() const;
  int slot_of(int e) const { return expert_slot_[e]; }

  uint64_t forwards = 0, hits = 0, misses = 0, evictions = 0, bytes_h2d = 0, waves = 0;

 private:
  bool before(int a, int b) const;  // a is a better victim than b
  int num_experts_ = 0, budget_ = 0, policy_ = kLRU;
  uint64_t expert_bytes_ = 0, n_ = 0;
  std::vector<int32_t> slot_expert_, expert_slot_;
  std::vector<uint64_t> last_use_, use_count_;
  std::vector<uint8_t> in_wave_;
};

}  // namespace strata
