#include "residency.h"

namespace strata {

void ResidencyManager::init(int num_experts, int budget, int policy, uint64_t expert_bytes) {
  num_experts_ = num_experts;
  budget_ = budget;
  policy_ = policy;
  expert_bytes_ = expert_bytes;
  n_ = 0;
  forwards = hits = misses = evictions = bytes_h2d = waves = 0;
  slot_expert_.assign(budget, -1);
  expert_slot_.assign(num_experts, -1);
  last_use_.assign(num_experts, 0);
  use_count_.assign(num_experts, 0);
  in_wave_.assign(num_experts, 0);
  for (int s = 0; s < budget; ++s) {
    slot_expert_[s] = s;
    expert_slot_[s] = s;
  }
}

int ResidencyManager::resident() const {
  int r = 0;
  for (int e : slot_expert_) r += (e >= 0);
  return r;
}

bool ResidencyManager::before(int a, int b) const {
  if (policy_ == kLFU && use_count_[a] != use_count_[b]) return use_count_[a] < use_count_[b];
  if (last_use_[a] != last_use_[b]) return last_use_[a] < last_use_[b];
  return a < b;
}

void ResidencyManager::forward(const std::vector<int32_t>& needed,
                               std::vector<std::vector<PlanEntry>>& plan) {
  plan.clear();
  if (needed.empty()) return;
  ++n_;
  ++forwards;
  std::vector<int32_t> order;
  order.reserve(needed.size());
  uint64_t nh = 0;
  for (int32_t e : needed)
    if (expert_slot_[e] >= 0) {
      order.push_back(e);
      ++nh;
    }
  for (int32_t e : needed)
    if (expert_slot_[e] < 0) order.push_back(e);
  const uint64_t nm = needed.size() - nh;

  for (size_t w0 = 0; w0 < order.size(); w0 += budget_) {
    const size_t w1 = (w0 + budget_ < order.size()) ? w0 + budget_ : order.size();
    for (size_t i = w0; i < w1; ++i) in_wave_[order[i]] = 1;
    std::vector<PlanEntry> wave;
    wave.reserve(w1 - w0);
    for (size_t i = w0; i < w1; ++i) {
      const int32_t e = order[i];
      if (expert_slot_[e] >= 0) {
        wave.push_back({e, expert_slot_[e], false});
        continue;
      }
      int slot = -1;
      for (int s = 0; s < budget_; ++s)
        if (slot_expert_[s] < 0) {
          slot = s;
          break;
        }
      if (slot < 0) {
        int victim = -1;
        for (int s = 0; s < budget_; ++s) {
          const int r = slot_expert_[s];
          if (in_wave_[r]) continue;
          if (victim < 0 || before(r, victim)) victim = r;
        }
        slot = expert_slot_[victim];
        expert_slot_[victim] = -1;
        ++evictions;
      }
      slot_expert_[slot] = e;
      expert_slot_[e] = slot;
      wave.push_back({e, slot, true});
    }
    for (size_t i = w0; i < w1; ++i) in_wave_[order[i]] = 0;
    plan.push_back(std::move(wave));
  }
  for (int32_t e : needed) {
    last_use_[e] = n_;
    ++use_count_[e];
  }
  hits += nh;
  misses += nm;
  bytes_h2d += nm * expert_bytes_;
  waves += plan.size();
}

}  // namespace strata
