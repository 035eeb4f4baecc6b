#include "residency.h"

#include <algorithm>

namespace strata {

void ResidencyManager::init(int num_experts, int budget, int policy, int decay_shift, int prefetch,
                            uint64_t expert_bytes) {
  num_experts_ = num_experts;
  budget_ = budget;
  policy_ = policy;
  decay_shift_ = policy == kWARM ? decay_shift : 0;
  prefetch_ = prefetch;
  expert_bytes_ = expert_bytes;
  n_ = 0;
  forwards = hits = misses = evictions = bytes_h2d = waves = 0;
  prefetched = prefetch_hits = host_experts = 0;
  slot_expert_.assign(budget, -1);
  expert_slot_.assign(num_experts, -1);
  last_use_.assign(num_experts, 0);
  score_.assign(num_experts, 0);
  in_wave_.assign(num_experts, 0);
  keep_.assign(num_experts, 0);
  wave_of_.assign(num_experts, -1);
  from_prefetch_.assign(num_experts, 0);
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

bool ResidencyManager::rank_less(int a, int b) const {
  if (policy_ != kLRU && score_[a] != score_[b]) return score_[a] < score_[b];
  return last_use_[a] < last_use_[b];
}

bool ResidencyManager::before(int a, int b) const {
  if (rank_less(a, b)) return true;
  if (rank_less(b, a)) return false;
  return a < b;
}

void ResidencyManager::page(int e, int slot, bool count, std::vector<PlanEntry>& pages) {
  const int old = slot_expert_[slot];
  if (old >= 0) {
    expert_slot_[old] = -1;
    from_prefetch_[old] = 0;
  }
  slot_expert_[slot] = e;
  expert_slot_[e] = slot;
  pages.push_back({e, slot, true});
  if (count) {
    if (old >= 0) ++evictions;
    ++prefetched;
    bytes_h2d += expert_bytes_;
    from_prefetch_[e] = 1;
  }
}

void ResidencyManager::load_profile(const uint64_t* scores, bool count, std::vector<PlanEntry>& pages) {
  pages.clear();
  score_.assign(scores, scores + num_experts_);
  std::vector<int32_t> order(num_experts_);
  for (int e = 0; e < num_experts_; ++e) order[e] = e;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return score_[a] > score_[b]; });
  std::vector<uint8_t> wanted(num_experts_, 0);
  for (int i = 0; i < budget_; ++i) wanted[order[i]] = 1;
  std::vector<int32_t> freed, newcomers;
  for (int s = 0; s < budget_; ++s)
    if (slot_expert_[s] < 0 || !wanted[slot_expert_[s]]) freed.push_back(s);
  for (int e = 0; e < num_experts_; ++e)
    if (wanted[e] && expert_slot_[e] < 0) newcomers.push_back(e);
  for (size_t i = 0; i < newcomers.size(); ++i) page(newcomers[i], freed[i], count, pages);
}

void ResidencyManager::forward(const std::vector<int32_t>& needed,
                               std::vector<std::vector<PlanEntry>>& plan, std::vector<PlanEntry>& ahead,
                               const int32_t* rows, int host_rows, std::vector<int32_t>* host) {
  plan.clear();
  ahead.clear();
  if (host) host->clear();
  if (needed.empty()) return;
  ++n_;
  ++forwards;
  std::vector<int32_t> order;
  order.reserve(needed.size());
  uint64_t nh = 0, nm = 0;
  for (int32_t e : needed)
    if (expert_slot_[e] >= 0) {
      order.push_back(e);
      ++nh;
      if (from_prefetch_[e]) {
        ++prefetch_hits;
        from_prefetch_[e] = 0;
      }
    }
  for (int32_t e : needed)
    if (expert_slot_[e] < 0) {
      if (host && host_rows > 0 && rows[e] <= host_rows) {
        host->push_back(e);  // hybrid prefill: computed by the host threads
      } else {
        order.push_back(e);
        ++nm;
      }
    }
  // misses coldest first (keys before this forward's updates)
  std::sort(order.begin() + nh, order.end(), [&](int a, int b) { return before(a, b); });

  // keep_: 1 = pinned for the forward; in_wave_: 1 = current wave, 2 = previous
  size_t W = budget_;
  bool prev_too = false;
  std::vector<int32_t> pinned;
  if (order.size() > (size_t)budget_) {
    pinned.assign(order.begin(), order.begin() + nh);  // the hits
    std::sort(pinned.begin(), pinned.end(), [&](int a, int b) { return before(b, a); });
    pinned.resize(std::min(pinned.size(), (size_t)(budget_ / 4)));
    for (int32_t e : pinned) keep_[e] = 1;
    const int S = budget_ - (int)pinned.size();
    W = S >= 2 ? S / 2 : 1;
    prev_too = S >= 2;
  }
  size_t p0 = 0, p1 = 0;  // previous wave: order[p0, p1)
  for (size_t w0 = 0; w0 < order.size(); w0 += W) {
    const size_t w1 = (w0 + W < order.size()) ? w0 + W : order.size();
    const int32_t wi = (int32_t)plan.size();
    for (size_t i = w0; i < w1; ++i) {
      in_wave_[order[i]] = 1;
      wave_of_[order[i]] = wi;
    }
    if (prev_too)
      for (size_t i = p0; i < p1; ++i) in_wave_[order[i]] = 2;
    std::vector<PlanEntry> wave;
    wave.reserve(w1 - w0);
    for (size_t i = w0; i < w1; ++i) {
      const int32_t e = order[i];
      if (expert_slot_[e] >= 0) {
        wave.push_back({e, expert_slot_[e], false});
        continue;
      }
      int slot = -1, after = -1;
      for (int s = 0; s < budget_; ++s)
        if (slot_expert_[s] < 0) {
          slot = s;
          break;
        }
      if (slot < 0) {
        int victim = -1;
        for (int s = 0; s < budget_; ++s) {
          const int r = slot_expert_[s];
          if (in_wave_[r] || keep_[r]) continue;
          if (victim < 0 || before(r, victim)) victim = r;
        }
        slot = expert_slot_[victim];
        after = wave_of_[victim];
        expert_slot_[victim] = -1;
        from_prefetch_[victim] = 0;
        ++evictions;
      }
      slot_expert_[slot] = e;
      expert_slot_[e] = slot;
      wave.push_back({e, slot, true, after});
    }
    for (size_t i = p0; i < w1; ++i) in_wave_[order[i]] = 0;
    p0 = w0;
    p1 = w1;
    plan.push_back(std::move(wave));
  }
  for (int32_t e : pinned) keep_[e] = 0;
  for (int32_t e : needed) wave_of_[e] = -1;
  hits += nh;
  misses += nm;
  bytes_h2d += nm * expert_bytes_;
  waves += plan.empty() ? 1 : plan.size();
  if (host) host_experts += host->size();
  finish(needed, ahead);
}

void ResidencyManager::forward_hybrid(const std::vector<int32_t>& needed, std::vector<PlanEntry>& hit_list,
                                      std::vector<int32_t>& host, std::vector<PlanEntry>& ahead) {
  hit_list.clear();
  host.clear();
  ahead.clear();
  if (needed.empty()) return;
  ++n_;
  ++forwards;
  for (int32_t e : needed) {
    if (expert_slot_[e] >= 0) {
      hit_list.push_back({e, expert_slot_[e], false});
      if (from_prefetch_[e]) {
        ++prefetch_hits;
        from_prefetch_[e] = 0;
      }
    } else {
      host.push_back(e);
    }
  }
  hits += hit_list.size();
  host_experts += host.size();
  ++waves;
  finish(needed, ahead);
}

// Score updates of a forward, then the policy's pages ahead of need.
void ResidencyManager::finish(const std::vector<int32_t>& needed, std::vector<PlanEntry>& ahead) {
  if (decay_shift_ > 0)
    for (int e = 0; e < num_experts_; ++e) score_[e] -= score_[e] >> decay_shift_;
  for (int32_t e : needed) {
    last_use_[e] = n_;
    score_[e] += kUnit;
  }
  if (prefetch_ > 0) {
    std::vector<int32_t> out, in;
    for (int e = 0; e < num_experts_; ++e) (expert_slot_[e] < 0 ? out : in).push_back(e);
    // candidates: decreasing rank, ties to the lower id; victims: increasing key
    std::stable_sort(out.begin(), out.end(), [&](int a, int b) { return rank_less(b, a); });
    std::sort(in.begin(), in.end(), [&](int a, int b) { return before(a, b); });
    const size_t np = std::min({out.size(), in.size(), (size_t)prefetch_});
    for (size_t i = 0; i < np; ++i) {
      if (!rank_less(in[i], out[i])) break;
      page(out[i], expert_slot_[in[i]], true, ahead);
    }
  }
}

}  // namespace strata
