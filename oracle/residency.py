"""Plain model of the expert-slot residency policy (test infrastructure only).

The pages state the problem, not the policy: a budget of experts stays
resident and the rest is streamed ("Documentation" page, Signature: `budget`
and `policy`); the GPU holds a cache of the most-used experts that adapts to
the conversation while every expert sits pinned in host RAM ("Strata,
Explained", section 2).  The exact rules are a reading (R9), written here as
plainly as possible:

* create fills slots 0..B-1 with experts 0..B-1, last_use = 0, use_count = 0;
* forward n (n = 1, 2, ...): N = experts with at least one token, ascending;
  hits = N that are resident when the call starts, misses = the rest;
* the needed list is hits (ascending) then misses (ascending), cut into waves
  of B experts; a wave is computed before any of its slots is reused;
* each miss, in list order, takes the lowest free slot, else evicts the
  resident with the smallest key among residents that are not in the current
  wave: LRU key (last_use, id), LFU key (use_count, last_use, id);
* afterwards every expert of N gets last_use = n and use_count += 1.

Outputs of the layer do not depend on any of this; only the counters do.
"""
from __future__ import annotations

LRU = "lru"
LFU = "lfu"


class ResidencyModel:
    def __init__(self, num_experts: int, budget: int, policy: str = LRU, expert_bytes: int = 0):
        if not 1 <= budget <= num_experts:
            raise ValueError("budget must be in [1, E]")
        if policy not in (LRU, LFU):
            raise ValueError("policy must be lru or lfu")
        self.E, self.B, self.policy, self.expert_bytes = num_experts, budget, policy, expert_bytes
        self.slot_expert = list(range(budget))          # slot -> expert (-1 free)
        self.last_use = [0] * num_experts
        self.use_count = [0] * num_experts
        self.n = 0
        self.forwards = self.hits = self.misses = self.evictions = self.bytes_h2d = self.waves = 0

    def resident(self) -> dict:
        return {e: s for s, e in enumerate(self.slot_expert) if e >= 0}

    def _key(self, e):
        if self.policy == LRU:
            return (self.last_use[e], e)
        return (self.use_count[e], self.last_use[e], e)

    def forward(self, needed):
        """Apply one forward with needed expert set `needed`; return the plan:
        a list of waves, each a list of (expert, slot, paged) tuples."""
        N = sorted(set(int(e) for e in needed))
        if not N:
            return []
        self.n += 1
        self.forwards += 1
        res = self.resident()
        hits = [e for e in N if e in res]
        misses = [e for e in N if e not in res]
        order = hits + misses
        plan = []
        for w0 in range(0, len(order), self.B):
            wave = order[w0:w0 + self.B]
            in_wave = set(wave)
            entries = []
            for e in wave:
                res = self.resident()
                if e in res:
                    entries.append((e, res[e], False))
                    continue
                free = [s for s, x in enumerate(self.slot_expert) if x < 0]
                if free:
                    slot = free[0]
                else:
                    cands = [x for x in res if x not in in_wave]
                    victim = min(cands, key=self._key)
                    slot = res[victim]
                    self.evictions += 1
                self.slot_expert[slot] = e
                entries.append((e, slot, True))
            plan.append(entries)
        for e in N:
            self.last_use[e] = self.n
            self.use_count[e] += 1
        self.hits += len(hits)
        self.misses += len(misses)
        self.bytes_h2d += len(misses) * self.expert_bytes
        self.waves += len(plan)
        return plan

    def stats(self) -> dict:
        resident = sum(1 for e in self.slot_expert if e >= 0)
        return dict(forwards=self.forwards, hits=self.hits, misses=self.misses,
                    evictions=self.evictions, bytes_h2d=self.bytes_h2d, waves=self.waves,
                    budget=self.B, resident=resident, resident_bytes=resident * self.expert_bytes)
