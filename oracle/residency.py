"""Plain model of the expert-slot residency policy (test infrastructure only).

The pages state the problem, not the policy: a budget of experts stays
resident and the rest is streamed ("Documentation" page, Signature: `budget`
and `policy`, whose values are none, warm, cache and hybrid); the GPU holds a
cache of the most-used experts that adapts to the conversation while every
expert sits pinned in host RAM ("Strata, Explained", section 2); the learned
cache can be saved and restored, one profile per kind of work, and how fast
the cache adapts is a tuning knob (same page, section 8); a predictor may
reorder work but never change what is computed (ro99/strata README, the list
of rules).  The exact rules are a reading, written here as plainly as
possible:

* every expert has last_use (forward number, 0 at create) and a frequency
  score (an unsigned integer, one use = UNIT = 2**16, 0 at create);
* create fills slots 0..B-1 with experts 0..B-1; if a profile (E scores) is
  given, the scores are set to it and the slots are then rebalanced (below);
* forward n (n = 1, 2, ...): N = experts with at least one token, ascending;
  hits = N that are resident when the call starts, misses = the rest;
* the needed list is hits (ascending) then misses by increasing key (keys
  below, as they stand when the call starts): the coldest misses stream
  first, so the hottest are still resident for the next forward.  If it holds
  at most B experts it is one wave.  Otherwise (a forward that streams more
  experts than there are slots) the P = floor(B/4) hits with the largest keys
  are pinned for the whole forward, so a long prompt does not flush the hot
  set; the other S = B - (pinned count) slots stream, and the list is cut into
  waves of W = floor(S/2) experts (1 if S < 2): while one wave computes, the
  next one's pages land in slots the computing wave does not read;
* each miss, in list order, takes the lowest free slot, else evicts the
  resident with the smallest key among the residents that are not in the
  current wave, not in the previous wave (multi-wave forwards with S >= 2)
  and not pinned.  Keys: LRU (last_use, id); LFU and WARM (score, last_use,
  id);
* afterwards every expert loses score >> d (d = decay_shift; WARM only, LRU
  and LFU use d = 0), every expert of N gains UNIT and gets last_use = n;
  so a use's weight falls by 1 - 2**-d per later forward (the adaptation rate);
* prefetch P > 0 (any policy), after those updates: with rank = the key
  without the id, pair the non-resident experts by decreasing rank (ties to
  the lower id) with the residents in increasing key order; while fewer than
  P pairs are taken and the candidate's rank is strictly larger than the
  resident's, the candidate is paged into that resident's slot (an eviction
  and a prefetch);
* rebalance (profile load): the wanted set is the B experts with the largest
  score, ties to the lower id; residents outside it free their slots (in
  ascending slot order), and the wanted experts that are not resident take
  them in ascending id order.  At run time each such page counts as an
  eviction and a prefetch; at create it counts nothing;
* prefetch_hits counts hits on an expert whose residency came from a prefetch
  or a run-time profile load, once, at its first use;
* hybrid forward (the Documentation page's policy value `hybrid`, undefined
  there; "Strata, Explained" section 2: the CPU computes the experts the GPU
  does not hold, at the same time): hits are run from their slots, every
  other needed expert is computed on the host and counted in host_experts;
  nothing is paged for them, so slots, misses, evictions and bytes do not
  move; the score updates and the prefetch step are those of any forward, and
  the forward is one wave;
* hybrid prefill (the same policy for forwards of more than eight tokens,
  with a row limit R): the needed experts that are not resident when the
  forward starts and have at most R tokens are computed on the host (counted
  in host_experts); the other needed experts run as an ordinary forward (hits,
  then misses paged in waves, as above, the pinned quarter chosen among the
  hits); the score updates and the prefetch step cover every needed expert,
  and the forward counts at least one wave.

Outputs of the layer do not depend on any of this; only the counters do.
"""
from __future__ import annotations

LRU = "lru"
LFU = "lfu"
WARM = "warm"
POLICIES = (LRU, LFU, WARM)
UNIT = 1 << 16
MAX_SCORE = 1 << 62


class ResidencyModel:
    def __init__(self, num_experts: int, budget: int, policy: str = LRU, expert_bytes: int = 0,
                 decay_shift: int = 0, prefetch: int = 0, profile=None):
        if not 1 <= budget <= num_experts:
            raise ValueError("budget must be in [1, E]")
        if policy not in POLICIES:
            raise ValueError("policy must be lru, lfu or warm")
        if policy == WARM and not 1 <= decay_shift <= 24:
            raise ValueError("warm needs decay_shift in [1, 24]")
        if policy != WARM and decay_shift != 0:
            raise ValueError("decay_shift applies to warm only")
        if not 0 <= prefetch <= budget:
            raise ValueError("prefetch must be in [0, B]")
        self.E, self.B, self.policy, self.expert_bytes = num_experts, budget, policy, expert_bytes
        self.d, self.P = decay_shift, prefetch
        self.slot_expert = list(range(budget))          # slot -> expert (-1 free)
        self.last_use = [0] * num_experts
        self.score = [0] * num_experts
        self.from_prefetch = [False] * num_experts
        self.n = 0
        self.forwards = self.hits = self.misses = self.evictions = self.bytes_h2d = self.waves = 0
        self.prefetched = self.prefetch_hits = self.host_experts = 0
        if profile is not None:
            self._set_profile(profile)
            self._rebalance(count=False)

    def resident(self) -> dict:
        return {e: s for s, e in enumerate(self.slot_expert) if e >= 0}

    def _rank(self, e):
        if self.policy == LRU:
            return (self.last_use[e],)
        return (self.score[e], self.last_use[e])

    def _key(self, e):
        return self._rank(e) + (e,)

    def _set_profile(self, profile):
        prof = [int(v) for v in profile]
        if len(prof) != self.E or any(not 0 <= v <= MAX_SCORE for v in prof):
            raise ValueError("profile must hold E scores in [0, 2**62]")
        self.score = prof

    def _page(self, e, slot, count):
        old = self.slot_expert[slot]
        if old >= 0:
            self.from_prefetch[old] = False
        self.slot_expert[slot] = e
        if count:
            if old >= 0:
                self.evictions += 1
            self.prefetched += 1
            self.bytes_h2d += self.expert_bytes
            self.from_prefetch[e] = True

    def _rebalance(self, count):
        ranked = sorted(range(self.E), key=lambda e: (-self.score[e], e))
        wanted = set(ranked[:self.B])
        res = self.resident()
        freed = sorted(s for e, s in res.items() if e not in wanted)
        freed += [s for s, e in enumerate(self.slot_expert) if e < 0]
        freed.sort()
        newcomers = sorted(e for e in wanted if e not in res)
        for e, slot in zip(newcomers, freed):
            self._page(e, slot, count)

    def load_profile(self, profile):
        """Run-time profile load: set the scores, then rebalance the slots."""
        self._set_profile(profile)
        self._rebalance(count=True)

    def profile(self):
        return list(self.score)

    def forward(self, needed):
        """Apply one forward with needed expert set `needed`; return the plan:
        a list of waves, each a list of (expert, slot, paged) tuples."""
        return self.forward_split(needed)[0]

    def forward_split(self, needed, rows=None, host_rows=0):
        """A forward whose non-resident experts with at most `host_rows` tokens
        (rows[e]) run on the host (hybrid prefill; host_rows 0: none).  Returns
        (plan of the others, host experts ascending)."""
        N = sorted(set(int(e) for e in needed))
        if not N:
            return [], []
        self.n += 1
        self.forwards += 1
        res = self.resident()
        host = [e for e in N if e not in res and host_rows > 0 and rows[e] <= host_rows]
        run = [e for e in N if e not in host]
        hits = [e for e in run if e in res]
        misses = sorted((e for e in run if e not in res), key=self._key)
        for e in hits:
            if self.from_prefetch[e]:
                self.prefetch_hits += 1
                self.from_prefetch[e] = False
        order = hits + misses
        pinned, W, prev_too = set(), self.B, False
        if len(order) > self.B:
            pinned = set(sorted(hits, key=self._key, reverse=True)[:self.B // 4])
            S = self.B - len(pinned)
            W = S // 2 if S >= 2 else 1
            prev_too = S >= 2
        plan = []
        prev = set()
        for w0 in range(0, len(order), W):
            wave = order[w0:w0 + W]
            in_wave = set(wave)
            keep = in_wave | pinned | (prev if prev_too else set())
            prev = in_wave
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
                    cands = [x for x in res if x not in keep]
                    victim = min(cands, key=self._key)
                    slot = res[victim]
                    self.from_prefetch[victim] = False
                    self.evictions += 1
                self.slot_expert[slot] = e
                entries.append((e, slot, True))
            plan.append(entries)
        if self.policy == WARM:
            for e in range(self.E):
                self.score[e] -= self.score[e] >> self.d
        for e in N:
            self.last_use[e] = self.n
            self.score[e] += UNIT
        self.hits += len(hits)
        self.misses += len(misses)
        self.bytes_h2d += len(misses) * self.expert_bytes
        self.waves += max(1, len(plan))
        self.host_experts += len(host)
        if self.P:
            self._prefetch()
        return plan, host

    def forward_hybrid(self, needed):
        """A hybrid forward: returns (hits as (expert, slot) pairs, host-computed experts)."""
        N = sorted(set(int(e) for e in needed))
        if not N:
            return [], []
        self.n += 1
        self.forwards += 1
        res = self.resident()
        hits = [(e, res[e]) for e in N if e in res]
        host = [e for e in N if e not in res]
        for e, _ in hits:
            if self.from_prefetch[e]:
                self.prefetch_hits += 1
                self.from_prefetch[e] = False
        if self.policy == WARM:
            for e in range(self.E):
                self.score[e] -= self.score[e] >> self.d
        for e in N:
            self.last_use[e] = self.n
            self.score[e] += UNIT
        self.hits += len(hits)
        self.host_experts += len(host)
        self.waves += 1
        if self.P:
            self._prefetch()
        return hits, host

    def _prefetch(self):
        res = self.resident()
        outside = sorted((e for e in range(self.E) if e not in res),
                         key=lambda e: tuple(-r for r in self._rank(e)) + (e,))
        inside = sorted(res, key=self._key)
        for c, v in list(zip(outside, inside))[:self.P]:
            if self._rank(c) <= self._rank(v):
                break
            self._page(c, res[v], count=True)

    def stats(self) -> dict:
        resident = sum(1 for e in self.slot_expert if e >= 0)
        return dict(forwards=self.forwards, hits=self.hits, misses=self.misses,
                    evictions=self.evictions, bytes_h2d=self.bytes_h2d, waves=self.waves,
                    budget=self.B, resident=resident, resident_bytes=resident * self.expert_bytes,
                    prefetched=self.prefetched, prefetch_hits=self.prefetch_hits,
                    host_experts=self.host_experts)
