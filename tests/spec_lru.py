"""An independent, list-based model of the slot-cache admission, used only
to brute-force the C oracle on tiny caches.

It is written from the same statement of the method (FreeToken PR #680,
section Solution; FreeToken PR #491, sections 4-5) but in a different
form: the cache is an explicit recency list of slots (least recently used
first), instead of per-slot clock stamps sorted on demand.  Slots used in
the same step are appended in ascending slot order, which is the tie rule
the oracle expresses as "(stamp, slot) ascending".

The look-ahead prefetch (llama.cpp fork PR #126, sections Consumer and
Eviction guard) is modelled the same way: candidates are read off the
recency list, skipping slots used since the latest demand step, and the
guard compares demand heat kept as per-expert counters and last-demand
ticks.
"""
from fractions import Fraction


class SpecCache:
    def __init__(self, L, E, S, one_call, query_width):
        self.L, self.E, self.S = L, E, S
        self.one_call, self.query_width = one_call, query_width
        self.recency = list(range(S))        # least recently used first
        self.holder = [None] * S             # (layer, expert) or None
        self.where = {}                      # (layer, expert) -> slot
        self.last_tick = [0] * S
        self.tick = 0
        self.calls = [0] * L
        self.met = [0] * L
        self.missed = [0] * L
        self.overflow = [0] * L
        self.invalid = [0] * L
        self.hist = [[0] * E for _ in range(L)]
        self.plan = []
        self.last_seen = {}                  # (layer, expert) -> tick of its last demand
        self.demand_tick = 0
        self.pf_calls = [0] * L
        self.pf_filled = [0] * L
        self.pf_dropped = [0] * L
        self.fills = []

    def step(self, layer, ids, max_fetch=-1):
        E = self.E
        self.tick += 1
        valid = [e for e in ids if 0 <= e < E]
        self.invalid[layer] += len(ids) - len(valid)
        for e in valid:
            self.hist[layer][e] += 1
            self.last_seen[(layer, e)] = self.tick
        self.demand_tick = self.tick

        if len(ids) <= self.one_call:
            queries = [sorted(set(valid))] if ids else []
        else:
            width = min(len(ids), E)
            padded = sorted(set(valid))
            padded += [None] * (width - len(padded))
            queries = []
            for a in range(0, width, self.query_width):
                chunk = [e for e in padded[a:a + self.query_width] if e is not None]
                queries.append(chunk)

        used = []           # slots used in this step, in order of use
        self.plan = []
        fetched = 0
        for q in queries:
            self.met[layer] += len(q)
            misses = []
            for e in q:
                if (layer, e) in self.where:
                    used.append(self.where[(layer, e)])
                else:
                    misses.append(e)
            self.missed[layer] += len(misses)
            free = [s for s in self.recency if s not in used]
            for j, e in enumerate(misses):
                capped = max_fetch >= 0 and fetched >= max_fetch
                if j >= len(free) or capped:
                    self.overflow[layer] += 1
                    continue
                s = free[j]
                if self.holder[s] is not None:
                    del self.where[self.holder[s]]
                self.holder[s] = (layer, e)
                self.where[(layer, e)] = s
                used.append(s)
                self.plan.append((s, e))
                fetched += 1
        self.calls[layer] += 1
        for s in used:
            self.last_tick[s] = self.tick
        self.recency = [s for s in self.recency if s not in used] + sorted(set(used))
        return [self.where.get((layer, e), -1) if 0 <= e < E else -1 for e in ids]

    def heat(self, key):
        """Demand frequency and a recency byte that is 255 right after a
        demand access and falls by one per tick, to 0 (0 if never)."""
        f = self.hist[key[0]][key[1]]
        if key not in self.last_seen:
            return f, 0
        return f, max(0, 255 - (self.tick - self.last_seen[key]))

    def warm_against(self, resident, predicted):
        f_r, r_r = self.heat(resident)
        f_p, r_p = self.heat(predicted)
        if f_r < 2:
            return False
        score_r = Fraction(f_r * 256 + r_r)
        score_p = Fraction(f_p * 256 + r_p)
        return score_r > score_p * Fraction(5, 4) + 4

    def prefetch(self, layer, ids):
        E = self.E
        self.fills = []
        if not ids:
            return
        self.tick += 1
        self.pf_calls[layer] += 1
        want = sorted({e for e in ids if 0 <= e < E})
        used = [self.where[(layer, e)] for e in want if (layer, e) in self.where]
        recent = {s for s in range(self.S)
                  if self.last_tick[s] != 0 and self.last_tick[s] >= self.demand_tick}
        candidates = [s for s in self.recency if s not in used and s not in recent]
        self.fills = []
        k = 0
        for e in want:
            if (layer, e) in self.where:
                continue
            if k == len(candidates):
                self.pf_dropped[layer] += 1
                continue
            s = candidates[k]
            if self.holder[s] is not None and self.warm_against(self.holder[s], (layer, e)):
                self.pf_dropped[layer] += 1
                continue
            if self.holder[s] is not None:
                del self.where[self.holder[s]]
            self.holder[s] = (layer, e)
            self.where[(layer, e)] = s
            used.append(s)
            self.fills.append((s, e))
            k += 1
        self.pf_filled[layer] += len(self.fills)
        for s in used:
            self.last_tick[s] = self.tick
        self.recency = [s for s in self.recency if s not in used] + sorted(set(used))

    # The same state in the oracle's array form.
    def arrays(self):
        import numpy as np

        res = np.full(self.L * self.E, -1, np.int32)
        own = np.full(self.S, -1, np.int32)
        for (l, e), s in self.where.items():
            res[l * self.E + e] = s
            own[s] = l * self.E + e
        stats = np.array(
            [[self.calls[l], self.met[l], self.missed[l], self.overflow[l], self.invalid[l],
              self.pf_calls[l], self.pf_filled[l], self.pf_dropped[l]]
             for l in range(self.L)], np.int64)
        freq = np.array([c for row in self.hist for c in row], np.int64)
        dlast = np.zeros(self.L * self.E, np.uint32)
        for (l, e), t in self.last_seen.items():
            dlast[l * self.E + e] = t
        return dict(res=res, own=own, stamp=np.array(self.last_tick, np.uint32),
                    clock=self.tick, stats=stats, freq=freq, dlast=dlast,
                    last_demand=self.demand_tick)
