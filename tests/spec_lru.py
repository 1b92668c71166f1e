"""An independent, list-based model of the slot-cache admission, used only
to brute-force the C oracle on tiny caches.

It is written from the same statement of the method (FreeToken PR #680,
section Solution; FreeToken PR #491, sections 4-5) but in a different
form: the cache is an explicit recency list of slots (least recently used
first), instead of per-slot clock stamps sorted on demand.  Slots used in
the same step are appended in ascending slot order, which is the tie rule
the oracle expresses as "(stamp, slot) ascending".
"""


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

    def step(self, layer, ids, max_fetch=-1):
        E = self.E
        self.tick += 1
        valid = [e for e in ids if 0 <= e < E]
        self.invalid[layer] += len(ids) - len(valid)
        for e in valid:
            self.hist[layer][e] += 1

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

    # The same state in the oracle's array form.
    def arrays(self):
        import numpy as np

        res = np.full(self.L * self.E, -1, np.int32)
        own = np.full(self.S, -1, np.int32)
        for (l, e), s in self.where.items():
            res[l * self.E + e] = s
            own[s] = l * self.E + e
        stats = np.array(
            [[self.calls[l], self.met[l], self.missed[l], self.overflow[l], self.invalid[l]]
             for l in range(self.L)], np.int64)
        freq = np.array([c for row in self.hist for c in row], np.int64)
        return dict(res=res, own=own, stamp=np.array(self.last_tick, np.uint32),
                    clock=self.tick, stats=stats, freq=freq)
