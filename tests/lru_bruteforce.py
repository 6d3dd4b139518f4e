"""Brute-force LRU simulator for tiny traces: an explicit recency list (least recent first)
and a free-slot set, independent of the oracle's stamp-based implementation."""


def simulate(L, E, C, steps, transferred=None):
    """steps: list of (layer, ids).  Returns (records, slots per step, counters).
    transferred(m) -> q: a hybrid step, in which only the first q of the m misses (ascending
    expert id) enter the cache; the others take no slot (slot -1) and change nothing."""
    recency = []          # keys, least recently used first
    where = {}            # key -> slot
    free = list(range(C))
    recs, slots_all = [], []
    hits = misses = evictions = host = 0
    for s, (layer, ids) in enumerate(steps):
        R = sorted(set(int(e) for e in ids))
        if len(R) > C:
            raise ValueError("capacity")
        hit_e = [e for e in R if layer * E + e in where]
        miss_e = [e for e in R if layer * E + e not in where]
        for e in hit_e:
            key = layer * E + e
            recency.remove(key)
            recency.append(key)
            hits += 1
            recs.append((s, layer, e, where[key], 1, -1))
        q = len(miss_e) if transferred is None else transferred(len(miss_e))
        for i, e in enumerate(miss_e):
            key = layer * E + e
            if i >= q:
                misses += 1
                host += 1
                recs.append((s, layer, e, -1, 0, -1))
                continue
            if free:
                v = min(free)
                free.remove(v)
                old = -1
            else:
                old = recency.pop(0)
                v = where.pop(old)
                evictions += 1
            where[key] = v
            recency.append(key)
            misses += 1
            recs.append((s, layer, e, v, 0, old))
        slots_all.append([where.get(layer * E + int(e), -1) for e in ids])
    return (recs, slots_all, {"hits": hits, "misses": misses, "evictions": evictions, "host": host}, recency,
            where)
