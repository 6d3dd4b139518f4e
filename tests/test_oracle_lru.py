"""Oracle global LRU cache pinned to a brute-force recency-list simulator and LRU facts."""
import numpy as np
import pytest

import oracle
from lru_bruteforce import simulate


def run_oracle(L, E, C, steps):
    c = oracle.Cache(L, E, C)
    recs, slots = [], []
    for s, (layer, ids) in enumerate(steps):
        sl, r = c.step(s, layer, ids)
        recs += [tuple(int(v) for v in rr) for rr in r]
        slots.append(list(sl))
    return recs, slots, c


@pytest.mark.parametrize("seed", range(40))
def test_random_traces_match_bruteforce(seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(1, 4))
    E = int(rng.integers(2, 17))
    C = int(rng.integers(1, 9))
    steps = []
    for _ in range(int(rng.integers(1, 65))):
        n = int(rng.integers(1, min(C, E) + 1))
        ids = rng.choice(E, size=n, replace=False)
        if rng.random() < 0.3:  # duplicates inside a step (several tokens pick the same expert)
            ids = np.concatenate([ids, ids[: max(1, n // 2)]])
        steps.append((int(rng.integers(0, L)), ids.astype(np.int32)))
    recs, slots, c = run_oracle(L, E, C, steps)
    brecs, bslots, bcnt, recency, where = simulate(L, E, C, steps)
    assert recs == brecs
    assert slots == bslots
    assert c.counters() == bcnt
    slot_of, key_of, stamp = c.state()
    # bijection between resident keys and occupied slots; recency order = stamp order
    for key, v in where.items():
        assert slot_of[key] == v and key_of[v] == key
    assert (slot_of >= 0).sum() == len(where) == (key_of >= 0).sum()
    occ = [v for v in range(C) if key_of[v] >= 0]
    assert [key_of[v] for v in sorted(occ, key=lambda v: stamp[v])] == recency


def test_cyclic_scan_over_c_plus_1_keys_always_misses():
    C, E = 5, 6
    steps = [(0, [e % (C + 1)]) for e in range(40)]
    recs, _, c = run_oracle(1, E, C, steps)
    assert all(r[4] == 0 for r in recs)
    cnt = c.counters()
    assert cnt["misses"] == 40 and cnt["evictions"] == 40 - C


def test_working_set_within_capacity_only_compulsory_misses():
    rng = np.random.default_rng(7)
    C, L, E = 8, 2, 16
    keys = [(0, 1), (0, 5), (1, 2), (1, 3), (1, 9), (0, 11), (1, 15), (0, 0)]
    steps = []
    for _ in range(50):
        l, e = keys[int(rng.integers(0, len(keys)))]
        steps.append((l, [e]))
    _, _, c = run_oracle(L, E, C, steps)
    distinct = len(set((l, e[0]) for l, e in steps))
    assert c.counters()["misses"] == distinct and c.counters()["evictions"] == 0


def test_resident_set_is_most_recent_keys():
    rng = np.random.default_rng(9)
    C, L, E = 6, 2, 12
    c = oracle.Cache(L, E, C)
    history = []
    for s in range(60):
        l = int(rng.integers(0, L))
        e = int(rng.integers(0, E))
        c.step(s, l, [e])
        history.append(l * E + e)
        recent = []
        for key in reversed(history):
            if key not in recent:
                recent.append(key)
        slot_of, _, _ = c.state()
        resident = set(int(k) for k in np.nonzero(slot_of >= 0)[0])
        assert resident == set(recent[:C])


def test_evictions_equal_misses_minus_capacity():
    rng = np.random.default_rng(11)
    C, L, E = 4, 3, 10
    steps = [(int(rng.integers(0, L)), rng.choice(E, 2, replace=False)) for _ in range(100)]
    _, _, c = run_oracle(L, E, C, steps)
    cnt = c.counters()
    assert cnt["evictions"] == max(0, cnt["misses"] - C)


def test_step_never_evicts_its_own_hits():
    C, E = 4, 8
    c = oracle.Cache(1, E, C)
    c.step(0, 0, [0, 1])
    c.step(1, 0, [2, 3])        # cache full: 0,1 (old), 2,3 (new)
    _, r = c.step(2, 0, [0, 4, 5])  # 0 hit (restamped first); misses evict 1 and 2
    assert [(int(x["expert"]), int(x["hit"]), int(x["evicted_key"])) for x in r] == [(0, 1, -1), (4, 0, 1), (5, 0, 2)]


def test_capacity_error():
    c = oracle.Cache(1, 8, 2)
    with pytest.raises(ValueError):
        c.step(0, 0, [0, 1, 2])
