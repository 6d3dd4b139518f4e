"""Pins of the oracle's static per-layer split (the comparator of the router-following cache)."""
import numpy as np
import pytest

import oracle
import synth

GOLDEN = "tests/golden/page_worked_numbers.txt"


def _golden(kind):
    out = []
    for line in open(GOLDEN):
        f = line.split()
        if f and f[0] == kind:
            out.append(tuple(float(v) for v in f[1:]))
    return out


def test_resident_keys_never_miss_and_others_always_do():
    L, E, C, T = 4, 16, 40, 6      # R = 34: layers 0, 1 whole, 2 of layer 2
    c = oracle.StaticCache(L, E, C, T)
    rng = np.random.default_rng(1)
    for s in range(50):
        l = int(rng.integers(0, L))
        ids = rng.choice(E, 3, replace=False).astype(np.int32)
        slots, recs = c.step(s, l, ids)
        for r in recs:
            key = l * E + r["expert"]
            assert r["hit"] == (1 if key < C - T else 0)
            if r["hit"]:
                assert r["slot"] == key
            else:
                assert C - T <= r["slot"] < C
        # hits first, then misses, each ascending by expert
        h = [r["expert"] for r in recs if r["hit"]]
        m = [r["expert"] for r in recs if not r["hit"]]
        assert h == sorted(h) and m == sorted(m) and list(recs["hit"]) == [1] * len(h) + [0] * len(m)


def test_transient_slots_rotate_and_evict_the_miss_t_before():
    L, E, C, T = 3, 8, 12, 4       # R = 8: layer 0 resident
    c = oracle.StaticCache(L, E, C, T)
    rng = np.random.default_rng(2)
    miss_keys, miss_slots, miss_old = [], [], []
    for s in range(40):
        l = 1 + int(rng.integers(0, 2))
        ids = rng.choice(E, 2, replace=False).astype(np.int32)
        _, recs = c.step(s, l, ids)
        for r in recs:
            if not r["hit"]:
                miss_keys.append(l * E + r["expert"])
                miss_slots.append(r["slot"])
                miss_old.append(r["evicted_key"])
    n = len(miss_keys)
    assert miss_slots == [C - T + (i % T) for i in range(n)]
    assert miss_old == [-1 if i < T else miss_keys[i - T] for i in range(n)]
    cnt = c.counters()
    assert cnt["misses"] == n and cnt["evictions"] == max(0, n - T)
    slot_of, key_of = c.state()
    assert all(slot_of[k] == k for k in range(C - T)) and (slot_of[C - T:] == -1).all()
    for i in range(max(0, n - T), n):   # the last T misses are still in their slots
        assert key_of[miss_slots[i]] == miss_keys[i]


def test_miss_rate_under_uniform_routing_is_the_non_resident_fraction():
    """Uniform routing reaches every key of a layer alike, so the expected miss rate is the
    non-resident fraction of the pool, 1 - (C - T) / (L * E)."""
    L, E, k, C, T = 12, 64, 4, 300, 8
    c = oracle.StaticCache(L, E, C, T)
    rng = np.random.default_rng(3)
    steps = 4000
    for s in range(steps):
        for l in range(L):
            c.step(s, l, rng.choice(E, k, replace=False).astype(np.int32))
    cnt = c.counters()
    rate = cnt["misses"] / (cnt["hits"] + cnt["misses"])
    expect = 1 - (C - T) / (L * E)
    assert abs(rate - expect) < 0.01, (rate, expect)


@pytest.mark.parametrize("name,frac_idx", [("qwen36_35b_a3b_shaped", 0), ("dsv4_flash_shaped", 1)])
def test_static_split_closed_form_matches_the_pages(name, frac_idx):
    """At the cache fractions the pages quote (37 % and 11 % of the pool) the static split's
    expected miss rate 1 - (C - T)/pool is within 2 points of the pages' 62 % and 89 %."""
    wl = synth.WORKLOADS[name]
    frac, page_rate = _golden("static_split")[frac_idx]
    assert abs(wl.cache_slots / wl.pool - frac / 100) < 0.005
    T = 2 * wl.top_k
    rate = 1 - (wl.cache_slots - T) / wl.pool
    assert abs(100 * rate - page_rate) < 2.0, (rate, page_rate)
