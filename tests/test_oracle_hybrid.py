"""Oracle hybrid cache step (only the transferred share of the misses enters the cache) pinned to
the brute-force recency-list simulator, to the plain LRU step where the host has no bandwidth to
spare, and to the split rule written out from the pages (q = m B_P / B_H, nearest integer)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from lru_bruteforce import simulate


def q_rule(pcie, host):
    """Misses transferred out of m: m if the host is no faster than PCIe, else the integer
    nearest m * B_P / B_H (halves up), evaluated exactly with fractions."""
    def q(m):
        if m <= 0:
            return 0
        if host <= pcie:
            return m
        x = Fraction(m) * Fraction(pcie) / Fraction(host)
        return int(x + Fraction(1, 2))  # floor(x + 1/2), x >= 0
    return q


def run(L, E, C, steps, split):
    c = oracle.Cache(L, E, C)
    recs, slots = [], []
    for s, (layer, ids) in enumerate(steps):
        sl, r = c.step(s, layer, ids, split)
        recs += [tuple(int(v) for v in rr) for rr in r]
        slots.append(list(sl))
    return recs, slots, c


def random_steps(rng, L, E, C, n):
    steps = []
    for _ in range(n):
        m = int(rng.integers(1, min(C, E) + 1))
        steps.append((int(rng.integers(0, L)), rng.choice(E, size=m, replace=False).astype(np.int32)))
    return steps


@pytest.mark.parametrize("seed", range(30))
def test_split_steps_match_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    L, E, C = int(rng.integers(1, 4)), int(rng.integers(4, 17)), int(rng.integers(2, 9))
    # B_P, B_H on a quarter-GB/s grid so that the exact rule and the double-precision one agree
    pcie = float(rng.integers(20, 240)) / 4
    host = pcie * float(rng.choice([0.5, 1.0, 1.5, 2.0, 3.25, 5.0, 40.0]))
    steps = random_steps(rng, L, E, C, int(rng.integers(1, 65)))
    recs, slots, c = run(L, E, C, steps, (pcie, host))
    brecs, bslots, bcnt, recency, where = simulate(L, E, C, steps, q_rule(pcie, host))
    assert recs == brecs
    assert slots == bslots
    assert c.counters() == bcnt
    slot_of, key_of, _ = c.state()
    for key, v in where.items():
        assert slot_of[key] == v and key_of[v] == key
    assert int((slot_of >= 0).sum()) == len(where)


def test_no_spare_host_bandwidth_is_the_plain_lru():
    rng = np.random.default_rng(7)
    steps = random_steps(rng, 3, 16, 8, 200)
    for pcie, host in ((50.0, 50.0), (56.0, 27.0)):
        r1, s1, c1 = run(3, 16, 8, steps, (pcie, host))
        r0, s0, c0 = run(3, 16, 8, steps, None)
        assert r1 == r0 and s1 == s0
        assert c1.counters() == c0.counters() and c1.counters()["host"] == 0
        for a, b in zip(c1.state(), c0.state()):
            np.testing.assert_array_equal(a, b)


def test_host_share_leaves_the_cache_untouched():
    # a host 40x faster than PCIe: q = round(m / 40) = 0 for m <= 19, every miss runs on the host
    c = oracle.Cache(2, 16, 8)
    before = [a.copy() for a in c.state()]
    slots, recs = c.step(0, 1, np.array([3, 5, 9], np.int32), (10.0, 400.0))
    assert list(slots) == [-1, -1, -1]
    assert [(int(r["slot"]), int(r["hit"]), int(r["evicted_key"])) for r in recs] == [(-1, 0, -1)] * 3
    for a, b in zip(c.state(), before):
        np.testing.assert_array_equal(a, b)
    assert c.counters() == {"hits": 0, "misses": 3, "evictions": 0, "host": 3}


def test_pages_calibration_split_of_ten_misses():
    # B_H = 45.5, B_P = 26.7 (the florigen.ai page's calibration): 10 misses -> 6 transferred, 4 host
    c = oracle.Cache(1, 32, 16)
    slots, recs = c.step(0, 0, np.arange(10, dtype=np.int32), (26.7, 45.5))
    assert list(slots[:6]) == list(range(6)) and list(slots[6:]) == [-1] * 4
    assert c.counters()["host"] == 4
