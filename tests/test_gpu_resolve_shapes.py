"""Decode parity at the resolve kernels' size limits: expert counts up to 1024, k = 16 and cache
sizes up to 16384 slots, so that every specialisation of the one-token resolve (logit candidates
per lane, order entries per lane) runs, with evictions where the pool exceeds the cache.

Bit-exact: ids, trace records and the final cache state.  Outputs (sampled vectors) within
relative L2 5e-3 and max|diff| 1e-2 * max|ref|."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import close_enough, make_moe, run_stack, trace_tuples

pytestmark = pytest.mark.gpu

# name, L, E, k, shared, H, I, C, decode tokens, requests, rho
SHAPES = [
    synth.Workload("e256_c3000", 24, 256, 8, 0, 64, 64, 3000, 96, 1, 0.8, seed=31),
    synth.Workload("e512_c4500", 24, 512, 10, 1, 96, 64, 4500, 96, 1, 0.6, seed=32),
    synth.Workload("e1024_k16_c16384", 3, 1024, 16, 0, 64, 64, 16384, 24, 1, 0.85, seed=33),
    synth.Workload("e1024_k16_c1200", 4, 1024, 16, 1, 128, 96, 1200, 64, 1, 0.7, seed=34),
]


@pytest.mark.parametrize("wl", SHAPES, ids=[w.name for w in SHAPES])
def test_one_token_resolve_at_size_limits(wl):
    X = synth.decode_inputs(wl)
    m, W = make_moe(wl)
    ids, w, y = run_stack(m, wl, X)
    cnt, recs = m.stats(trace_cap=1 << 22)
    ref = oracle.decode_trace(wl, W, X)
    np.testing.assert_array_equal(ids, ref["ids"])
    assert np.max(np.abs(w - ref["w"])) <= 1e-5
    assert trace_tuples(recs) == trace_tuples(ref["trace"])
    slot_of, key_of, stamp = m.cache_state()
    r_slot, r_key, r_stamp = ref["cache"].state()
    np.testing.assert_array_equal(slot_of, r_slot)
    np.testing.assert_array_equal(key_of, r_key)
    np.testing.assert_array_equal(stamp, r_stamp)
    c = ref["counters"]
    assert (cnt["hits"], cnt["misses"], cnt["evictions"]) == (c["hits"], c["misses"], c["evictions"])
    T = X.shape[0]
    for t in sorted({0, 1, T // 2, T - 1}):
        for l in range(wl.n_layers):
            r = oracle.moe_output(wl, l, X[t, 0], ref["ids"][t, l, 0], ref["w"][t, l, 0])
            rel, mx, ok = close_enough(y[t, l, 0], r)
            assert ok, (t, l, rel, mx)
    print(wl.name, "hits", cnt["hits"], "misses", cnt["misses"], "evictions", cnt["evictions"])
    m.close()
