"""Cache auto-sizing on the device: the slot count comes from the HBM left after the workspace
(the --moe-cache-auto option of the pages' server), and a context built that way decodes exactly
like the oracle with the same cache size."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import close_enough, make_moe, run_stack, trace_tuples

pytestmark = pytest.mark.gpu


def test_auto_cache_slots_follows_device_free_memory():
    import torch

    import moe_expert_offload_amd as M
    wl = synth.WORKLOADS["gptoss120b_shaped"]
    cfg = M.make_config(wl.n_layers, wl.n_experts, wl.top_k, wl.hidden, wl.inter, wl.n_shared, 0, 1)
    blob = M.query_sizes(cfg)[0]
    router = wl.n_layers * wl.n_experts * wl.hidden * 2
    torch.cuda.synchronize()
    free, total = torch.cuda.mem_get_info()
    budget = 30 * 10**9
    reserve = free - budget
    assert reserve > 0, (free, total)
    C_dev = M.auto_cache_slots(cfg, 0, reserve)          # the library asks the runtime
    C_host = M.auto_cache_slots(cfg, free, reserve)      # the same free bytes, given
    print("free", free, "auto slots", C_dev, C_host)
    assert abs(C_dev - C_host) <= 1                     # free memory may move by a page meanwhile
    assert C_host * blob + router <= budget
    assert (C_host + 1) * blob + router + (8 << 20) > budget
    # the whole 60.9 GB pool fits in what is free on an idle MI355X
    assert M.auto_cache_slots(cfg, 0, 4 << 30) == wl.n_layers * wl.n_experts


def test_auto_sized_context_decodes_like_the_oracle():
    wl = synth.WORKLOADS["toy"]
    X = synth.decode_inputs(wl)[:24]
    m, W = make_moe(wl, cache_slots=0)
    C = m.cfg.cache_slots
    assert C == wl.n_layers * wl.n_experts  # a 6.7 MB pool fits whole
    ids, w, y = run_stack(m, wl, X)
    cnt, recs = m.stats(trace_cap=1 << 20)
    wl_c = dataclasses.replace(wl, cache_slots=C)
    ref = oracle.decode_trace(wl_c, W, X)
    np.testing.assert_array_equal(ids, ref["ids"])
    assert np.max(np.abs(w - ref["w"])) <= 1e-5
    assert trace_tuples(recs) == trace_tuples(ref["trace"])
    # a cache as large as the pool only takes compulsory misses and never evicts
    assert cnt["evictions"] == 0
    assert cnt["misses"] == len({(r[1], r[2]) for r in trace_tuples(recs)})
    for t in range(X.shape[0]):
        for l in range(wl.n_layers):
            r = oracle.moe_output(wl, l, X[t, 0], ref["ids"][t, l, 0], ref["w"][t, l, 0])
            assert close_enough(y[t, l, 0], r)[2], (t, l)
    m.close()
