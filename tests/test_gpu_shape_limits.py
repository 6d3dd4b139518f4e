"""Parity at the accepted shape limits (H and I up to 16384) and rejection of token counts outside
[1, max_tokens].  Bit-exact ids, traces and cache state; outputs within relative L2 5e-3 and
max|diff| 1e-2 * max|ref|."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import close_enough, make_moe, run_stack, run_steps, trace_tuples

pytestmark = pytest.mark.gpu

# name, L, E, k, shared, H, I, C, decode tokens, requests, rho
WIDE_H = synth.Workload("h16384", 3, 8, 2, 1, 16384, 64, 16, 6, 1, 0.8, prefill_tokens=40, seed=61)
WIDE_I = synth.Workload("i16384", 2, 4, 1, 0, 64, 16384, 4, 6, 1, 0.8, seed=62)


def test_hidden_16384_prefill_and_decode():
    wl = WIDE_H
    P = synth.prefill_inputs(wl)
    X = synth.decode_inputs(wl)
    steps = [P] + [X[t] for t in range(X.shape[0])]
    m, W = make_moe(wl, max_tokens=wl.prefill_tokens)
    ids, w, y = run_steps(m, wl, steps)
    cnt, recs = m.stats(trace_cap=1 << 16)
    ref = oracle.run_trace(wl, W, steps)
    for t in range(len(steps)):
        np.testing.assert_array_equal(ids[t], ref["ids"][t])
    assert trace_tuples(recs) == trace_tuples(ref["trace"])
    for t, toks in ((0, [0, 1, 17, 39]), (1, [0]), (len(steps) - 1, [0])):
        for l in range(wl.n_layers):
            for b in toks:
                r = oracle.moe_output(wl, l, steps[t][b], ref["ids"][t][l, b], ref["w"][t][l, b])
                rel, mx, ok = close_enough(y[t][l, b], r)
                assert ok, (t, l, b, rel, mx)
    m.close()


def test_inter_16384_decode():
    wl = WIDE_I
    X = synth.decode_inputs(wl)
    m, W = make_moe(wl)
    ids, w, y = run_stack(m, wl, X)
    cnt, recs = m.stats(trace_cap=1 << 16)
    ref = oracle.decode_trace(wl, W, X)
    np.testing.assert_array_equal(ids, ref["ids"])
    assert trace_tuples(recs) == trace_tuples(ref["trace"])
    for t in range(X.shape[0]):
        for l in range(wl.n_layers):
            r = oracle.moe_output(wl, l, X[t, 0], ref["ids"][t, l, 0], ref["w"][t, l, 0])
            rel, mx, ok = close_enough(y[t, l, 0], r)
            assert ok, (t, l, rel, mx)
    m.close()


def test_token_counts_outside_the_configured_range_are_rejected():
    import torch

    import moe_expert_offload_amd as M
    wl = synth.WORKLOADS["toy"]
    m, _ = make_moe(wl, max_tokens=4, cache_slots=16)  # 2 * min(4 * k, E) slots
    lib = M.lib()
    x = torch.zeros((8, wl.hidden), dtype=torch.int16, device=m.device)
    y = torch.empty((wl.n_layers, 8, wl.hidden), dtype=torch.int16, device=m.device)
    for n in (0, 5, -1):
        with pytest.raises(M.MoeError) as ei:
            m._check(lib.moe_layer_forward(m.ctx, 0, 0, M._ptr(x), n, M._ptr(y), None, None), "layer_forward")
        assert ei.value.status == -1
        with pytest.raises(M.MoeError) as ei:
            m._check(lib.moe_stack_forward(m.ctx, 0, M._ptr(x), 0, n, M._ptr(y), 8 * wl.hidden, None, None),
                     "stack_forward")
        assert ei.value.status == -1
    # the context stays usable after the rejected calls
    run_stack(m, wl, synth.decode_inputs(wl)[:2])
    m.close()
