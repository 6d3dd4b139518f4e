"""The oracle's run over steps with different token counts (a prefill chunk, then decode)."""
import dataclasses

import numpy as np

import oracle
import synth


def test_run_trace_equals_decode_trace_for_a_fixed_batch():
    wl = dataclasses.replace(synth.WORKLOADS["toy"], n_requests=3, decode_tokens=10, cache_slots=12)
    X = synth.decode_inputs(wl)
    W = synth.router_weights(wl)
    a = oracle.decode_trace(wl, W, X)
    b = oracle.run_trace(wl, W, [X[t] for t in range(X.shape[0])])
    for t in range(X.shape[0]):
        np.testing.assert_array_equal(b["ids"][t], a["ids"][t])
        np.testing.assert_array_equal(b["w"][t], a["w"][t])
        np.testing.assert_array_equal(b["slots"][t], a["slots"][t])
    assert b["trace"].tobytes() == a["trace"].tobytes()
    assert b["counters"] == a["counters"]


def test_prefill_step_requests_each_expert_once():
    """A prefill chunk is one step per layer: every distinct expert of the chunk is one access,
    so a cold cache records exactly one miss per distinct (layer, expert) and no hit."""
    wl = dataclasses.replace(synth.WORKLOADS["toy"], cache_slots=32)
    W = synth.router_weights(wl)
    P = synth.hidden_stream(wl.seed, synth.PREFILL_REQUEST_ID, 50, wl.hidden, wl.rho)
    r = oracle.run_trace(wl, W, [P])
    for l in range(wl.n_layers):
        distinct = np.unique(r["ids"][0][l])
        recs = r["trace"][r["trace"]["layer"] == l]
        assert list(recs["expert"]) == list(distinct)
        assert (recs["hit"] == 0).all()
    assert r["counters"]["hits"] == 0
