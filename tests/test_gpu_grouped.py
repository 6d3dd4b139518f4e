"""GPU parity of the grouped (B > 1) path: prefill chunks and multi-request decode steps.

The grouped matrix-core kernels run whenever a call has more than one token.  Every case runs a
prefill chunk (one step with many tokens) followed by lock-step decode steps, through
moe_stack_forward, and compares with the CPU oracle:
- bit-exact: expert ids, cache trace, final cache state;
- routing weights |diff| <= 1e-5;
- outputs per (step, layer, token): relative L2 <= 5e-3 and max|diff| <= 1e-2 * max|ref|.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import close_enough, make_moe, run_steps, trace_tuples

pytestmark = pytest.mark.gpu


def _steps(wl, prefill, B, T):
    steps = []
    if prefill:
        steps.append(synth.hidden_stream(wl.seed, synth.PREFILL_REQUEST_ID, prefill, wl.hidden, wl.rho))
    streams = [synth.hidden_stream(wl.seed, r, T, wl.hidden, wl.rho) for r in range(B)]
    for t in range(T):
        steps.append(np.stack([s[t] for s in streams]))
    return steps


def _check(wl, steps, ids, w, y, m, recs, token_sample=None):
    ref = oracle.run_trace(wl, synth.router_weights(wl), steps)
    for t in range(len(steps)):
        np.testing.assert_array_equal(ids[t], ref["ids"][t])
        assert np.max(np.abs(w[t] - ref["w"][t])) <= 1e-5
    assert trace_tuples(recs) == trace_tuples(ref["trace"])
    slot_of, key_of, stamp = m.cache_state()
    r_slot, r_key, r_stamp = ref["cache"].state()
    np.testing.assert_array_equal(slot_of, r_slot)
    np.testing.assert_array_equal(key_of, r_key)
    np.testing.assert_array_equal(stamp, r_stamp)
    worst = 0.0
    for t, x in enumerate(steps):
        toks = range(len(x)) if token_sample is None else token_sample(t, len(x))
        for l in range(wl.n_layers):
            for b in toks:
                r = oracle.moe_output(wl, l, x[b], ref["ids"][t][l, b], ref["w"][t][l, b])
                rel, mx, ok = close_enough(y[t][l, b], r)
                worst = max(worst, rel)
                assert ok, (t, l, b, rel, mx)
    return ref, worst


# prefill lengths chosen to give groups above and below one 64-row chunk and ragged tails
GROUPED = [
    (synth.Workload("toy_grouped", 2, 16, 2, 0, 256, 512, 40, 6, 4, 0.9, prefill_tokens=100, seed=21)),
    (synth.Workload("shared_k8_grouped", 2, 32, 8, 1, 2048, 512, 80, 4, 3, 0.9, prefill_tokens=70, seed=22)),
    (synth.Workload("odd_grouped", 2, 24, 3, 1, 800, 96, 60, 3, 5, 0.85, prefill_tokens=37, seed=23)),
    (synth.Workload("ragged_2880_grouped", 2, 8, 2, 0, 2880, 2880, 16, 3, 2, 0.9, prefill_tokens=20, seed=24)),
]


@pytest.mark.parametrize("wl", GROUPED, ids=[w.name for w in GROUPED])
def test_grouped_prefill_then_decode(wl):
    steps = _steps(wl, wl.prefill_tokens, wl.n_requests, wl.decode_tokens)
    m, _ = make_moe(wl, max_tokens=max(wl.prefill_tokens, wl.n_requests))
    ids, w, y = run_steps(m, wl, steps)
    _, recs = m.stats(trace_cap=1 << 20)
    _, worst = _check(wl, steps, ids, w, y, m, recs)
    print(wl.name, "worst rel-L2", worst)
    m.close()


def test_grouped_e512_k10_shared_prefill_and_b16_decode():
    """The 512-expert, top-10 + shared shape: a 130-token prefill chunk then B = 16 decode steps
    (sampled prefill tokens: both sides of a 64-row chunk boundary, and the last)."""
    wl = synth.Workload("e512_grouped", 2, 512, 10, 1, 3072, 768, 1024, 3, 16, 0.9,
                        prefill_tokens=130, seed=25)
    steps = _steps(wl, wl.prefill_tokens, wl.n_requests, wl.decode_tokens)
    m, _ = make_moe(wl, max_tokens=wl.prefill_tokens)
    ids, w, y = run_steps(m, wl, steps)
    _, recs = m.stats(trace_cap=1 << 20)

    def sample(t, B):
        return [0, 1, 63, 64, 65, 127, 128, 129] if t == 0 else [0, 5, 15]

    _, worst = _check(wl, steps, ids, w, y, m, recs, token_sample=sample)
    print("e512_grouped worst rel-L2", worst)
    m.close()


def test_per_token_path_for_batches_matches_oracle():
    """MOE_FLAG_PER_TOKEN_FFN: the per-token GEMV kernels on a B > 1 step, same bar."""
    import moe_expert_offload_amd as M
    wl = GROUPED[1]
    steps = _steps(wl, 0, wl.n_requests, wl.decode_tokens)
    m, _ = make_moe(wl, max_tokens=wl.n_requests, flags=M.MOE_FLAG_PER_TOKEN_FFN)
    ids, w, y = run_steps(m, wl, steps)
    _, recs = m.stats(trace_cap=1 << 20)
    _check(wl, steps, ids, w, y, m, recs)
    m.close()


def test_grouped_identical_tokens_give_identical_outputs():
    """Every token of the batch is the same vector: one group holds all B rows of each expert;
    the outputs are bitwise equal across tokens and match the oracle."""
    wl = dataclasses.replace(GROUPED[1], name="dup", n_requests=24, decode_tokens=2, prefill_tokens=0)
    x = synth.hidden_stream(wl.seed, 0, 2, wl.hidden, wl.rho)
    steps = [np.repeat(x[t][None], 24, axis=0) for t in range(2)]
    m, _ = make_moe(wl, max_tokens=24)
    ids, w, y = run_steps(m, wl, steps)
    _, recs = m.stats(trace_cap=1 << 20)
    for t in range(2):
        for b in range(1, 24):
            np.testing.assert_array_equal(y[t][:, b].view(np.uint32), y[t][:, 0].view(np.uint32))
    _check(wl, steps, ids, w, y, m, recs, token_sample=lambda t, B: [0, B - 1])
    m.close()


def test_grouped_lookahead_and_causal_are_bitwise_equal():
    wl = GROUPED[2]
    steps = _steps(wl, wl.prefill_tokens, wl.n_requests, wl.decode_tokens)
    m1, _ = make_moe(wl, lookahead=1, max_tokens=wl.prefill_tokens)
    _, _, y1 = run_steps(m1, wl, steps)
    m1.close()
    m0, _ = make_moe(wl, lookahead=0, max_tokens=wl.prefill_tokens)
    _, _, y0 = run_steps(m0, wl, steps)
    m0.close()
    for a, b in zip(y0, y1):
        np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


def test_grouped_expert_forward_rejects_bad_slots_with_nan():
    """A slot outside [0, C) in moe_expert_forward's input: no work runs and every output of the
    call is NaN (the kernels never touch memory for it)."""
    import torch
    wl = GROUPED[0]
    m, _ = make_moe(wl, max_tokens=4)
    dev = m.device
    x = torch.zeros((4, wl.hidden), dtype=torch.int16, device=dev)
    slots = torch.tensor([[0, 1], [2, 3], [4, wl.cache_slots + 7], [5, 6]], dtype=torch.int32, device=dev)
    wts = torch.full((4, 2), 0.5, dtype=torch.float32, device=dev)
    y = torch.zeros((4, wl.hidden), dtype=torch.int16, device=dev)
    with torch.cuda.stream(m.compute_stream):
        m.expert_forward(0, x, slots, wts, y)
    m.compute_stream.synchronize()
    yf = y.view(torch.bfloat16).float().cpu().numpy()
    assert np.isnan(yf).all()
    m.close()


def test_grouped_prefill_with_pageable_pool_part():
    """A prefill chunk whose misses mostly come from the pageable part of the pool (pinned part
    capped at 2 MiB), then decode steps; same bar."""
    wl = GROUPED[1]
    steps = _steps(wl, wl.prefill_tokens, wl.n_requests, wl.decode_tokens)
    m, _ = make_moe(wl, max_tokens=wl.prefill_tokens, pinned_mb=2)
    ids, w, y = run_steps(m, wl, steps)
    cnt, recs = m.stats(trace_cap=1 << 20)
    assert cnt["h2d_bounced"] > 0
    _check(wl, steps, ids, w, y, m, recs)
    m.close()


@pytest.mark.parametrize("case", ["decode_b1", "prefill_then_b4"])
def test_static_split_policy_matches_oracle(case):
    """MOE_POLICY_STATIC: keys below R = C - T resident from init, every other access streamed
    into T transient slots in rotation.  ids, trace (hit/miss, slot, evicted key), the resident
    table and outputs against the oracle's static split."""
    import moe_expert_offload_amd as M
    if case == "decode_b1":
        wl = synth.Workload("static_b1", 3, 16, 2, 0, 256, 512, 20, 24, 1, 0.9, seed=31)
        steps = _steps(wl, 0, 1, wl.decode_tokens)
        max_tokens = 1
    else:
        wl = GROUPED[0]
        steps = _steps(wl, wl.prefill_tokens, wl.n_requests, wl.decode_tokens)
        max_tokens = wl.prefill_tokens
    T = 2 * min(max_tokens * wl.top_k, wl.n_experts)
    m, _ = make_moe(wl, max_tokens=max_tokens, policy=M.MOE_POLICY_STATIC)
    ids, w, y = run_steps(m, wl, steps)
    cnt, recs = m.stats(trace_cap=1 << 20)
    ref = oracle.run_trace(wl, synth.router_weights(wl), steps, static_transient=T)
    for t in range(len(steps)):
        np.testing.assert_array_equal(ids[t], ref["ids"][t])
    assert trace_tuples(recs) == trace_tuples(ref["trace"])
    rc = ref["counters"]
    assert (cnt["hits"], cnt["misses"], cnt["evictions"]) == (rc["hits"], rc["misses"], rc["evictions"])
    slot_of, key_of, _ = m.cache_state()
    r_slot, r_key = ref["cache"].state()
    np.testing.assert_array_equal(slot_of, r_slot)
    np.testing.assert_array_equal(key_of, r_key)
    for t, x in enumerate(steps):
        for l in range(wl.n_layers):
            for b in range(len(x)):
                r = oracle.moe_output(wl, l, x[b], ref["ids"][t][l, b], ref["w"][t][l, b])
                rel, mx, ok = close_enough(y[t][l, b], r)
                assert ok, (t, l, b, rel, mx)
    assert cnt["misses"] > 0 and cnt["hits"] > 0
    m.close()


def test_grouped_wide_4096_shape():
    """H = 4096, I = 2048, top-6 (the DeepSeek-shaped expert) through the grouped path."""
    wl = synth.Workload("wide_4096_grouped", 2, 16, 6, 0, 4096, 2048, 40, 2, 3, 0.85,
                        prefill_tokens=40, seed=26)
    steps = _steps(wl, wl.prefill_tokens, wl.n_requests, wl.decode_tokens)
    m, _ = make_moe(wl, max_tokens=wl.prefill_tokens)
    ids, w, y = run_steps(m, wl, steps)
    _, recs = m.stats(trace_cap=1 << 20)
    _, worst = _check(wl, steps, ids, w, y, m, recs, token_sample=lambda t, B: [0, B // 2, B - 1])
    print("wide_4096_grouped worst rel-L2", worst)
    m.close()


def test_layer_forward_on_a_batch_matches_the_stack():
    """moe_layer_forward (causal, one layer per call) and moe_stack_forward (lookahead 1) give
    bitwise equal outputs for a batch step: the same kernels in the same order per layer."""
    import torch
    wl = GROUPED[0]
    steps = _steps(wl, 0, wl.n_requests, 3)
    m, _ = make_moe(wl, max_tokens=wl.n_requests)
    _, _, ys = run_steps(m, wl, steps)
    m.close()
    m, _ = make_moe(wl, lookahead=0, max_tokens=wl.n_requests)
    dev = m.device
    for t, x in enumerate(steps):
        xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev)
        y = torch.empty((wl.n_layers, len(x), wl.hidden), dtype=torch.int16, device=dev)
        with torch.cuda.stream(m.compute_stream):
            for l in range(wl.n_layers):
                m.layer_forward(t, l, xd, y[l])
        m.compute_stream.synchronize()
        from gpu_helpers import bf16_to_f32
        np.testing.assert_array_equal(bf16_to_f32(y).view(np.uint32), ys[t].view(np.uint32))
    m.close()


def test_cache_resolve_then_grouped_expert_forward():
    """The boundary's two halves on a batch: moe_cache_resolve with oracle ids, then
    moe_expert_forward on the returned slots, against the oracle's layer output."""
    import torch
    wl = GROUPED[1]
    x = synth.decode_inputs(dataclasses.replace(wl, decode_tokens=1))[0]     # [B][H]
    W = synth.router_weights(wl)
    ref = oracle.run_trace(wl, W, [x])
    m, _ = make_moe(wl, max_tokens=wl.n_requests)
    dev = m.device
    l = 1
    ids = torch.from_numpy(ref["ids"][0][l].astype(np.int32)).to(dev)
    wts = torch.from_numpy(ref["w"][0][l].astype(np.float32)).to(dev)
    slots = torch.empty_like(ids)
    xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev)
    y = torch.empty((len(x), wl.hidden), dtype=torch.int16, device=dev)
    with torch.cuda.stream(m.compute_stream):
        nm = m.cache_resolve(0, l, ids, slots)
        m.expert_forward(l, xd, slots, wts, y)
    m.compute_stream.synchronize()
    assert nm == len(np.unique(ref["ids"][0][l]))     # cold cache: every distinct expert misses
    from gpu_helpers import bf16_to_f32
    yf = bf16_to_f32(y)
    for b in range(len(x)):
        r = oracle.moe_output(wl, l, x[b], ref["ids"][0][l, b], ref["w"][0][l, b])
        rel, mx, ok = close_enough(yf[b], r)
        assert ok, (b, rel, mx)
    m.close()
