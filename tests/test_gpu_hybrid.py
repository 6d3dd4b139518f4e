"""Hybrid backend on the device: a decode step (one token, or a batch of at most 16 lock-step
requests) transfers q = m B_P / B_H of its m misses and the host workers compute the rest, for
every token that selected them.  Against the oracle: ids, cache trace (host misses carry slot -1),
final cache state and counters bit-exact with the oracle's hybrid steps; outputs within relative
L2 5e-3 and max|diff| 1e-2 * max|ref| of the plain MoE output (placement does not change it)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import close_enough, make_moe, run_stack, trace_tuples

pytestmark = pytest.mark.gpu

TOY = synth.WORKLOADS["toy"]
SHARED = synth.Workload("hyb_shared_k8", 3, 32, 8, 1, 2048, 512, 20, 12, 1, 0.8, seed=51)
WIDE = synth.Workload("hyb_2880", 3, 16, 4, 0, 2880, 2880, 10, 10, 1, 0.7, seed=52)
# batches of lock-step requests (the grouped FFN path); capacity C >= 2 min(B k, E)
BATCH4 = synth.Workload("hyb_b4", 3, 32, 4, 1, 512, 256, 40, 10, 4, 0.8, seed=53)
BATCH16 = synth.Workload("hyb_b16_k8", 3, 64, 8, 0, 1024, 512, 130, 8, 16, 0.8, seed=54)
BATCH8W = synth.Workload("hyb_b8_2880", 2, 16, 4, 1, 2880, 2880, 32, 6, 8, 0.7, seed=55)

# (B_P, B_H): every miss on the host (q = round(m / 40) = 0 for m < 20), the pages' calibration
# (q = 0.59 m), a ratio measured on an MI355X host with 16 EPYC cores (q = 0.19 m), and no spare
# host bandwidth (offload)
SPLITS = [(10.0, 400.0), (26.7, 45.5), (56.0, 290.0), (50.0, 50.0)]


def _hybrid(wl, split, threads=4, **kw):
    m, W = make_moe(wl, **kw)
    m.set_backend("hybrid", split[0], split[1], threads)
    return m, W


def _check(wl, X, W, m, ids, w, y, split):
    cnt, recs = m.stats(trace_cap=1 << 20)
    ref = oracle.decode_trace(wl, W, X, split=split)
    np.testing.assert_array_equal(ids, ref["ids"])
    assert np.max(np.abs(w - ref["w"])) <= 1e-5
    assert trace_tuples(recs) == trace_tuples(ref["trace"])
    slot_of, key_of, stamp = m.cache_state()
    r_slot, r_key, r_stamp = ref["cache"].state()
    np.testing.assert_array_equal(slot_of, r_slot)
    np.testing.assert_array_equal(key_of, r_key)
    np.testing.assert_array_equal(stamp, r_stamp)
    c = ref["counters"]
    assert (cnt["hits"], cnt["misses"], cnt["evictions"], cnt["host_experts"]) == \
        (c["hits"], c["misses"], c["evictions"], c["host"])
    assert cnt["h2d_copies"] == c["misses"] - c["host"]
    worst = 0.0
    T, B = X.shape[:2]
    for t in range(T):
        for l in range(wl.n_layers):
            for b in range(B):
                r = oracle.moe_output(wl, l, X[t, b], ref["ids"][t, l, b], ref["w"][t, l, b])
                rel, mx, ok = close_enough(y[t, l, b], r)
                worst = max(worst, rel)
                assert ok, (t, l, b, rel, mx)
    return c, worst


@pytest.mark.parametrize("split", SPLITS, ids=[f"{a}_{b}" for a, b in SPLITS])
@pytest.mark.parametrize("wl", [TOY, SHARED, WIDE], ids=lambda w: w.name)
def test_hybrid_decode_matches_oracle(wl, split):
    X = synth.decode_inputs(wl)[:24]
    m, W = _hybrid(wl, split)
    ids, w, y = run_stack(m, wl, X)
    c, worst = _check(wl, X, W, m, ids, w, y, split)
    print(wl.name, split, c, "worst rel-L2 %.2e" % worst)
    if split[1] > split[0]:
        assert c["host"] > 0
    m.close()


@pytest.mark.parametrize("split", SPLITS[:3], ids=[f"{a}_{b}" for a, b in SPLITS[:3]])
@pytest.mark.parametrize("wl", [BATCH4, BATCH16, BATCH8W], ids=lambda w: w.name)
def test_hybrid_batch_decode_matches_oracle(wl, split):
    X = synth.decode_inputs(wl)
    m, W = _hybrid(wl, split)
    ids, w, y = run_stack(m, wl, X)
    c, worst = _check(wl, X, W, m, ids, w, y, split)
    print(wl.name, split, c, "worst rel-L2 %.2e" % worst)
    assert c["host"] > 0
    cnt, _ = m.stats()
    assert cnt["host_tasks"] > 0
    m.close()


def test_hybrid_batch_is_bitwise_independent_of_workers_and_lookahead():
    wl = BATCH8W
    X = synth.decode_inputs(wl)[:4]
    outs = []
    for threads, la in ((1, 1), (9, 1), (4, 0)):
        m, _ = _hybrid(wl, (26.7, 45.5), threads=threads, lookahead=la)
        outs.append(run_stack(m, wl, X)[2])
        m.close()
    for o in outs[1:]:
        np.testing.assert_array_equal(o.view(np.uint32), outs[0].view(np.uint32))


def test_hybrid_batches_beyond_16_tokens_and_per_token_ffn_run_offload_steps():
    import moe_expert_offload_amd as M
    big = synth.Workload("hyb_b20", 2, 32, 4, 0, 512, 256, 64, 4, 20, 0.8, seed=56)
    for wl, flags in ((big, 0), (BATCH4, M.MOE_FLAG_PER_TOKEN_FFN)):
        X = synth.decode_inputs(wl)
        m, W = _hybrid(wl, (10.0, 400.0), flags=flags)
        ids, w, y = run_stack(m, wl, X)
        c, _ = _check(wl, X, W, m, ids, w, y, None)
        assert c["host"] == 0
        m.close()


def test_hybrid_is_bitwise_independent_of_workers_and_lookahead():
    wl = WIDE
    X = synth.decode_inputs(wl)[:12]
    outs = []
    for threads, la in ((1, 1), (7, 1), (4, 0)):
        m, _ = _hybrid(wl, (26.7, 45.5), threads=threads, lookahead=la)
        outs.append(run_stack(m, wl, X)[2])
        m.close()
    for o in outs[1:]:
        np.testing.assert_array_equal(o.view(np.uint32), outs[0].view(np.uint32))


# caches of at least 8 k B slots: stack calls run seven layers ahead, the host tasks queued
WIDE_DEEP = synth.Workload("hyb_2880_deep", 6, 16, 4, 0, 2880, 2880, 32, 10, 1, 0.7, seed=57)
SHARED_DEEP = synth.Workload("hyb_shared_deep", 6, 32, 8, 1, 2048, 512, 64, 12, 1, 0.8, seed=58)
BATCH4_DEEP = synth.Workload("hyb_b4_deep", 6, 32, 4, 1, 512, 256, 128, 10, 4, 0.8, seed=59)


@pytest.mark.parametrize("split", SPLITS[:3], ids=[f"{a}_{b}" for a, b in SPLITS[:3]])
@pytest.mark.parametrize("wl", [WIDE_DEEP, SHARED_DEEP, BATCH4_DEEP], ids=lambda w: w.name)
def test_hybrid_with_queued_host_tasks_matches_oracle(wl, split):
    """Lookahead 7: the host tasks of up to seven layer steps are queued ahead of their FFNs, and
    the compute stream waits for each layer's task.  Same bar as the other hybrid tests."""
    X = synth.decode_inputs(wl)
    m, W = _hybrid(wl, split)
    ids, w, y = run_stack(m, wl, X)
    c, worst = _check(wl, X, W, m, ids, w, y, split)
    print(wl.name, split, c, "worst rel-L2 %.2e" % worst)
    assert c["host"] > 0
    m.close()


@pytest.mark.parametrize("wl", [WIDE_DEEP, BATCH4_DEEP], ids=lambda w: w.name)
def test_queued_host_tasks_are_bitwise_equal_to_lookahead_1_and_0(wl):
    X = synth.decode_inputs(wl)
    outs = []
    for threads, la in ((4, 7), (9, 7), (4, 3), (1, 1), (4, 0)):
        m, _ = _hybrid(wl, (26.7, 45.5), threads=threads, lookahead=la)
        ids, w, y = run_stack(m, wl, X)
        outs.append((ids, y, m.cache_state()))
        m.close()
    for ids, y, st in outs[1:]:
        np.testing.assert_array_equal(ids, outs[0][0])
        np.testing.assert_array_equal(y.view(np.uint32), outs[0][1].view(np.uint32))
        for u, v in zip(st, outs[0][2]):
            np.testing.assert_array_equal(u, v)


@pytest.mark.parametrize("wl", [SHARED, BATCH4], ids=lambda w: w.name)
def test_hybrid_layer_forward_matches_stack_and_pageable_pool(wl):
    import torch
    X = synth.decode_inputs(wl)[:8]
    B = X.shape[1]
    m, W = _hybrid(wl, (10.0, 400.0), pinned_mb=1)   # most of the pool pageable
    _, _, ys = run_stack(m, wl, X)
    m.close()
    m, W = _hybrid(wl, (10.0, 400.0), lookahead=0, pinned_mb=1)
    dev = m.device
    H = wl.hidden
    xd = torch.from_numpy(X.view(np.int16)).to(dev)
    y = torch.empty((X.shape[0], wl.n_layers, B, H), dtype=torch.int16, device=dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(m.compute_stream):
        for t in range(X.shape[0]):
            for l in range(wl.n_layers):
                m.layer_forward(t, l, xd[t], y[t, l])
    m.compute_stream.synchronize()
    yl = y.view(torch.bfloat16).float().cpu().numpy()
    np.testing.assert_array_equal(yl.view(np.uint32), ys.view(np.uint32))
    cnt, _ = m.stats()
    assert cnt["host_experts"] > 0 and cnt["host_tasks"] > 0
    m.close()


@pytest.mark.parametrize("wl", [SHARED, BATCH4], ids=lambda w: w.name)
def test_hybrid_stack_with_its_own_input_per_layer(wl):
    """moe_stack_forward with a different hidden state per layer (layer stride B*H): every
    layer's host share reads its own layer's inputs.  Equal bit for bit to moe_layer_forward
    calls in the same order, and within tolerance of the plain MoE output."""
    import torch
    T, L = 5, wl.n_layers
    X = synth.decode_inputs(wl)[:T]
    B, H = X.shape[1], wl.hidden
    # layer l of step t sees step (t + 3 l) mod T's states: distinct per layer, same shapes
    XL = np.stack([np.stack([X[(t + 3 * l) % T] for l in range(L)]) for t in range(T)])  # [T][L][B][H]
    split = (26.7, 45.5)
    outs, traces = [], []
    for by_layer in (False, True):
        m, W = _hybrid(wl, split)
        dev = m.device
        xd = torch.from_numpy(np.ascontiguousarray(XL).view(np.int16)).to(dev)
        y = torch.empty((T, L, B, H), dtype=torch.int16, device=dev)
        torch.cuda.synchronize()
        with torch.cuda.stream(m.compute_stream):
            for t in range(T):
                if by_layer:
                    for l in range(L):
                        m.layer_forward(t, l, xd[t, l], y[t, l])
                else:
                    m.stack_forward(t, xd[t], B * H, B, y[t], B * H)
        m.compute_stream.synchronize()
        outs.append(y.view(torch.bfloat16).float().cpu().numpy())
        cnt, recs = m.stats(trace_cap=1 << 16)
        traces.append(trace_tuples(recs))
        assert cnt["host_experts"] > 0
        m.close()
    np.testing.assert_array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    assert traces[0] == traces[1]
    for (t, l, b) in [(0, 0, 0), (T - 1, L - 1, B - 1), (2, L // 2, 0)]:
        ids, w = oracle.route_batch(W, XL[t, l, b:b + 1], wl.top_k, np.array([l]), np.array([0]))
        r = oracle.moe_output(wl, l, XL[t, l, b], ids[0], w[0])
        rel, mx, ok = close_enough(outs[0][t, l, b], r)
        assert ok, (t, l, b, rel, mx)


def test_set_backend_rejects_bad_arguments_and_switches_back():
    import moe_expert_offload_amd as M
    m, W = make_moe(TOY)
    for args in (("hybrid", 0.0, 10.0, 2), ("hybrid", 10.0, -1.0, 2), ("hybrid", 10.0, 20.0, 0)):
        with pytest.raises(M.MoeError):
            m.set_backend(*args)
    X = synth.decode_inputs(TOY)[:6]
    m.set_backend("hybrid", 10.0, 400.0, 2)
    run_stack(m, TOY, X[:3])
    m.set_backend("offload")
    run_stack(m, TOY, X[3:], step0=3)
    cnt, recs = m.stats(trace_cap=1 << 16)
    # the steps after the switch transfer every miss
    late = [r for r in trace_tuples(recs) if r[0] >= 3 and r[4] == 0]
    assert late and all(r[3] >= 0 for r in late)
    m.close()
    ms, _ = make_moe(TOY, policy=1)
    with pytest.raises(M.MoeError):
        ms.set_backend("hybrid", 10.0, 20.0, 2)
    ms.close()
