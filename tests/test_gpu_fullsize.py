"""Full-size parity on every workload shape: gpt-oss-120b (36 x 128 experts, H = I = 2880, top-4,
1862 of 4608 experts cached, the full 60.9 GB pool in pinned host RAM), Qwen3.6-35B-A3B,
DeepSeek-V4-Flash (a 147 GB pool, partly pageable) and Qwen3.8-Flash-Next (prefill and 16-request
decode), in the launch configuration the benchmark times (lookahead 7), with the offload and the
hybrid backends.  Routing ids and the cache trace are checked bit-exactly for every step run;
outputs at sampled (step, layer[, token]) points."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import close_enough, make_moe, run_stack, trace_tuples

pytestmark = pytest.mark.gpu


def test_gptoss_shaped_sampled():
    wl = synth.WORKLOADS["gptoss120b_shaped"]
    T = 48
    X = synth.decode_inputs(wl)[:T]
    m, W = make_moe(wl)
    ids, w, y = run_stack(m, wl, X)
    _, recs = m.stats(trace_cap=1 << 20)
    ref = oracle.decode_trace(wl, W, X)
    np.testing.assert_array_equal(ids, ref["ids"])
    assert np.max(np.abs(w - ref["w"])) <= 1e-5
    assert trace_tuples(recs) == trace_tuples(ref["trace"])
    for (t, l) in [(0, 0), (1, 35), (5, 17), (T // 2, 3), (T - 1, 0), (T - 1, 35)]:
        r = oracle.moe_output(wl, l, X[t, 0], ref["ids"][t, l, 0], ref["w"][t, l, 0])
        rel, mx, ok = close_enough(y[t, l, 0], r)
        print("t", t, "l", l, "rel-L2", rel)
        assert ok, (t, l, rel, mx)
    m.close()


def test_qwen38_shaped_prefill_and_b16_decode_sampled():
    """The 48 x 512-expert, top-10 + shared workload at full size (92.4 GB pool, 6144 slots): the
    2048-token prefill chunk (grouped MFMA path, every layer's experts missing on a cold cache),
    then 8 lock-step decode steps of 16 requests.  ids, weights and the whole trace are checked
    for every step; outputs at sampled (step, layer, token) points: prefill tokens on both
    sides of 64-row chunk boundaries and the last token, decode tokens 0, 7 and 15."""
    import gc
    from gpu_helpers import run_steps
    wl = synth.WORKLOADS["qwen38_flash_next_shaped"]
    T = 8
    X = synth.decode_inputs(wl)[:T]
    steps = [synth.prefill_inputs(wl)] + [X[t] for t in range(T)]
    m, W = make_moe(wl)
    ids, w, y = run_steps(m, wl, steps)
    _, recs = m.stats(trace_cap=1 << 20)
    m.close()
    del m
    gc.collect()
    ref = oracle.run_trace(wl, W, steps)
    for t in range(len(steps)):
        np.testing.assert_array_equal(ids[t], ref["ids"][t])
        assert np.max(np.abs(w[t] - ref["w"][t])) <= 1e-5
    assert trace_tuples(recs) == trace_tuples(ref["trace"])
    L = wl.n_layers
    points = [(0, 0, 0), (0, L - 1, 63), (0, 7, 64), (0, 30, 1000), (0, L - 1, 2047),
              (1, 0, 0), (1, L - 1, 15), (T, 20, 7), (T, L - 1, 0)]
    for (t, l, b) in points:
        r = oracle.moe_output(wl, l, steps[t][b], ref["ids"][t][l, b], ref["w"][t][l, b])
        rel, mx, ok = close_enough(y[t][l, b], r)
        print("t", t, "l", l, "b", b, "rel-L2", rel)
        assert ok, (t, l, b, rel, mx)


def test_gptoss_shaped_hybrid_sampled():
    """The same workload with the hybrid backend at a split like the one calibrated on these hosts
    (B_P 56 GB/s, B_H 290 GB/s: about one miss in five transferred) and 15 host workers: ids, the
    trace (host misses with slot -1) and the final cache state bit-exact with the oracle's hybrid
    steps; outputs at sampled points against the plain MoE output."""
    wl = synth.WORKLOADS["gptoss120b_shaped"]
    T = 32
    X = synth.decode_inputs(wl)[:T]
    m, W = make_moe(wl)
    split = (56.0, 290.0)
    m.set_backend("hybrid", split[0], split[1], 15)
    ids, w, y = run_stack(m, wl, X)
    cnt, recs = m.stats(trace_cap=1 << 20)
    ref = oracle.decode_trace(wl, W, X, split=split)
    np.testing.assert_array_equal(ids, ref["ids"])
    assert np.max(np.abs(w - ref["w"])) <= 1e-5
    assert trace_tuples(recs) == trace_tuples(ref["trace"])
    slot_of, key_of, _ = m.cache_state()
    r_slot, r_key, _ = ref["cache"].state()
    np.testing.assert_array_equal(slot_of, r_slot)
    np.testing.assert_array_equal(key_of, r_key)
    assert cnt["host_experts"] == ref["counters"]["host"] > 0
    for (t, l) in [(0, 0), (2, 35), (9, 17), (T // 2, 3), (T - 1, 0), (T - 1, 35)]:
        r = oracle.moe_output(wl, l, X[t, 0], ref["ids"][t, l, 0], ref["w"][t, l, 0])
        rel, mx, ok = close_enough(y[t, l, 0], r)
        print("hybrid t", t, "l", l, "rel-L2", rel)
        assert ok, (t, l, rel, mx)
    m.close()


def test_qwen38_shaped_hybrid_prefill_and_b16_decode_sampled():
    """The 48 x 512-expert workload with the hybrid backend (B_P 56 GB/s, B_H 290 GB/s, 14 host
    workers): the 2048-token prefill chunk transfers all of its misses, the 16-request decode
    steps split theirs.  ids, weights, the whole trace (host misses with slot -1) and the final
    cache state bit-exact with the oracle; outputs at sampled (step, layer, token) points."""
    import gc
    from gpu_helpers import run_steps
    wl = synth.WORKLOADS["qwen38_flash_next_shaped"]
    T = 6
    X = synth.decode_inputs(wl)[:T]
    steps = [synth.prefill_inputs(wl)] + [X[t] for t in range(T)]
    split = (56.0, 290.0)
    m, W = make_moe(wl)
    m.set_backend("hybrid", split[0], split[1], 14)
    ids, w, y = run_steps(m, wl, steps)
    cnt, recs = m.stats(trace_cap=1 << 21)
    slot_of, key_of, _ = m.cache_state()
    m.close()
    del m
    gc.collect()
    ref = oracle.run_trace(wl, W, steps, split=split)
    for t in range(len(steps)):
        np.testing.assert_array_equal(ids[t], ref["ids"][t])
        assert np.max(np.abs(w[t] - ref["w"][t])) <= 1e-5
    assert trace_tuples(recs) == trace_tuples(ref["trace"])
    r_slot, r_key, _ = ref["cache"].state()
    np.testing.assert_array_equal(slot_of, r_slot)
    np.testing.assert_array_equal(key_of, r_key)
    assert cnt["host_experts"] == ref["counters"]["host"] > 0
    L = wl.n_layers
    for (t, l, b) in [(0, 5, 2047), (1, 0, 0), (1, L - 1, 15), (3, 20, 7), (T, L - 1, 0), (T, 11, 9)]:
        r = oracle.moe_output(wl, l, steps[t][b], ref["ids"][t][l, b], ref["w"][t][l, b])
        rel, mx, ok = close_enough(y[t][l, b], r)
        print("hybrid t", t, "l", l, "b", b, "rel-L2", rel)
        assert ok, (t, l, b, rel, mx)


@pytest.mark.parametrize("name,T,points", [
    ("qwen36_35b_a3b_shaped", 64, [(0, 0), (1, 39), (7, 20), (40, 3), (63, 0), (63, 39)]),
    ("dsv4_flash_shaped", 24, [(0, 0), (1, 42), (5, 21), (12, 3), (23, 0), (23, 42)]),
], ids=["qwen36_35b_a3b_shaped", "dsv4_flash_shaped"])
def test_other_shapes_sampled(name, T, points):
    """The Qwen3.6-shaped (40 x 256 experts, top-8 + shared, 17.1 GB pool, 3789 slots) and the
    DeepSeek-V4-Flash-shaped (43 x 256, top-6, H = 4096, I = 2048, 147 GB pool, 1211 slots; the
    pool's unpinned part goes through the bounce ring) workloads at full size, in the benchmark's
    launch configuration (batch 1, lookahead 7): ids, weights and the whole trace bit-exact for
    every step run, outputs at sampled (step, layer) points."""
    wl = synth.WORKLOADS[name]
    X = synth.decode_inputs(wl)[:T]
    m, W = make_moe(wl)
    ids, w, y = run_stack(m, wl, X)
    _, recs = m.stats(trace_cap=1 << 20)
    m.close()
    ref = oracle.decode_trace(wl, W, X)
    np.testing.assert_array_equal(ids, ref["ids"])
    assert np.max(np.abs(w - ref["w"])) <= 1e-5
    assert trace_tuples(recs) == trace_tuples(ref["trace"])
    assert ref["counters"]["evictions"] > 0
    for (t, l) in points:
        r = oracle.moe_output(wl, l, X[t, 0], ref["ids"][t, l, 0], ref["w"][t, l, 0])
        rel, mx, ok = close_enough(y[t, l, 0], r)
        print(name, "t", t, "l", l, "rel-L2", rel)
        assert ok, (t, l, rel, mx)


def test_dsv4_shaped_hybrid_sampled():
    """The DeepSeek-shaped workload with the hybrid backend (B_P 56 GB/s, B_H 240 GB/s, 10 host
    workers, as the benchmark runs it on a partly pageable pool): the route-stream schedule, the
    bounce ring and the host workers together.  ids, trace (host misses with slot -1) and final
    cache state bit-exact with the oracle's hybrid steps; outputs at sampled points."""
    wl = synth.WORKLOADS["dsv4_flash_shaped"]
    T = 40   # long enough for the transferred misses to fill the 1211 slots and start evicting
    X = synth.decode_inputs(wl)[:T]
    m, W = make_moe(wl)
    split = (56.0, 240.0)
    m.set_backend("hybrid", split[0], split[1], 10)
    ids, w, y = run_stack(m, wl, X)
    cnt, recs = m.stats(trace_cap=1 << 20)
    slot_of, key_of, _ = m.cache_state()
    m.close()
    ref = oracle.decode_trace(wl, W, X, split=split)
    np.testing.assert_array_equal(ids, ref["ids"])
    assert trace_tuples(recs) == trace_tuples(ref["trace"])
    r_slot, r_key, _ = ref["cache"].state()
    np.testing.assert_array_equal(slot_of, r_slot)
    np.testing.assert_array_equal(key_of, r_key)
    assert cnt["host_experts"] == ref["counters"]["host"] > 0 and ref["counters"]["evictions"] > 0
    for (t, l) in [(0, 0), (3, 42), (17, 17), (T - 1, 0), (T - 1, 42)]:
        r = oracle.moe_output(wl, l, X[t, 0], ref["ids"][t, l, 0], ref["w"][t, l, 0])
        rel, mx, ok = close_enough(y[t, l, 0], r)
        print("hybrid t", t, "l", l, "rel-L2", rel)
        assert ok, (t, l, rel, mx)


def test_gptoss_shaped_whole_pool_schedule_sampled():
    """C = L E = 4608 slots (the whole 60.9 GB pool cached, as auto sizing gives on this GPU): one-token
    stack calls then resolve on the route stream, launched by a helper host thread, and the host
    stages layer l+1's copies once layer l-1's FFN has ended.  48 tokens: ids, weights, the whole
    trace and the final cache state bit-exact with the oracle; outputs at sampled (step, layer)
    points."""
    import dataclasses
    wl = dataclasses.replace(synth.WORKLOADS["gptoss120b_shaped"], name="gptoss_whole_pool", cache_slots=36 * 128)
    T = 48
    X = synth.decode_inputs(wl)[:T]
    m, W = make_moe(wl)
    ids, w, y = run_stack(m, wl, X)
    _, recs = m.stats(trace_cap=1 << 20)
    state = m.cache_state()
    m.close()
    ref = oracle.decode_trace(wl, W, X)
    np.testing.assert_array_equal(ids, ref["ids"])
    assert np.max(np.abs(w - ref["w"])) <= 1e-5
    assert trace_tuples(recs) == trace_tuples(ref["trace"])
    for u, v in zip(state, ref["cache"].state()):
        np.testing.assert_array_equal(u, v)
    assert ref["counters"]["evictions"] == 0
    for (t, l) in [(0, 0), (1, 35), (9, 18), (T // 2, 2), (T - 1, 1), (T - 1, 35)]:
        r = oracle.moe_output(wl, l, X[t, 0], ref["ids"][t, l, 0], ref["w"][t, l, 0])
        rel, mx, ok = close_enough(y[t, l, 0], r)
        print("whole pool t", t, "l", l, "rel-L2", rel)
        assert ok, (t, l, rel, mx)
