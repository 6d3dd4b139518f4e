"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded inputs.

Bit-exact: expert ids, cache trace records, slots and final cache state.
Tolerance: routing weights |diff| <= 1e-5; layer outputs per (step, layer, token) vector
relative L2 <= 5e-3 and max|diff| <= 1e-2 * max|ref| (bf16 activations, FP32 accumulation).
"""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import close_enough, make_moe, run_stack, trace_tuples

pytestmark = pytest.mark.gpu


def _ref_outputs(wl, X, ref, points):
    out = {}
    for (t, l, b) in points:
        out[(t, l, b)] = oracle.moe_output(wl, l, X[t, b], ref["ids"][t, l, b], ref["w"][t, l, b])
    return out


def _check_run(wl, X, ids, w, y, recs, m, points, ref=None):
    ref = ref or oracle.decode_trace(wl, synth.router_weights(wl), X)
    np.testing.assert_array_equal(ids, ref["ids"])
    assert np.max(np.abs(w - ref["w"])) <= 1e-5
    assert trace_tuples(recs) == trace_tuples(ref["trace"])
    slot_of, key_of, stamp = m.cache_state()
    r_slot, r_key, r_stamp = ref["cache"].state()
    np.testing.assert_array_equal(slot_of, r_slot)
    np.testing.assert_array_equal(key_of, r_key)
    np.testing.assert_array_equal(stamp, r_stamp)
    worst = 0.0
    for (t, l, b), r in _ref_outputs(wl, X, ref, points).items():
        rel, mx, ok = close_enough(y[t, l, b], r)
        worst = max(worst, rel)
        assert ok, (t, l, b, rel, mx)
    return ref, worst


def test_toy_decode_all_outputs():
    wl = synth.WORKLOADS["toy"]
    X = synth.decode_inputs(wl)
    m, _ = make_moe(wl)
    ids, w, y = run_stack(m, wl, X)
    cnt, recs = m.stats(trace_cap=1 << 20)
    T = X.shape[0]
    points = [(t, l, 0) for t in range(T) for l in range(wl.n_layers)]
    ref, worst = _check_run(wl, X, ids, w, y, recs, m, points)
    c = ref["counters"]
    assert (cnt["hits"], cnt["misses"], cnt["evictions"]) == (c["hits"], c["misses"], c["evictions"])
    assert cnt["h2d_bytes"] == c["misses"] * wl.blob_bytes
    print("toy worst rel-L2", worst)
    m.close()


def test_lookahead_and_causal_are_bitwise_equal():
    wl = synth.WORKLOADS["toy"]
    X = synth.decode_inputs(wl)[:24]
    ys = []
    for la in (7, 3, 2, 1, 0):
        m, _ = make_moe(wl, lookahead=la)
        _, _, y = run_stack(m, wl, X)
        m.close()
        ys.append(y)
    for y in ys[1:]:
        np.testing.assert_array_equal(ys[0].view(np.uint32), y.view(np.uint32))


@pytest.mark.parametrize("D,B", [(2, 1), (2, 4), (3, 1), (3, 4), (5, 2), (7, 1), (7, 2)])
def test_deep_lookahead_stack_at_its_cache_bound_matches_causal_and_oracle(D, B):
    """Lookahead D (2 .. 7) enqueues the resolve of layer l+D before layer l's FFN, so layer
    l+D's copies can land while the FFNs of layers l .. l+D-1 are still pending; the library
    takes it when C >= (D + 1) k B, where a step's LRU victims are always older than the D steps
    before it.  max(8, 2 D) layers at exactly C = (D + 1) k B (evictions on most steps), B tokens
    per step: ids, weights, trace, final cache state and outputs equal the causal schedule's bit
    for bit and the oracle's (outputs within tolerance, every step and layer)."""
    k = 2
    L = max(8, 2 * D)
    wl = synth.Workload(f"la{D}_l{L}_b{B}", L, 16, k, 0, 256, 512, (D + 1) * k * B, 24, B, 0.9, seed=23)
    X = synth.decode_inputs(wl)
    runs = []
    for la in (D, 0):
        m, _ = make_moe(wl, lookahead=la)
        ids, w, y = run_stack(m, wl, X)
        _, recs = m.stats(trace_cap=1 << 16)
        if la == D:
            points = [(t, l, b) for t in range(X.shape[0]) for l in range(wl.n_layers) for b in range(B)]
            ref = oracle.decode_trace(wl, synth.router_weights(wl), X)
            assert ref["counters"]["evictions"] > X.shape[0] * wl.n_layers // 2
            _check_run(wl, X, ids, w, y, recs, m, points, ref=ref)
        runs.append((ids, w, y, trace_tuples(recs), m.cache_state()))
        m.close()
    np.testing.assert_array_equal(runs[0][0], runs[1][0])
    np.testing.assert_array_equal(runs[0][1].view(np.uint32), runs[1][1].view(np.uint32))
    np.testing.assert_array_equal(runs[0][2].view(np.uint32), runs[1][2].view(np.uint32))
    assert runs[0][3] == runs[1][3]
    for u, v in zip(runs[0][4], runs[1][4]):
        np.testing.assert_array_equal(u, v)


@pytest.mark.parametrize("la_cfg,fits", [(3, 2), (7, 4)])
def test_deep_lookahead_with_a_smaller_cache_runs_the_deepest_that_fits(la_cfg, fits):
    """Configured lookahead la_cfg but C = (fits + 1) k B: the call runs `fits` layers ahead (the
    deepest that fits) and still equals the causal schedule bit for bit."""
    k, B = 2, 2
    wl = synth.Workload(f"la{la_cfg}_c{fits + 1}kb", 10, 16, k, 0, 256, 512, (fits + 1) * k * B, 16, B, 0.9,
                        seed=29)
    X = synth.decode_inputs(wl)
    runs = []
    for la in (la_cfg, 0):
        m, _ = make_moe(wl, lookahead=la)
        ids, w, y = run_stack(m, wl, X)
        _, recs = m.stats(trace_cap=1 << 16)
        runs.append((ids, w, y, trace_tuples(recs)))
        m.close()
    np.testing.assert_array_equal(runs[0][0], runs[1][0])
    np.testing.assert_array_equal(runs[0][2].view(np.uint32), runs[1][2].view(np.uint32))
    assert runs[0][3] == runs[1][3]


def test_whole_pool_cache_route_stream_matches_causal_and_oracle():
    """With the whole pool in the cache (C = L E) one-token stack calls resolve on the route stream
    and the host gates the copies on the FFN two layers back.  Ids, trace and outputs equal the
    causal schedule's bit for bit and the oracle's within tolerance."""
    wl = dataclasses.replace(synth.WORKLOADS["toy"], name="toy_whole_pool", cache_slots=32, decode_tokens=24)
    assert wl.cache_slots == wl.n_layers * wl.n_experts
    X = synth.decode_inputs(wl)
    runs = []
    for la in (1, 0):
        m, _ = make_moe(wl, lookahead=la)
        ids, w, y = run_stack(m, wl, X)
        _, recs = m.stats(trace_cap=1 << 16)
        if la == 1:
            points = [(t, l, 0) for t in range(X.shape[0]) for l in range(wl.n_layers)]
            _check_run(wl, X, ids, w, y, recs, m, points)
        runs.append((ids, y, trace_tuples(recs)))
        m.close()
    np.testing.assert_array_equal(runs[0][0], runs[1][0])
    np.testing.assert_array_equal(runs[0][1].view(np.uint32), runs[1][1].view(np.uint32))
    assert runs[0][2] == runs[1][2]


def test_whole_pool_schedule_deep_stack_matches_causal_and_oracle():
    """The whole-pool one-token schedule with 8 layers: the helper thread's resolve of layer r
    waits until layer r-2's miss list, which it rewrites, has been staged, a gate that only blocks
    with more than two layers in flight.  Ids, trace, final cache state and outputs equal the causal
    schedule's bit for bit and the oracle's (outputs within tolerance) over every step."""
    wl = synth.Workload("whole_pool_l8", 8, 16, 2, 0, 256, 512, 8 * 16, 24, 1, 0.9, seed=21)
    X = synth.decode_inputs(wl)
    runs = []
    for la in (1, 0):
        m, _ = make_moe(wl, lookahead=la)
        ids, w, y = run_stack(m, wl, X)
        _, recs = m.stats(trace_cap=1 << 16)
        if la == 1:
            points = [(t, l, 0) for t in range(X.shape[0]) for l in range(wl.n_layers)]
            _check_run(wl, X, ids, w, y, recs, m, points)
        runs.append((ids, y, trace_tuples(recs), m.cache_state()))
        m.close()
    np.testing.assert_array_equal(runs[0][0], runs[1][0])
    np.testing.assert_array_equal(runs[0][1].view(np.uint32), runs[1][1].view(np.uint32))
    assert runs[0][2] == runs[1][2]
    for u, v in zip(runs[0][3], runs[1][3]):
        np.testing.assert_array_equal(u, v)


def test_layer_forward_matches_stack():
    import torch
    wl = synth.WORKLOADS["toy"]
    X = synth.decode_inputs(wl)[:8]
    m, _ = make_moe(wl, lookahead=1)
    _, _, ys = run_stack(m, wl, X)
    m.close()
    m, _ = make_moe(wl, lookahead=0)
    dev = m.device
    xd = torch.from_numpy(X.view(np.int16)).to(dev)
    y = torch.empty((X.shape[0], wl.n_layers, 1, wl.hidden), dtype=torch.int16, device=dev)
    with torch.cuda.stream(m.compute_stream):
        for t in range(X.shape[0]):
            for l in range(wl.n_layers):
                m.layer_forward(t, l, xd[t], y[t, l])
    m.compute_stream.synchronize()
    from gpu_helpers import bf16_to_f32
    np.testing.assert_array_equal(bf16_to_f32(y).view(np.uint32), ys.view(np.uint32))
    m.close()


# several tiles, ragged segment tails (H = 2880 -> 90 blocks over 16 segments) and a shared expert
SMALL = [
    synth.Workload("ragged_2880", 3, 8, 2, 0, 2880, 2880, 6, 12, 1, 0.9, seed=11),
    synth.Workload("shared_k8", 3, 32, 8, 1, 2048, 512, 20, 16, 1, 0.9, seed=12),
    synth.Workload("odd_blocks", 2, 24, 3, 1, 800, 96, 8, 16, 1, 0.85, seed=13),
    synth.Workload("wide_4096", 2, 16, 6, 0, 4096, 2048, 14, 10, 1, 0.85, seed=14),
    synth.Workload("e512_k10", 2, 512, 10, 1, 3072, 768, 24, 10, 1, 0.9, seed=15),
]


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_small_shapes_all_outputs(wl):
    X = synth.decode_inputs(wl)
    m, _ = make_moe(wl)
    ids, w, y = run_stack(m, wl, X)
    _, recs = m.stats(trace_cap=1 << 20)
    points = [(t, l, 0) for t in range(X.shape[0]) for l in range(wl.n_layers)]
    _, worst = _check_run(wl, X, ids, w, y, recs, m, points)
    print(wl.name, "worst rel-L2", worst)
    m.close()


def test_zero_input_edge_case():
    wl = synth.WORKLOADS["toy"]
    X = np.zeros((3, 1, wl.hidden), np.uint16)
    m, _ = make_moe(wl)
    ids, w, y = run_stack(m, wl, X)
    assert np.all(ids == np.arange(wl.top_k))
    np.testing.assert_allclose(w, 1.0 / wl.top_k, atol=1e-7)
    assert np.all(y == 0)
    m.close()


def test_every_expert_selected():
    """k = E: every step selects all experts of every layer (softmax over all of them, ids in
    rank order); with C = L E the whole pool fits, so after the first step every access hits."""
    wl = synth.Workload("k_eq_e", 3, 4, 4, 1, 256, 128, 12, 10, 1, 0.9, seed=71)
    X = synth.decode_inputs(wl)
    m, _ = make_moe(wl)
    ids, w, y = run_stack(m, wl, X)
    cnt, recs = m.stats(trace_cap=1 << 16)
    points = [(t, l, 0) for t in range(X.shape[0]) for l in range(wl.n_layers)]
    ref, _ = _check_run(wl, X, ids, w, y, recs, m, points)
    assert np.all(np.sort(ids, axis=-1) == np.arange(wl.top_k))
    assert cnt["misses"] == wl.n_layers * wl.n_experts and cnt["evictions"] == 0
    m.close()


def test_exact_logit_ties_take_the_lower_expert():
    """Router rows duplicated in pairs (expert 2i+1 = expert 2i) make every logit an exact tie
    with its partner at a non-zero input: both sides pick the lower index first, so ids, trace,
    weights and outputs match the oracle bit for bit / within tolerance."""
    import ctypes
    import moe_expert_offload_amd as M
    wl = dataclasses.replace(synth.WORKLOADS["toy"], name="toy_ties", decode_tokens=12)
    W = synth.router_weights(wl).copy()
    W[:, 1::2, :] = W[:, 0::2, :]
    X = synth.decode_inputs(wl)
    cfg = M.make_config(wl.n_layers, wl.n_experts, wl.top_k, wl.hidden, wl.inter, wl.n_shared, wl.cache_slots,
                        wl.max_tokens, 1, 1 << 16, 0, 0, 0, 0)
    fptr, FillArgs = synth.fill_callback()
    fa = FillArgs(wl.seed, wl.hidden, wl.inter)
    m = M.OffloadMoE(cfg, (fptr, ctypes.addressof(fa)), W)
    ids, w, y = run_stack(m, wl, X)
    _, recs = m.stats(trace_cap=1 << 16)
    ref = oracle.decode_trace(wl, W, X)
    points = [(t, l, 0) for t in range(X.shape[0]) for l in range(wl.n_layers)]
    _check_run(wl, X, ids, w, y, recs, m, points, ref=ref)
    # each top-2 pick is a tied pair (2i, 2i+1) in that order, with equal weights
    assert np.all(ids[..., 0] % 2 == 0) and np.all(ids[..., 1] == ids[..., 0] + 1)
    np.testing.assert_array_equal(w[..., 0], w[..., 1])
    m.close()


@pytest.mark.parametrize("seed", range(3))
def test_cache_resolve_random_batches(seed):
    """moe_cache_resolve with caller ids (several tokens, duplicates) against the oracle LRU."""
    import torch
    rng = np.random.default_rng(seed)
    wl = synth.Workload("resolve", 3, 16, 3, 0, 256, 64, 24, 1, 4, 0.9, seed=seed)
    m, _ = make_moe(wl, max_tokens=4)
    cache = oracle.Cache(wl.n_layers, wl.n_experts, wl.cache_slots)
    recs_ref = []
    for s in range(60):
        l = int(rng.integers(0, wl.n_layers))
        B = int(rng.integers(1, 5))
        ids = rng.integers(0, wl.n_experts, size=(B, wl.top_k)).astype(np.int32)
        idd = torch.from_numpy(ids).to(m.device)
        sl = torch.empty_like(idd)
        with torch.cuda.stream(m.compute_stream):
            nm = m.cache_resolve(s, l, idd, sl)
        m.compute_stream.synchronize()
        slots_ref, r = cache.step(s, l, ids)
        recs_ref.append(r)
        assert nm == int((r["hit"] == 0).sum())
        np.testing.assert_array_equal(sl.cpu().numpy().ravel(), slots_ref)
    _, recs = m.stats(trace_cap=1 << 16)
    assert trace_tuples(recs) == trace_tuples(np.concatenate(recs_ref))
    m.close()


def test_slot_bytes_equal_pool_blob_after_fill():
    """After misses land, the FFN of a slot equals the FFN of the pool blob: checked through
    outputs at a cache size that forces evictions every step (C = 2 * k)."""
    wl = dataclasses.replace(synth.WORKLOADS["toy"], cache_slots=4)
    X = synth.decode_inputs(wl)[:16]
    m, _ = make_moe(wl)
    ids, w, y = run_stack(m, wl, X)
    _, recs = m.stats(trace_cap=1 << 16)
    points = [(t, l, 0) for t in range(16) for l in range(wl.n_layers)]
    ref, _ = _check_run(wl, X, ids, w, y, recs, m, points)
    assert ref["counters"]["evictions"] > 0
    m.close()


def test_expert_forward_with_resolved_slots_matches_stack():
    """moe_expert_forward on slots from the cache state reproduces the stack's output bitwise."""
    import torch
    wl = synth.WORKLOADS["toy"]
    X = synth.decode_inputs(wl)[:6]
    m, _ = make_moe(wl)
    ids, w, y = run_stack(m, wl, X)
    slot_of, _, _ = m.cache_state()
    t = X.shape[0] - 1
    dev = m.device
    xd = torch.from_numpy(X[t].view(np.int16)).to(dev)
    for l in range(wl.n_layers):
        slots = torch.from_numpy(slot_of[l * wl.n_experts + ids[t, l]].astype(np.int32)).to(dev)
        wd = torch.from_numpy(w[t, l].astype(np.float32)).to(dev)
        yo = torch.empty((1, wl.hidden), dtype=torch.int16, device=dev)
        with torch.cuda.stream(m.compute_stream):
            m.expert_forward(l, xd, slots, wd, yo)
        m.compute_stream.synchronize()
        from gpu_helpers import bf16_to_f32
        np.testing.assert_array_equal(bf16_to_f32(yo)[0].view(np.uint32), y[t, l, 0].view(np.uint32))
    m.close()


def test_pageable_pool_part_through_bounce_ring():
    """pinned_mb caps the pinned part of the pool at 1 MiB (5 of 32 toy blobs); every other miss
    is copied through the pinned bounce ring.  Same bar as the fully pinned pool, at a cache
    size that forces evictions every step."""
    wl = dataclasses.replace(synth.WORKLOADS["toy"], cache_slots=4)
    X = synth.decode_inputs(wl)[:24]
    m, _ = make_moe(wl, pinned_mb=1)
    ids, w, y = run_stack(m, wl, X)
    cnt, recs = m.stats(trace_cap=1 << 16)
    assert cnt["pool_pinned_bytes"] == (1 << 20) // wl.blob_bytes * wl.blob_bytes
    assert cnt["h2d_bounced"] > 0 and cnt["h2d_bounced"] < cnt["h2d_copies"]
    points = [(t, l, 0) for t in range(24) for l in range(wl.n_layers)]
    _check_run(wl, X, ids, w, y, recs, m, points)
    m.close()


@pytest.mark.parametrize("B", [1, 2])
def test_deep_lookahead_with_a_pageable_pool_part_matches_causal_and_oracle(B):
    """A pool about half pageable with lookahead 7 (C = 16 k B): pinned misses on the second copy
    stream, pageable ones through the bounce ring on the first, seven layers of them queued.  Ids,
    weights, trace, cache state, copy counts and outputs equal the causal schedule's bit for bit
    and the oracle's (outputs within tolerance)."""
    k, L = 2, 12
    wl = synth.Workload(f"la7_pageable_b{B}", L, 16, k, 0, 256, 512, 16 * k * B, 24, B, 0.9, seed=41)
    X = synth.decode_inputs(wl)
    pinned_mb = (wl.pool * wl.blob_bytes // 2) >> 20
    runs = []
    for la in (7, 0):
        m, _ = make_moe(wl, lookahead=la, pinned_mb=pinned_mb)
        ids, w, y = run_stack(m, wl, X)
        cnt, recs = m.stats(trace_cap=1 << 16)
        assert 0 < cnt["h2d_bounced"] < cnt["h2d_copies"], cnt
        if la == 7:
            points = [(t, l, b) for t in range(X.shape[0]) for l in range(L) for b in range(B)]
            _check_run(wl, X, ids, w, y, recs, m, points)
        runs.append((ids, w, y, trace_tuples(recs), m.cache_state(), cnt["h2d_copies"], cnt["h2d_bounced"]))
        m.close()
    np.testing.assert_array_equal(runs[0][0], runs[1][0])
    np.testing.assert_array_equal(runs[0][1].view(np.uint32), runs[1][1].view(np.uint32))
    np.testing.assert_array_equal(runs[0][2].view(np.uint32), runs[1][2].view(np.uint32))
    assert runs[0][3] == runs[1][3]
    for u, v in zip(runs[0][4], runs[1][4]):
        np.testing.assert_array_equal(u, v)
    assert runs[0][5:] == runs[1][5:]


def test_profile_counters_and_h2d_measurement():
    """MOE_FLAG_PROFILE times every layer FFN with HIP events; moe_measure_h2d returns a plausible
    copy-path bandwidth (PCIe: between 1 and 70 GB/s)."""
    import moe_expert_offload_amd as M
    wl = synth.WORKLOADS["toy"]
    X = synth.decode_inputs(wl)[:5]
    m, _ = make_moe(wl, flags=M.MOE_FLAG_PROFILE)
    run_stack(m, wl, X)
    cnt, _ = m.stats()
    assert cnt["ffn_launches"] == 5 * wl.n_layers
    assert cnt["k3_ms"] > 0 and cnt["k4_ms"] > 0
    assert cnt["pool_pinned_bytes"] == wl.pool * wl.blob_bytes and cnt["h2d_bounced"] == 0
    g = m.measure_h2d(wl.blob_bytes, 16)
    assert 1.0 < g < 70.0, g
    m.close()


def test_out_of_range_ids_are_rejected_and_leave_no_trace():
    """Ids outside [0, E) given to moe_cache_resolve are counted by the resolve kernel (never used
    as an index) and the whole step is rejected with MOE_EINVAL before any state changes: slot
    table, reverse map, stamps, counters and trace stay as they were and every slot output is -1.
    The context keeps working: a run with rejected calls between its steps equals, in ids, trace,
    cache state and outputs, the oracle run that never saw them."""
    import torch
    import moe_expert_offload_amd as M
    from gpu_helpers import bf16_to_f32
    wl = dataclasses.replace(synth.WORKLOADS["toy"], name="toy_reject", decode_tokens=10)
    X = synth.decode_inputs(wl)  # [T][1][H]: one token per step through the stack
    W = synth.router_weights(wl)
    m, _ = make_moe(wl, max_tokens=2)
    dev = m.device
    xd = torch.from_numpy(np.ascontiguousarray(X).view(np.int16)).to(dev)
    T, L, H, k = X.shape[0], wl.n_layers, wl.hidden, wl.top_k
    y = torch.empty((T, L, 1, H), dtype=torch.int16, device=dev)
    ids = torch.empty((T, L, 1, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, L, 1, k), dtype=torch.float32, device=dev)
    # the oracle: the same stack steps plus the valid caller-id steps, none of the rejected ones
    ref_ids, ref_w = oracle.route_batch(W, X.reshape(T, H), k, np.tile(np.arange(L), T), np.repeat(np.arange(T), L))
    ref_ids, ref_w = ref_ids.reshape(T, L, 1, k), ref_w.reshape(T, L, 1, k)
    cache = oracle.Cache(L, wl.n_experts, wl.cache_slots)
    recs_ref = []
    valid = np.array([[3, 9], [9, 14]], np.int32)
    bad = {3: np.array([[0, wl.n_experts + 5], [1, 2]], np.int32), 7: np.array([[-1, 4], [7, 7]], np.int32)}

    def drain_and_check():
        _, recs = m.stats(trace_cap=1 << 12)
        want = np.concatenate(recs_ref) if recs_ref else np.empty(0, oracle.TRACE_DTYPE)
        assert trace_tuples(recs) == trace_tuples(want)
        recs_ref.clear()

    for t in range(T):
        if t in bad:
            drain_and_check()
            before = m.cache_state()
            c0, _ = m.stats()
            sl = torch.full((2, k), 123, dtype=torch.int32, device=dev)
            with pytest.raises(M.MoeError) as ei:
                with torch.cuda.stream(m.compute_stream):
                    m.cache_resolve(100 + t, t % L, torch.from_numpy(bad[t]).to(dev), sl)
            assert ei.value.status == M.MOE_EINVAL
            m.compute_stream.synchronize()
            assert np.all(sl.cpu().numpy() == -1)
            for u, v in zip(before, m.cache_state()):
                np.testing.assert_array_equal(u, v)
            c1, recs_mid = m.stats(trace_cap=1 << 10)
            assert len(recs_mid) == 0
            assert all(c0[f] == c1[f] for f in ("hits", "misses", "evictions", "resolves", "h2d_copies"))
            # then a valid caller-id step on the same context
            sl2 = torch.empty((2, k), dtype=torch.int32, device=dev)
            with torch.cuda.stream(m.compute_stream):
                nm = m.cache_resolve(200 + t, (t + 1) % L, torch.from_numpy(valid).to(dev), sl2)
            m.compute_stream.synchronize()
            slots_ref, r = cache.step(200 + t, (t + 1) % L, valid)
            recs_ref.append(r)
            assert nm == int((r["hit"] == 0).sum())
            np.testing.assert_array_equal(sl2.cpu().numpy().ravel(), slots_ref)
        with torch.cuda.stream(m.compute_stream):
            m.stack_forward(t, xd[t], 0, 1, y[t], H, ids[t], w[t])
        for l in range(L):
            _, r = cache.step(t, l, ref_ids[t, l])
            recs_ref.append(r)
    m.compute_stream.synchronize()
    drain_and_check()
    np.testing.assert_array_equal(ids.cpu().numpy(), ref_ids)
    assert np.max(np.abs(w.cpu().numpy() - ref_w)) <= 1e-5
    for u, v in zip(m.cache_state(), cache.state()):
        np.testing.assert_array_equal(u, v)
    yf = bf16_to_f32(y)
    for t in range(T):
        for l in range(L):
            r = oracle.moe_output(wl, l, X[t, 0], ref_ids[t, l, 0], ref_w[t, l, 0])
            rel, mx, ok = close_enough(yf[t, l, 0], r)
            assert ok, (t, l, rel, mx)
    m.close()
