"""Failure handling through the C ABI, every failure forced from the host (no kernel faults).

- An injected host-to-device copy failure (MOE_FAULT=h2d_fail_at=N: the stager reports the N-th
  miss copy as a failed HIP call instead of issuing it) fails the call with MOE_EHIP; from then on
  every call on the context returns MOE_ESTATE until moe_destroy, and a fresh context replays the
  run exactly (cold start, deterministic).
- Verify mode reads every filled slot back and compares it with its pool blob: clean runs pass and
  are bitwise equal to runs without it; a copy of the wrong blob (MOE_FAULT=h2d_corrupt_at=N) is
  caught with MOE_EVERIFY, which is sticky too.
- The copy-path and FFN timing counters are filled without the profile flag.

The pages record failures of this kind without a mechanism (pirouter.ai "FreeToken × RTX 5090——120B
MoE が 127 tok/s、その請求書", sections on the three measurements and the operating-cost line: a
backend that failed to load, and silent fallbacks).
"""
import contextlib
import dataclasses
import os

import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import close_enough, make_moe, run_stack, trace_tuples

pytestmark = pytest.mark.gpu


@contextlib.contextmanager
def env(name, value):
    old = os.environ.get(name)
    os.environ[name] = value
    try:
        yield
    finally:
        if old is None:
            del os.environ[name]
        else:
            os.environ[name] = old


def _every_call_is_estate(m, wl):
    import torch
    import moe_expert_offload_amd as M
    dev = m.device
    x = torch.zeros((1, wl.hidden), dtype=torch.int16, device=dev)
    y = torch.empty_like(x)
    ids = torch.zeros((1, wl.top_k), dtype=torch.int32, device=dev)
    w = torch.full((1, wl.top_k), 0.5, dtype=torch.float32, device=dev)
    ys = torch.empty((wl.n_layers, 1, wl.hidden), dtype=torch.int16, device=dev)
    calls = [
        lambda: m.stack_forward(0, x, 0, 1, ys, wl.hidden),
        lambda: m.layer_forward(0, 0, x, y),
        lambda: m.cache_resolve(0, 0, ids),
        lambda: m.expert_forward(0, x, ids, w, y),
        lambda: m.stats(),
        lambda: m.cache_state(),
        lambda: m.measure_h2d(wl.blob_bytes, 2),
        lambda: m.set_backend("offload"),
        lambda: m.calibrate_backend(1, 0.1),
    ]
    for f in calls:
        with pytest.raises(M.MoeError) as ei:
            with torch.cuda.stream(m.compute_stream):
                f()
        assert ei.value.status == M.MOE_ESTATE


def _check_against_oracle(m, wl, X, ids, w, y):
    ref = oracle.decode_trace(wl, synth.router_weights(wl), X)
    _, recs = m.stats(trace_cap=1 << 16)
    np.testing.assert_array_equal(ids, ref["ids"])
    assert trace_tuples(recs) == trace_tuples(ref["trace"])
    for u, v in zip(m.cache_state(), ref["cache"].state()):
        np.testing.assert_array_equal(u, v)
    for t in range(X.shape[0]):
        for l in range(wl.n_layers):
            r = oracle.moe_output(wl, l, X[t, 0], ref["ids"][t, l, 0], ref["w"][t, l, 0])
            assert close_enough(y[t, l, 0], r)[2], (t, l)


def test_injected_copy_failure_is_sticky_and_a_fresh_context_replays_exactly():
    import torch
    import moe_expert_offload_amd as M
    wl = dataclasses.replace(synth.WORKLOADS["toy"], cache_slots=4)
    X = synth.decode_inputs(wl)[:12]
    with env("MOE_FAULT", "h2d_fail_at=7"):
        m, _ = make_moe(wl)
    dev = m.device
    xd = torch.from_numpy(X.view(np.int16)).to(dev)
    y = torch.empty((wl.n_layers, 1, wl.hidden), dtype=torch.int16, device=dev)
    failed_at = None
    for t in range(X.shape[0]):
        try:
            with torch.cuda.stream(m.compute_stream):
                m.stack_forward(t, xd[t], 0, 1, y, wl.hidden)
        except M.MoeError as e:
            assert e.status == M.MOE_EHIP and "injected" in str(e), str(e)
            failed_at = t
            break
    assert failed_at is not None, "the injected copy failure never fired"
    _every_call_is_estate(m, wl)
    m.close()
    # a fresh context (no injection) from a cold cache replays the oracle exactly
    m2, _ = make_moe(wl)
    ids, w, yy = run_stack(m2, wl, X)
    _check_against_oracle(m2, wl, X, ids, w, yy)
    m2.close()


def test_verify_mode_passes_clean_runs_bitwise():
    import moe_expert_offload_amd as M
    wl = dataclasses.replace(synth.WORKLOADS["toy"], cache_slots=4)
    X = synth.decode_inputs(wl)[:16]
    m, _ = make_moe(wl, flags=M.MOE_FLAG_VERIFY)
    ids, w, y = run_stack(m, wl, X)
    cnt, _ = m.stats()
    assert cnt["evictions"] > 0
    m.close()
    m, _ = make_moe(wl)
    ids0, w0, y0 = run_stack(m, wl, X)
    _check_against_oracle(m, wl, X, ids0, w0, y0)
    m.close()
    np.testing.assert_array_equal(ids, ids0)
    np.testing.assert_array_equal(y.view(np.uint32), y0.view(np.uint32))


def test_verify_mode_catches_a_wrong_blob_and_stays_failed():
    import torch
    import moe_expert_offload_amd as M
    wl = dataclasses.replace(synth.WORKLOADS["toy"], cache_slots=4)
    X = synth.decode_inputs(wl)[:12]
    with env("MOE_FAULT", "h2d_corrupt_at=5"), env("MOE_VERIFY", "1"):
        m, _ = make_moe(wl)
    xd = torch.from_numpy(X.view(np.int16)).to(m.device)
    y = torch.empty((wl.n_layers, 1, wl.hidden), dtype=torch.int16, device=m.device)
    with pytest.raises(M.MoeError) as ei:
        with torch.cuda.stream(m.compute_stream):
            for t in range(X.shape[0]):
                m.stack_forward(t, xd[t], 0, 1, y, wl.hidden)
    assert ei.value.status == M.MOE_EVERIFY, str(ei.value)
    _every_call_is_estate(m, wl)
    m.close()


def test_bad_fault_spec_is_rejected_at_init():
    import moe_expert_offload_amd as M
    wl = synth.WORKLOADS["toy"]
    with env("MOE_FAULT", "h2d_fail_at=x"):
        with pytest.raises(M.MoeError) as ei:
            make_moe(wl)
    assert ei.value.status == M.MOE_EINVAL


def test_copy_and_ffn_timing_counters():
    """h2d_ns / h2d_timed_bytes: the copy path's busy time (merged over both copy streams) and the
    bytes moved in it, over every copy of one stack call in seven; ffn_ns / ffn_timed: one layer
    FFN in 17 timed.  Both filled without MOE_FLAG_PROFILE."""
    wl = dataclasses.replace(synth.WORKLOADS["toy"], cache_slots=4)
    X = synth.decode_inputs(wl)[:40]
    m, _ = make_moe(wl)
    run_stack(m, wl, X)
    cnt, _ = m.stats()
    launches = X.shape[0] * wl.n_layers
    assert cnt["ffn_timed"] == (launches + 16) // 17
    assert cnt["ffn_ns"] > 0 and cnt["ffn_ns"] / cnt["ffn_timed"] < 5e6
    assert cnt["h2d_copies"] > 0 and cnt["h2d_ns"] > 0
    assert 0 < cnt["h2d_timed_bytes"] < cnt["h2d_bytes"]
    assert cnt["h2d_timed_bytes"] % wl.blob_bytes == 0
    gbps = cnt["h2d_timed_bytes"] / cnt["h2d_ns"]
    assert 0.05 < gbps < 80.0, gbps
    # cumulative: a second stats call without work reports the same figures
    cnt2, _ = m.stats()
    keys = ("h2d_ns", "h2d_timed_bytes", "ffn_ns", "ffn_timed")
    assert tuple(cnt2[k] for k in keys) == tuple(cnt[k] for k in keys)
    m.close()
