"""The allocation-free expert FFN (moe_expert_forward_noalloc) against moe_expert_forward of a
context with the same kernels (MOE_FLAG_PER_TOKEN_FFN), bit for bit, and against the oracle within
the output tolerance: two calls in a row, the second with fewer tokens, on the same static scratch
array; a slot outside the arena gives NaN outputs for its token only."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import bf16_to_f32, close_enough, make_moe, run_stack

pytestmark = pytest.mark.gpu


def test_noalloc_expert_forward_matches_the_context_entry_point():
    import torch
    import moe_expert_offload_amd as M
    wl = synth.Workload("noalloc_shared_k8", 2, 48, 8, 1, 2048, 512, 64, 6, 1, 0.9, seed=31)
    m, _ = make_moe(wl, flags=M.MOE_FLAG_PER_TOKEN_FFN, max_tokens=4)
    X = synth.decode_inputs(wl)
    run_stack(m, wl, X)  # fills the cache with each layer's recent experts
    slot_of, _, _ = m.cache_state()
    dev = m.device
    l = 1
    resident = np.nonzero(slot_of[l * wl.n_experts:(l + 1) * wl.n_experts] >= 0)[0]
    assert len(resident) >= wl.top_k
    rng = np.random.default_rng(5)
    cfg = M.make_config(wl.n_layers, wl.n_experts, wl.top_k, wl.hidden, wl.inter, wl.n_shared, wl.cache_slots, 4)
    shared = torch.from_numpy(M.pack_blob(cfg, synth.blob(wl.seed, l, -1, wl.hidden, wl.inter))).to(dev)
    xs = synth.decode_inputs(synth.Workload("noalloc_x", 1, 1, 1, 0, wl.hidden, 32, 2, 4, 4, 0.5, seed=9))[0]
    for B in (4, 2):  # the second call is smaller
        ids = np.stack([rng.choice(resident, wl.top_k, replace=False) for _ in range(B)]).astype(np.int32)
        w = rng.random((B, wl.top_k)).astype(np.float32)
        w /= w.sum(axis=1, keepdims=True)
        slots = slot_of[l * wl.n_experts + ids].astype(np.int32)
        x = torch.from_numpy(np.ascontiguousarray(xs[:B]).view(np.int16)).to(dev)
        sd, wd = torch.from_numpy(slots).to(dev), torch.from_numpy(w).to(dev)
        y_ctx = torch.empty((B, wl.hidden), dtype=torch.int16, device=dev)
        y_na = torch.full((B, wl.hidden), 0x7FC0, dtype=torch.int16, device=dev)
        with torch.cuda.stream(m.compute_stream):
            m.expert_forward(l, x, sd, wd, y_ctx)
            M.expert_forward_noalloc(cfg, m.arena, shared, x, sd, wd, y_na, stream=m.compute_stream)
        m.compute_stream.synchronize()
        np.testing.assert_array_equal(y_na.cpu().numpy(), y_ctx.cpu().numpy())
        yf = bf16_to_f32(y_na)
        for b in range(B):
            r = oracle.moe_output(wl, l, xs[b], ids[b], w[b])
            rel, mx, ok = close_enough(yf[b], r)
            assert ok, (B, b, rel, mx)
    # a slot outside the arena is never read: its token's outputs are NaN, the others unchanged
    bad = slots.copy()
    bad[1, 3] = wl.cache_slots + 7
    y_bad = torch.empty((B, wl.hidden), dtype=torch.int16, device=dev)
    with torch.cuda.stream(m.compute_stream):
        M.expert_forward_noalloc(cfg, m.arena, shared, x, torch.from_numpy(bad).to(dev), wd, y_bad,
                                 stream=m.compute_stream)
    m.compute_stream.synchronize()
    yb = bf16_to_f32(y_bad)
    assert np.all(np.isnan(yb[1]))
    np.testing.assert_array_equal(y_bad.cpu().numpy()[0], y_na.cpu().numpy()[0])
    m.close()


def test_noalloc_rejects_tokens_beyond_its_limit():
    import torch
    import moe_expert_offload_amd as M
    cfg = M.make_config(1, 16, 2, 256, 512, 0, 8, 32)
    t = torch.zeros(17 * 256, dtype=torch.int16, device="cuda")
    x = t.view(17, 256)
    with pytest.raises(M.MoeError) as ei:
        M.expert_forward_noalloc(cfg, t, None, x, t, t, t)
    assert ei.value.status == M.MOE_EINVAL
