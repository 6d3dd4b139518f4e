"""Helpers for the GPU parity tests: build a library context for a workload and run it."""
import ctypes

import numpy as np

import synth


def bf16_to_f32(t):
    """torch int16/uint16 tensor of bf16 bits -> numpy float32."""
    import torch
    return t.view(torch.bfloat16).float().cpu().numpy()


def make_moe(wl, lookahead=7, trace_capacity=1 << 20, flags=0, max_tokens=None, cache_slots=None, pinned_mb=0,
             policy=0):
    import moe_expert_offload_amd as M
    cfg = M.make_config(wl.n_layers, wl.n_experts, wl.top_k, wl.hidden, wl.inter, wl.n_shared,
                        wl.cache_slots if cache_slots is None else cache_slots, max_tokens or wl.max_tokens, lookahead,
                        trace_capacity, 0, flags, pinned_mb, policy)
    fptr, FillArgs = synth.fill_callback()
    args = FillArgs(wl.seed, wl.hidden, wl.inter)
    W = synth.router_weights(wl)
    m = M.OffloadMoE(cfg, (fptr, ctypes.addressof(args)), W)
    m._keep.append(args)
    return m, W


def run_stack(m, wl, X, steps=None, step0=0):
    """Run moe_stack_forward for every step of X [T][B][H] (bf16 bits, same input for every
    layer).  Returns ids [T][L][B][k], w [T][L][B][k], y [T][L][B][H] float32."""
    import torch
    T, B, H = X.shape
    L, k = wl.n_layers, wl.top_k
    steps = range(T) if steps is None else steps
    dev = m.device
    xd = torch.from_numpy(X.view(np.int16)).to(dev)
    y = torch.empty((len(steps), L, B, H), dtype=torch.int16, device=dev)
    ids = torch.empty((len(steps), L, B, k), dtype=torch.int32, device=dev)
    w = torch.empty((len(steps), L, B, k), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(m.compute_stream):
        for i, t in enumerate(steps):
            m.stack_forward(step0 + t, xd[t], 0, B, y[i], B * H, ids[i], w[i])
    m.compute_stream.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy(), bf16_to_f32(y)


def close_enough(y, ref):
    """Per-vector tolerance: relative L2 <= 5e-3 and max|diff| <= 1e-2 * max|ref|."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    nr = np.linalg.norm(ref)
    rel = np.linalg.norm(y - ref) / nr if nr > 0 else np.linalg.norm(y)
    mx = np.max(np.abs(y - ref))
    return rel, mx, (rel <= 5e-3 and mx <= 1e-2 * max(np.max(np.abs(ref)), 1e-30))


def trace_tuples(recs):
    return [tuple(int(r[f]) for f in ("step", "layer", "expert", "slot", "hit", "evicted_key")) for r in recs]


def run_steps(m, wl, steps_X):
    """moe_stack_forward once per step, step t with its own token count B_t (steps_X: list of
    [B_t][H] bf16 bits).  Returns per-step lists ids [L][B_t][k], w, y [L][B_t][H] float32."""
    import torch
    L, k, H = wl.n_layers, wl.top_k, wl.hidden
    dev = m.device
    outs = []
    torch.cuda.synchronize()
    with torch.cuda.stream(m.compute_stream):
        for t, x in enumerate(steps_X):
            B = len(x)
            xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev)
            y = torch.empty((L, B, H), dtype=torch.int16, device=dev)
            ids = torch.empty((L, B, k), dtype=torch.int32, device=dev)
            w = torch.empty((L, B, k), dtype=torch.float32, device=dev)
            m.stack_forward(t, xd, 0, B, y, B * H, ids, w)
            outs.append((ids, w, y))
    m.compute_stream.synchronize()
    return ([o[0].cpu().numpy() for o in outs], [o[1].cpu().numpy() for o in outs],
            [bf16_to_f32(o[2]) for o in outs])
