"""Decode benchmark of the MoE expert-offload path on one MI355X.

A step is one decode token through the whole MoE stack (all layers): router + top-k, cache
resolve, miss copies over PCIe, expert FFNs and combine, with inputs resident in HBM and the
expert pool in pinned host RAM.  Default workload: the gpt-oss-120b-shaped decode (36 layers x
128 experts, top-4, H = I = 2880, MXFP4, batch 1, 1862 of 4608 experts cached, AR(1) hidden
states with rho = 0.9).  W warm-up tokens, then K timed tokens (the cache keeps its state).

Prints one JSON line with the decode rate, the expert-FFN kernel roofline (HIP events around
every K3/K4 launch on the compute stream), the miss rate, the effective and measured
host-to-device bandwidth, and the CPU oracle timed on a bounded sample on the host cores.
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E


def decode_rate(tokens, total_s, ttft_s):
    """Completion tokens / (total - time to first token)."""
    return tokens / (total_s - ttft_s)


def pcie_payload_gbps(gt_per_s, lanes):
    """Per-direction payload bandwidth of a PCIe link with 128b/130b encoding (GB/s)."""
    return gt_per_s * 128.0 / 130.0 * lanes / 8.0


def per_token_budget_gb(link_gbps, tok_per_s):
    """Bytes of expert weights one token may transfer at a given decode rate (GB)."""
    return link_gbps / tok_per_s


def ffn_bytes(wl):
    """Algorithmic HBM bytes of one token-layer expert FFN: K3 reads the selected (and shared)
    experts' MXFP4 gate/up weights and x and writes the intermediate vector; K4 reads the down
    weights and the intermediate vector and writes y."""
    H, I, nE = wl.hidden, wl.inter, wl.top_k + wl.n_shared
    k3 = nE * (I * H * 34 // 32) + H * 2 + nE * I * 2
    k4 = nE * (H * I * 17 // 32) + nE * I * 2 + H * 2
    return k3, k4


def cpu_baseline(wl, W, X, budget_s=20.0):
    """The oracle as it stands, on the host cores: routing, LRU step and FFN of one decode
    token through every layer, repeated while the budget lasts (at least one token)."""
    import numpy as np

    import oracle
    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    cache = oracle.Cache(wl.n_layers, wl.n_experts, wl.cache_slots)
    t0 = time.perf_counter()
    done = 0
    for t in range(X.shape[0]):
        for l in range(wl.n_layers):
            z = oracle.router_logits(W[l], X[t, 0])
            ids, w = oracle.topk_softmax(z, wl.top_k)
            cache.step(t, l, ids)
            oracle.moe_output(wl, l, X[t, 0], ids, w)
        done += 1
        if time.perf_counter() - t0 > budget_s * 0.5:
            break
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "tok/s", "cores": int(os.environ.get("OMP_NUM_THREADS", cores)),
            "kind": "oracle",
            "sample": f"{done} decode token(s) x {wl.n_layers} layers of {wl.name}: FP32 router, "
                      f"top-{wl.top_k}, LRU step, FP64 MXFP4 SwiGLU FFN of the selected experts"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=448)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default="gptoss120b_shaped")
    ap.add_argument("--lookahead", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ffn-rounds", type=int, default=20)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the path has no multi-GPU "
              "sharding in this build", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import moe_expert_offload_amd as M

    wl = synth.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    X = synth.decode_inputs(wl)
    T = X.shape[0]
    W_, K = args.warmup, args.steps
    if W_ + K > T:
        K = T - W_
    flags = 0
    cfg = M.make_config(wl.n_layers, wl.n_experts, wl.top_k, wl.hidden, wl.inter, wl.n_shared,
                        wl.cache_slots, wl.n_requests, args.lookahead, 0, 0, flags)
    fptr, FillArgs = synth.fill_callback()
    fa = FillArgs(wl.seed, wl.hidden, wl.inter)
    Wr = synth.router_weights(wl)
    t0 = time.perf_counter()
    m = M.OffloadMoE(cfg, (fptr, ctypes.addressof(fa)), Wr)
    init_s = time.perf_counter() - t0
    print(f"# pool {wl.pool} x {m.blob_bytes} B = {wl.pool * m.blob_bytes / 1e9:.2f} GB pinned, "
          f"cache {wl.cache_slots} slots, init {init_s:.1f} s", file=sys.stderr, flush=True)

    # measured host-to-device bandwidth of the copy path (>= 2 GB of blob-sized copies)
    n_cp = max(8, int(2e9 // m.blob_bytes) + 1)
    h2d_meas = m.measure_h2d(m.blob_bytes, n_cp)
    h2d_big = m.measure_h2d(64 << 20, 32)

    B, L, H = wl.n_requests, wl.n_layers, wl.hidden
    xd = torch.from_numpy(X.view(np.int16)).to(dev)
    y = torch.empty((L, B, H), dtype=torch.int16, device=dev)
    cs = m.compute_stream
    torch.cuda.synchronize()
    with torch.cuda.stream(cs):
        for t in range(W_):
            m.stack_forward(t, xd[t], 0, B, y, B * H)
    cs.synchronize()
    c_warm, _ = m.stats()
    ids = torch.empty((L, B, wl.top_k), dtype=torch.int32, device=dev)
    wts = torch.empty((L, B, wl.top_k), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(cs):
        for t in range(W_, W_ + K):
            last = t == W_ + K - 1
            m.stack_forward(t, xd[t], 0, B, y, B * H, ids if last else None, wts if last else None)
    cs.synchronize()
    m.copy_stream.synchronize()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    c_all, _ = m.stats()
    # device and host counters are cumulative: take the timed region's share
    c = dict(c_all)
    for key in ("hits", "misses", "evictions", "resolves", "h2d_bytes", "h2d_copies"):
        c[key] = c_all[key] - c_warm[key]
    tok_s = K * B / dt

    # Expert-FFN kernel timing: the last token's experts of every layer are resident; run K3+K4
    # for layer 0..L-1 back to back, several rounds, between two HIP events on the compute
    # stream (consecutive launches read different experts, so nothing is served from a cache).
    slot_of, _, _ = m.cache_state()
    ids_h = ids.cpu().numpy()
    slots_h = np.stack([slot_of[l * wl.n_experts + ids_h[l]] for l in range(L)]).astype(np.int32)
    assert (slots_h >= 0).all()
    slots_d = torch.from_numpy(slots_h).to(dev)
    xt = xd[W_ + K - 1]
    y_eager = torch.empty_like(y)
    with torch.cuda.stream(cs):
        for l in range(L):
            m.expert_forward(l, xt, slots_d[l], wts[l], y_eager[l])
    cs.synchronize()
    # one pass over the L layers captured in a HIP graph, so that launch overhead on the host
    # does not leave gaps between the kernels; replayed between two events
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cs):
        for l in range(L):
            m.expert_forward(l, xt, slots_d[l], wts[l], y[l])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(cs):
        graph.replay()
        cs.synchronize()
        assert torch.equal(y, y_eager), "graph replay differs from the eager FFN"
        e0.record(cs)
        for r in range(args.ffn_rounds):
            graph.replay()
        e1.record(cs)
    cs.synchronize()
    assert torch.equal(y, y_eager), "graph replay differs from the eager FFN"
    ffn_launches = args.ffn_rounds * L
    ffn_us = e0.elapsed_time(e1) * 1e3 / ffn_launches

    k3b, k4b = ffn_bytes(wl)
    acc = c["hits"] + c["misses"]
    extra = {}
    gbs = (k3b + k4b) / (ffn_us * 1e-6) / 1e9
    roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
            "kernel": "expert FFN of one layer: k3_gate_up + k4_down (MXFP4 GEMVs, SwiGLU, weighted combine)",
            "bytes_per_launch": k3b + k4b, "bytes_k3": k3b, "bytes_k4": k4b,
            "avg_us": round(ffn_us, 2), "launches": ffn_launches}
    # miss bytes over the whole timed region: a lower bound on the copy path's achieved rate
    eff = c["h2d_bytes"] / dt / 1e9
    extra["h2d"] = {"effective_GBps": round(eff, 2), "measured_GBps": round(h2d_meas, 2),
                    "measured_64MB_GBps": round(h2d_big, 2), "frac_of_measured": round(eff / h2d_meas, 4)}
    extra["miss_rate"] = round(c["misses"] / acc, 4) if acc else None
    extra["miss_rate_warmup"] = round(c_warm["misses"] / max(1, c_warm["hits"] + c_warm["misses"]), 4)
    extra["misses_per_token"] = round(c["misses"] / K, 2)
    extra["h2d_GB_per_token"] = round(c["h2d_bytes"] / K / 1e9, 4)
    miss_bytes_tok = c["h2d_bytes"] / K
    hbm_bytes_tok = L * (k3b + k4b)
    roof_tok = 1.0 / max(hbm_bytes_tok / (HBM_PEAK_GBS * 1e9), miss_bytes_tok / (h2d_meas * 1e9))
    extra["decode_roofline_tok_s"] = round(roof_tok, 1)
    extra["decode_frac_of_roofline"] = round(tok_s / roof_tok, 4)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, Wr, X)
    m.close()
    out = {
        "metric": "decode tok/s per MoE stack at batch 1",
        "value": round(tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W_,
        "ms_per_step": round(dt * 1e3 / K, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4-w/bf16-a/fp32-acc",
        "data": "synthetic (seeded MXFP4 experts, N(0,0.02) bf16 router, AR(1) hidden states)",
        "config": {"workload": wl.name, "layers": L, "experts": wl.n_experts, "top_k": wl.top_k,
                   "shared": wl.n_shared, "hidden": H, "inter": wl.inter, "cache_slots": wl.cache_slots,
                   "pool_GB": round(wl.pool * m.blob_bytes / 1e9, 2), "batch": B, "lookahead": args.lookahead},
        "roofline": roof,
        "cpu_baseline": cpu,
        **extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
