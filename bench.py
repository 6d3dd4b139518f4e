"""Decode benchmark of the MoE expert-offload path on one MI355X.

A step is one decode token through the whole MoE stack (all layers): router + top-k, cache
resolve, miss copies over PCIe, expert FFNs and combine, with inputs resident in HBM and the
expert pool in host RAM.  Default workload: the DeepSeek-V4-Flash-shaped decode, the largest
batch-1 shape and the pages' stress case for the miss path (43 layers x 256 experts, top-6,
H = 4096, I = 2048, MXFP4, batch 1, 1211 of 11008 experts cached (11 %), a 147 GB pool, AR(1)
hidden states with rho = 0.85).  W warm-up tokens, then K timed tokens (the cache keeps its state).

Prints one JSON line with the decode rate, the expert-FFN kernel roofline (HIP events around
graph replays of the layer FFNs on the compute stream, and the same kernels timed inside the
decode loop), the miss rate, the copy path's achieved and measured host-to-device bandwidth, and
the CPU oracle timed on a bounded sample on the host cores.
"""
import argparse
import ctypes
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores

# HBM bytes moved per layer FFN launch (k3_gate_up + k4_down, batch 1) from the FETCH_SIZE and
# WRITE_SIZE counter runs, scaled by a device copy of known size in the same process
# (profiles/expert_ffn_*_traffic.md, profiles/decode_qwen36_*_traffic.md).  Set an entry to None when
# those kernels change.
FFN_TRAFFIC_BYTES = {"gptoss120b_shaped": 53743002, "dsv4_flash_shaped": 80790742, "qwen36_35b_a3b_shaped": 15382205}


def decode_rate(tokens, total_s, ttft_s):
    """Completion tokens / (total - time to first token)."""
    return tokens / (total_s - ttft_s)


def pcie_payload_gbps(gt_per_s, lanes):
    """Per-direction payload bandwidth of a PCIe link with 128b/130b encoding (GB/s)."""
    return gt_per_s * 128.0 / 130.0 * lanes / 8.0


def per_token_budget_gb(link_gbps, tok_per_s):
    """Bytes of expert weights one token may transfer at a given decode rate (GB)."""
    return link_gbps / tok_per_s


def pcie_link(dev_index=0):
    """PCIe link of the GPU from sysfs (speed, width, NUMA node), or None where unreadable."""
    import torch
    try:
        p = torch.cuda.get_device_properties(dev_index)
        bdf = "%04x:%02x:%02x.0" % (getattr(p, "pci_domain_id", 0), p.pci_bus_id, p.pci_device_id)
        base = "/sys/bus/pci/devices/" + bdf + "/"
        rd = lambda f: open(base + f).read().strip()
        return {"bdf": bdf, "speed": rd("current_link_speed"), "width": int(rd("current_link_width")),
                "max_speed": rd("max_link_speed"), "max_width": int(rd("max_link_width")),
                "numa_node": int(rd("numa_node"))}
    except Exception:
        return None


def ffn_bytes_split(wl):
    """Algorithmic HBM bytes of one token-layer expert FFN at batch 1: K3 reads the selected (and
    shared) experts' MXFP4 gate/up weights and x and writes the intermediate vector; K4 reads
    the down weights and the intermediate vector and writes y."""
    H, I, nE = wl.hidden, wl.inter, wl.top_k + wl.n_shared
    k3 = nE * (I * H * 34 // 32) + H * 2 + nE * I * 2
    k4 = nE * (H * I * 17 // 32) + nE * I * 2 + H * 2
    return k3, k4


def ffn_bytes(wl, B, n_distinct):
    """Algorithmic HBM bytes of one layer's expert FFN for B tokens: the weights of the distinct
    selected experts and the shared expert, read once; x read and y written; the bf16
    intermediate vector of every (token, expert) row written and read back."""
    H, I, nE = wl.hidden, wl.inter, wl.top_k + wl.n_shared
    blob = 3 * H * I * 17 // 32
    return (n_distinct + wl.n_shared) * blob + 2 * B * H * 2 + 2 * B * nE * I * 2


def ffn_flops(wl, rows):
    """Multiply-add flops of `rows` (token, expert) rows through one expert FFN (gate, up, down)."""
    return 2 * rows * 3 * wl.hidden * wl.inter


def time_ffn_pass(m, x, layers, slots, w, y, rounds):
    """Mean time (us) of one layer's expert FFN: moe_expert_forward for each of `layers` (slots,
    w, y indexed like `layers`), captured as one HIP graph and replayed `rounds` times between
    two events on the compute stream."""
    import torch
    cs = m.compute_stream
    L = len(layers)
    y_eager = torch.empty_like(y)
    with torch.cuda.stream(cs):
        for i, l in enumerate(layers):
            m.expert_forward(l, x, slots[i], w[i], y_eager[i])
    cs.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cs):
        for i, l in enumerate(layers):
            m.expert_forward(l, x, slots[i], w[i], y[i])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(cs):
        graph.replay()
        cs.synchronize()
        assert torch.equal(y, y_eager), "graph replay differs from the eager FFN"
        e0.record(cs)
        for _ in range(rounds):
            graph.replay()
        e1.record(cs)
    cs.synchronize()
    assert torch.equal(y, y_eager), "graph replay differs from the eager FFN"
    return e0.elapsed_time(e1) * 1e3 / (rounds * L)


def time_read_pass(m, byte_counts, n_layers, rounds):
    """Mean time (us) per layer of plain streaming reads (moe_hbm_read): one launch per entry of
    byte_counts, for each of n_layers layers from its own region of the slot arena (consecutive
    layers read different bytes, as the FFN's layers read different slots), captured as one HIP
    graph and replayed `rounds` times between two events on the compute stream."""
    import torch

    import moe_expert_offload_amd as M
    cs = m.compute_stream
    counts = [b // 16 * 16 for b in byte_counts]
    stride = (sum(counts) + 4095) // 4096 * 4096
    total = m.arena.numel()
    n_regions = max(1, (total - stride) // stride + 1) if total >= stride else 0
    if not n_regions:
        return None

    def one_pass():
        for i in range(n_layers):
            o = (i % n_regions) * stride
            for b in counts:
                M.hbm_read(m.arena, o, b, cs)
                o += b

    with torch.cuda.stream(cs):
        one_pass()
    cs.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cs):
        one_pass()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(cs):
        graph.replay()
        e0.record(cs)
        for _ in range(rounds):
            graph.replay()
        e1.record(cs)
    cs.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (rounds * n_layers)


def run_prefill(m, wl, dev, rounds):
    """The prefill chunk: one step of all its tokens through every layer (cold cache), then the
    last layer's grouped expert FFN on the chunk timed alone (its experts are all resident)."""
    import numpy as np
    import torch
    import synth
    P = synth.prefill_inputs(wl)
    n, L, H, k = P.shape[0], wl.n_layers, wl.hidden, wl.top_k
    xp = torch.from_numpy(P.view(np.int16)).to(dev)
    yp = torch.empty((L, n, H), dtype=torch.int16, device=dev)
    ids = torch.empty((L, n, k), dtype=torch.int32, device=dev)
    w = torch.empty((L, n, k), dtype=torch.float32, device=dev)
    cs = m.compute_stream
    c0, _ = m.stats()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(cs):
        m.stack_forward(0, xp, 0, n, yp, n * H, ids, w)
    cs.synchronize()
    m.copy_stream.synchronize()
    dt = time.perf_counter() - t0
    c1, _ = m.stats()
    slot_of, _, _ = m.cache_state()
    l = L - 1
    ids_l = ids[l].cpu().numpy()
    slots = slot_of[l * wl.n_experts + ids_l].astype(np.int32)
    assert (slots >= 0).all()
    sd = torch.from_numpy(slots[None]).to(dev)
    us = time_ffn_pass(m, xp, [l], sd, w[l:l + 1], yp[l:l + 1], rounds)
    rows = n * (k + wl.n_shared)
    fl = ffn_flops(wl, rows)
    nb = ffn_bytes(wl, n, len(np.unique(slots)))
    tf = fl / (us * 1e-6) / 1e12
    gbs = nb / (us * 1e-6) / 1e9
    h2d = c1["h2d_bytes"] - c0["h2d_bytes"]
    return {"tokens": n, "wall_s": round(dt, 3), "tok_s": round(n / dt, 1),
            "h2d_GB": round(h2d / 1e9, 2), "h2d_GBps": round(h2d / dt / 1e9, 2),
            "ffn_layer_us": round(us, 1),
            "ffn_mfma": {"achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / BF16_PEAK_TFLOPS, 4), "flops_per_launch": fl},
            "ffn_hbm": {"achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": nb}}


def cpu_baseline(wl, W, X, C, n_trace, budget_s=20.0):
    """The oracle as it stands, on the host cores: routing, LRU step and FFN of every token of
    one decode step through every layer, repeated while the budget lasts (at least one step);
    and, apart, the oracle's routing and LRU trace alone over the first n_trace tokens (every
    layer), the part of the method that decides ids and slots."""
    import numpy as np

    import oracle
    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    wtr = dataclasses.replace(wl, cache_slots=C)
    t0 = time.perf_counter()
    oracle.decode_trace(wtr, W, X[:n_trace])
    trace_s = time.perf_counter() - t0
    cache = oracle.Cache(wl.n_layers, wl.n_experts, C)
    B = X.shape[1]
    t0 = time.perf_counter()
    done = 0
    for t in range(X.shape[0]):
        for l in range(wl.n_layers):
            step_ids = []
            for b in range(B):
                z = oracle.router_logits(W[l], X[t, b])
                ids, w = oracle.topk_softmax(z, wl.top_k)
                step_ids.append(ids)
                oracle.moe_output(wl, l, X[t, b], ids, w)
            cache.step(t, l, np.stack(step_ids))
        done += 1
        if time.perf_counter() - t0 > budget_s * 0.5:
            break
    dt = time.perf_counter() - t0
    return {"value": done * B / dt, "unit": "tok/s", "cores": int(os.environ.get("OMP_NUM_THREADS", cores)),
            "kind": "oracle",
            "sample": f"{done} decode step(s) of {B} token(s) x {wl.n_layers} layers of {wl.name}: FP32 router, "
                      f"top-{wl.top_k}, LRU step, FP64 MXFP4 SwiGLU FFN of the selected experts",
            "trace_only_tok_s": round(n_trace * B / trace_s, 2),
            "trace_only_sample": f"routing (FP32 logits, top-{wl.top_k}, softmax) and the LRU cache step of "
                                 f"{n_trace} step(s) x {B} token(s) x {wl.n_layers} layers (warm-up + timed "
                                 "tokens of this run), no FFN"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=448)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default="dsv4_flash_shaped")
    ap.add_argument("--lookahead", type=int, default=7, choices=tuple(range(8)))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ffn-rounds", type=int, default=20)
    ap.add_argument("--calib-copy", action="store_true",
                    help="end with 3 device copies of 256 MiB (reference dispatches for counter scaling)")
    ap.add_argument("--policy", choices=("lru", "static"), default="lru",
                    help="cache policy: router-following LRU, or the static per-layer split comparator")
    ap.add_argument("--cache-slots", default="config",
                    help="'config' (the workload's cache fraction), 'auto' (as many slots as free HBM holds, "
                         "whole pool at most), or a slot count")
    ap.add_argument("--backend", choices=("offload", "hybrid", "auto"), default="offload",
                    help="offload: every miss over PCIe; hybrid: the calibrated split between PCIe and host "
                         "workers; auto: hybrid when the calibration says the host is more than twice as fast")
    ap.add_argument("--host-workers", type=int, default=0,
                    help="host worker threads of the hybrid backend (0: this process's cores - 2, at most 14; "
                         "4 fewer when part of the pool is pageable)")
    ap.add_argument("--auto-reserve-gb", type=float, default=4.0,
                    help="HBM kept free by --cache-slots auto (the KV cache's share in a server)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the path has no multi-GPU "
              "sharding", file=sys.stderr)
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
    policy = M.MOE_POLICY_STATIC if args.policy == "static" else M.MOE_POLICY_LRU
    C = {"config": wl.cache_slots, "auto": 0}.get(args.cache_slots)
    if C is None:
        C = int(args.cache_slots)
    cfg = M.make_config(wl.n_layers, wl.n_experts, wl.top_k, wl.hidden, wl.inter, wl.n_shared,
                        C, wl.max_tokens, args.lookahead, 0, 0, flags, 0, policy)
    fptr, FillArgs = synth.fill_callback()
    fa = FillArgs(wl.seed, wl.hidden, wl.inter)
    Wr = synth.router_weights(wl)
    t0 = time.perf_counter()
    m = M.OffloadMoE(cfg, (fptr, ctypes.addressof(fa)), Wr, auto_reserve_bytes=int(args.auto_reserve_gb * 2**30))
    init_s = time.perf_counter() - t0
    C = m.cfg.cache_slots
    c_init, _ = m.stats()
    pinned_gb = c_init["pool_pinned_bytes"] / 1e9
    print(f"# pool {wl.pool} x {m.blob_bytes} B = {wl.pool * m.blob_bytes / 1e9:.2f} GB ({pinned_gb:.2f} GB pinned), "
          f"cache {C} slots ({args.cache_slots}), init {init_s:.1f} s", file=sys.stderr, flush=True)

    # measured host-to-device bandwidth of the copy path (>= 2 GB of blob-sized copies)
    n_cp = max(8, int(2e9 // m.blob_bytes) + 1)
    h2d_meas = m.measure_h2d(m.blob_bytes, n_cp)
    h2d_big = m.measure_h2d(64 << 20, 32)
    # backend calibration: B_P (blob copies) vs B_H (the host expert kernel on the cores the host
    # workers would use: all of this process's cores but two, one for the thread that drives the
    # GPU and one for the HIP runtime's own threads (measured: 14 workers on 16 cores beat 15);
    # a pool with a pageable part also leaves the bounce ring's 4 copy threads their cores
    # (measured on 16 cores: 10 workers beat 14 there, DeepSeek-shaped 82 -> 90 tok/s)
    cores = min(16, len(os.sched_getaffinity(0)))
    pageable = c_init["pool_pinned_bytes"] < wl.pool * m.blob_bytes
    workers = args.host_workers or max(1, cores - 2 - (min(4, cores // 4) if pageable else 0))
    calib = m.calibrate_backend(workers, host_seconds=2.0)
    backend = args.backend if args.backend != "auto" else calib["backend"]
    if backend == "hybrid":
        m.set_backend("hybrid", calib["pcie_GBps"], calib["host_GBps"], workers)

    B, L, H = wl.n_requests, wl.n_layers, wl.hidden
    cs = m.compute_stream
    extra = {}
    prefill = None
    if wl.prefill_tokens:
        prefill = run_prefill(m, wl, dev, args.ffn_rounds)
        extra["prefill"] = prefill
    xd = torch.from_numpy(X.view(np.int16)).to(dev)
    y = torch.empty((L, B, H), dtype=torch.int16, device=dev)
    s0 = 1 if wl.prefill_tokens else 0
    torch.cuda.synchronize()
    tw0 = time.perf_counter()
    with torch.cuda.stream(cs):
        for t in range(W_):
            m.stack_forward(s0 + t, xd[t], 0, B, y, B * H)
    cs.synchronize()
    m.copy_stream.synchronize()
    warm_s = time.perf_counter() - tw0
    c_warm, _ = m.stats()
    ids = torch.empty((L, B, wl.top_k), dtype=torch.int32, device=dev)
    wts = torch.empty((L, B, wl.top_k), dtype=torch.float32, device=dev)
    # the timed region, in 5 equal segments (each ends with the streams drained) for the
    # run-to-run spread; value is the whole region's rate
    nseg = 5 if K >= 5 else 1
    bounds = [W_ + (K * i) // nseg for i in range(nseg + 1)]
    seg_rates = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for si in range(nseg):
        ts = time.perf_counter()
        with torch.cuda.stream(cs):
            for t in range(bounds[si], bounds[si + 1]):
                last = t == W_ + K - 1
                m.stack_forward(s0 + t, xd[t], 0, B, y, B * H, ids if last else None, wts if last else None)
        cs.synchronize()
        m.copy_stream.synchronize()
        seg_rates.append((bounds[si + 1] - bounds[si]) * B / (time.perf_counter() - ts))
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    c_all, _ = m.stats()
    # device and host counters are cumulative: take the timed region's share
    c = dict(c_all)
    for key in ("hits", "misses", "evictions", "resolves", "h2d_bytes", "h2d_copies", "h2d_bounced", "host_experts",
                "host_tasks", "host_busy_ms", "host_wait_ms"):
        c[key] = c_all[key] - c_warm[key]
    tok_s = K * B / dt

    # Expert-FFN kernel timing on the last step's experts: one pass over the layers whose
    # selected experts are all still resident (all of them at batch 1; a 16-request step can
    # touch more experts than there are slots, evicting its own early layers) is captured in a
    # HIP graph and replayed between two HIP events on the compute stream.  Every layer's
    # experts sit in their own slots, so consecutive launches read different weights.
    slot_of, _, _ = m.cache_state()
    ids_h = ids.cpu().numpy()
    slots_all = np.stack([slot_of[l * wl.n_experts + ids_h[l]] for l in range(L)]).astype(np.int32)
    layers = [l for l in range(L) if (slots_all[l] >= 0).all()]
    if layers:
        slots_h = slots_all[layers]
    else:
        # hybrid steps can leave no layer fully in slots: time the same kernels on distinct
        # slots per layer (the kernels' time does not depend on the weights' values)
        layers = list(range(L))
        kk = slots_all.shape[-1]
        slots_h = ((np.arange(L)[:, None, None] * kk + np.arange(kk)[None, None, :]) % wl.cache_slots
                   ).astype(np.int32).repeat(B, axis=1)
    ffn_us = time_ffn_pass(m, xd[W_ + K - 1], layers, torch.from_numpy(slots_h).to(dev), wts[layers],
                           y[layers], args.ffn_rounds)

    nbytes = [ffn_bytes(wl, B, len(np.unique(slots_h[i]))) for i in range(len(layers))]
    bytes_layer = sum(nbytes) / len(layers)
    acc = c["hits"] + c["misses"]
    gbs = bytes_layer / (ffn_us * 1e-6) / 1e9
    roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": FFN_TRAFFIC_BYTES.get(wl.name) if B == 1 and args.policy == "lru" else None,
            "kernel": ("expert FFN of one layer: k3_gate_up + k4_down (MXFP4 GEMVs, SwiGLU, weighted combine)"
                       if B == 1 else
                       "expert FFN of one layer: k2g_group + k5_gate_up + k5_down + k5_combine (grouped MXFP4 MFMA)"),
            "bytes_per_launch": round(bytes_layer), "avg_us": round(ffn_us, 2),
            "launches": args.ffn_rounds * len(layers), "layers_timed": len(layers)}
    if B == 1:
        roof["bytes_k3"], roof["bytes_k4"] = ffn_bytes_split(wl)
        # the plain-read floor of the same byte counts on this GPU: two launches (k3's bytes, then
        # k4's) and one launch of both, per layer, replayed like the FFN
        two = time_read_pass(m, [roof["bytes_k3"], roof["bytes_k4"]], len(layers), args.ffn_rounds)
        one = time_read_pass(m, [roof["bytes_k3"] + roof["bytes_k4"]], len(layers), args.ffn_rounds)
        if two and one:
            fb = roof["bytes_k3"] + roof["bytes_k4"]
            roof["plain_read"] = {
                "kernel": "moe_hbm_read: 16-byte nontemporal loads, 8 per lane, one round, from the slot arena",
                "two_launches_us": round(two, 2), "two_launches_frac": round(fb / (two * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "one_launch_us": round(one, 2), "one_launch_frac": round(fb / (one * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "ffn_frac_of_two_launches": round(two / ffn_us, 4)}
    # the same kernels inside the timed decode loop (one layer FFN in 17 timed by the library,
    # with the miss copies streaming beside them), against the same algorithmic bytes
    n_ffn = c_all["ffn_timed"] - c_warm["ffn_timed"]
    if n_ffn > 0 and not c["host_experts"]:
        us_loop = (c_all["ffn_ns"] - c_warm["ffn_ns"]) / n_ffn / 1e3
        b_loop = ffn_bytes(wl, B, min(B * wl.top_k, wl.n_experts)) if B == 1 else None
        roof["in_loop"] = {"avg_us": round(us_loop, 2), "launches_timed": n_ffn}
        if b_loop:
            g_loop = b_loop / (us_loop * 1e-6) / 1e9
            roof["in_loop"].update({"achieved": round(g_loop, 1), "frac": round(g_loop / HBM_PEAK_GBS, 4),
                                    "bytes_per_launch": b_loop})
    # miss bytes over the time the copy path was busy (the library times every copy of one call in
    # 7: per layer step and copy stream, first copy start to last copy end, merged over both
    # streams; those calls' bytes over that time), and over the whole timed region (a lower bound).
    # The busy share of the wall time scales the sampled busy time by all bytes over timed bytes.
    eff = c["h2d_bytes"] / dt / 1e9
    busy_ns = c_all["h2d_ns"] - c_warm["h2d_ns"]
    timed_b = c_all["h2d_timed_bytes"] - c_warm["h2d_timed_bytes"]
    ach = timed_b / busy_ns if busy_ns > 0 else None
    extra["h2d"] = {"achieved_GBps": round(ach, 2) if ach else None,
                    "achieved_frac_of_measured": round(ach / h2d_meas, 4) if ach else None,
                    "busy_frac_of_wall": round(busy_ns * 1e-9 * c["h2d_bytes"] / timed_b / dt, 4) if timed_b else None,
                    "effective_GBps": round(eff, 2), "measured_GBps": round(h2d_meas, 2),
                    "measured_64MB_GBps": round(h2d_big, 2), "frac_of_measured": round(eff / h2d_meas, 4),
                    "link": pcie_link(0)}
    extra["pool"] = {"GB": round(wl.pool * m.blob_bytes / 1e9, 2), "pinned_GB": round(pinned_gb, 2),
                     "bounced_copies": c["h2d_bounced"], "copies": c["h2d_copies"]}
    srt = sorted(seg_rates)
    extra["segments"] = {"n": nseg, "median_tok_s": round(srt[len(srt) // 2], 2), "min_tok_s": round(srt[0], 2),
                         "max_tok_s": round(srt[-1], 2)}
    # cold = every token from the empty cache on (warm-up + timed); steady = the timed region
    extra["cold_tok_s"] = round((W_ + K) * B / (warm_s + dt), 2)
    if B > 1:
        extra["per_request_tok_s"] = round(tok_s / B, 2)
    extra["miss_rate"] = round(c["misses"] / acc, 4) if acc else None
    extra["miss_rate_cumulative"] = round(c_all["misses"] / max(1, c_all["hits"] + c_all["misses"]), 4)
    extra["miss_rate_warmup"] = round(c_warm["misses"] / max(1, c_warm["hits"] + c_warm["misses"]), 4)
    extra["misses_per_step"] = round(c["misses"] / K, 2)
    extra["h2d_GB_per_step"] = round(c["h2d_bytes"] / K / 1e9, 4)
    miss_bytes_step = c["h2d_bytes"] / K
    host_bytes_step = c["host_experts"] * m.blob_bytes / K
    roof_step = 1.0 / max(L * bytes_layer / (HBM_PEAK_GBS * 1e9), miss_bytes_step / (h2d_meas * 1e9),
                          host_bytes_step / (calib["host_GBps"] * 1e9))
    if backend == "hybrid":
        extra["host"] = {"workers": workers, "experts_per_step": round(c["host_experts"] / K, 2),
                         "GB_per_step": round(host_bytes_step / 1e9, 4),
                         "effective_GBps": round(c["host_experts"] * m.blob_bytes / dt / 1e9, 2),
                         "calibrated_GBps": round(calib["host_GBps"], 2),
                         "tasks_per_step": round(c["host_tasks"] / K, 2),
                         "busy_ms_per_step": round(c["host_busy_ms"] / K, 3),
                         "wait_ms_per_step": round(c["host_wait_ms"] / K, 3)}
    extra["decode_roofline_tok_s"] = round(roof_step * B, 1)
    extra["decode_frac_of_roofline"] = round(tok_s / (roof_step * B), 4)

    if args.calib_copy:
        # plain device copies of known size: under a counter profiler their FETCH_SIZE /
        # WRITE_SIZE per dispatch give the scale from counter units to bytes
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, Wr, X, C, W_ + K)
    m.close()
    out = {
        "metric": ("decode tok/s per MoE stack at batch 1" if B == 1 else
                   f"decode tok/s per MoE stack, {B} requests in lock-step (aggregate)"),
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
                   "shared": wl.n_shared, "hidden": H, "inter": wl.inter, "cache_slots": C, "cache_sizing": args.cache_slots,
                   "pool_GB": round(wl.pool * m.blob_bytes / 1e9, 2), "batch": B, "lookahead": args.lookahead,
                   "policy": args.policy, "backend": backend},
        "roofline": roof,
        "backend_calibration": {k: (round(v, 2) if isinstance(v, float) else v) for k, v in calib.items()},
        "cpu_baseline": cpu,
        **extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
