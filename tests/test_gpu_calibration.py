"""Backend calibration on the device: B_P from the copy path, B_H from the host expert kernel over
pool blobs, and the recommendation the auto rule gives for them."""
import ctypes
import os

import pytest

import synth

pytestmark = pytest.mark.gpu


def test_calibration_measures_both_paths_and_recommends():
    import moe_expert_offload_amd as M
    wl = synth.Workload("calib_2880", 4, 32, 4, 0, 2880, 2880, 16, 4, 1, 0.9, seed=41)
    cfg = M.make_config(wl.n_layers, wl.n_experts, wl.top_k, wl.hidden, wl.inter, wl.n_shared, wl.cache_slots, 1)
    fptr, FillArgs = synth.fill_callback()
    fa = FillArgs(wl.seed, wl.hidden, wl.inter)
    m = M.OffloadMoE(cfg, (fptr, ctypes.addressof(fa)), synth.router_weights(wl))
    threads = min(16, len(os.sched_getaffinity(0)))
    p = m.calibrate_backend(threads, host_seconds=1.0)
    print(p)
    assert 5.0 < p["pcie_GBps"] < 200.0
    assert p["host_GBps"] > 0.1
    assert abs(p["ratio"] - p["host_GBps"] / p["pcie_GBps"]) < 1e-9 * p["ratio"]
    assert p["backend"] == M.select_backend(p["pcie_GBps"], p["host_GBps"], 2.0)
    assert p["host_isa"] in ("avx512", "scalar") and p["host_threads"] == threads
    # the calibration leaves the (cold) cache untouched
    slot_of, key_of, _ = m.cache_state()
    assert (slot_of == -1).all() and (key_of == -1).all()
    m.close()
