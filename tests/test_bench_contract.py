"""bench.py on the CPU: the one-GPU contract and the arithmetic behind its roofline fields.

The algorithmic bytes are checked against the MXFP4 blob size written out from the format (E2M1
codes: half a byte per element; one E8M0 byte per 32 elements; three matrices of H x I), not
against bench.py's own formula."""
import importlib.util
import os
import subprocess
import sys

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_ffn_algorithmic_bytes_at_gptoss_shape():
    b = _bench()
    wl = synth.WORKLOADS["gptoss120b_shaped"]
    H, I, k = wl.hidden, wl.inter, wl.top_k
    matrix = H * I // 2 + H * I // 32          # codes + scales of one H x I matrix
    assert 3 * matrix == wl.blob_bytes == 13_219_200
    act = H * 2 + k * I * 2                    # x (or y) and the intermediate vectors, bf16
    gate_up, down = b.ffn_bytes_split(wl)
    assert gate_up == k * 2 * matrix + act == 35_280_000
    assert down == k * matrix + act == 17_654_400
    # one token, k distinct experts: the same bytes as the two parts together
    assert b.ffn_bytes(wl, 1, k) == gate_up + down == 52_934_400


def test_ffn_bytes_count_distinct_experts_once():
    b = _bench()
    wl = synth.WORKLOADS["qwen38_flash_next_shaped"]
    blob = wl.blob_bytes
    B, nE = 16, wl.top_k + wl.n_shared
    # 139 distinct routed experts plus the shared one, each read once for the 16 tokens
    expect = (139 + 1) * blob + 2 * B * wl.hidden * 2 + 2 * B * nE * wl.inter * 2
    assert b.ffn_bytes(wl, B, 139) == expect


def test_pcie_and_budget_arithmetic():
    b = _bench()
    # PCIe 5.0 x16: 32 GT/s per lane, 128b/130b encoding
    assert abs(b.pcie_payload_gbps(32.0, 16) - 63.0154) < 1e-3
    # a 49 GB/s link at 127 tok/s leaves 0.386 GB of expert transfers per token
    assert abs(b.per_token_budget_gb(49.0, 127.0) - 0.38583) < 1e-4
    assert b.decode_rate(100, 11.0, 1.0) == 10.0
    assert b.ffn_flops(synth.WORKLOADS["toy"], 3) == 2 * 3 * 3 * 256 * 512


GOLDEN = os.path.join(ROOT, "tests", "golden", "page_worked_numbers.txt")


def _golden(tag):
    return [[float(v) for v in line.split()[1:]] for line in open(GOLDEN) if line.split()[:1] == [tag]]


def test_decode_rate_reproduces_the_pages_runs():
    """blog.florigen.ai Qwen3.8-Flash-Next page, speed section: three runs printed as completion
    tokens, total seconds and time to first token, with their decode rates and mean."""
    b = _bench()
    rows = _golden("decode")
    assert len(rows) == 3
    rates = []
    for tokens, total, ttft, printed in rows:
        r = b.decode_rate(tokens, total, ttft)
        assert abs(r - printed) < 0.005 + 1e-9, (tokens, total, ttft, r, printed)
        rates.append(r)
    (mean,), = _golden("decode_mean")
    assert abs(sum(rates) / 3 - mean) < 0.005


def test_pcie_payload_reproduces_the_pages_link_figures():
    """Same page, PCIe efficiency section: PCIe 5.0 x8 carries 31.5 GB/s per direction, and
    the measured 28.9 GB/s is 91.7 % of it."""
    b = _bench()
    (gt, lanes, printed), = _golden("pcie")
    assert abs(b.pcie_payload_gbps(gt, lanes) - printed) < 0.05
    (meas, link, pct), = _golden("pcie_eff")
    assert abs(100.0 * meas / b.pcie_payload_gbps(gt, lanes) - pct) < 0.1
    assert abs(100.0 * meas / link - pct) < 0.1


def test_per_token_budget_reproduces_the_pages_ceiling():
    """pirouter.ai "FreeToken x RTX 5090" page, expert-path section: the per-token transfer
    ceiling is the link rate over the decode rate (0.39 GB at 127.1 tok/s, 1.53 GB at 32 tok/s)."""
    b = _bench()
    rows = _golden("budget")
    assert len(rows) == 2
    for link, tok_s, printed in rows:
        assert abs(b.per_token_budget_gb(link, tok_s) - printed) < 0.005 + 1e-9, (link, tok_s, printed)
