"""The host expert kernel (timed by the backend calibration) against the oracle, the pool-layout
packing, and the hybrid split and auto-selection rules against the pages' worked numbers.
Host code only: no GPU."""
import os

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden", "page_worked_numbers.txt")


def _cfg(H, I):
    import moe_expert_offload_amd as M
    return M.make_config(1, 8, 2, H, I, 0, 0, 1)


def _golden(tag):
    rows = []
    for line in open(GOLDEN):
        f = line.split()
        if f and f[0] == tag:
            rows.append(f[1:])
    return rows


def _close(y, ref):
    nr = np.linalg.norm(ref)
    rel = np.linalg.norm(y - ref) / nr if nr > 0 else np.linalg.norm(y)
    return rel, np.max(np.abs(y - ref)), rel <= 5e-3 and np.max(np.abs(y - ref)) <= 1e-2 * max(np.max(np.abs(ref)), 1e-30)


def test_pack_blob_is_a_permutation_of_the_bytes():
    import moe_expert_offload_amd as M
    H, I = 800, 96
    logical = synth.blob(3, 0, 5, H, I)
    packed = M.pack_blob(_cfg(H, I), logical)
    assert packed.size == logical.size == 3 * H * I * 17 // 32
    np.testing.assert_array_equal(np.sort(packed), np.sort(logical))
    assert not np.array_equal(packed, logical)


# (H, I): one tile row; segments of unequal length (H/32 = 25 and 90 blocks); the gpt-oss shape
SHAPES = [(256, 512), (800, 96), (3072, 768), (2880, 2880)]


@pytest.mark.parametrize("isa", ["native", "scalar"])
@pytest.mark.parametrize("H,I", SHAPES, ids=[f"{h}x{i}" for h, i in SHAPES])
def test_host_kernel_matches_oracle(H, I, isa, monkeypatch):
    import moe_expert_offload_amd as M
    if isa == "scalar":
        monkeypatch.setenv("MOE_HOST_FFN_SCALAR", "1")
    cfg = _cfg(H, I)
    rng = np.random.default_rng(H + I)
    x = synth.f32_to_bf16_bits(rng.standard_normal(H).astype(np.float32))
    experts = [0, 3, 7]
    w = np.array([0.5, 0.3, 0.2], dtype=np.float32)
    logical = [synth.blob(9, 1, e, H, I) for e in experts]
    packed = [M.pack_blob(cfg, b) for b in logical]
    ref = sum(float(wj) * oracle.expert_ffn(b, H, I, x) for wj, b in zip(w, logical))
    for threads in (1, 2):
        y = M.host_expert_ffn(cfg, packed, w, x, threads=threads)
        rel, mx, ok = _close(y.astype(np.float64), ref)
        assert ok, (isa, threads, rel, mx)


def test_host_kernel_degenerate_inputs():
    import moe_expert_offload_amd as M
    H, I = 256, 512
    cfg = _cfg(H, I)
    packed = [M.pack_blob(cfg, synth.blob(1, 0, 0, H, I))]
    zero_x = np.zeros(H, dtype=np.uint16)
    assert not np.any(M.host_expert_ffn(cfg, packed, [1.0], zero_x))      # silu(0) * 0 = 0
    x = synth.f32_to_bf16_bits(np.ones(H, dtype=np.float32))
    assert not np.any(M.host_expert_ffn(cfg, [], [], x))                   # no experts
    assert not np.any(M.host_expert_ffn(cfg, packed, [0.0], x))            # zero weight
    y1 = M.host_expert_ffn(cfg, packed, [1.0], x)
    y2 = M.host_expert_ffn(cfg, packed, [2.0], x)
    np.testing.assert_array_equal(y2, 2.0 * y1)                            # linear in the weight


def test_auto_selection_matches_the_pages_worked_case():
    import moe_expert_offload_amd as M
    (threshold,), = _golden("threshold")
    for host, pcie, ratio, backend in _golden("calib"):
        host, pcie = float(host), float(pcie)
        assert round(host / pcie, 2) == float(ratio)
        assert M.select_backend(pcie, host, float(threshold)) == backend
    t = float(threshold)
    assert M.select_backend(10.0, 20.0, t) == "offload"          # exactly twice: not above the threshold
    assert M.select_backend(10.0, 20.01, t) == "hybrid"
    assert M.select_backend(0.0, 50.0, t) == "offload"           # no PCIe measurement


def test_hybrid_split_balances_finishing_times():
    import moe_expert_offload_amd as M
    assert M.hybrid_split(0, 26.7, 45.5) == 0
    assert M.hybrid_split(-3, 26.7, 45.5) == 0
    # host no faster than PCIe: nothing is left for the host while the DMA reads host memory
    assert M.hybrid_split(7, 49.0, 27.0) == 7
    assert M.hybrid_split(7, 30.0, 30.0) == 7
    # the pages' calibration numbers: 10 misses -> 10 * 26.7 / 45.5 = 5.87 -> 6 transferred
    assert M.hybrid_split(10, 26.7, 45.5) == 6
    assert M.hybrid_split(5, 10.0, 20.0) == 3                    # 2.5 rounds half up
    rng = np.random.default_rng(0)
    for _ in range(500):
        m = int(rng.integers(1, 200))
        bp = float(rng.uniform(5, 60))
        bh = bp * float(rng.uniform(1.01, 6.0))
        q = M.hybrid_split(m, bp, bh)
        assert 0 <= q <= m
        # q is the integer nearest the point where q / B_P = (m - q) / (B_H - B_P)
        q_star = m * bp / bh
        assert abs(q_star / bp - (m - q_star) / (bh - bp)) < 1e-9 * m
        assert abs(q - q_star) <= 0.5 + 1e-9


# the hybrid backend's host workers on one task: (expert, token) entries over up to 16 tokens
BATCH_SHAPES = [(256, 512), (800, 96), (2880, 2880)]


def _batch_case(H, I, n_tok, seed):
    import moe_expert_offload_amd as M
    cfg = _cfg(H, I)
    rng = np.random.default_rng(seed)
    x = synth.f32_to_bf16_bits(rng.standard_normal((n_tok, H)).astype(np.float32))
    n_exp = 5
    logical = [synth.blob(seed, 2, e, H, I) for e in range(n_exp)]
    packed = [M.pack_blob(cfg, b) for b in logical]
    ent = []   # (expert, weight, token); token 1 selects nothing
    for b in range(n_tok):
        if b == 1:
            continue
        for e in rng.choice(n_exp, size=int(rng.integers(1, 4)), replace=False):
            ent.append((int(e), float(rng.uniform(0.05, 1.0)), b))
    order = rng.permutation(len(ent))            # tokens interleaved in the entry list
    ent = [ent[i] for i in order]
    return cfg, x, logical, packed, ent


@pytest.mark.parametrize("H,I", BATCH_SHAPES, ids=[f"{h}x{i}" for h, i in BATCH_SHAPES])
def test_host_batch_matches_oracle_per_token(H, I):
    import moe_expert_offload_amd as M
    n_tok = 5
    cfg, x, logical, packed, ent = _batch_case(H, I, n_tok, H + 7)
    y = M.host_expert_batch(cfg, [packed[e] for e, _, _ in ent], [w for _, w, _ in ent],
                            [b for _, _, b in ent], x, threads=3)
    for b in range(n_tok):
        ref = np.zeros(H)
        for e, w, t in ent:
            if t == b:
                ref += w * oracle.expert_ffn(logical[e], H, I, x[b])
        if b == 1:
            assert not np.any(y[b])
            continue
        rel, mx, ok = _close(y[b].astype(np.float64), ref)
        assert ok, (b, rel, mx)


def test_host_batch_is_bitwise_independent_of_threads_and_matches_the_single_token_kernel():
    import moe_expert_offload_amd as M
    H, I, n_tok = 800, 96, 16
    cfg, x, _, packed, ent = _batch_case(H, I, n_tok, 11)
    args = ([packed[e] for e, _, _ in ent], [w for _, w, _ in ent], [b for _, _, b in ent], x)
    ys = [M.host_expert_batch(cfg, *args, threads=t) for t in (1, 4, 9)]
    for y in ys[1:]:
        np.testing.assert_array_equal(y.view(np.uint32), ys[0].view(np.uint32))
    # one thread of the single-token kernel adds a token's experts in the same order
    for b in range(n_tok):
        mine = [(e, w) for e, w, t in ent if t == b]
        y1 = M.host_expert_ffn(cfg, [packed[e] for e, _ in mine], [w for _, w in mine], x[b], threads=1)
        np.testing.assert_array_equal(y1.view(np.uint32), ys[0][b].view(np.uint32))


def test_host_batch_rejects_bad_arguments():
    import moe_expert_offload_amd as M
    H, I = 256, 512
    cfg = _cfg(H, I)
    p = M.pack_blob(cfg, synth.blob(1, 0, 0, H, I))
    x = np.zeros((2, H), dtype=np.uint16)
    for blobs, w, tok, xx, th in (([p], [1.0], [2], x, 1),                            # token out of range
                                  ([p], [1.0], [-1], x, 1),
                                  ([p], [1.0], [0], np.zeros((17, H), np.uint16), 1),  # more than 16 tokens
                                  ([p] * 257, [1.0] * 257, [0] * 257, x, 1),           # more than 256 entries
                                  ([p], [1.0], [0], x, 0)):                            # no worker
        with pytest.raises(M.MoeError):
            M.host_expert_batch(cfg, blobs, w, tok, xx, threads=th)
    y = M.host_expert_batch(cfg, [], [], [], x, threads=2)
    assert y.shape == (2, H) and not np.any(y)
