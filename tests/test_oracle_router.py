"""Oracle routing: fixed-order FP32 logits, top-k with ties to the lower index, softmax."""
import math

import numpy as np
import pytest

import oracle
import synth


def bf16(a):
    return synth.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def test_fold_order_hand_derived():
    # H = 16: elements 0..7 belong to lane 0, 8..15 to lane 1.  Lane 0 adds 2^24 then
    # seven 1s: each 2^24 + 1 rounds back to 2^24 (tie to even).  Lane 1 sums eight 1s = 8.
    # The butterfly gives 2^24 + 8, while the exact sum is 2^24 + 15.
    w = np.ones(16, np.float32)
    w[0] = 2.0 ** 24
    z = oracle.router_logits(bf16(w)[None, :], bf16(np.ones(16)))
    assert z[0] == np.float32(2.0 ** 24 + 8)
    # Same values, but the big term is last in lane 0: 1+..+1 (7) = 7, + 2^24 -> 2^24 + 8
    # (2^24 + 7 rounds to 2^24 + 8), lane 1 = 8, total 2^24 + 16.
    w2 = np.ones(16, np.float32)
    w2[7] = 2.0 ** 24
    z2 = oracle.router_logits(bf16(w2)[None, :], bf16(np.ones(16)))
    assert z2[0] == np.float32(2.0 ** 24 + 16)


def test_lane_wraps_every_512_elements():
    # H = 1024: elements 512..519 form group 64, which belongs to lane 0 again, so they are
    # folded into lane 0 after element 0 = 2^24 and each 1.0 is absorbed (ties to even):
    # z = 2^24.  Elements 520..527 (group 65) belong to lane 1, which sums them to 8 on its
    # own; the butterfly then gives 2^24 + 8.
    H = 1024
    w = np.zeros(H, np.float32)
    w[0] = 2.0 ** 24
    w[512:520] = 1.0
    z = oracle.router_logits(bf16(w)[None, :], bf16(np.ones(H)))
    assert z[0] == np.float32(2.0 ** 24)
    w[512:520] = 0.0
    w[520:528] = 1.0
    z = oracle.router_logits(bf16(w)[None, :], bf16(np.ones(H)))
    assert z[0] == np.float32(2.0 ** 24 + 8.0)


def test_logits_close_to_exact_sum():
    rng = np.random.default_rng(0)
    for H in (256, 2880, 4096):
        W = bf16(rng.normal(0, 0.02, (8, H)))
        x = bf16(rng.normal(0, 1, H))
        z = oracle.router_logits(W, x)
        Wf, xf = synth.bf16_bits_to_f32(W).astype(np.float64), synth.bf16_bits_to_f32(x).astype(np.float64)
        for e in range(8):
            exact = math.fsum(Wf[e] * xf)
            scale = math.fsum(np.abs(Wf[e] * xf))
            assert abs(float(z[e]) - exact) <= 1e-6 * scale


def test_zero_input_and_one_hot():
    rng = np.random.default_rng(1)
    W = bf16(rng.normal(0, 0.02, (16, 256)))
    z = oracle.router_logits(W, bf16(np.zeros(256)))
    assert np.all(z == 0)
    ids, w = oracle.topk_softmax(z, 4)
    assert list(ids) == [0, 1, 2, 3]
    np.testing.assert_allclose(w, 0.25, rtol=0, atol=1e-15)
    x = np.zeros(256, np.float32)
    x[37] = 1.5
    z = oracle.router_logits(W, bf16(x))
    np.testing.assert_array_equal(z, synth.bf16_bits_to_f32(W)[:, 37] * np.float32(1.5))


def brute_topk(z, k):
    order = sorted(range(len(z)), key=lambda e: (-float(z[e]), e))
    return order[:k]


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(2)
    for trial in range(200):
        E = int(rng.choice([16, 128, 256, 512]))
        k = int(rng.integers(1, 11))
        z = rng.normal(0, 1, E).astype(np.float32)
        if trial % 3 == 0:  # heavy ties
            z = np.round(z * 2).astype(np.float32) / 2
        if trial % 7 == 0:
            z[rng.integers(0, E, 5)] = -0.0
            z[rng.integers(0, E, 5)] = 0.0
        ids, w = oracle.topk_softmax(z, k)
        assert list(ids) == brute_topk(z, k)
        assert abs(w.sum() - 1.0) < 1e-12
        assert np.all(np.diff(w) <= 0)


def test_softmax_closed_form_k2():
    z = np.array([0.3, 1.7, -0.2, 1.2], np.float32)
    ids, w = oracle.topk_softmax(z, 2)
    assert list(ids) == [1, 3]
    w0 = 1.0 / (1.0 + math.exp(float(z[3]) - float(z[1])))
    assert abs(w[0] - w0) < 1e-15 and abs(w[1] - (1 - w0)) < 1e-15


def test_duplicate_router_rows_tie_to_lower_index():
    rng = np.random.default_rng(3)
    W = bf16(rng.normal(0, 0.02, (32, 512)))
    x = bf16(rng.normal(0, 1, 512))
    z = oracle.router_logits(W, x)
    top = int(np.argmax(z))
    W2 = W.copy()
    W2[31] = W[top]
    W2[top] = W[top]
    z2 = oracle.router_logits(W2, x)
    assert z2[31] == z2[top]
    ids, _ = oracle.topk_softmax(z2, 2)
    assert list(ids) == [top, 31]


def test_route_batch_matches_single_calls():
    wl = synth.WORKLOADS["toy"]
    W = synth.router_weights(wl)
    X = synth.decode_inputs(wl)[:5, 0]
    ids, w = oracle.route_batch(W, X, wl.top_k, [0, 1, 1, 0, 1], [0, 1, 2, 3, 4])
    for i, (l, t) in enumerate(zip([0, 1, 1, 0, 1], [0, 1, 2, 3, 4])):
        z = oracle.router_logits(W[l], X[t])
        i2, w2 = oracle.topk_softmax(z, wl.top_k)
        np.testing.assert_array_equal(ids[i], i2)
        np.testing.assert_array_equal(w[i], w2)
