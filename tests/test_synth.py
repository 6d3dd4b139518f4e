"""Seeded input generator: determinism, C generator == numpy twin, distributions."""
import numpy as np
import pytest

import synth


def test_c_generator_matches_numpy_twin():
    for (l, e, H, I) in [(0, 0, 64, 32), (1, 5, 256, 512), (3, -1, 96, 64), (0, 127, 32, 96)]:
        a = synth.blob(7, l, e, H, I)
        b = synth.blob_numpy(7, l, e, H, I)
        assert a.size == 3 * H * I * 17 // 32
        np.testing.assert_array_equal(a, b)


def test_key_matches_c():
    L = synth.lib()
    for args in [(0, 1, 0, 0, 0), (5, 22, 3, 9, 1), (2**40, 11, 47, 511, 0)]:
        assert int(synth.key(*args)) == L.synth_key(*args)


def test_blob_determinism_and_distinct_streams():
    a = synth.blob(0, 1, 2, 256, 512)
    np.testing.assert_array_equal(a, synth.blob(0, 1, 2, 256, 512))
    assert not np.array_equal(a, synth.blob(1, 1, 2, 256, 512))
    assert not np.array_equal(a, synth.blob(0, 1, 3, 256, 512))
    assert not np.array_equal(a, synth.blob(0, 0, 2, 256, 512))
    assert not np.array_equal(a, synth.blob(0, 1, -1, 256, 512))


def test_code_and_scale_distributions():
    H, I = 512, 1024
    b = synth.blob(3, 0, 0, H, I)
    secs = {n: b[o:o + int(np.prod(s))].reshape(s) for n, o, s in synth.blob_sections(H, I)}
    codes = np.concatenate([secs[m + "_codes"].ravel() for m in ("gate", "up", "down")])
    nib = np.concatenate([codes & 15, codes >> 4])
    cnt = np.bincount(nib, minlength=16)
    exp = nib.size / 16
    chi2 = ((cnt - exp) ** 2 / exp).sum()
    assert chi2 < 45.0  # 15 dof, p ~ 1e-4
    sc = np.concatenate([secs[m + "_scales"].ravel() for m in ("gate", "up", "down")])
    assert sc.min() == 123 and sc.max() == 127
    cnt = np.bincount(sc - 123, minlength=5)
    exp = sc.size / 5
    assert ((cnt - exp) ** 2 / exp).sum() < 25.0  # 4 dof


def test_ar1_statistics():
    rho = 0.9
    x = synth.bf16_bits_to_f32(synth.hidden_stream(0, 0, 4096, 128, rho)).astype(np.float64)
    assert abs(x.var() - 1.0) < 0.05
    lag1 = (x[1:] * x[:-1]).mean() / np.sqrt(x[1:].var() * x[:-1].var())
    assert abs(lag1 - rho) < 0.02
    x2 = synth.bf16_bits_to_f32(synth.hidden_stream(0, 1, 4096, 128, 0.85)).astype(np.float64)
    lag1 = (x2[1:] * x2[:-1]).mean() / np.sqrt(x2[1:].var() * x2[:-1].var())
    assert abs(lag1 - 0.85) < 0.02


def test_router_distribution():
    wl = synth.WORKLOADS["toy"]
    W = synth.bf16_bits_to_f32(synth.router_weights(wl)).astype(np.float64)
    assert W.shape == (2, 16, 256)
    assert abs(W.mean()) < 0.002
    assert abs(W.std() - 0.02) < 0.001


def test_bf16_rounding_ties_to_even():
    f = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5], dtype=np.float32)
    got = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(f))
    np.testing.assert_array_equal(got, np.array([1.0, 1.0, 1.0 + 2**-6, 1.0, -2.5], dtype=np.float32))


def test_workload_shapes():
    W = synth.WORKLOADS
    assert W["gptoss120b_shaped"].pool == 4608
    assert W["gptoss120b_shaped"].cache_slots == 1862
    assert W["gptoss120b_shaped"].blob_bytes == 13_219_200
    assert W["qwen36_35b_a3b_shaped"].cache_slots == 3789
    assert W["dsv4_flash_shaped"].cache_slots == 1211
    assert W["qwen38_flash_next_shaped"].cache_slots == 6144
    for wl in W.values():
        # capacity rule: twice the largest distinct set one step can request
        per_step = min(wl.max_tokens * wl.top_k, wl.n_experts)
        assert wl.cache_slots >= 2 * per_step
