"""Router logits through the C ABI (moe_router_logits) against the oracle's FP32 logits in the
canonical summation order, bit for bit.

Both router kernels are covered: the one-wave-per-(expert, token) kernel (1 and 16 tokens) and
the tiled kernel (more than 16 tokens).  The hidden sizes fill every lane's groups exactly (256,
3072, 4096) or leave a partial last group (2880: 360 groups of 8 over 64 lanes; 800: 100; 3584:
448, so the tiled kernel's eighth group of every lane is past the row; 1056: 132).
All-zero activations make every product zero.  Ids being bit-exact does not show that the logits
are: a change in the order of the additions moves a logit by an ulp, which almost never changes
a top-k choice."""
import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import make_moe

pytestmark = pytest.mark.gpu

# (name, layers, experts, top_k, shared, H, I, cache slots, decode tokens, requests, rho,
# prefill tokens = the largest token count of a call); cache slots at the capacity rule's minimum,
# 2 * min(24 * k, E)
CASES = [
    synth.Workload("router_256", 2, 16, 2, 0, 256, 512, 32, 1, 1, 0.9, prefill_tokens=24, seed=31),
    synth.Workload("router_2880", 2, 32, 4, 0, 2880, 256, 64, 1, 1, 0.9, prefill_tokens=24, seed=32),
    synth.Workload("router_3072_e512", 1, 512, 10, 1, 3072, 256, 480, 1, 1, 0.9, prefill_tokens=24, seed=33),
    synth.Workload("router_4096", 2, 256, 6, 0, 4096, 256, 288, 1, 1, 0.9, prefill_tokens=24, seed=34),
    synth.Workload("router_800", 2, 24, 3, 1, 800, 96, 48, 1, 1, 0.85, prefill_tokens=24, seed=35),
    synth.Workload("router_3584", 2, 64, 4, 0, 3584, 128, 128, 1, 1, 0.9, prefill_tokens=24, seed=36),
    synth.Workload("router_1056", 2, 48, 2, 0, 1056, 64, 96, 1, 1, 0.9, prefill_tokens=24, seed=37),
]


def _logits(m, layer, X):
    import torch
    xd = torch.from_numpy(np.ascontiguousarray(X).view(np.int16)).to(m.device)
    z = torch.full((X.shape[0], m.cfg.n_experts), float("nan"), dtype=torch.float32, device=m.device)
    torch.cuda.synchronize()
    with torch.cuda.stream(m.compute_stream):
        m.router_logits(layer, xd, z)
    m.compute_stream.synchronize()
    return z.cpu().numpy()


def _oracle(W, X):
    return np.stack([oracle.router_logits(W, X[t]) for t in range(X.shape[0])])


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_router_logits_are_bit_exact(wl):
    m, W = make_moe(wl)
    X = synth.prefill_inputs(wl)
    for layer in range(wl.n_layers):
        ref_all = _oracle(W[layer], X)
        for n in (1, 16, 17, X.shape[0]):
            got = _logits(m, layer, X[:n])
            ref = ref_all[:n]
            bad = np.argwhere(got.view(np.uint32) != ref.view(np.uint32))
            assert bad.size == 0, (wl.name, layer, n, bad[:5].tolist(),
                                   [(float(got[t, e]), float(ref[t, e])) for t, e in bad[:5]])


def test_router_logits_of_zero_activations_are_zero():
    wl = CASES[2]
    m, W = make_moe(wl)
    X = np.zeros((20, wl.hidden), dtype=np.uint16)
    for n in (1, 20):
        got = _logits(m, 0, X[:n])
        assert np.array_equal(got.view(np.uint32), np.zeros_like(got.view(np.uint32))), "expected +0.0 logits"
        assert np.array_equal(got.view(np.uint32), _oracle(W[0], X[:n]).view(np.uint32))


def test_router_logits_rejects_bad_arguments():
    import torch
    import moe_expert_offload_amd as M
    wl = CASES[0]
    m, _ = make_moe(wl)
    x = torch.zeros((4, wl.hidden), dtype=torch.int16, device=m.device)
    z = torch.zeros((4, wl.n_experts), dtype=torch.float32, device=m.device)
    for layer in (-1, wl.n_layers):
        with pytest.raises(M.MoeError) as e:
            m.router_logits(layer, x, z)
        assert e.value.status == M.MOE_EINVAL
    big = torch.zeros((wl.max_tokens + 1, wl.hidden), dtype=torch.int16, device=m.device)
    with pytest.raises(M.MoeError) as e:
        m.router_logits(0, big, z)
    assert e.value.status == M.MOE_EINVAL
    # the context stays usable
    m.router_logits(0, x, z)
    m.compute_stream.synchronize()
