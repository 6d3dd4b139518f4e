"""Seeded synthetic inputs for the decode-time MoE expert-offload workloads.

This package is the only code shared by the HIP library's callers and the CPU
oracle.  It generates inputs and holds none of the method's arithmetic (no
dequantisation, routing, caching or FFN):

* expert weight blobs in the logical MXFP4 layout (bulk bytes come from the C
  generator in ``synth.c``; ``blob_numpy`` is a slow pure-numpy twin used to
  check it),
* router weights, N(0, 0.02^2) rounded to bfloat16,
* hidden states, one AR(1) stream per request, rounded to bfloat16,
* the workload shapes (layers, experts, top-k, hidden and intermediate sizes,
  cache size, token counts, AR(1) coefficient).

Shapes follow the models the FreeToken pages discuss (pirouter.ai "FreeToken x
RTX 5090 -- 120B MoE が 127 tok/s、その請求書", section on how 65 GB fits into
32 GB: 36 x 128 experts, 4 per layer, 40.4 % resident; ai-hardware-zukan.com
FreeToken vs Ollama page, section on cache misses: caches of 37 % and 11 % of the
expert pool; gaming-st.com DeepSeek page, MoE background section: 43 layers x 256
experts, 6 active; blog.florigen.ai Qwen3.8-Flash-Next page, model section: 48
layers, 512 routed + 1 shared expert, 10 routed per token).  Hidden and
intermediate sizes are not on the pages; they are fixed here as part of the
workload definition.

Random numbers: SplitMix64 used counter-style (see ``synth.c``).  Gaussians use
the cosine branch of Box-Muller on two consecutive words.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
import subprocess

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

KIND_CODES = 1
KIND_SCALES = 11
KIND_ROUTER = 21
KIND_HIDDEN = 22
SHARED_ID_BASE = 1000000
PREFILL_REQUEST_ID = 100000

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")


# ----------------------------------------------------------------------------
# workload shapes
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_layers: int
    n_experts: int
    top_k: int
    n_shared: int
    hidden: int
    inter: int
    cache_slots: int
    decode_tokens: int      # decode steps per request
    n_requests: int         # requests decoded in lock-step (batch of one token each)
    rho: float              # AR(1) coefficient of the hidden-state stream
    prefill_tokens: int = 0  # tokens of one prefill chunk processed before decode
    seed: int = 0

    @property
    def pool(self) -> int:
        return self.n_layers * self.n_experts

    @property
    def blob_bytes(self) -> int:
        return 3 * self.hidden * self.inter * 17 // 32

    @property
    def max_tokens(self) -> int:
        return max(self.n_requests, self.prefill_tokens)


def cache_slots_for(fraction: float, pool: int) -> int:
    """round-half-up(fraction * pool)"""
    return int(math.floor(fraction * pool + 0.5))


WORKLOADS = {
    "toy": Workload("toy", 2, 16, 2, 0, 256, 512, 8, 64, 1, 0.9),
    "gptoss120b_shaped": Workload("gptoss120b_shaped", 36, 128, 4, 0, 2880, 2880,
                                  cache_slots_for(0.404, 36 * 128), 512, 1, 0.9),
    "qwen36_35b_a3b_shaped": Workload("qwen36_35b_a3b_shaped", 40, 256, 8, 1, 2048, 512,
                                      cache_slots_for(0.37, 40 * 256), 512, 1, 0.9),
    "dsv4_flash_shaped": Workload("dsv4_flash_shaped", 43, 256, 6, 0, 4096, 2048,
                                  cache_slots_for(0.11, 43 * 256), 512, 1, 0.85),
    "qwen38_flash_next_shaped": Workload("qwen38_flash_next_shaped", 48, 512, 10, 1, 3072, 768,
                                         cache_slots_for(0.25, 48 * 512), 256, 16, 0.9,
                                         prefill_tokens=2048),
}


# ----------------------------------------------------------------------------
# SplitMix64, numpy twin of synth.c
# ----------------------------------------------------------------------------
def mix64(z):
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def key(seed: int, kind: int, a: int = 0, b: int = 0, c: int = 0) -> np.uint64:
    with np.errstate(over="ignore"):
        k = mix64(np.uint64(seed) + GAMMA)
        for v in (kind, a, b, c):
            k = mix64(k + GAMMA * np.uint64(v + 1))
    return np.uint64(k)


def words(k: np.uint64, start: int, n: int) -> np.ndarray:
    idx = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(np.uint64(k) + GAMMA * idx)


def bytes_numpy(k: np.uint64, n: int) -> np.ndarray:
    w = words(k, 0, (n + 7) // 8)
    return w.astype("<u8").view(np.uint8)[:n].copy()


def scales_numpy(k: np.uint64, n: int, lo: int = 123, span: int = 5) -> np.ndarray:
    hi = words(k, 0, n) >> np.uint64(32)
    with np.errstate(over="ignore"):
        return (np.uint64(lo) + ((hi * np.uint64(span)) >> np.uint64(32))).astype(np.uint8)


def expert_id(expert: int) -> int:
    """Stream id of a routed expert (>= 0) or of shared expert s (passed as -1-s)."""
    return expert if expert >= 0 else SHARED_ID_BASE + (-1 - expert)


def blob_numpy(seed: int, layer: int, expert: int, H: int, I: int) -> np.ndarray:
    """Logical blob of one expert, pure numpy (slow; used to check the C generator)."""
    eid = expert_id(expert)
    parts = []
    for m in range(3):
        parts.append(bytes_numpy(key(seed, KIND_CODES + m, layer, eid, 0), H * I // 2))
        parts.append(scales_numpy(key(seed, KIND_SCALES + m, layer, eid, 0), H * I // 32))
    return np.concatenate(parts)


def blob_sections(H: int, I: int):
    """(name, offset, shape) of the six arrays inside a logical blob."""
    out, off = [], 0
    for name, rows, cols in (("gate", I, H), ("up", I, H), ("down", H, I)):
        out.append((name + "_codes", off, (rows, cols // 2)))
        off += rows * cols // 2
        out.append((name + "_scales", off, (rows, cols // 32)))
        off += rows * cols // 32
    return out


# ----------------------------------------------------------------------------
# C generator (bulk bytes)
# ----------------------------------------------------------------------------
class FillArgs(ctypes.Structure):
    _fields_ = [("seed", ctypes.c_uint64), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32)]


def build_lib(force: bool = False) -> str:
    src = os.path.join(_HERE, "synth.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", src, "-o", tmp])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build_lib()
        L = ctypes.CDLL(_LIB_PATH)
        L.synth_key.restype = ctypes.c_uint64
        L.synth_key.argtypes = [ctypes.c_uint64] * 5
        L.synth_bytes.argtypes = [ctypes.c_uint64, ctypes.c_void_p, ctypes.c_size_t]
        L.synth_scales.argtypes = [ctypes.c_uint64, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_uint32, ctypes.c_uint32]
        L.synth_expert_blob.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
        _lib = L
    return _lib


def blob(seed: int, layer: int, expert: int, H: int, I: int, out: np.ndarray | None = None) -> np.ndarray:
    """Logical blob of one routed expert (expert >= 0) or shared expert s (expert = -1-s)."""
    n = 3 * H * I * 17 // 32
    if out is None:
        out = np.empty(n, dtype=np.uint8)
    assert out.dtype == np.uint8 and out.size == n and out.flags.c_contiguous
    lib().synth_expert_blob(seed, layer, expert, H, I, out.ctypes.data)
    return out


def fill_callback():
    """(function pointer, FillArgs type) for the library's pool filler."""
    return ctypes.cast(lib().synth_fill_cb, ctypes.c_void_p).value, FillArgs


# ----------------------------------------------------------------------------
# bfloat16 helpers (storage rounding of generated values only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(u) -> np.ndarray:
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normals(k: np.uint64, start: int, n: int) -> np.ndarray:
    """n standard normals: Box-Muller (cosine branch) on words 2j and 2j+1 of the stream."""
    w = words(k, 2 * start, 2 * n).reshape(n, 2)
    u1 = ((w[:, 0] >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53   # (0, 1]
    u2 = (w[:, 1] >> np.uint64(11)).astype(np.float64) * 2.0 ** -53           # [0, 1)
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)


def router_weights(wl: Workload, layer: int | None = None) -> np.ndarray:
    """Router W as bf16 bits: [E][H] for one layer, or [L][E][H]."""
    layers = range(wl.n_layers) if layer is None else [layer]
    out = []
    for l in layers:
        z = normals(key(wl.seed, KIND_ROUTER, l, 0, 0), 0, wl.n_experts * wl.hidden)
        out.append(f32_to_bf16_bits((0.02 * z).astype(np.float32)).reshape(wl.n_experts, wl.hidden))
    return out[0] if layer is not None else np.stack(out)


def hidden_stream(seed: int, request: int, T: int, H: int, rho: float) -> np.ndarray:
    """AR(1) stream of T hidden states of width H as bf16 bits [T][H]:
    x[0] = eps_0, x[t] = rho*x[t-1] + sqrt(1-rho^2)*eps_t (float64), stored rounded to bf16."""
    eps = normals(key(seed, KIND_HIDDEN, request, 0, 0), 0, T * H).reshape(T, H)
    x = np.empty((T, H), dtype=np.float64)
    c = math.sqrt(1.0 - rho * rho)
    x[0] = eps[0]
    for t in range(1, T):
        x[t] = rho * x[t - 1] + c * eps[t]
    return f32_to_bf16_bits(x.astype(np.float32))


def decode_inputs(wl: Workload) -> np.ndarray:
    """Decode hidden states as bf16 bits [T][B][H] (B = requests, one stream each)."""
    streams = [hidden_stream(wl.seed, r, wl.decode_tokens, wl.hidden, wl.rho) for r in range(wl.n_requests)]
    return np.stack(streams, axis=1)


def prefill_inputs(wl: Workload) -> np.ndarray:
    """The prefill chunk as bf16 bits [P][H]: one AR(1) stream of its own."""
    return hidden_stream(wl.seed, PREFILL_REQUEST_ID, wl.prefill_tokens, wl.hidden, wl.rho)
