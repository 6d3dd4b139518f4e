"""CPU oracle for decode-time MoE layers over a router-following LRU expert cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the library and its
Python binding never do, and the two share no code (only the seeded input
generator in ``synth``).

The arithmetic lives in ``oracle.c`` (plain C, FP32 canonical-order logits, FP64
routing weights and FFN); this module wraps it with ctypes and strings the
steps together exactly as the FreeToken pages describe the offload backend
(pirouter.ai "FreeToken x RTX 5090 -- 120B MoE が 127 tok/s、その請求書", section
on how 65 GB runs on a 32 GB GPU): for each token and layer the router picks
experts, the (layer, expert) pairs are looked up in one global LRU cache of
GPU slots, misses are loaded from host RAM into evicted slots, and the
selected experts' outputs are combined with the routing weights.

Combine (not stated on the pages; reading): out = sum_j w_j * y_j plus the
shared expert's output with weight 1 when the model has one.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

import synth

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")


def build_lib(force: bool = False) -> str:
    src = os.path.join(_HERE, "oracle.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-shared",
                               "-fPIC", src, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class TraceRec(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("step", "layer", "expert", "slot", "hit", "evicted_key")]


TRACE_DTYPE = np.dtype([(n, np.int32) for n in ("step", "layer", "expert", "slot", "hit", "evicted_key")])

_lib = None
_P = ctypes.c_void_p


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build_lib()
        L = ctypes.CDLL(_LIB_PATH)
        L.orc_e2m1_value.restype = ctypes.c_double
        L.orc_e2m1_value.argtypes = [ctypes.c_uint]
        L.orc_e8m0_scale.restype = ctypes.c_double
        L.orc_e8m0_scale.argtypes = [ctypes.c_uint]
        L.orc_dequant_row.argtypes = [_P, _P, ctypes.c_int, _P]
        L.orc_router_logits.argtypes = [_P, _P, ctypes.c_int, ctypes.c_int, _P]
        L.orc_topk_softmax.argtypes = [_P, ctypes.c_int, ctypes.c_int, _P, _P]
        L.orc_route_batch.argtypes = [_P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      _P, _P, _P, _P, _P]
        L.orc_expert_ffn.argtypes = [_P, ctypes.c_int, ctypes.c_int, _P, _P]
        L.orc_cache_new.restype = _P
        L.orc_cache_new.argtypes = [ctypes.c_int] * 3
        L.orc_cache_free.argtypes = [_P]
        L.orc_cache_counters.argtypes = [_P, _P]
        L.orc_cache_state.argtypes = [_P, _P, _P, _P]
        L.orc_cache_step.restype = ctypes.c_int
        L.orc_cache_step.argtypes = [_P, ctypes.c_int, ctypes.c_int, _P, ctypes.c_int, _P, _P]
        L.orc_cache_step_split.restype = ctypes.c_int
        L.orc_cache_step_split.argtypes = [_P, ctypes.c_int, ctypes.c_int, _P, ctypes.c_int, ctypes.c_double,
                                           ctypes.c_double, _P, _P]
        L.orc_cache_host.restype = ctypes.c_uint64
        L.orc_cache_host.argtypes = [_P]
        L.orc_static_new.restype = _P
        L.orc_static_new.argtypes = [ctypes.c_int] * 4
        L.orc_static_free.argtypes = [_P]
        L.orc_static_counters.argtypes = [_P, _P]
        L.orc_static_state.argtypes = [_P, _P, _P]
        L.orc_static_step.restype = ctypes.c_int
        L.orc_static_step.argtypes = [_P, ctypes.c_int, ctypes.c_int, _P, ctypes.c_int, _P, _P]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags.c_contiguous
    return a.ctypes.data


# ---------------------------------------------------------------- dequant --
def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(code)


def e8m0_scale(e: int) -> float:
    return lib().orc_e8m0_scale(e)


def dequant_row(codes: np.ndarray, scales: np.ndarray, K: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    assert codes.size == K // 2 and scales.size == K // 32
    out = np.empty(K, dtype=np.float64)
    lib().orc_dequant_row(_ptr(codes), _ptr(scales), K, _ptr(out))
    return out


# ----------------------------------------------------------------- router --
def router_logits(W: np.ndarray, x: np.ndarray) -> np.ndarray:
    """W: [E][H] bf16 bits, x: [H] bf16 bits -> z [E] float32 (fixed summation order)."""
    W = np.ascontiguousarray(W, dtype=np.uint16)
    x = np.ascontiguousarray(x, dtype=np.uint16)
    E, H = W.shape
    z = np.empty(E, dtype=np.float32)
    lib().orc_router_logits(_ptr(W), _ptr(x), E, H, _ptr(z))
    return z


def topk_softmax(z: np.ndarray, k: int):
    z = np.ascontiguousarray(z, dtype=np.float32)
    ids = np.empty(k, dtype=np.int32)
    w = np.empty(k, dtype=np.float64)
    lib().orc_topk_softmax(_ptr(z), z.size, k, _ptr(ids), _ptr(w))
    return ids, w


def route_batch(W_all: np.ndarray, X: np.ndarray, k: int, layers, toks, want_z: bool = False):
    """Routing of (layer, token) items.  W_all [L][E][H], X [n_tok][H] (bf16 bits)."""
    W_all = np.ascontiguousarray(W_all, dtype=np.uint16)
    X = np.ascontiguousarray(X, dtype=np.uint16)
    L, E, H = W_all.shape
    layers = np.ascontiguousarray(layers, dtype=np.int32)
    toks = np.ascontiguousarray(toks, dtype=np.int32)
    n = layers.size
    ids = np.empty((n, k), dtype=np.int32)
    w = np.empty((n, k), dtype=np.float64)
    z = np.empty((n, E), dtype=np.float32) if want_z else None
    lib().orc_route_batch(_ptr(W_all), _ptr(X), E, H, k, n, _ptr(layers), _ptr(toks),
                          _ptr(z) if want_z else None, _ptr(ids), _ptr(w))
    return (ids, w, z) if want_z else (ids, w)


# -------------------------------------------------------------------- FFN --
def expert_ffn(blob: np.ndarray, H: int, I: int, x: np.ndarray) -> np.ndarray:
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.uint16)
    assert blob.size == 3 * H * I * 17 // 32 and x.size == H
    y = np.empty(H, dtype=np.float64)
    lib().orc_expert_ffn(_ptr(blob), H, I, _ptr(x), _ptr(y))
    return y


def moe_output(wl: "synth.Workload", layer: int, x: np.ndarray, ids, w) -> np.ndarray:
    """Output of layer `layer` for one token: sum_j w_j * FFN_{ids_j}(x) (+ shared, weight 1)."""
    H, I = wl.hidden, wl.inter
    out = np.zeros(H, dtype=np.float64)
    for e, wj in zip(ids, w):
        out += float(wj) * expert_ffn(synth.blob(wl.seed, layer, int(e), H, I), H, I, x)
    for s in range(wl.n_shared):
        out += expert_ffn(synth.blob(wl.seed, layer, -1 - s, H, I), H, I, x)
    return out


# ------------------------------------------------------------------ cache --
class Cache:
    """Global LRU over C slots keyed by (layer, expert); cold start."""

    def __init__(self, L: int, E: int, C: int):
        self.L, self.E, self.C = L, E, C
        self._h = lib().orc_cache_new(L, E, C)

    def __del__(self):
        if getattr(self, "_h", None):
            lib().orc_cache_free(self._h)
            self._h = None

    def step(self, step: int, layer: int, ids, split=None):
        """split = (pcie_GBps, host_GBps): a hybrid step (oracle.c, the hybrid split)."""
        ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32).ravel())
        slots = np.empty(ids.size, dtype=np.int32)
        rec = np.empty(max(1, min(ids.size, self.E)), dtype=TRACE_DTYPE)
        if split is None:
            n = lib().orc_cache_step(self._h, step, layer, _ptr(ids), ids.size, _ptr(slots), _ptr(rec))
        else:
            n = lib().orc_cache_step_split(self._h, step, layer, _ptr(ids), ids.size, float(split[0]),
                                           float(split[1]), _ptr(slots), _ptr(rec))
        if n < 0:
            raise ValueError("step requests more distinct experts than the cache has slots")
        return slots, rec[:n].copy()

    def counters(self):
        c = np.empty(3, dtype=np.uint64)
        lib().orc_cache_counters(self._h, _ptr(c))
        return {"hits": int(c[0]), "misses": int(c[1]), "evictions": int(c[2]),
                "host": int(lib().orc_cache_host(self._h))}

    def state(self):
        slot_of = np.empty(self.L * self.E, dtype=np.int32)
        key_of = np.empty(self.C, dtype=np.int32)
        stamp = np.empty(self.C, dtype=np.int64)
        lib().orc_cache_state(self._h, _ptr(slot_of), _ptr(key_of), _ptr(stamp))
        return slot_of, key_of, stamp


class StaticCache:
    """Static per-layer split over C slots: keys [0, C - T) resident for good, T transient
    slots in rotation for every other access (see oracle.c, static per-layer split)."""

    def __init__(self, L: int, E: int, C: int, T: int):
        self.L, self.E, self.C, self.T = L, E, C, T
        self._h = lib().orc_static_new(L, E, C, T)
        if not self._h:
            raise ValueError("need 1 <= T <= C")

    def __del__(self):
        if getattr(self, "_h", None):
            lib().orc_static_free(self._h)
            self._h = None

    def step(self, step: int, layer: int, ids):
        ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32).ravel())
        slots = np.empty(ids.size, dtype=np.int32)
        rec = np.empty(max(1, min(ids.size, self.E)), dtype=TRACE_DTYPE)
        n = lib().orc_static_step(self._h, step, layer, _ptr(ids), ids.size, _ptr(slots), _ptr(rec))
        if n < 0:
            raise ValueError("step misses more distinct experts than there are transient slots")
        return slots, rec[:n].copy()

    def counters(self):
        c = np.empty(3, dtype=np.uint64)
        lib().orc_static_counters(self._h, _ptr(c))
        return {"hits": int(c[0]), "misses": int(c[1]), "evictions": int(c[2])}

    def state(self):
        slot_of = np.empty(self.L * self.E, dtype=np.int32)
        key_of = np.empty(self.C, dtype=np.int32)
        lib().orc_static_state(self._h, _ptr(slot_of), _ptr(key_of))
        return slot_of, key_of


# ------------------------------------------------------------ whole runs --
# Steps of more tokens than this run every miss through the cache even under the hybrid
# backend (the host share is a decode-time split; a prefill chunk transfers all of its misses).
HYBRID_MAX_TOKENS = 16


def decode_trace(wl: "synth.Workload", W_all: np.ndarray, X: np.ndarray, steps=None, split=None):
    """Routing and cache trace of a decode run.

    X: [T][B][H] bf16 bits (B lock-step requests); every layer of step t sees
    X[t] (the hidden state of a request is fed unchanged to every layer).
    Steps run in order t = 0..T-1, layers 0..L-1 inside a step.
    Returns dict with ids [T][L][B][k], w [T][L][B][k], slots [T][L][B][k],
    trace (structured array), counters.  split = (pcie_GBps, host_GBps) runs the hybrid
    backend's cache steps (misses beyond the transferred share take no slot) when B is at
    most HYBRID_MAX_TOKENS.
    """
    T, B, H = X.shape
    if B > HYBRID_MAX_TOKENS:
        split = None
    L, k = wl.n_layers, wl.top_k
    steps = range(T) if steps is None else steps
    Xf = X.reshape(T * B, H)
    tt, ll, bb = np.meshgrid(np.arange(T), np.arange(L), np.arange(B), indexing="ij")
    ids, w = route_batch(W_all, Xf, k, ll.ravel(), (tt * B + bb).ravel())
    ids = ids.reshape(T, L, B, k)
    w = w.reshape(T, L, B, k)
    cache = Cache(L, wl.n_experts, wl.cache_slots)
    slots = np.empty_like(ids)
    recs = []
    for t in steps:
        for l in range(L):
            s, r = cache.step(t, l, ids[t, l], split)
            slots[t, l] = s.reshape(B, k)
            recs.append(r)
    return {"ids": ids, "w": w, "slots": slots,
            "trace": np.concatenate(recs) if recs else np.empty(0, TRACE_DTYPE),
            "counters": cache.counters(), "cache": cache}


def run_trace(wl: "synth.Workload", W_all: np.ndarray, steps_X, static_transient: int = 0, split=None):
    """Routing and cache trace of a run whose steps have their own token counts.

    steps_X: list of [B_t][H] bf16-bit arrays; step t feeds X_t to every layer (a prefill
    chunk is one step whose B_t is the chunk length).  Steps run in order, layers 0..L-1
    inside a step.  Returns dict with per-step lists ids[t] [L][B_t][k], w[t], slots[t],
    the trace (structured array), counters and the cache.  static_transient > 0 runs the static
    per-layer split with that many transient slots instead of the LRU cache.  split =
    (pcie_GBps, host_GBps) runs the hybrid backend's cache steps for the steps of at most
    HYBRID_MAX_TOKENS tokens.
    """
    assert not (split and static_transient), "the hybrid split runs on the LRU cache"
    L, k = wl.n_layers, wl.top_k
    Xc = np.concatenate([np.asarray(x, dtype=np.uint16).reshape(-1, wl.hidden) for x in steps_X])
    layers, toks, shapes = [], [], []
    base = 0
    for x in steps_X:
        B = len(x)
        ll, bb = np.meshgrid(np.arange(L), np.arange(B), indexing="ij")
        layers.append(ll.ravel())
        toks.append(base + bb.ravel())
        shapes.append(B)
        base += B
    ids_all, w_all = route_batch(W_all, Xc, k, np.concatenate(layers), np.concatenate(toks))
    cache = (StaticCache(L, wl.n_experts, wl.cache_slots, static_transient) if static_transient
             else Cache(L, wl.n_experts, wl.cache_slots))
    out = {"ids": [], "w": [], "slots": []}
    recs = []
    pos = 0
    for t, B in enumerate(shapes):
        ids = ids_all[pos:pos + L * B].reshape(L, B, k)
        w = w_all[pos:pos + L * B].reshape(L, B, k)
        pos += L * B
        slots = np.empty_like(ids)
        sp = split if B <= HYBRID_MAX_TOKENS else None
        for l in range(L):
            s, r = cache.step(t, l, ids[l], sp) if sp else cache.step(t, l, ids[l])
            slots[l] = s.reshape(B, k)
            recs.append(r)
        out["ids"].append(ids)
        out["w"].append(w)
        out["slots"].append(slots)
    out["trace"] = np.concatenate(recs) if recs else np.empty(0, TRACE_DTYPE)
    out["counters"] = cache.counters()
    out["cache"] = cache
    return out
