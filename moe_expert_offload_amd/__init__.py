"""Python binding of libmoe.so: decode-time MoE layers over a router-following
LRU cache of expert slots on an MI355X (gfx950).

Argument marshalling only: every step of the path runs in the HIP library
(see ``include/moe.h`` for the C ABI).  PyTorch provides device memory and
streams.  Importing this package fails loudly when the library is missing.
"""
from __future__ import annotations

import ctypes
import os

# PyTorch ships its own HIP runtime with the same soname (libamdhip64.so.7) as the system one.
# Import it first so the dynamic loader binds libmoe.so to that runtime: the streams and device
# pointers torch hands over are only valid inside the runtime that created them.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it first (python -m moe_expert_offload_amd.build "
        "or __graft_entry__.build())")

_lib = ctypes.CDLL(LIB_PATH)

MOE_OK, MOE_EINVAL, MOE_ENOMEM, MOE_EHIP, MOE_ECAPACITY, MOE_ESTATE, MOE_EVERIFY = 0, -1, -2, -3, -4, -5, -6
MOE_FLAG_PROFILE = 1
MOE_FLAG_PER_TOKEN_FFN = 2
MOE_FLAG_VERIFY = 4
MOE_POLICY_LRU, MOE_POLICY_STATIC = 0, 1
_STATUS = {0: "MOE_OK", -1: "MOE_EINVAL", -2: "MOE_ENOMEM", -3: "MOE_EHIP", -4: "MOE_ECAPACITY",
           -5: "MOE_ESTATE", -6: "MOE_EVERIFY"}


class MoeConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "n_experts", "top_k", "hidden", "inter", "n_shared", "cache_slots", "max_tokens",
        "lookahead", "trace_capacity", "fill_threads", "flags", "pinned_mb", "policy")]


class MoeCounters(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "hits", "misses", "evictions", "resolves", "h2d_bytes", "h2d_copies", "trace_records",
        "trace_dropped", "ffn_launches", "h2d_bounced", "pool_pinned_bytes")] + [
        ("k3_ms", ctypes.c_double), ("k4_ms", ctypes.c_double),
        ("host_experts", ctypes.c_uint64), ("host_tasks", ctypes.c_uint64),
        ("host_busy_ms", ctypes.c_double), ("host_wait_ms", ctypes.c_double),
        ("h2d_ns", ctypes.c_uint64), ("ffn_ns", ctypes.c_uint64), ("ffn_timed", ctypes.c_uint64),
        ("h2d_timed_bytes", ctypes.c_uint64)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class MoeTraceRec(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("step", "layer", "expert", "slot", "hit", "evicted_key")]


FILL_FN = ctypes.CFUNCTYPE(None, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_uint8))

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_st = ctypes.c_int

_lib.moe_query_sizes.restype = _st
_lib.moe_query_sizes.argtypes = [ctypes.POINTER(MoeConfig), ctypes.POINTER(ctypes.c_size_t),
                                 ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
_lib.moe_auto_cache_slots.restype = _st
_lib.moe_auto_cache_slots.argtypes = [ctypes.POINTER(MoeConfig), ctypes.c_uint64, ctypes.c_uint64,
                                      ctypes.POINTER(_I32)]
_lib.moe_init_pool.restype = _st
_lib.moe_pack_blob.restype = _st
_lib.moe_pack_blob.argtypes = [ctypes.POINTER(MoeConfig), _P, _P]
_lib.moe_host_expert_ffn.restype = _st
_lib.moe_host_expert_ffn.argtypes = [ctypes.POINTER(MoeConfig), _P, _P, _I32, _P, _P, _I32]
_lib.moe_host_expert_batch.restype = _st
_lib.moe_host_expert_batch.argtypes = [ctypes.POINTER(MoeConfig), _I32, _P, _P, _P, _P, _P, _I32, _I32]
_lib.moe_hybrid_split.restype = _I32
_lib.moe_hybrid_split.argtypes = [_I32, ctypes.c_double, ctypes.c_double]
_lib.moe_set_backend.restype = _st
_lib.moe_set_backend.argtypes = [_P, _I32, ctypes.c_double, ctypes.c_double, _I32]
_lib.moe_select_backend.restype = _I32
_lib.moe_select_backend.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_double]
_lib.moe_calibrate_backend.restype = _st
_lib.moe_calibrate_backend.argtypes = [_P, _I32, ctypes.c_double, ctypes.c_double, ctypes.c_void_p]
_lib.moe_init_pool.argtypes = [ctypes.POINTER(MoeConfig), _P, _P, _P, _P, ctypes.c_size_t, _P,
                               ctypes.c_size_t, _P, _P, ctypes.POINTER(_P)]
_lib.moe_cache_resolve.restype = _st
_lib.moe_cache_resolve.argtypes = [_P, _I32, _I32, _P, _I32, _P, ctypes.POINTER(_I32)]
_lib.moe_layer_forward.restype = _st
_lib.moe_layer_forward.argtypes = [_P, _I32, _I32, _P, _I32, _P, _P, _P]
_lib.moe_stack_forward.restype = _st
_lib.moe_stack_forward.argtypes = [_P, _I32, _P, ctypes.c_int64, _I32, _P, ctypes.c_int64, _P, _P]
_lib.moe_expert_forward.restype = _st
_lib.moe_expert_forward.argtypes = [_P, _I32, _P, _I32, _P, _P, _P]
_lib.moe_router_logits.restype = _st
_lib.moe_router_logits.argtypes = [_P, _I32, _P, _I32, _P]
_lib.moe_expert_forward_noalloc.restype = _st
_lib.moe_expert_forward_noalloc.argtypes = [ctypes.POINTER(MoeConfig), _P, _P, _P, _I32, _P, _P, _P, _P]
_lib.moe_stats.restype = _st
_lib.moe_stats.argtypes = [_P, ctypes.POINTER(MoeCounters), _P, ctypes.c_size_t, ctypes.POINTER(ctypes.c_size_t)]
_lib.moe_measure_h2d.restype = _st
_lib.moe_measure_h2d.argtypes = [_P, ctypes.c_size_t, _I32, ctypes.POINTER(ctypes.c_double)]
_lib.moe_hbm_read.restype = _st
_lib.moe_hbm_read.argtypes = [_P, ctypes.c_size_t, _P]
_lib.moe_cache_state.restype = _st
_lib.moe_cache_state.argtypes = [_P, _P, _P, _P]
_lib.moe_destroy.restype = None
_lib.moe_destroy.argtypes = [_P]
_lib.moe_last_error.restype = ctypes.c_char_p
_lib.moe_last_error.argtypes = [_P]

EXPORTED = ("moe_query_sizes", "moe_auto_cache_slots", "moe_pack_blob", "moe_host_expert_ffn", "moe_host_expert_batch",
            "moe_hybrid_split",
            "moe_select_backend", "moe_calibrate_backend", "moe_set_backend", "moe_init_pool", "moe_cache_resolve", "moe_layer_forward", "moe_stack_forward",
            "moe_expert_forward", "moe_expert_forward_noalloc", "moe_router_logits", "moe_stats", "moe_measure_h2d", "moe_hbm_read", "moe_cache_state", "moe_destroy", "moe_last_error")


class MoeError(RuntimeError):
    def __init__(self, status, msg=""):
        self.status = status
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")


def lib():
    return _lib


def make_config(n_layers, n_experts, top_k, hidden, inter, n_shared, cache_slots, max_tokens,
                lookahead=1, trace_capacity=0, fill_threads=0, flags=0, pinned_mb=0, policy=0) -> MoeConfig:
    return MoeConfig(n_layers, n_experts, top_k, hidden, inter, n_shared, cache_slots, max_tokens,
                     lookahead, trace_capacity, fill_threads, flags, pinned_mb, policy)


def query_sizes(cfg: MoeConfig):
    b, a, w = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    st = _lib.moe_query_sizes(ctypes.byref(cfg), ctypes.byref(b), ctypes.byref(a), ctypes.byref(w))
    if st:
        raise MoeError(st, "moe_query_sizes")
    return b.value, a.value, w.value


def auto_cache_slots(cfg: MoeConfig, free_bytes: int = 0, reserve_bytes: int = 0) -> int:
    """Largest cache_slots that fits the device memory left (moe_auto_cache_slots).

    free_bytes 0 asks the runtime for the current device's free memory."""
    out = _I32()
    st = _lib.moe_auto_cache_slots(ctypes.byref(cfg), free_bytes, reserve_bytes, ctypes.byref(out))
    if st:
        raise MoeError(st, f"moe_auto_cache_slots (fits {out.value} slots)")
    return out.value


MOE_BACKEND_OFFLOAD, MOE_BACKEND_HYBRID = 0, 1


class MoeBwProfile(ctypes.Structure):
    _fields_ = [("pcie_gbps", ctypes.c_double), ("host_gbps", ctypes.c_double), ("ratio", ctypes.c_double),
                ("threshold", ctypes.c_double), ("host_threads", _I32), ("backend", _I32),
                ("host_isa", ctypes.c_char * 16)]


def pack_blob(cfg: MoeConfig, logical):
    """Logical expert blob (numpy uint8) -> the pool's layout (moe_pack_blob)."""
    import numpy as np
    src = np.ascontiguousarray(logical, dtype=np.uint8)
    dst = np.empty_like(src)
    st = _lib.moe_pack_blob(ctypes.byref(cfg), src.ctypes.data, dst.ctypes.data)
    if st:
        raise MoeError(st, "moe_pack_blob")
    return dst


def host_expert_ffn(cfg: MoeConfig, packed_blobs, w, x, threads=1):
    """Host expert kernel (moe_host_expert_ffn): float32 [H] = sum_j w[j] * FFN_j(x)."""
    import numpy as np
    blobs = [np.ascontiguousarray(b, dtype=np.uint8) for b in packed_blobs]
    ptrs = (ctypes.c_void_p * max(len(blobs), 1))(*[b.ctypes.data for b in blobs])
    wv = np.ascontiguousarray(w, dtype=np.float32)
    xv = np.ascontiguousarray(x, dtype=np.uint16)
    y = np.empty(cfg.hidden, dtype=np.float32)
    st = _lib.moe_host_expert_ffn(ctypes.byref(cfg), ptrs, wv.ctypes.data, len(blobs), xv.ctypes.data,
                                  y.ctypes.data, threads)
    if st:
        raise MoeError(st, "moe_host_expert_ffn")
    return y


def host_expert_batch(cfg: MoeConfig, packed_blobs, w, tok, x, threads=1):
    """The hybrid backend's host workers on one task (moe_host_expert_batch): x bf16 bits
    [n_tok][H]; returns float32 [n_tok][H], row b = the sum over the entries j with tok[j] == b,
    in order, of w[j] * FFN_j(x[b])."""
    import numpy as np
    blobs = [np.ascontiguousarray(b, dtype=np.uint8) for b in packed_blobs]
    ptrs = (ctypes.c_void_p * max(len(blobs), 1))(*[b.ctypes.data for b in blobs])
    wv = np.ascontiguousarray(w, dtype=np.float32)
    tv = np.ascontiguousarray(tok, dtype=np.int32)
    xv = np.ascontiguousarray(x, dtype=np.uint16)
    if xv.ndim != 2 or xv.shape[1] != cfg.hidden or len(wv) != len(blobs) or len(tv) != len(blobs):
        raise ValueError("x must be [n_tok][hidden]; w and tok one per blob")
    y = np.empty(xv.shape, dtype=np.float32)
    st = _lib.moe_host_expert_batch(ctypes.byref(cfg), xv.shape[0], xv.ctypes.data, y.ctypes.data, ptrs,
                                    wv.ctypes.data, tv.ctypes.data, len(blobs), threads)
    if st:
        raise MoeError(st, "moe_host_expert_batch")
    return y


def select_backend(pcie_gbps: float, host_gbps: float, threshold: float = 2.0) -> str:
    """The auto rule (moe_select_backend): "hybrid" or "offload"."""
    return "hybrid" if _lib.moe_select_backend(pcie_gbps, host_gbps, threshold) == MOE_BACKEND_HYBRID else "offload"


def hybrid_split(n_miss: int, pcie_gbps: float, host_gbps: float) -> int:
    """Misses that go over PCIe in the hybrid split (moe_hybrid_split)."""
    return int(_lib.moe_hybrid_split(n_miss, pcie_gbps, host_gbps))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


NOALLOC_SCRATCH_BYTES = 1 << 20
NOALLOC_MAX_TOKENS = 16


def expert_forward_noalloc(cfg: MoeConfig, arena, shared_blob, x, slots, w, y, stream=None):
    """moe_expert_forward_noalloc: the expert FFN on caller slots with no context and no device
    allocation (device tensors; stream: a torch stream or None for the current one)."""
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    st = _lib.moe_expert_forward_noalloc(ctypes.byref(cfg), _ptr(arena), _ptr(shared_blob), _ptr(x), x.shape[0],
                                         _ptr(slots), _ptr(w), _ptr(y), ctypes.c_void_p(s.cuda_stream))
    if st:
        raise MoeError(st, "moe_expert_forward_noalloc: " + _lib.moe_last_error(None).decode())


def hbm_read(buf, offset, nbytes, stream=None):
    """moe_hbm_read: one streaming-read launch over nbytes of the device tensor buf from byte
    offset (stream: a torch stream or None for the current one)."""
    import torch
    if offset < 0 or offset + nbytes > buf.numel() * buf.element_size():
        raise MoeError(MOE_EINVAL, "moe_hbm_read: range outside the buffer")
    s = stream if stream is not None else torch.cuda.current_stream()
    st = _lib.moe_hbm_read(ctypes.c_void_p(buf.data_ptr() + offset), nbytes, ctypes.c_void_p(s.cuda_stream))
    if st:
        raise MoeError(st, "moe_hbm_read")


class OffloadMoE:
    """One context: pinned expert pool, slot arena and workspace (torch device tensors), streams.

    fill: (function pointer int, user pointer int) of a C callback, or a Python callable
    fill(layer, expert, numpy_uint8_view) (slow; serialised by the GIL).
    router_w: host numpy uint16 array [L][E][H] (bf16 bits).
    cfg.cache_slots == 0 sizes the cache from the device memory left once the workspace is
    allocated (moe_auto_cache_slots), keeping auto_reserve_bytes free; self.cfg holds the result.
    """

    def __init__(self, cfg: MoeConfig, fill, router_w, device=None, compute_stream=None, copy_stream=None,
                 auto_reserve_bytes=2 << 30):
        import numpy as np
        import torch

        cfg = MoeConfig.from_buffer_copy(cfg)
        self.cfg = cfg
        self.torch = torch
        self.device = torch.device("cuda", torch.cuda.current_device() if device is None else device)
        self.blob_bytes, arena_bytes, ws_bytes = query_sizes(cfg)
        self.workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=self.device)
        if cfg.cache_slots == 0:
            with torch.cuda.device(self.device):
                torch.cuda.synchronize()
                cfg.cache_slots = auto_cache_slots(cfg, 0, auto_reserve_bytes)
            arena_bytes = cfg.cache_slots * self.blob_bytes
        self.arena = torch.empty(arena_bytes, dtype=torch.uint8, device=self.device)
        self.compute_stream = compute_stream or torch.cuda.Stream(device=self.device)
        self.copy_stream = copy_stream or torch.cuda.Stream(device=self.device)
        rw = np.ascontiguousarray(router_w, dtype=np.uint16)
        assert rw.shape == (cfg.n_layers, cfg.n_experts, cfg.hidden)
        self._keep = [rw]
        if callable(fill):
            n = self.blob_bytes

            def _cb(user, layer, expert, dst):
                buf = np.ctypeslib.as_array(dst, shape=(n,))
                fill(layer, expert, buf)

            cb = FILL_FN(_cb)
            self._keep.append(cb)
            fptr, uptr = ctypes.cast(cb, ctypes.c_void_p).value, None
        else:
            fptr, uptr = fill
        ctx = ctypes.c_void_p()
        torch.cuda.synchronize(self.device)
        st = _lib.moe_init_pool(ctypes.byref(cfg), fptr, uptr, rw.ctypes.data, _ptr(self.arena), arena_bytes,
                                _ptr(self.workspace), ws_bytes, ctypes.c_void_p(self.compute_stream.cuda_stream),
                                ctypes.c_void_p(self.copy_stream.cuda_stream), ctypes.byref(ctx))
        if st:
            raise MoeError(st, "moe_init_pool: " + _lib.moe_last_error(None).decode())
        self.ctx = ctx

    def _check(self, st, what):
        if st:
            raise MoeError(st, f"{what}: {_lib.moe_last_error(self.ctx).decode()}")

    def close(self):
        if getattr(self, "ctx", None):
            _lib.moe_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- calls (device tensors; all work is ordered on the compute stream) --
    def cache_resolve(self, step, layer, ids, slots=None):
        n = ctypes.c_int32()
        self._check(_lib.moe_cache_resolve(self.ctx, step, layer, _ptr(ids), ids.shape[0], _ptr(slots),
                                           ctypes.byref(n)), "moe_cache_resolve")
        return n.value

    def layer_forward(self, step, layer, x, y, ids=None, w=None):
        self._check(_lib.moe_layer_forward(self.ctx, step, layer, _ptr(x), x.shape[0], _ptr(y), _ptr(ids), _ptr(w)),
                    "moe_layer_forward")

    def stack_forward(self, step, x, x_layer_stride, n_tokens, y, y_layer_stride, ids=None, w=None):
        self._check(_lib.moe_stack_forward(self.ctx, step, _ptr(x), x_layer_stride, n_tokens, _ptr(y),
                                           y_layer_stride, _ptr(ids), _ptr(w)), "moe_stack_forward")

    def expert_forward(self, layer, x, slots, w, y):
        self._check(_lib.moe_expert_forward(self.ctx, layer, _ptr(x), x.shape[0], _ptr(slots), _ptr(w), _ptr(y)),
                    "moe_expert_forward")

    def router_logits(self, layer, x, z):
        """z [n][E] float32 device tensor <- the layer's router logits of x [n][H] (moe_router_logits)."""
        self._check(_lib.moe_router_logits(self.ctx, layer, _ptr(x), x.shape[0], _ptr(z)), "moe_router_logits")

    def set_backend(self, backend, pcie_gbps=0.0, host_gbps=0.0, host_threads=1):
        """backend "offload" or "hybrid" (moe_set_backend)."""
        b = {"offload": MOE_BACKEND_OFFLOAD, "hybrid": MOE_BACKEND_HYBRID}[backend]
        self._check(_lib.moe_set_backend(self.ctx, b, pcie_gbps, host_gbps, host_threads), "moe_set_backend")

    def calibrate_backend(self, host_threads, host_seconds=2.0, threshold=2.0):
        p = MoeBwProfile()
        self._check(_lib.moe_calibrate_backend(self.ctx, host_threads, host_seconds, threshold, ctypes.byref(p)),
                    "moe_calibrate_backend")
        return {"pcie_GBps": p.pcie_gbps, "host_GBps": p.host_gbps, "ratio": p.ratio, "threshold": p.threshold,
                "host_threads": p.host_threads, "host_isa": p.host_isa.decode(),
                "backend": "hybrid" if p.backend == MOE_BACKEND_HYBRID else "offload"}

    def stats(self, trace_cap=0):
        import numpy as np
        c = MoeCounters()
        buf = (MoeTraceRec * max(trace_cap, 1))()
        n = ctypes.c_size_t()
        self._check(_lib.moe_stats(self.ctx, ctypes.byref(c), ctypes.cast(buf, ctypes.c_void_p) if trace_cap else None,
                                   trace_cap, ctypes.byref(n)), "moe_stats")
        dt = np.dtype([(f, np.int32) for f in ("step", "layer", "expert", "slot", "hit", "evicted_key")])
        recs = np.frombuffer(bytes(buf), dtype=dt, count=n.value).copy() if trace_cap else np.empty(0, dt)
        return c.as_dict(), recs

    def measure_h2d(self, bytes_per_copy, n_copies):
        g = ctypes.c_double()
        self._check(_lib.moe_measure_h2d(self.ctx, bytes_per_copy, n_copies, ctypes.byref(g)), "moe_measure_h2d")
        return g.value

    def cache_state(self):
        import numpy as np
        cfg = self.cfg
        slot_of = np.empty(cfg.n_layers * cfg.n_experts, np.int32)
        key_of = np.empty(cfg.cache_slots, np.int32)
        stamp = np.empty(cfg.cache_slots, np.int64)
        self._check(_lib.moe_cache_state(self.ctx, slot_of.ctypes.data, key_of.ctypes.data, stamp.ctypes.data),
                    "moe_cache_state")
        return slot_of, key_of, stamp
