"""ctypes binding of libmoecache (argument marshalling only).

Every step of the layer runs in the library; this module converts Python and
torch objects into the pointers and sizes of include/moe_cache.h.  There is no
fallback: when the library is missing, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libmoecache.so"

MISS_STREAM = 0
MISS_HOST = 1
_STATUS = {0: "MOE_OK", -1: "MOE_EINVAL", -2: "MOE_ENOMEM", -3: "MOE_EHIP", -4: "MOE_ESTATE"}


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class Opts(ctypes.Structure):
    _fields_ = [("top_k", ctypes.c_int32), ("miss_mode", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("norm_topk", ctypes.c_int32),
                ("host_threads", ctypes.c_int32), ("max_fills_per_call", ctypes.c_int32),
                ("keep_debug", ctypes.c_int32), ("timing", ctypes.c_int32),
                ("policy", ctypes.c_int32), ("preheat", ctypes.c_int32),
                ("adopt", ctypes.c_int32), ("reserved", ctypes.c_int32 * 5)]


class Stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in
                ("calls", "tokens", "selections", "hits", "misses", "unique", "fills", "fill_bytes",
                 "evictions", "host_selections", "stages")] + \
               [(n, ctypes.c_double) for n in ("plan_s", "h2d_s", "host_s", "gpu_s")]


class EvictRec(ctypes.Structure):
    _fields_ = [("call", ctypes.c_int64), ("stage", ctypes.c_int32), ("slot", ctypes.c_int32),
                ("evicted_expert", ctypes.c_int32), ("inserted_expert", ctypes.c_int32)]


_lib = None


def lib_path() -> str:
    return os.path.join(_HERE, LIB_NAME)


def load_library():
    """Loads the in-tree libmoecache.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m expert_cache_host_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "moe_cache_default_opts": (None, [ctypes.POINTER(Opts)]),
        "moe_cache_create": (I32, [I32, I32, I32, I32, I32, P, ctypes.POINTER(Opts), ctypes.POINTER(P)]),
        "moe_layer_forward": (I32, [P, I32, P, I32, P, P, P, P]),
        "moe_layer_forward_noalloc": (I32, [P, I32, P, I32, P, P, P, P]),
        "moe_cache_stats": (I32, [P, I32, ctypes.POINTER(Stats)]),
        "moe_cache_reset_stats": (I32, [P]),
        "moe_cache_set_timing": (I32, [P, I32]),
        "moe_cache_set_kernel_timing": (I32, [P, ctypes.c_uint32]),
        "moe_cache_kernel_stats": (I32, [P, I32, ctypes.POINTER(ctypes.c_int64),
                                         ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]),
        "moe_cache_sync": (I32, [P]),
        "moe_cache_destroy": (None, [P]),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_slot_bytes": (I64, [I32, I32]),
        "moe_debug_last_call": (I32, [P, I32, P, P]),
        "moe_debug_routing": (I32, [P, I32, P, P]),
        "moe_debug_views": (I32, [P, I32, I32, P, P]),
        "moe_debug_slots": (I32, [P, I32, P, P]),
        "moe_debug_scores": (I32, [P, I32, P]),
        "moe_debug_evictions": (I32, [P, I32, P, SZ, ctypes.POINTER(SZ)]),
        "moe_debug_partials": (I32, [P, I32, P, P]),
        "moe_debug_logits": (I32, [P, I32, P]),
        "moe_planner_create": (I32, [I32, I32, I32, I32, I32, ctypes.POINTER(P)]),
        "moe_planner_plan": (I32, [P, P, I32, I32, P, P, P]),
        "moe_planner_set_adopt": (I32, [P, I32]),
        "moe_planner_scores": (I32, [P, P]),
        "moe_planner_usage": (I32, [P, P]),
        "moe_planner_preload": (I32, [P, P]),
        "moe_cache_usage": (I32, [P, P]),
        "moe_cache_preload": (I32, [P, P]),
        "moe_planner_views": (I32, [P, I32, P, P]),
        "moe_planner_slots": (I32, [P, P, P]),
        "moe_planner_evictions": (I32, [P, P, SZ, ctypes.POINTER(SZ)]),
        "moe_planner_destroy": (None, [P]),
        "moe_debug_fill_delay": (I32, [P, I32]),
        "moe_debug_fail_alloc": (I32, [I32]),
        "moe_host_topk": (I32, [P, I32, I32, I32, I32, P, P]),
        "moe_host_expert_forward": (I32, [P, I32, I32, P, I32, P, I32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


POLICY_LRU, POLICY_SCORE = 0, 1


def _policy(name: str) -> int:
    if name not in ("lru", "score"):
        raise ValueError("policy must be 'lru' or 'score'")
    return POLICY_SCORE if name == "score" else POLICY_LRU


def _check(rc: int):
    if rc != 0:
        raise MoeError(rc, load_library().moe_last_error().decode(errors="replace"))


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def slot_bytes(d_model: int, d_ff: int) -> int:
    return int(load_library().moe_slot_bytes(d_model, d_ff))


def _evictions(fn, handle, *pre) -> list:
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check(fn(handle, *pre, None, 0, ctypes.byref(n)))
    buf = (EvictRec * max(1, n.value))()
    _check(fn(handle, *pre, buf, n.value, ctypes.byref(n)))
    del lib
    return [(r.call, r.stage, r.slot, r.evicted_expert, r.inserted_expert) for r in buf[:n.value]]


class MoECache:
    """One cache: layers x (slots + shared) device records over a pinned host arena."""

    def __init__(self, layers: int, n_experts: int, slots: int, d_model: int, d_ff: int,
                 host_weights: np.ndarray, top_k: int = 8, miss_mode: str = "stream",
                 n_shared: int = 0, norm_topk: bool = True, host_threads: int = 0,
                 max_fills_per_call: int = -1, keep_debug: bool = False, timing: bool = False,
                 policy: str = "lru", adopt: int = -1):
        """adopt: prefill preheat share of the slots per mille (0..1000), -1 = off."""
        lib = load_library()
        w = np.ascontiguousarray(host_weights, dtype=np.uint8)
        need = layers * (n_experts + n_shared) * (3 * d_model * d_ff // 32 * 18)
        if w.size < need:
            raise ValueError(f"host_weights holds {w.size} bytes, {need} needed")
        o = Opts()
        lib.moe_cache_default_opts(ctypes.byref(o))
        o.top_k = top_k
        o.miss_mode = MISS_HOST if miss_mode == "host" else MISS_STREAM
        o.n_shared = n_shared
        o.norm_topk = 1 if norm_topk else 0
        o.host_threads = host_threads
        o.max_fills_per_call = max_fills_per_call
        o.keep_debug = 1 if keep_debug else 0
        o.timing = 1 if timing else 0
        o.policy = _policy(policy)
        if adopt >= 0:
            o.preheat = 1
            o.adopt = adopt
        h = ctypes.c_void_p()
        _check(lib.moe_cache_create(layers, n_experts, slots, d_model, d_ff, _ptr(w), ctypes.byref(o),
                                    ctypes.byref(h)))
        self._h = h
        self.layers, self.n_experts, self.slots = layers, n_experts, slots
        self.d_model, self.d_ff, self.top_k, self.n_shared = d_model, d_ff, top_k, n_shared
        self.miss_mode = miss_mode
        self.policy = policy
        self.adopt = adopt

    # -- compute ---------------------------------------------------------------
    def forward(self, layer: int, x, router_w, router_bias=None, out=None, stream=None,
                noalloc: bool = False):
        """out [T, d] = layer(x) for torch float32 CUDA tensors (contiguous).
        noalloc: through moe_layer_forward_noalloc (the library's fixed scratch;
        `out` must then be given, since creating it would allocate)."""
        import torch
        if noalloc and out is None:
            raise ValueError("noalloc calls need a preallocated out")
        if out is None:
            out = torch.empty_like(x)
        for t in (x, router_w, out) + ((router_bias,) if router_bias is not None else ()):
            if not (t.is_cuda and t.dtype == torch.float32 and t.is_contiguous()):
                raise ValueError("tensors must be contiguous float32 on the GPU")
        if x.dim() != 2 or x.shape[1] != self.d_model or out.shape != x.shape:
            raise ValueError("x and out must be [T, d_model]")
        if tuple(router_w.shape) != (self.n_experts, self.d_model):
            raise ValueError("router_w must be [n_experts, d_model]")
        s = torch.cuda.current_stream() if stream is None else stream
        fn = load_library().moe_layer_forward_noalloc if noalloc else load_library().moe_layer_forward
        rc = fn(
            self._h, layer, x.data_ptr(), x.shape[0], router_w.data_ptr(),
            router_bias.data_ptr() if router_bias is not None else None, out.data_ptr(),
            s.cuda_stream)
        _check(rc)
        return out

    # -- counters and inspection -------------------------------------------------
    def stats(self, layer: int = -1) -> dict:
        st = Stats()
        _check(load_library().moe_cache_stats(self._h, layer, ctypes.byref(st)))
        return {n: getattr(st, n) for n, _ in Stats._fields_}

    KERNELS = ("router", "topk", "remap", "gateup", "down", "combine", "fill", "prep")

    def set_timing(self, on: bool):
        _check(load_library().moe_cache_set_timing(self._h, 1 if on else 0))

    def set_kernel_timing(self, kernels):
        """Times only the named kernels (names from KERNELS) from now on."""
        mask = 0
        for k in kernels:
            mask |= 1 << self.KERNELS.index(k)
        _check(load_library().moe_cache_set_kernel_timing(self._h, mask))

    def kernel_stats(self) -> dict:
        """{kernel: (launches, device seconds, algorithmic bytes)} while timing was on."""
        out = {}
        for i, name in enumerate(self.KERNELS):
            n, sec, by = ctypes.c_int64(), ctypes.c_double(), ctypes.c_double()
            _check(load_library().moe_cache_kernel_stats(self._h, i, ctypes.byref(n), ctypes.byref(sec),
                                                         ctypes.byref(by)))
            out[name] = (n.value, sec.value, by.value)
        return out

    def reset_stats(self):
        _check(load_library().moe_cache_reset_stats(self._h))

    def sync(self):
        _check(load_library().moe_cache_sync(self._h))

    def last_call(self, layer: int):
        ns, nt = ctypes.c_int32(), ctypes.c_int32()
        _check(load_library().moe_debug_last_call(self._h, layer, ctypes.byref(ns), ctypes.byref(nt)))
        return ns.value, nt.value

    def routing(self, layer: int):
        _, t = self.last_call(layer)
        idx = np.empty((t, self.top_k), np.int32)
        w = np.empty((t, self.top_k), np.float32)
        _check(load_library().moe_debug_routing(self._h, layer, _ptr(idx), _ptr(w)))
        return idx, w

    def views(self, layer: int, stage: int):
        sv = np.empty(self.n_experts, np.int32)
        hv = np.empty(self.n_experts, np.int32)
        _check(load_library().moe_debug_views(self._h, layer, stage, _ptr(sv), _ptr(hv)))
        return sv, hv

    def slot_state(self, layer: int):
        ein = np.empty(self.slots, np.int32)
        lu = np.empty(self.slots, np.uint64)
        _check(load_library().moe_debug_slots(self._h, layer, _ptr(ein), _ptr(lu)))
        return ein, lu

    def evictions(self, layer: int) -> list:
        return _evictions(load_library().moe_debug_evictions, self._h, layer)

    def scores(self, layer: int) -> np.ndarray:
        sc = np.empty(self.n_experts, np.float64)
        _check(load_library().moe_debug_scores(self._h, layer, _ptr(sc)))
        return sc

    def usage(self) -> np.ndarray:
        """Lifetime selection counts [layers, n_experts] (uint32)."""
        u = np.empty((self.layers, self.n_experts), np.uint32)
        _check(load_library().moe_cache_usage(self._h, _ptr(u)))
        return u

    def preload(self, counts):
        """Puts each layer's most-used experts (counts [layers, n_experts]) in its slots."""
        a = np.ascontiguousarray(counts, dtype=np.uint32)
        if a.shape != (self.layers, self.n_experts):
            raise ValueError("counts must be [layers, n_experts]")
        _check(load_library().moe_cache_preload(self._h, _ptr(a)))

    def partials(self, layer: int):
        _, t = self.last_call(layer)
        g = np.empty((t, self.d_model), np.float32)
        h = np.empty((t, self.d_model), np.float32)
        _check(load_library().moe_debug_partials(self._h, layer, _ptr(g), _ptr(h)))
        return g, h

    def logits(self, layer: int):
        _, t = self.last_call(layer)
        z = np.empty((t, self.n_experts), np.float32)
        _check(load_library().moe_debug_logits(self._h, layer, _ptr(z)))
        return z

    def close(self):
        if getattr(self, "_h", None):
            load_library().moe_cache_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Planner:
    """The library's per-layer slot planner alone (host only, no GPU)."""

    def __init__(self, n_experts: int, slots: int, miss_mode: str = "stream",
                 max_fills_per_call: int = -1, policy: str = "lru", adopt: int = -1):
        h = ctypes.c_void_p()
        _check(load_library().moe_planner_create(n_experts, slots,
                                                 MISS_HOST if miss_mode == "host" else MISS_STREAM,
                                                 max_fills_per_call, _policy(policy),
                                                 ctypes.byref(h)))
        self._h = h
        if adopt != -1:
            _check(load_library().moe_planner_set_adopt(h, adopt))
        self.n_experts, self.slots = n_experts, slots

    def plan(self, idx, tokens: int = 1):
        a = np.ascontiguousarray(idx, dtype=np.int32).ravel()
        ns, hi, mi = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(load_library().moe_planner_plan(self._h, _ptr(a), a.size, tokens, ctypes.byref(ns),
                                               ctypes.byref(hi), ctypes.byref(mi)))
        return ns.value, hi.value, mi.value

    def scores(self) -> np.ndarray:
        sc = np.empty(self.n_experts, np.float64)
        _check(load_library().moe_planner_scores(self._h, _ptr(sc)))
        return sc

    def usage(self) -> np.ndarray:
        u = np.empty(self.n_experts, np.uint32)
        _check(load_library().moe_planner_usage(self._h, _ptr(u)))
        return u

    def preload(self, counts):
        a = np.ascontiguousarray(counts, dtype=np.uint32)
        if a.shape != (self.n_experts,):
            raise ValueError("counts must be [n_experts]")
        _check(load_library().moe_planner_preload(self._h, _ptr(a)))

    def views(self, stage: int):
        sv = np.empty(self.n_experts, np.int32)
        hv = np.empty(self.n_experts, np.int32)
        _check(load_library().moe_planner_views(self._h, stage, _ptr(sv), _ptr(hv)))
        return sv, hv

    def slot_state(self):
        ein = np.empty(self.slots, np.int32)
        lu = np.empty(self.slots, np.uint64)
        _check(load_library().moe_planner_slots(self._h, _ptr(ein), _ptr(lu)))
        return ein, lu

    def evictions(self) -> list:
        return _evictions(load_library().moe_planner_evictions, self._h)

    def close(self):
        if getattr(self, "_h", None):
            load_library().moe_planner_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def host_expert_forward(expert_q4: np.ndarray, d_model: int, d_ff: int, x: np.ndarray,
                        threads: int = 0) -> np.ndarray:
    """y [T, d] of one expert (interchange bytes) on host cores."""
    e = np.ascontiguousarray(expert_q4, dtype=np.uint8)
    xx = np.ascontiguousarray(x, dtype=np.float32)
    if xx.ndim != 2 or xx.shape[1] != d_model:
        raise ValueError("x must be [T, d_model]")
    y = np.empty_like(xx)
    _check(load_library().moe_host_expert_forward(_ptr(e), d_model, d_ff, _ptr(xx), xx.shape[0],
                                                  _ptr(y), threads))
    return y


def host_topk(z: np.ndarray, top_k: int, norm_topk: bool = True):
    """(idx [T, k] int32, w [T, k] float32): the host's selection on logits z [T, E]."""
    zz = np.ascontiguousarray(z, dtype=np.float32)
    if zz.ndim != 2:
        raise ValueError("z must be [T, E]")
    idx = np.empty((zz.shape[0], top_k), np.int32)
    w = np.empty((zz.shape[0], top_k), np.float32)
    _check(load_library().moe_host_topk(_ptr(zz), zz.shape[0], zz.shape[1], top_k,
                                        1 if norm_topk else 0, _ptr(idx), _ptr(w)))
    return idx, w
