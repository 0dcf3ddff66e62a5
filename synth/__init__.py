"""Seeded synthetic workloads for the routed-MoE expert-cache layer.

This package produces INPUTS only (Q4_0 expert bytes, router matrices and
biases, hidden states) and is the one input source that both the oracle side
and the library side use.  It holds none of the layer's arithmetic.

Workloads (shapes follow the pages; values are synthetic):

* tiny      -- 1 layer, d=256, f=512, 8 experts, top-2, 4 slots, 64 decode
               tokens (the small case of the first expert-cache pull request).
* gemma     -- 30 layers, d=2816, f=704, 128 experts, top-8, 32 slots, 512 decode
               tokens; the Gemma 4 26B-A4B shape of the laptop-GPU fork
               ("How it works": 30 layers x 128 experts of ~3.35 MB, top-8).
* qwen      -- 48 layers, d=2048, f=768, 128 experts, top-8, 16 slots, batches of
               1, 2 or 4 independent streams x 256 steps.
* large     -- 8 layers, d=6144, f=2048, 256 routed experts + 1 resident shared
               expert, top-8, 64 slots, 256 decode tokens, misses on host cores.
* prefill   -- the `large` layer shape, a 12288-token prompt in ubatches of 512,
               i.i.d. N(0,1) hidden states, routed experts streamed into slots.

Recipe (the pages give none; these are the plainest readings):

* expert weights ~ N(0, 0.02^2), quantised per 32-weight block (q4gen.c);
* router W_r ~ N(0, sigma_r^2) with sigma_r = 0.1 at d=256 and 1.6/sqrt(d)
  otherwise (same logit variance); Zipf skew as a per-expert bias
  b_e = -s * ln(rank_e), rank_e a seeded permutation of 1..E;
* hidden states: AR(1), x_t = rho * x_{t-1} + eps_t, eps ~ N(0, 1), stationary
  start x_0 ~ N(0, 1 / (1 - rho^2)); i.i.d. N(0, 1) for the prefill workload;
* every stream is seeded by numpy SeedSequence([workload id, layer, purpose]).
"""
from __future__ import annotations

import ctypes
import math
import os
import statistics
import subprocess
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "_q4gen.so")
_SRC = os.path.join(_HERE, "q4gen.c")

PURPOSE_X = 0
PURPOSE_ROUTER = 1
PURPOSE_BIAS = 2


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int                 # workload id used in every seed
    layers: int
    d_model: int
    d_ff: int
    n_experts: int
    top_k: int
    slots: int
    n_shared: int = 0
    sigma_w: float = 0.02
    router_sigma: float = 0.0
    zipf_s: Optional[float] = None
    rho: Optional[float] = 0.8   # None -> i.i.d. N(0,1) hidden states
    tokens: int = 1              # tokens per stream
    batch: int = 1               # tokens per call (independent streams or ubatch)
    miss_mode: str = "stream"
    weight_wid: Optional[int] = None  # reuse another workload's expert bytes and router
    modes: tuple = field(default=("stream",))

    @property
    def expert_bytes(self) -> int:
        return expert_bytes(self.d_model, self.d_ff)

    @property
    def n_total_experts(self) -> int:
        return self.n_experts + self.n_shared

    @property
    def layer_bytes(self) -> int:
        return self.n_total_experts * self.expert_bytes

    @property
    def total_bytes(self) -> int:
        return self.layers * self.layer_bytes

    @property
    def calls_per_layer(self) -> int:
        if self.rho is None:
            return self.tokens // self.batch
        return self.tokens


def expert_bytes(d_model: int, d_ff: int) -> int:
    """Bytes of one expert in 18-byte / 32-weight blocks: gate, up and down."""
    return 3 * d_model * d_ff // 32 * 18


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 256, 512, 8, 2, 4, router_sigma=0.1, rho=0.8,
                     tokens=64, batch=1, modes=("stream", "host")),
    "gemma": Workload("gemma", 2, 30, 2816, 704, 128, 8, 32,
                      router_sigma=1.6 / math.sqrt(2816), zipf_s=1.1, rho=0.8,
                      tokens=512, batch=1, miss_mode="host", modes=("host", "stream")),
    "qwen": Workload("qwen", 3, 48, 2048, 768, 128, 8, 16,
                     router_sigma=1.6 / math.sqrt(2048), zipf_s=1.0, rho=0.7,
                     tokens=256, batch=1, miss_mode="host", modes=("host", "stream")),
    "large": Workload("large", 4, 8, 6144, 2048, 256, 8, 64, n_shared=1,
                      router_sigma=1.6 / math.sqrt(6144), zipf_s=1.2, rho=0.8,
                      tokens=256, batch=1, miss_mode="host", modes=("host",)),
    "prefill": Workload("prefill", 5, 8, 6144, 2048, 256, 8, 64, n_shared=1,
                        router_sigma=1.6 / math.sqrt(6144), zipf_s=None, rho=None,
                        tokens=12288, batch=512, weight_wid=4),
}


def qwen_batch(b: int) -> Workload:
    """The qwen workload with `b` independent streams per call (b in 1, 2, 4)."""
    base = WORKLOADS["qwen"]
    return Workload(**{**base.__dict__, "name": f"qwen_b{b}", "batch": b})


# ---------------------------------------------------------------- native helper

_lib = None
_table = None


def build(force: bool = False) -> str:
    """Compile q4gen.c with gcc into an in-tree shared object."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_SO)
        lib.q4gen_experts.restype = ctypes.c_int
        lib.q4gen_experts.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p,
                                      ctypes.c_int]
        lib.q4gen_values.restype = ctypes.c_int
        lib.q4gen_values.argtypes = lib.q4gen_experts.argtypes
        _lib = lib
    return _lib


def normal_table() -> np.ndarray:
    """Inverse normal CDF at the 65536 midpoints (u + 0.5) / 65536, float32."""
    global _table
    if _table is None:
        nd = statistics.NormalDist()
        _table = np.array([nd.inv_cdf((u + 0.5) / 65536.0) for u in range(65536)], dtype=np.float32)
    return _table


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _weight_seed(wl: Workload, layer: int) -> int:
    wid = wl.weight_wid or wl.wid
    return (wid << 40) | (layer << 8) | 0x5A


def gen_experts(wl: Workload, layer: int, e_begin: int = 0, e_end: Optional[int] = None,
                out: Optional[np.ndarray] = None, threads: Optional[int] = None) -> np.ndarray:
    """Q4_0 bytes of experts [e_begin, e_end) of `layer` (ids >= n_experts are shared)."""
    if e_end is None:
        e_end = wl.n_total_experts
    n = (e_end - e_begin) * wl.expert_bytes
    if out is None:
        out = np.empty(n, dtype=np.uint8)
    if out.dtype != np.uint8 or out.size < n or not out.flags["C_CONTIGUOUS"]:
        raise ValueError("out must be a contiguous uint8 array of the right size")
    tab = normal_table()
    rc = _load().q4gen_experts(out.ctypes.data, _weight_seed(wl, layer), e_begin, e_end,
                               wl.d_model, wl.d_ff, wl.sigma_w, tab.ctypes.data,
                               threads or default_threads())
    if rc != 0:
        raise RuntimeError("q4gen_experts failed")
    return out[:n]


def gen_values(wl: Workload, layer: int, e_begin: int = 0, e_end: Optional[int] = None,
               threads: Optional[int] = None) -> np.ndarray:
    """The unquantised float32 values behind gen_experts (3*d*f per expert)."""
    if e_end is None:
        e_end = wl.n_total_experts
    out = np.empty((e_end - e_begin) * 3 * wl.d_model * wl.d_ff, dtype=np.float32)
    rc = _load().q4gen_values(out.ctypes.data, _weight_seed(wl, layer), e_begin, e_end,
                              wl.d_model, wl.d_ff, wl.sigma_w, normal_table().ctypes.data,
                              threads or default_threads())
    if rc != 0:
        raise RuntimeError("q4gen_values failed")
    return out


def gen_all_weights(wl: Workload, out: Optional[np.ndarray] = None,
                    threads: Optional[int] = None) -> np.ndarray:
    """Interchange bytes of every layer: [layer][expert (routed, then shared)][gate|up|down]."""
    if out is None:
        out = np.empty(wl.total_bytes, dtype=np.uint8)
    for l in range(wl.layers):
        gen_experts(wl, l, out=out[l * wl.layer_bytes:(l + 1) * wl.layer_bytes], threads=threads)
    return out


def _rng(wl_id: int, layer: int, purpose: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([wl_id, layer, purpose]))


def gen_router(wl: Workload, layer: int):
    """Router matrix W_r [E, d] float32 and bias [E] float32 (or None)."""
    wid = wl.weight_wid or wl.wid
    w = (_rng(wid, layer, PURPOSE_ROUTER).standard_normal((wl.n_experts, wl.d_model))
         * wl.router_sigma).astype(np.float32)
    bias = None
    if wl.zipf_s is not None:
        rank = _rng(wl.wid, layer, PURPOSE_BIAS).permutation(wl.n_experts) + 1
        bias = (-wl.zipf_s * np.log(rank.astype(np.float64))).astype(np.float32)
    return w, bias


def gen_hidden(wl: Workload, layer: int, n_calls: Optional[int] = None) -> np.ndarray:
    """Hidden states [n_calls, batch, d] float32 for `layer`.

    AR(1) workloads: `batch` independent streams, call t holds step t of every
    stream.  i.i.d. workloads: call t holds tokens [t*batch, (t+1)*batch).
    """
    total = wl.calls_per_layer if n_calls is None else n_calls
    rng = _rng(wl.wid, layer, PURPOSE_X)
    d = wl.d_model
    if wl.rho is None:
        return rng.standard_normal((total, wl.batch, d), dtype=np.float32)
    rho = wl.rho
    x = np.empty((total, wl.batch, d), dtype=np.float64)
    cur = rng.standard_normal((wl.batch, d)) / math.sqrt(1.0 - rho * rho)
    x[0] = cur
    for t in range(1, total):
        cur = rho * cur + rng.standard_normal((wl.batch, d))
        x[t] = cur
    return x.astype(np.float32)
