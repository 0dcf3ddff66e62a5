"""Router logits, top-k selection and gating weights (oracle side).

The router picks k experts per token per layer ("How it works", llama.cpp + MoE
expert cache, step 1); the expert weights are applied after the partial results
are added (step 4).  The pages fix neither the precision nor the summation
order, nor the tie rule, nor the form of the gating weights.  Readings taken:

* logits in fp32, in one fixed order (router_logits_fp32) so that a GPU
  implementation can reproduce every top-k decision bit for bit;
* top-k on the biased logits, ordered by (-z, expert id): ties go to the lower id;
* gating weights: softmax over all E biased logits, renormalised over the k
  selected (norm_topk=True) or kept as they are (norm_topk=False); fp64.
"""
from __future__ import annotations

import numpy as np

LANES = 64


def router_logits_fp32(x: np.ndarray, w: np.ndarray, bias=None) -> np.ndarray:
    """z[t, e] = x[t] . w[e] + bias[e] in fp32, in this order:

    1. 64 lane partials p[l], all 0;
    2. for i = l, l+64, l+128, ... ascending: p[l] = fl(p[l] + fl(x[t,i] * w[e,i]))
       (product and sum rounded separately, no fused multiply-add);
    3. for off = 32, 16, 8, 4, 2, 1: p[l] = fl(p[l] + p[l + off]) for l < off;
    4. z = fl(p[0] + bias[e]).
    Round to nearest even, subnormals kept.  Requires d % 64 == 0.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    t, d = x.shape
    e, d2 = w.shape
    if d != d2 or d % LANES:
        raise ValueError("x and w need the same d, a multiple of 64")
    xs = x.reshape(t, d // LANES, LANES)
    ws = w.reshape(e, d // LANES, LANES)
    p = np.zeros((t, e, LANES), dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        for m in range(d // LANES):
            prod = xs[:, None, m, :] * ws[None, :, m, :]
            p = p + prod
        off = LANES // 2
        while off >= 1:
            p[..., :off] = p[..., :off] + p[..., off:2 * off]
            off //= 2
        z = p[..., 0].copy()
        if bias is not None:
            z = z + np.asarray(bias, dtype=np.float32)[None, :]
    return z


def topk(z: np.ndarray, k: int) -> np.ndarray:
    """First k experts of each row in (-z, expert id) order, int32 [T, k]."""
    z = np.asarray(z, dtype=np.float32)
    t, e = z.shape
    if not 1 <= k <= e:
        raise ValueError("k must be in [1, E]")
    if not np.all(np.isfinite(z)):
        raise ValueError("non-finite logit")
    ids = np.arange(e)
    out = np.empty((t, k), dtype=np.int32)
    for r in range(t):
        order = np.lexsort((ids, -z[r].astype(np.float64)))
        out[r] = order[:k]
    return out


def gate_weights(z: np.ndarray, idx: np.ndarray, norm_topk: bool = True) -> np.ndarray:
    """Softmax over all E logits at the selected ids, optionally renormalised; fp64."""
    z64 = np.asarray(z, dtype=np.float64)
    m = z64.max(axis=1, keepdims=True)
    ez = np.exp(z64 - m)
    p = ez / ez.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, np.asarray(idx, dtype=np.int64), axis=1)
    if norm_topk:
        sel = sel / sel.sum(axis=1, keepdims=True)
    return sel
