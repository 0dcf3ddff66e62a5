"""The full routed-MoE layer over all experts (oracle side).

The cache changes where each selected expert is computed, never the result:
every selected expert is computed exactly once, on the GPU or on the host, the
partial results are added and the gating weights applied ("How it works",
llama.cpp + MoE expert cache, steps 1-4 and the note above "Quick start").  So
the oracle is the plain layer with every routed expert evaluated from the
interchange bytes, independent of slots, cache state and miss mode:

    out[t] = sum_j w[t, j] * y_{idx[t, j]}(x_t) + sum_s y_shared_s(x_t)

Shared experts are always resident and enter with weight 1 (longhaul.md keeps
shared experts resident and streams only the routed banks; their weight is not
stated -- reading taken: 1).  Sums in fp64, rounded to fp32 at the end.
"""
from __future__ import annotations

import numpy as np

from .expert import expert_hidden
from .q4 import BLOCK, BLOCK_BYTES, decode_matrix, expert_nbytes
from .routing import gate_weights, router_logits_fp32, topk


def _expert_parts(layer_buf, e, d_model, d_ff, out_cols=None):
    eb = expert_nbytes(d_model, d_ff)
    gu = d_ff * d_model // BLOCK * BLOCK_BYTES
    b = np.asarray(layer_buf, dtype=np.uint8)
    base = e * eb
    g = decode_matrix(b[base:base + gu], d_ff, d_model)
    u = decode_matrix(b[base + gu:base + 2 * gu], d_ff, d_model)
    row_bytes = d_ff // BLOCK * BLOCK_BYTES
    dbase = base + 2 * gu
    if out_cols is None:
        dn = decode_matrix(b[dbase:dbase + d_model * row_bytes], d_model, d_ff)
    else:
        rows = [b[dbase + int(r) * row_bytes: dbase + (int(r) + 1) * row_bytes] for r in out_cols]
        dn = decode_matrix(np.concatenate(rows), len(rows), d_ff) if rows else np.zeros((0, d_ff))
    return g, u, dn


def expert_output(layer_buf, e, d_model, d_ff, x, out_cols=None):
    """y [n, d] (or [n, len(out_cols)]) of expert e for token rows x [n, d]."""
    g, u, dn = _expert_parts(layer_buf, e, d_model, d_ff, out_cols)
    return expert_hidden(g, u, x) @ dn.T


def moe_layer(x, w_r, bias, layer_buf, d_model, d_ff, n_experts, top_k,
              n_shared=0, norm_topk=True, out_cols=None):
    """Returns dict(out [T, d or |out_cols|] f32, out64 (fp64), idx, w, z).

    layer_buf holds the layer's experts in the interchange layout: routed
    experts 0..E-1, then the shared experts E..E+n_shared-1.
    """
    x = np.asarray(x, dtype=np.float32)
    z = router_logits_fp32(x, w_r, bias)
    idx = topk(z, top_k)
    w = gate_weights(z, idx, norm_topk)
    ncol = d_model if out_cols is None else len(out_cols)
    out = np.zeros((x.shape[0], ncol), dtype=np.float64)
    x64 = x.astype(np.float64)
    for e in np.unique(idx):
        tok, j = np.nonzero(idx == e)
        y = expert_output(layer_buf, int(e), d_model, d_ff, x64[tok], out_cols)
        out[tok] += w[tok, j][:, None] * y
    for s in range(n_shared):
        out += expert_output(layer_buf, n_experts + s, d_model, d_ff, x64, out_cols)
    return {"out": out.astype(np.float32), "out64": out, "idx": idx, "w": w, "z": z}


def dense_mixture(x, w_r, bias, layer_buf, d_model, d_ff, n_experts, top_k,
                  n_shared=0, norm_topk=True):
    """Brute force: every expert on every token, masked by the routing.

    Used as a pin of moe_layer: sum_e [e selected] * w * y_e equals the sparse
    sum in which each selected expert is evaluated once.
    """
    x = np.asarray(x, dtype=np.float32)
    z = router_logits_fp32(x, w_r, bias)
    idx = topk(z, top_k)
    w = gate_weights(z, idx, norm_topk)
    x64 = x.astype(np.float64)
    out = np.zeros((x.shape[0], d_model))
    for e in range(n_experts):
        y = expert_output(layer_buf, e, d_model, d_ff, x64)
        mask = (idx == e)
        coef = (w * mask).sum(axis=1)
        out += coef[:, None] * y
    for s in range(n_shared):
        out += expert_output(layer_buf, n_experts + s, d_model, d_ff, x64)
    return out
