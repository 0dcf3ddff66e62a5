"""The expert MLP (oracle side).

An expert is a gated feed-forward network without biases whose activation is
GELU or SiLU ("Limitations", llama.cpp + MoE expert cache: merged gate/up expert
tensors, no expert biases, GELU or SiLU).  Reading taken: SwiGLU,
h = silu(G x) * (U x), y = D h, with silu(v) = v / (1 + exp(-v)); fp64.
"""
from __future__ import annotations

import numpy as np


def silu(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def expert_hidden(g_mat: np.ndarray, u_mat: np.ndarray, x: np.ndarray) -> np.ndarray:
    """h [n, f] = silu(x G^T) * (x U^T) for token rows x [n, d]."""
    x = np.asarray(x, dtype=np.float64)
    return silu(x @ g_mat.T) * (x @ u_mat.T)


def expert_forward(g_mat, u_mat, d_mat, x, out_rows=None) -> np.ndarray:
    """y [n, d] = h D^T, or only the output columns listed in out_rows."""
    h = expert_hidden(g_mat, u_mat, x)
    dm = d_mat if out_rows is None else d_mat[np.asarray(out_rows)]
    return h @ dm.T
