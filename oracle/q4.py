"""Q4_0 block decoding (oracle side).

Block format: 32 weights in 18 bytes -- the 18/32 bytes per parameter that the
calculator page gives for Q4_0 ("Multi-GPU LLM Calculator", Memory placement,
which defers to the GGML block definitions).  Reading taken here (GGML's Q4_0):

* bytes 0-1: IEEE binary16 scale d, little-endian;
* bytes 2-17: qs[16]; element i < 16 is the low nibble of qs[i], element
  i >= 16 the high nibble of qs[i - 16];
* value w_i = d * (q_i - 8).

Expert layout of the interchange buffer: gate [f][d], up [f][d], down [d][f],
each row quantised along its reduction dimension, blocks in K order, no padding;
experts are consecutive, layers are consecutive.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
BLOCK_BYTES = 18


def decode_blocks(raw: np.ndarray) -> np.ndarray:
    """Decode a uint8 array [..., 18] of blocks into float64 [..., 32]."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    if raw.shape[-1] != BLOCK_BYTES:
        raise ValueError("last axis must hold 18-byte blocks")
    d = raw[..., 0:2].copy().view("<f2")[..., 0].astype(np.float64)
    qs = raw[..., 2:18]
    q = np.empty(raw.shape[:-1] + (BLOCK,), dtype=np.int8)
    q[..., :16] = qs & 0x0F                        # elements 0..15: low nibbles
    q[..., 16:] = qs >> 4                          # elements 16..31: high nibbles
    q -= 8                                         # q - 8 in [-8, 7]
    return d[..., None] * q                        # float64, exact


def decode_matrix(buf: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Dequantise a [rows][cols] Q4_0 matrix (rows quantised along cols)."""
    if cols % BLOCK:
        raise ValueError("cols must be a multiple of 32")
    nb = cols // BLOCK
    need = rows * nb * BLOCK_BYTES
    blocks = np.asarray(buf, dtype=np.uint8)[:need].reshape(rows, nb, BLOCK_BYTES)
    return decode_blocks(blocks).reshape(rows, cols)


def expert_nbytes(d_model: int, d_ff: int) -> int:
    return 3 * d_model * d_ff // BLOCK * BLOCK_BYTES
