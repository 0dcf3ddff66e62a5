"""Pins of the oracle's Q4_0 decoding (oracle/q4.py) against hand-worked blocks,
closed-form sizes quoted on the pages, and the seeded generator's round trip."""
import os

import numpy as np
import pytest

from oracle.q4 import decode_blocks, decode_matrix, expert_nbytes
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "q4_blocks.txt")


def _golden_blocks():
    out = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, hx, vals = [p.strip() for p in line.split("|")]
        raw = np.array([int(b, 16) for b in hx.split()], dtype=np.uint8)
        exp = np.array([float(v) for v in vals.split()])
        out.append((name, raw, exp))
    return out


@pytest.mark.parametrize("name,raw,exp", _golden_blocks())
def test_hand_blocks(name, raw, exp):
    assert raw.size == 18 and exp.size == 32
    got = decode_blocks(raw)
    np.testing.assert_array_equal(got, exp)


def test_expert_size_matches_pages():
    # "How it works" (llama.cpp + MoE expert cache): experts of ~3.35 MB at 4-bit
    # for the Gemma 4 26B-A4B shape (d=2816, f=704, three matrices).
    eb = expert_nbytes(2816, 704)
    assert eb == 3 * 2816 * 704 * 18 // 32 == 3_345_408
    assert round(eb / 1e6, 2) == 3.35
    # "Settings": 28 slots x 26 layers = 2.4 GB.
    assert round(28 * 26 * eb / 1e9, 1) == 2.4
    # "The problem": a token reads ~1 GB (8 experts x 30 layers).
    assert 0.75e9 < 8 * 30 * eb < 1.05e9
    # "Memory placement" (calculator page): Q4_0 = 18/32 bytes per parameter.
    assert eb * 32 == 3 * 2816 * 704 * 18


def test_decode_matrix_row_major():
    # Row r of a 3 x 64 matrix: two blocks with scale r+1 and all q = 9 -> value r+1.
    rows, cols = 3, 64
    blocks = []
    for r in range(rows):
        for b in range(2):
            d = np.float16(r + 1 + 0.5 * b).tobytes()
            blocks.append(np.frombuffer(d + bytes([0x99] * 16), dtype=np.uint8))
    buf = np.concatenate(blocks)
    m = decode_matrix(buf, rows, cols)
    for r in range(rows):
        np.testing.assert_array_equal(m[r, :32], r + 1)
        np.testing.assert_array_equal(m[r, 32:], r + 1.5)


def test_generator_round_trip():
    """Decoding the generator's bytes recovers its normals within half a step.

    The generator (synth/q4gen.c) and the decoder are written independently;
    the bound |w - x| <= |d|/2 holds except where q is clamped (|w - x| <= |d|,
    up to the fp16 rounding of d, a relative 2^-11 of the block maximum).
    """
    wl = synth.WORKLOADS["tiny"]
    raw = synth.gen_experts(wl, 0, 0, 1)
    vals = synth.gen_values(wl, 0, 0, 1)
    d, f = wl.d_model, wl.d_ff
    gu = f * d // 32 * 18
    mats = [(raw[:gu], f, d), (raw[gu:2 * gu], f, d), (raw[2 * gu:], d, f)]
    off = 0
    for buf, r, c in mats:
        w = decode_matrix(buf, r, c)
        x = vals[off:off + r * c].reshape(r, c).astype(np.float64)
        off += r * c
        blocks = buf.reshape(r, c // 32, 18)
        scale = np.abs(blocks[..., 0:2].copy().view("<f2")[..., 0].astype(np.float64))
        step = np.repeat(scale, 32, axis=1)
        err = np.abs(w - x)
        assert np.all(err <= step * (1.0 + 2.0 ** -10))
        assert np.mean(err <= step * 0.5 + 1e-9) > 0.99
        # values are ~N(0, 0.02^2)
        assert 0.015 < x.std() < 0.025
