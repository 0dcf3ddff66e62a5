"""Error of the GPU path's activation encodings, emulated in numpy on the CPU.

The GPU path never multiplies float activations by float weights.  It encodes
them, and the layer's accuracy bar (max |out - oracle| <= 2e-3 * RMS) holds only
if the encodings lose less than that on every input the layer may see:

* decode GEMV (gate/up input x, down input h): 16-bit fixed point with one scale
  per 32-element block, X = rint(v * (30000 / m)) in float32, m = the block's
  max |v| (floored at 2^-100), value = X * (m / 30000);
* matrix-core GEMM (prefill; gate/up input x, down input h): per row a power of
  two 2^-e brings max |v| into [2^13, 2^14) (e = frexp exponent - 14, clamped
  to [-126, 127]), then binary16 hi = fp16(v 2^-e) and lo = fp16(v 2^-e - hi),
  value = (hi + lo) 2^e.

This module emulates exactly those encodings through one SwiGLU expert with
float64 weights (the weights' Q4 form is exact on both sides and plays no part
in the encoding error) and compares with the float64 expert on the unencoded
input, for inputs from RMS 2^-20 to 2^20 and with one channel at 10x, 100x and
1000x the rest.  The earlier designs (one scale per token for x; a scale that
only ever shrinks rows, max(0, e)) are kept as planted mistakes: each must fail
the bar at a corner, so that the test would catch a regression to either.
"""
import numpy as np
import pytest

TOL = 2e-3
D_MODEL, D_FF = 2816, 704  # the Gemma-like expert


def silu(v):
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


@pytest.fixture(scope="module")
def expert():
    rng = np.random.default_rng(11)
    return (rng.standard_normal((D_FF, D_MODEL)) * 0.02,
            rng.standard_normal((D_FF, D_MODEL)) * 0.02,
            rng.standard_normal((D_MODEL, D_FF)) * 0.02)


def fixed16_blocks(v):
    v32 = np.asarray(v, np.float32).reshape(-1, 32)
    m = np.max(np.abs(v32), axis=1)
    ms = np.maximum(m, np.float32(2.0 ** -100))
    inv = np.where(m > 0, np.float32(30000.0) / ms, np.float32(0.0)).astype(np.float32)
    x = np.rint((v32 * inv[:, None]).astype(np.float32))
    assert np.all(np.abs(x) <= 30001)
    s = np.where(m > 0, ms / np.float32(30000.0), np.float32(0.0)).astype(np.float32)
    return (x.astype(np.float64) * s[:, None].astype(np.float64)).reshape(-1)


def fixed16_token(v):
    """Planted mistake: one scale for the whole vector."""
    v32 = np.asarray(v, np.float32)
    m = np.max(np.abs(v32))
    x = np.rint((v32 * (np.float32(30000.0) / m)).astype(np.float32))
    return x.astype(np.float64) * np.float64(np.float32(m / np.float32(30000.0)))


def hilo_pow2(v, signed=True):
    """signed=False is the planted mistake: the scale only ever shrinks rows."""
    v32 = np.asarray(v, np.float32)
    m = float(np.max(np.abs(v32)))
    e = 0
    if m > 0:
        fe = np.frexp(m)[1]
        e = min(127, max(-126, fe - 14)) if signed else max(0, fe - 14)
    sc = np.float32(2.0 ** -e)
    a = (v32 * sc).astype(np.float32)
    hi = a.astype(np.float16).astype(np.float32)
    lo = (a - hi).astype(np.float16).astype(np.float32)
    return (hi.astype(np.float64) + lo.astype(np.float64)) * 2.0 ** e


def rel_err(expert, x, enc_x, enc_h):
    g, u, dn = expert
    y_ref = dn @ (silu(g @ x) * (u @ x))
    xe = enc_x(x)
    y = dn @ enc_h(silu(g @ xe) * (u @ xe))
    return float(np.max(np.abs(y - y_ref)) / np.sqrt(np.mean(y_ref ** 2)))


def inputs(seed, rms, outlier):
    x = np.random.default_rng(seed).standard_normal(D_MODEL) * rms
    if outlier:
        x[701] *= outlier
    return x.astype(np.float32).astype(np.float64)


SCALES = [2.0 ** p for p in range(-20, 21, 4)]
OUTLIERS = [None, 10, 100, 1000]


@pytest.mark.parametrize("outlier", OUTLIERS)
def test_decode_block_scale_within_bar(expert, outlier):
    worst = max(rel_err(expert, inputs(i, rms, outlier), fixed16_blocks, fixed16_blocks)
                for i, rms in enumerate(SCALES))
    assert worst <= TOL / 4, worst


@pytest.mark.parametrize("outlier", OUTLIERS)
def test_prefill_hilo_within_bar(expert, outlier):
    worst = max(rel_err(expert, inputs(i, rms, outlier), hilo_pow2, hilo_pow2)
                for i, rms in enumerate(SCALES))
    assert worst <= 1e-5, worst


def test_planted_token_scale_fails_on_outlier(expert):
    errs = [rel_err(expert, inputs(s, 1.0, 1000), fixed16_token, fixed16_blocks)
            for s in range(4)]
    assert max(errs) > TOL, errs


def test_planted_shrink_only_scale_fails_on_small_rows(expert):
    assert rel_err(expert, inputs(0, 1e-5, None), lambda v: hilo_pow2(v, False),
                   lambda v: hilo_pow2(v, False)) > TOL


def test_hilo_exponent_clamp():
    """Row maxima at the ends of float32 keep a finite scale and lose no more
    than the split's 22 bits on their largest elements."""
    for m in [np.float32(1e-38), np.float32(2.0 ** -126), np.float32(3.0e38), np.float32(1.0)]:
        v = np.array([m, m / 3, -m / 7] + [0.0] * 29, np.float32)
        got = hilo_pow2(v)
        assert np.all(np.isfinite(got))
        assert abs(got[0] - float(m)) <= abs(float(m)) * 2.0 ** -21


def test_fixed16_zero_and_tiny_blocks():
    v = np.zeros(64, np.float32)
    v[40] = np.float32(1e-35)  # below the 2^-100 floor: encoded on the floor's scale
    got = fixed16_blocks(v)
    assert np.all(got[:32] == 0.0)
    assert abs(got[40] - 1e-35) <= 2.0 ** -100 / 60000
