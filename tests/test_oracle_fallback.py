"""Pins of the oracle's Outlier Fallback (MXFP4 error-decomposition abstract:
the fallback recovers the deadzone entries), reading: an entry the quantizer
sends to zero keeps its own BF16 value, every other entry is dequantized.

  * hand-worked 1 x 32 MXFP4 and 1 x 16 NVFP4 blocks (tests/golden/
    fallback_blocks.json), ties and signed zeros included;
  * against the three-way split (pinned separately): outside the deadzone
    the output is the quantizer's value Q_s(x) = x - total, rounded once to
    FP32, and inside it the output is x itself; so x - out is exactly
    scale_bias + grid_noise (the deadzone component is gone) for MXFP4, and
    within half an FP32 ulp of it for NVFP4 (whose Q_s is a real product);
  * the fallback count equals the split's deadzone count;
  * grid inputs at an exact scale need no fallback; tiny entries beside an
    outlier come back unchanged.
"""
import json
import os

import numpy as np
import pytest

from workloads import bf16_bits, bf16_to_f32, dense_case

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "fallback_blocks.json")


def _golden(fmt_key, cols):
    g = json.load(open(GOLDEN))[fmt_key]
    x = np.zeros((1, cols), np.uint16)
    want = np.zeros((1, cols), np.float32)
    for e in g["elements"]:
        x[0, e["col"]] = int(e["bits"], 16)
        want[0, e["col"]] = np.float32(e["out"])
    return x, want, g["n_fallback"]


@pytest.mark.parametrize("fmt,key,cols", [(1, "mxfp4", 32), (0, "nvfp4", 16)])
def test_golden_blocks(orc, fmt, key, cols):
    x, want, n = _golden(key, cols)
    out, nfb = orc.qdq_fallback(fmt, x)
    assert np.array_equal(out.view(np.uint32), want.view(np.uint32)), (out, want)
    assert nfb == n


@pytest.mark.parametrize("fmt", [0, 1])
def test_split_identity(orc, fmt):
    """out = x on the deadzone, fl32(x - total) elsewhere, from the pinned
    per-element components (times 6)."""
    d = dense_case(48, 512, 8, x_dist="t4", n_out=6, out_mult=30.0, seed=41 + fmt)
    x = d["x"]
    out, _ = orc.qdq_fallback(fmt, x)
    c6 = orc.error_components6(x, fmt=fmt)
    xv = bf16_to_f32(x).astype(np.float64)
    qs = (6.0 * xv - c6[0]) / 6.0          # Q_s(x): exact in FP64
    dz = c6[2] != 0.0
    q = orc.quantize(fmt, x)["q"]
    codes = np.stack([q & 15, q >> 4], -1).reshape(x.shape)
    zero_code = (codes & 7) == 0
    # the deadzone of the split is exactly the non-zero entries with code 0
    assert np.array_equal(dz, zero_code & (xv != 0.0))
    assert np.array_equal(out[zero_code].view(np.uint32),
                          bf16_to_f32(x)[zero_code].view(np.uint32))
    assert np.array_equal(out[~zero_code], qs[~zero_code].astype(np.float32))
    resid6 = 6.0 * (xv - out.astype(np.float64))
    sb_gn = c6[1] + c6[3]
    if fmt == 1:
        assert np.array_equal(resid6, sb_gn)          # the deadzone component is gone
    else:
        half_ulp6 = 3.0 * np.spacing(np.abs(out)).astype(np.float64)
        assert np.all(np.abs(resid6 - sb_gn) <= half_ulp6)
    assert np.all(resid6[zero_code] == 0.0)


@pytest.mark.parametrize("fmt", [0, 1])
def test_count_is_the_deadzone_count(orc, fmt):
    x = dense_case(64, 1024, 8, n_out=10, out_mult=30.0, seed=77 + fmt)["x"]
    _, nfb = orc.qdq_fallback(fmt, x)
    assert nfb == orc.error_decompose(x, fmt=fmt)["n_deadzone"]
    assert nfb > 0


def test_grid_inputs_need_no_fallback(orc):
    """Non-zero E2M1 grid values times 2^-3 with a 6 in every block: MXFP4
    scale 2^-3 exactly, every entry on the grid, nothing falls back."""
    rng = np.random.default_rng(3)
    mags = np.array([0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    v = rng.choice(mags, (8, 64)) * rng.choice([-1.0, 1.0], (8, 64)).astype(np.float32)
    v[:, ::32] = 6.0
    v *= np.float32(2.0 ** -3)
    out, nfb = orc.qdq_fallback(1, bf16_bits(v))
    assert nfb == 0
    assert np.array_equal(out, v)


@pytest.mark.parametrize("fmt,blk", [(0, 16), (1, 32)])
def test_tiny_entries_beside_an_outlier(orc, fmt, blk):
    """A block holding 1000 and entries below 1000/24 in magnitude: the small
    entries are deadzone and come back exactly; the outlier is on the grid."""
    x = np.zeros((2, blk), np.float32)
    x[:, 0] = 1000.0
    x[:, 1:] = np.linspace(-9.0, 9.0, blk - 1, dtype=np.float32)
    xb = bf16_bits(x)
    out, nfb = orc.qdq_fallback(fmt, xb)
    xv = bf16_to_f32(xb)
    assert np.array_equal(out[:, 1:], xv[:, 1:])
    assert nfb == int(np.count_nonzero(xv[:, 1:]))
    assert out[0, 0] != 0.0
