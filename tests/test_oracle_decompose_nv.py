"""Pins for the oracle's three-way error decomposition under the NVFP4
quantizer (CPU only).  The split follows the MXFP4 decomposition's
definitions (actual scale vs the ideal scale amax/6); with NVFP4 the actual
scale is the E4M3 block scale times the FP32 tensor scale.  Pins: the
actual quantization term against the already-pinned quantizer, the ideal
term and the sums against exact rational arithmetic on small tensors, the
per-element identity, and cases where a component must vanish."""
from fractions import Fraction

import numpy as np
import pytest

from workloads import bf16_bits, bf16_to_f32, dense_case

GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
        Fraction(4), Fraction(6)]


def _e4m3(code):
    e, m = (code >> 3) & 15, code & 7
    return Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def _qstar_index(ax, A):
    """Nearest E2M1 point to 6|x|/A, ties to the even mantissa bit."""
    if A == 0:
        return 0
    v = 6 * ax / A
    best = 0
    for c in range(1, 8):
        d, bd = abs(v - GRID[c]), abs(v - GRID[best])
        if d < bd or (d == bd and c % 2 == 0 and best % 2 == 1):
            best = c
    return best


def _exact_components(orc, xb):
    """Components (not times 6) as Fractions, from the pinned quantizer's
    codes and scales and an independent Q* in rational arithmetic."""
    qx = orc.quantize(0, xb)
    t = Fraction(float(qx["tscale"][0]))
    x = bf16_to_f32(xb).astype(np.float64)
    rows, cols = x.shape
    out = np.empty((4, rows, cols), object)
    for r in range(rows):
        for c in range(cols):
            xv = Fraction(float(x[r, c]))
            A = max(abs(Fraction(float(v))) for v in x[r, (c // 16) * 16:(c // 16) * 16 + 16])
            byte = int(qx["q"][r, c // 2])
            code = (byte >> 4) if c & 1 else (byte & 15)
            sgn = -1 if np.signbit(x[r, c]) else 1
            qs = sgn * GRID[code & 7] * _e4m3(int(qx["scales"][r, c // 16])) * t
            qst = sgn * GRID[_qstar_index(abs(xv), A)] * A / 6
            g = code & 7
            out[0, r, c] = xv - qs
            out[1, r, c] = (qst - qs) if g else Fraction(0)
            out[2, r, c] = Fraction(0) if g else xv
            out[3, r, c] = (xv - qst) if g else Fraction(0)
    return out


@pytest.mark.parametrize("seed", [3, 4])
def test_components_match_exact_rational(orc, seed):
    xb = dense_case(6, 64, 8, x_dist="t4", n_out=2, seed=seed)["x"]
    c6 = orc.error_components6(xb, fmt=0)
    ref = _exact_components(orc, xb)
    for c in range(4):
        for idx in np.ndindex(ref[c].shape):
            assert Fraction(c6[c][idx]) == 6 * ref[c][idx], (c, idx)


@pytest.mark.parametrize("seed", [5, 6])
def test_sums_are_exact(orc, seed):
    xb = dense_case(5, 48, 8, x_dist="t4", n_out=2, seed=seed)["x"]
    st = orc.error_decompose(xb, fmt=0)
    ref = _exact_components(orc, xb)
    for c in range(4):
        want = sum(ref[c].ravel(), Fraction(0)) * 6 * (Fraction(2) ** 136)
        assert want.denominator == 1
        assert st["exact_int"][c] == want.numerator, c
    # the three parts add up to the total, bit for bit
    assert st["exact_int"][0] == st["exact_int"][1] + st["exact_int"][2] + st["exact_int"][3]
    nz = bf16_to_f32(xb) != 0
    assert st["n_deadzone"] == int(np.sum((ref[2] != 0) & nz))


def test_identity_and_disjoint_support(orc):
    xb = dense_case(64, 256, 8, n_out=5, seed=31)["x"]
    c6 = orc.error_components6(xb, fmt=0)
    assert np.array_equal(c6[1] + c6[2] + c6[3], c6[0])
    assert not np.any((c6[2] != 0) & ((c6[1] != 0) | (c6[3] != 0)))


def test_exact_scale_block_has_no_scale_bias(orc):
    """A tensor whose amax is 21 * 2^k: t = amax / 2688 = 2^(k-7) exactly, and
    the amax block's scale 448 t equals amax / 6, so in that block the actual
    and ideal quantizations coincide (no scale bias) and the amax itself is
    represented exactly."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 32)).astype(np.float32)
    x = np.clip(x, -5, 5)
    x[0, 3] = 21.0 * 0.25            # the tensor amax, in block 0 of row 0
    xb = bf16_bits(x)
    c6 = orc.error_components6(xb, fmt=0)
    assert np.all(c6[1][0, :16] == 0)
    assert c6[0][0, 3] == 0
    assert np.any(c6[1] != 0)        # the other blocks do have scale bias


def test_small_entries_next_to_a_large_one_are_deadzone(orc):
    """Block amax 64 and entries of 1/4: 6 * (1/4) / 64 is far below 0.25, so
    Q* is zero too; the quantizer's code is zero, so they are deadzone, and
    the deadzone sum is their exact sum."""
    x = np.full((2, 16), 0.25, np.float32)
    x[:, 0] = 64.0
    x[1, 5] = -0.25
    xb = bf16_bits(x)
    st = orc.error_decompose(xb, fmt=0)
    want = (15 * Fraction(1, 4) + 14 * Fraction(1, 4) - Fraction(1, 4)) * 6 * Fraction(2) ** 136
    assert st["exact_int"][2] == want.numerator
    assert st["n_deadzone"] == 30


def test_grid_values_at_exact_scales_have_no_error(orc):
    """Tensor amax 5.25 = 21 * 2^-2, so t = 2^-9 exactly.  Block scales:
    amax 5.25 -> 448 t = 0.875; amax 3 -> 256 t = 0.5; amax 1.5 -> 128 t =
    0.25, each exactly amax / 6.  Every element is a grid point times its
    block's scale, so every sum is zero and nothing is deadzone or clipped."""
    g = np.array([6, 4, 3, 2, 1.5, 1, 0.5, 0], np.float32)
    x = np.zeros((2, 32), np.float32)
    x[0, :8] = g * 0.875
    x[0, 16:24] = -g * 0.5
    x[1, :8] = g * 0.25
    x[1, 16:24] = g[::-1] * 0.25
    xb = bf16_bits(x)
    assert np.array_equal(bf16_to_f32(xb), x)
    st = orc.error_decompose(xb, fmt=0)
    assert st["exact_int"] == [0, 0, 0, 0]
    assert st["n_deadzone"] == 0 and st["n_clipped"] == 0


def test_tiny_tensor_rejected(orc):
    """Amax 2^-120: the tensor scale 2^-127/21 is an FP32 subnormal, odd
    multiple of 2^-149, so 6 Q_s(amax) = 16128 t is not a multiple of 2^-136
    and the fixed point cannot hold it: rejected.  A tensor of 1e-30 still
    fits (its terms are multiples of 2^-127) and is accepted."""
    x = np.full((1, 16), 2.0 ** -120, np.float32)
    with pytest.raises(ValueError):
        orc.error_decompose(bf16_bits(x), fmt=0)
    st = orc.error_decompose(bf16_bits(np.full((1, 16), 1e-30, np.float32)), fmt=0)
    assert st["n_elems"] == 16


def test_scale_rounded_down_clips_the_block_amax(orc):
    """Tensor amax 5.25 (t = 2^-9).  A block with amax 0.96875 wants the scale
    code of 0.96875 / 6 / t = 82.67, which E4M3 rounds down to 80, so the
    block's largest value is 6 * 80 t = 0.9375 and only its amax element is
    clipped; a block with amax 1 rounds its scale up (88) and clips nothing."""
    x = np.zeros((1, 48), np.float32)
    x[0, 0] = 5.25
    x[0, 16:20] = [0.96875, 0.5, -0.25, 0.9375]
    x[0, 32:35] = [1.0, -0.75, 0.5]
    xb = bf16_bits(x)
    qx = orc.quantize(0, xb)
    assert float(qx["tscale"][0]) == 2.0 ** -9
    assert float(_e4m3(int(qx["scales"][0, 1]))) == 80.0
    assert float(_e4m3(int(qx["scales"][0, 2]))) == 88.0
    st = orc.error_decompose(xb, fmt=0)
    assert st["n_clipped"] == 1
    c6 = orc.error_components6(xb, fmt=0)
    assert c6[0][0, 16] == 6 * (0.96875 - 0.9375)
