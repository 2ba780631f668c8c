"""Pins for the oracle's exact three-way MXFP4 error decomposition (CPU only).

The MXFP4 error-decomposition abstract states the split is exact and
additive: scale bias (power-of-two rounding of the scale), deadzone
truncation (small values zeroed) and grid noise (rounding to the grid).
Pins: a hand-derived block, the per-element identity, special cases where a
component must vanish, and the fixed-point sums against Python's exact
integers."""
import json
import os
from fractions import Fraction

import numpy as np

from workloads import bf16_bits, bf16_to_f32, dense_case

GOLD = os.path.join(os.path.dirname(__file__), "golden")
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
NAMES = ("total6", "scale_bias6", "deadzone6", "grid_noise6")


def test_golden_block(orc):
    g = json.load(open(os.path.join(GOLD, "mxfp4_decompose_block0.json")))
    a = json.load(open(os.path.join(GOLD, g["activation_fixture"])))
    x = bf16_bits(np.array([a["x"]], np.float32))
    c6 = orc.error_components6(x)
    for k, ent in g["elements"].items():
        k = int(k)
        assert bf16_to_f32(x)[0, k] == ent["x"]
        for c, name in enumerate(NAMES):
            assert c6[c, 0, k] == ent[name], (k, name)


def test_identity_per_element(orc):
    x = dense_case(64, 512, 8, n_out=5, seed=31)["x"]
    c6 = orc.error_components6(x)
    assert np.array_equal(c6[1] + c6[2] + c6[3], c6[0])
    # disjoint support: the deadzone part never overlaps the other two
    assert not np.any((c6[2] != 0) & ((c6[1] != 0) | (c6[3] != 0)))


def test_power_of_two_amax_has_no_scale_bias(orc):
    """Block amax = 6*2^k: the ideal scale amax/6 is already a power of two,
    so Q* = Q_s and the scale-bias part vanishes."""
    rng = np.random.default_rng(32)
    xv = rng.standard_normal((8, 128)).astype(np.float32)
    for r in range(8):
        for b in range(4):
            blk = xv[r, 32 * b:32 * b + 32]
            blk /= np.abs(blk).max()
            blk *= 6.0 * 2.0 ** (b - 2)
    x = bf16_bits(xv)
    c6 = orc.error_components6(x)
    assert not np.any(c6[1])


def test_grid_input_has_no_error(orc):
    rng = np.random.default_rng(33)
    codes = rng.integers(0, 16, (4, 128)).astype(np.uint8)
    codes[:, ::32] = 7
    e = np.repeat(rng.integers(-5, 5, (4, 4)), 32, axis=1)
    xv = (np.where(codes & 8, -1.0, 1.0) * GRID[codes & 7] * np.exp2(e.astype(float)))
    c6 = orc.error_components6(bf16_bits(xv.astype(np.float32)))
    assert not np.any(c6)


def test_tiny_elements_are_pure_deadzone(orc):
    """|x| <= s/4 rounds to zero under the actual scale s: total = deadzone = x."""
    rng = np.random.default_rng(34)
    xv = rng.standard_normal((16, 64)).astype(np.float32)
    x = bf16_bits(xv)
    xf = bf16_to_f32(x).reshape(16, 2, 32)
    e = np.array([[orc.mx_exponent(float(np.abs(b).max())) for b in row] for row in xf])
    s = np.exp2(e.astype(float))[..., None]
    tiny = (np.abs(xf) <= s / 4).reshape(16, 64)
    c6 = orc.error_components6(x)
    x6 = 6.0 * bf16_to_f32(x).astype(np.float64)
    assert tiny.any()
    assert np.array_equal(c6[0][tiny], x6[tiny])
    assert np.array_equal(c6[2][tiny], x6[tiny])


def test_fixed_point_sums_are_exact(orc):
    """The 320-bit fixed-point totals equal Python's exact integer sums of the
    per-element components (each times 6, in units of 2^-136), and the three
    parts add up to the total exactly."""
    x = dense_case(24, 256, 8, n_out=3, seed=35)["x"]
    # include extreme magnitudes: bf16 subnormals and huge values
    x[0, :4] = [0x0001, 0x8003, 0x7F00, 0xFF00]
    st = orc.error_decompose(x)
    c6 = orc.error_components6(x)
    for c in range(4):
        want = sum(Fraction(v) * 2 ** 136 for v in c6[c].ravel().tolist())
        assert want.denominator == 1
        assert st["exact_int"][c] == int(want)
    t, sb, dz, gn = st["exact_int"]
    assert sb + dz + gn == t
    assert st["n_elems"] == x.size
    assert st["n_clipped"] == 0
    nz = bf16_to_f32(x) != 0
    assert st["n_deadzone"] == int(((c6[2] != 0) & nz).sum())
    for c in range(4):
        comp = c6[c] / 6.0
        assert np.isclose(st["sum"][c], comp.sum(), rtol=1e-12, atol=0)
        assert np.isclose(st["sumsq"][c], (comp ** 2).sum(), rtol=1e-12)
    assert np.isclose(st["cross_sb_gn"], ((c6[1] / 6) * (c6[3] / 6)).sum(), rtol=1e-12)


def test_squared_norm_split(orc):
    """Deadzone has disjoint support, so ||e||^2 = ||sb||^2 + ||dz||^2 +
    ||gn||^2 + 2<sb, gn> (real arithmetic; FP64 here)."""
    x = dense_case(32, 256, 8, n_out=3, seed=36)["x"]
    st = orc.error_decompose(x)
    lhs = st["sumsq"][0]
    rhs = st["sumsq"][1] + st["sumsq"][2] + st["sumsq"][3] + 2 * st["cross_sb_gn"]
    assert np.isclose(lhs, rhs, rtol=1e-10)
