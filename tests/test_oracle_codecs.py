"""Pins for the oracle's number formats (CPU only).

Each codec of the oracle is written as a nearest-value search; these tests
hold it against independent facts: the closed-form E2M1 grid and its
midpoint table, torch's own float8_e4m3fn and bfloat16 conversions (library
routines), the float32 exponent field for E8M0, and exhaustive brute force.
"""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

from workloads import bf16_to_f32

pytestmark = pytest.mark.filterwarnings("ignore")

# E2M1 magnitudes: 8 levels per sign with zero counted (QUADS explainer,
# section 1; grid values as read from the task's format statement).
GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_values_closed_form(orc):
    for c in range(16):
        v = orc.e2m1_value(c)
        assert abs(v) == GRID[c & 7]
        assert math.copysign(1.0, v) == (-1.0 if c & 8 else 1.0)


def _e2m1_by_midpoints(a: float) -> int:
    # Round to nearest on the grid: the decision points are the midpoints
    # 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5; at a midpoint the code with an even
    # mantissa bit wins, i.e. 0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2,
    # 3.5->4, 5->4; everything above 5 saturates to 6.
    table = [(0.25, False), (0.75, True), (1.25, False), (1.75, True), (2.5, False),
             (3.5, True), (5.0, False)]
    code = 0
    for mid, inclusive in table:
        if a > mid or (inclusive and a == mid):
            code += 1
    return code


def test_e2m1_encode_every_bf16_pattern(orc):
    """All 65536 BF16 patterns at unit scale: oracle == midpoint table ==
    exact brute force over the grid with Fractions."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bf16_to_f32(bits)
    for h, v in zip(bits.tolist(), vals.tolist()):
        if not math.isfinite(v):
            continue
        a = abs(v)
        got = orc.e2m1_encode_mag(a)
        assert got == _e2m1_by_midpoints(a), (hex(h), v)
        if a < 16.0 and (h & 0x7F) % 7 == 0:  # brute force on a spread subset
            fa = Fraction(a)
            dists = [abs(fa - Fraction(g)) for g in GRID]
            best = min(dists)
            cands = [c for c in range(8) if dists[c] == best]
            want = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
            assert got == want


@pytest.mark.parametrize("a,code", [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4),
                                    (3.5, 6), (5.0, 6), (5.0000005, 7), (1e30, 7), (0.0, 0),
                                    (0.2500001, 1)])
def test_e2m1_ties_and_saturation(orc, a, code):
    assert orc.e2m1_encode_mag(a) == code


def test_e4m3_decode_matches_torch(orc):
    codes = torch.arange(0, 256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).tolist()
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue  # NaN code, never produced
        assert orc.e4m3_value(c) == ref[c], c
    assert orc.e4m3_value(0x7E) == 448.0
    assert orc.e4m3_value(0x01) == 2.0 ** -9


def test_e4m3_encode_matches_torch_rne(orc):
    rng = np.random.default_rng(7)
    # random values across the whole range, plus every midpoint between
    # adjacent finite codes (the tie cases)
    v = np.concatenate([
        rng.uniform(0, 2.0 ** -6, 20000), np.exp2(rng.uniform(-12, 8.8, 60000)),
    ]).astype(np.float32)
    finite = [orc.e4m3_value(c) for c in range(0x7F)]
    mids = np.array([(finite[i] + finite[i + 1]) / 2 for i in range(len(finite) - 1)],
                    np.float32)
    v = np.concatenate([v, mids])
    v = v[v < 448.0]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.e4m3_encode(float(x)) for x in v], np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(v[i]), int(got[i]), int(ref[i])) for i in bad[:5]]


@pytest.mark.parametrize("v", [448.0, 460.0, 463.99, 464.0, 500.0, 1e9, 3.0e38])
def test_e4m3_saturates(orc, v):
    assert orc.e4m3_encode(v) == 0x7E


def test_e4m3_underflow(orc):
    assert orc.e4m3_encode(2.0 ** -10) == 0      # tie between 0 and 2^-9: even code 0
    assert orc.e4m3_encode(2.0 ** -10 * 1.0001) == 1
    assert orc.e4m3_encode(0.0) == 0


def test_e8m0_is_float_exponent(orc):
    for c in range(1, 255):
        f = struct.unpack("<f", struct.pack("<I", c << 23))[0]  # exponent field c, mantissa 0
        assert orc.e8m0_value(c) == f
    assert orc.e8m0_value(0) == 2.0 ** -127


def test_bf16_rne_matches_torch(orc):
    rng = np.random.default_rng(3)
    u = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    # force exact ties (low 16 bits 0x8000) in a quarter of the samples
    u[::4] = (u[::4] & 0xFFFF0000) | 0x8000
    f = u.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3.0e38)]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.bf16_from_f32(float(x)) for x in f[:20000]], np.uint16)
    assert np.array_equal(got, ref[:20000])


def test_mx_exponent_integer_form(orc):
    """Smallest e with 6*2^e >= amax equals the integer rule: amax = f*2^E,
    f in [1,2): e = E-2 if f <= 1.5 else E-1 (clamped at -127); and every
    BF16 amax then satisfies 3 < amax/2^e <= 6 (no element clips)."""
    bits = np.arange(1, 0x7F80, dtype=np.uint32).astype(np.uint16)  # positive finite
    vals = bf16_to_f32(bits)
    for v in vals[::3].tolist():
        m, E = math.frexp(v)        # v = m * 2^E, m in [0.5, 1)
        f, E = 2 * m, E - 1
        e = E - 2 if f <= 1.5 else E - 1
        e = max(e, -127)
        assert orc.mx_exponent(v) == e, v
        r = v / 2.0 ** e
        assert r <= 6.0
        if e > -127:
            assert r > 3.0
    assert orc.mx_exponent(0.0) == -127


def test_nv_tensor_scale(orc):
    assert orc.nv_tensor_scale(10.5) == 2.0 ** -8
    assert orc.nv_tensor_scale(0.0) == 1.0
    for a in [1.0, 3.14159, 1e-30, 65504.0]:
        assert orc.nv_tensor_scale(a) == float(np.float32(a) / np.float32(2688.0))
