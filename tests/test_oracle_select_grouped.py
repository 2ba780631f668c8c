"""Pins for the oracle's grouped online channel selection (CPU only): the MoE
form of the QUADS explainer's top-k residual mask (section 2.2 B; the QUADS
abstract places the method in MoE rollout).  Checked against what the
definition forces: one group is the pinned single-group selection; each
group's choice is the single-group selection over its rows quantized on
their own (the grouped quantizer's per-group tensor scale is pinned equal to
that); an empty group has all-zero magnitudes and takes the first k
channels; a group's choice does not depend on the other groups' rows; k =
cols gives every channel and the quantizer's own residual."""
import numpy as np
import pytest

from workloads import dense_case


def _x(rows, cols, seed):
    return dense_case(rows, cols, 8, n_out=4, out_mult=30.0, seed=seed)["x"]


@pytest.mark.parametrize("fmt", [0, 1])
def test_one_group_is_the_single_group_selection(orc, fmt):
    x = _x(40, 256, 5 + fmt)
    off = np.array([0, 40], np.int32)
    qx = orc.quantize(fmt, x, offsets=off)
    chan, R = orc.select_channels_grouped(fmt, x, qx, off, 24)
    c1, R1 = orc.select_channels(fmt, x, orc.quantize(fmt, x), 24)
    assert np.array_equal(chan[0], c1) and np.array_equal(R, R1)


@pytest.mark.parametrize("fmt", [0, 1])
def test_each_group_selects_from_its_own_rows(orc, fmt):
    off = np.array([0, 7, 7, 30, 31, 64], np.int32)
    x = _x(64, 256, 11 + fmt)
    qx = orc.quantize(fmt, x, offsets=off)
    k = 16
    chan, R = orc.select_channels_grouped(fmt, x, qx, off, k)
    for g in range(off.size - 1):
        r0, r1 = off[g], off[g + 1]
        if r1 == r0:
            assert np.array_equal(chan[g], np.arange(k))   # all magnitudes zero: the tie rule
            continue
        cg, Rg = orc.select_channels(fmt, x[r0:r1], orc.quantize(fmt, x[r0:r1]), k)
        assert np.array_equal(chan[g], cg)
        assert np.array_equal(R[r0:r1], Rg)
    assert not all(np.array_equal(chan[0], chan[g]) for g in (2, 4))


def test_groups_are_independent(orc):
    fmt = 0
    off = np.array([0, 20, 45], np.int32)
    x = _x(45, 256, 21)
    y = x.copy()
    y[:20] = _x(20, 256, 99)                 # other rows in group 0
    ca, Ra = orc.select_channels_grouped(fmt, x, orc.quantize(fmt, x, offsets=off), off, 12)
    cb, Rb = orc.select_channels_grouped(fmt, y, orc.quantize(fmt, y, offsets=off), off, 12)
    assert np.array_equal(ca[1], cb[1]) and np.array_equal(Ra[20:], Rb[20:])
    assert not np.array_equal(ca[0], cb[0])


@pytest.mark.parametrize("fmt", [0, 1])
def test_all_channels(orc, fmt):
    off = np.array([0, 9, 30], np.int32)
    x = _x(30, 128, 31 + fmt)
    qx = orc.quantize(fmt, x, offsets=off)
    chan, R = orc.select_channels_grouped(fmt, x, qx, off, 128)
    assert np.array_equal(chan, np.tile(np.arange(128), (2, 1)))
    full = orc.quantize(fmt, x, offsets=off, chan_idx=np.tile(np.arange(128, dtype=np.int32),
                                                              (2, 1)))
    assert np.array_equal(R, full["resid"])
