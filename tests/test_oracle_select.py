"""Pins for the oracle's online channel selection (CPU only): the channels
of largest residual magnitude, max over rows of |R|, with R the BF16
residual the quantizer emits.  Checked against the already-pinned quantizer
residual (S = every channel) plus a numpy sort, against constructed ties,
and at the edges k = 0 and k = cols."""
import numpy as np
import pytest

from workloads import bf16_bits, bf16_to_f32, dense_case


def _scores_via_quantizer(orc, fmt, x):
    """Per-channel magnitudes from the quantizer's own residual output with
    every channel selected -- independent of the selection code."""
    K = x.shape[1]
    q = orc.quantize(fmt, x, chan_idx=np.arange(K, dtype=np.int32))
    return np.abs(bf16_to_f32(q["resid"]).astype(np.float64)).max(axis=0), q


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("k", [1, 7, 64, 128])
def test_topk_matches_numpy_sort(orc, fmt, k):
    d = dense_case(40, 256, 8, n_out=5, seed=100 + k + fmt)
    x = d["x"]
    score, _ = _scores_via_quantizer(orc, fmt, x)
    order = np.lexsort((np.arange(score.size), -score))   # score desc, index asc
    want = np.sort(order[:k]).astype(np.int32)
    qx = orc.quantize(fmt, x)
    chan, R = orc.select_channels(fmt, x, qx, k)
    assert np.array_equal(chan, want)
    # the emitted residual is the quantizer's residual on those channels
    ref = orc.quantize(fmt, x, chan_idx=want)["resid"]
    assert np.array_equal(R, ref)


@pytest.mark.parametrize("fmt", [0, 1])
def test_all_and_no_channels(orc, fmt):
    d = dense_case(16, 128, 8, n_out=2, seed=7 + fmt)
    x = d["x"]
    qx = orc.quantize(fmt, x)
    chan, R = orc.select_channels(fmt, x, qx, 128)
    assert np.array_equal(chan, np.arange(128))
    assert np.array_equal(R, orc.quantize(fmt, x, chan_idx=np.arange(128, dtype=np.int32))["resid"])
    chan0, R0 = orc.select_channels(fmt, x, qx, 0)
    assert chan0.size == 0 and R0.shape == (16, 0)
    with pytest.raises(ValueError):
        orc.select_channels(fmt, x, qx, 129)


def test_ties_go_to_the_lower_index(orc):
    """Columns 5, 9, 20 and 33 are copies of one column, so their residual
    magnitudes tie; with the top-2 boundary inside the tie, 5 and 9 win.
    Every other column is zero (zero residual, ranked last)."""
    rng = np.random.default_rng(3)
    x = np.zeros((8, 128), np.float32)
    col = rng.standard_normal(8).astype(np.float32) * 3.0
    for c in (5, 9, 20, 33):
        x[:, c] = col
    xb = bf16_bits(x)
    for fmt in (0, 1):
        qx = orc.quantize(fmt, xb)
        score, _ = _scores_via_quantizer(orc, fmt, xb)
        assert score[5] == score[9] == score[20] == score[33] > 0
        chan, _ = orc.select_channels(fmt, xb, qx, 2)
        assert chan.tolist() == [5, 9]
        chan, _ = orc.select_channels(fmt, xb, qx, 6)   # 4 tied, then the zero columns 0, 1
        assert chan.tolist() == [0, 1, 5, 9, 20, 33]


def test_grid_exact_columns_rank_last(orc):
    """A block of columns already on the MXFP4 grid (every entry +-0.5, so
    the block scale is 2^-3 and 0.5 is code 4) has zero residual; its
    columns are picked only after every column with a nonzero residual."""
    d = dense_case(24, 128, 8, x_dist="normal", seed=12)
    x = bf16_to_f32(d["x"]).copy()
    x[:, 32:64] = np.where(x[:, 32:64] < 0, -0.5, 0.5)
    xb = bf16_bits(x)
    qx = orc.quantize(1, xb)
    score, _ = _scores_via_quantizer(orc, 1, xb)
    assert np.all(score[32:64] == 0)
    nz = int((score > 0).sum())
    chan, _ = orc.select_channels(1, xb, qx, nz)
    assert not set(range(32, 64)) & set(chan.tolist())
    chan, _ = orc.select_channels(1, xb, qx, nz + 3)     # then the lowest zero-score ones
    assert set(chan.tolist()) - set(np.flatnonzero(score > 0).tolist()) == {32, 33, 34}
