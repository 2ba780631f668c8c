"""Pins for the oracle's grouped second-pass residual (CPU only): the MoE
form of the QUADS explainer's second-pass quantization (section 2.2 B; the
QUADS abstract places the method in MoE rollout), each expert's residual
R[rows_g, S_g] quantized with its own tensor scale.  Checked against what the
definition forces: one group is the pinned dense form; residuals that
quantize losslessly reduce it exactly to the pinned grouped BF16
compensation (empty and single-row groups included); a group's residual
scale changes that group's rows only, as the dense form of those rows
predicts."""
import numpy as np
import pytest

from workloads import bf16_bits, bf16_to_f32, dense_case

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
BLK = {0: 16, 1: 32}


def _lossless_resid(rng, fmt, rows, nS):
    """R whose second-pass quantization is exact (per group: a full-scale
    entry in every block; NVFP4 amax 10.5 gives t = 2^-8 and d = 1.75)."""
    blk = BLK[fmt]
    codes = rng.integers(0, 16, (rows, nS)).astype(np.uint8)
    codes[:, ::blk] = 7
    mag = GRID[codes & 7] * np.where(codes & 8, -1.0, 1.0)
    if fmt == 1:
        e = rng.integers(-9, -2, (rows, nS // blk))
        v = mag * np.exp2(np.repeat(e, blk, axis=1).astype(np.float64))
    else:
        v = mag * 1.75
    return v.astype(np.float32)


def _operands(orc, fmt, off, K, N, nS, seed):
    G = len(off) - 1
    x = dense_case(int(off[-1]), K, 8, n_out=3, seed=seed)["x"]
    wts = [dense_case(1, K, N, seed=seed + 10 + g)["wt"] for g in range(G)]
    rng = np.random.default_rng(seed)
    chan = np.sort(np.stack([rng.choice(K, nS, replace=False) for _ in range(G)]), 1)
    chan = chan.astype(np.int32)
    qa = orc.quantize(fmt, x, offsets=off, chan_idx=chan)
    qbs = [orc.quantize(fmt, w) for w in wts]
    bq = np.stack([q["q"] for q in qbs])
    bs = np.stack([q["scales"] for q in qbs])
    bts = np.array([q["tscale"][0] for q in qbs], np.float32) if fmt == 0 else None
    ats = qa["tscale"] if fmt == 0 else None
    return qa, ats, bq, bs, bts, chan


def _points(rows, N):
    return np.repeat(np.arange(rows), N), np.tile(np.arange(N), rows)


def _r4(orc, fmt, off, qa, ats, bq, bs, bts, chan, R_bits):
    qr = orc.quantize(fmt, R_bits, offsets=off)
    pm, pn = _points(int(off[-1]), bq.shape[1])
    return orc.grouped_gemm_points_r4(fmt, off, qa["q"], qa["scales"], ats, bq, bs, bts, chan,
                                      qr["q"], qr["scales"], qr["tscale"], pm, pn), qr


@pytest.mark.parametrize("fmt", [0, 1])
def test_one_group_is_the_dense_form(orc, fmt):
    off = np.array([0, 24], np.int32)
    K, N, nS = 256, 12, 2 * BLK[fmt]
    qa, ats, bq, bs, bts, chan = _operands(orc, fmt, off, K, N, nS, seed=61 + fmt)
    (y, ya), qr = _r4(orc, fmt, off, qa, ats, bq, bs, bts, chan, qa["resid"])
    qd = orc.quantize_residual(fmt, qa["resid"])
    assert np.array_equal(qr["q"], qd["q"]) and np.array_equal(qr["scales"], qd["scales"])
    pm, pn = _points(24, N)
    yd, yad = orc.gemm_points_r4(fmt, qa["q"], qa["scales"], 1.0 if ats is None else ats[0],
                                 bq[0], bs[0], 1.0 if bts is None else bts[0], chan[0],
                                 qd["q"], qd["scales"],
                                 1.0 if fmt == 1 else float(qd["tscale"][0]), pm, pn)
    assert np.array_equal(y, yd) and np.array_equal(ya, yad)


@pytest.mark.parametrize("fmt", [0, 1])
def test_lossless_residual_equals_grouped_bf16_compensation(orc, fmt):
    off = np.array([0, 5, 5, 17, 18, 40], np.int32)   # an empty and a single-row group
    K, N, nS = 256, 10, 2 * BLK[fmt]
    qa, ats, bq, bs, bts, chan = _operands(orc, fmt, off, K, N, nS, seed=71 + fmt)
    rng = np.random.default_rng(3 + fmt)
    Rf = np.concatenate([_lossless_resid(rng, fmt, int(off[g + 1] - off[g]), nS)
                         for g in range(off.size - 1)])
    R = bf16_bits(Rf)
    assert np.array_equal(bf16_to_f32(R), Rf)
    (y4, ya4), _ = _r4(orc, fmt, off, qa, ats, bq, bs, bts, chan, R)
    pm, pn = _points(int(off[-1]), N)
    y, ya = orc.grouped_gemm_points(fmt, off, qa["q"], qa["scales"], ats, bq, bs, bts, chan, R,
                                    pm, pn)
    assert np.array_equal(y4, y) and np.array_equal(ya4, ya)


def test_each_group_has_its_own_residual_scale(orc):
    """NVFP4: four times group 1's residual gives group 1 a four times larger
    residual tensor scale (same codes); every other group's output is
    unchanged bit for bit, and group 1's equals the dense form of its rows
    with the scaled residual."""
    fmt = 0
    off = np.array([0, 9, 30, 44], np.int32)
    K, N, nS = 256, 8, 32
    qa, ats, bq, bs, bts, chan = _operands(orc, fmt, off, K, N, nS, seed=83)
    R = qa["resid"]
    R4 = R.copy()
    R4[9:30] = bf16_bits(bf16_to_f32(R[9:30]) * np.float32(4.0))
    (y, _), qr = _r4(orc, fmt, off, qa, ats, bq, bs, bts, chan, R)
    (y4, _), qr4 = _r4(orc, fmt, off, qa, ats, bq, bs, bts, chan, R4)
    assert qr4["tscale"][1] == 4 * qr["tscale"][1]
    assert qr4["tscale"][0] == qr["tscale"][0] and qr4["tscale"][2] == qr["tscale"][2]
    assert np.array_equal(qr4["q"], qr["q"])
    rows = np.repeat(np.arange(44), N)
    other = (rows < 9) | (rows >= 30)
    assert np.array_equal(y4[other], y[other])
    assert not np.array_equal(y4[~other], y[~other])
    qd = orc.quantize_residual(fmt, R4[9:30])
    pm, pn = _points(21, N)
    yd, _ = orc.gemm_points_r4(fmt, qa["q"][9:30], qa["scales"][9:30], ats[1], bq[1], bs[1],
                               bts[1], chan[1], qd["q"], qd["scales"], float(qd["tscale"][0]),
                               pm, pn)
    assert np.array_equal(y4[~other], yd)
