"""Pins for the oracle's second-pass residual (CPU only): the compensation
term deq(Q(R)) * deq(W)[:,S]^T, with R[:,S] quantized a second time as an
M x |S| tensor.  Checked against what the definition forces, not against a
retyping of it: residuals that quantize losslessly reduce it exactly to the
already-pinned BF16 compensation; a zero residual adds nothing; negating R
negates the term; and its distance from the BF16 compensation stays inside
the FP4 error bound of the residual blocks."""
import numpy as np
import pytest

from workloads import bf16_bits, bf16_to_f32, dense_case

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
BLK = {0: 16, 1: 32}


def _lossless_resid(rng, fmt, rows, nS):
    """R whose second-pass quantization is exact.  MXFP4: grid * 2^e with a
    6 * 2^e in every block.  NVFP4: grid * 1.75 with 10.5 = 6 * 1.75 in every
    block, so t = 10.5 / 2688 = 2^-8, the block scale is 448 and d = 1.75."""
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


def _operands(orc, fmt, M, K, N, nS, seed):
    d = dense_case(M, K, N, n_out=3, seed=seed)
    S = np.sort(np.random.default_rng(seed).choice(K, nS, replace=False)).astype(np.int32)
    qa = orc.quantize(fmt, d["x"], chan_idx=S)
    qb = orc.quantize(fmt, d["wt"])
    ta = float(qa["tscale"][0]) if fmt == 0 else 1.0
    tb = float(qb["tscale"][0]) if fmt == 0 else 1.0
    return qa, qb, ta, tb, S


def _r4(orc, fmt, qa, qb, ta, tb, S, R_bits):
    qr = orc.quantize_residual(fmt, R_bits)
    tr = float(qr["tscale"][0]) if fmt == 0 else 1.0
    return orc.gemm_full_r4(fmt, qa["q"], qa["scales"], ta, qb["q"], qb["scales"], tb, S,
                            qr["q"], qr["scales"], tr)


@pytest.mark.parametrize("fmt", [0, 1])
def test_lossless_residual_equals_bf16_compensation(orc, fmt):
    M, K, N, nS = 12, 256, 20, 2 * BLK[fmt]
    qa, qb, ta, tb, S = _operands(orc, fmt, M, K, N, nS, seed=31 + fmt)
    R = bf16_bits(_lossless_resid(np.random.default_rng(5 + fmt), fmt, M, nS))
    assert np.array_equal(bf16_to_f32(R), _lossless_resid(np.random.default_rng(5 + fmt), fmt, M, nS))
    y4, ya4 = _r4(orc, fmt, qa, qb, ta, tb, S, R)
    y, ya = orc.gemm_full(fmt, qa["q"], qa["scales"], ta, qb["q"], qb["scales"], tb, S, R)
    assert np.array_equal(y4, y) and np.array_equal(ya4, ya)


@pytest.mark.parametrize("fmt", [0, 1])
def test_zero_residual_adds_nothing(orc, fmt):
    M, K, N, nS = 9, 128, 17, BLK[fmt]
    qa, qb, ta, tb, S = _operands(orc, fmt, M, K, N, nS, seed=41 + fmt)
    Z = np.zeros((M, nS), np.uint16)
    y4, _ = _r4(orc, fmt, qa, qb, ta, tb, S, Z)
    y0, _ = orc.gemm_full(fmt, qa["q"], qa["scales"], ta, qb["q"], qb["scales"], tb, None, None)
    assert np.array_equal(y4, y0)


@pytest.mark.parametrize("fmt", [0, 1])
def test_negated_residual_negates_the_term(orc, fmt):
    M, K, N, nS = 10, 256, 24, 2 * BLK[fmt]
    qa, qb, ta, tb, S = _operands(orc, fmt, M, K, N, nS, seed=51 + fmt)
    R = qa["resid"]
    y_pos, _ = _r4(orc, fmt, qa, qb, ta, tb, S, R)
    y_neg, _ = _r4(orc, fmt, qa, qb, ta, tb, S, R ^ np.uint16(0x8000))
    y0, ya0 = orc.gemm_full(fmt, qa["q"], qa["scales"], ta, qb["q"], qb["scales"], tb, None, None)
    assert np.allclose((y_pos + y_neg) / 2, y0, rtol=0, atol=1e-12 * ya0.max())
    assert not np.allclose(y_pos, y0)          # the term is really there


@pytest.mark.parametrize("fmt", [0, 1])
def test_distance_from_bf16_compensation_within_fp4_bound(orc, fmt):
    """|deq(Q(r)) - r| <= amax_block / 4 for every element (half the widest
    grid gap, 1 of 6, plus scale rounding), so the two compensations differ
    by at most sum_j amax_block(j) / 4 * |W_deq[n, S_j]|."""
    M, K, N, nS = 16, 256, 20, 2 * BLK[fmt]
    qa, qb, ta, tb, S = _operands(orc, fmt, M, K, N, nS, seed=61 + fmt)
    R = qa["resid"]
    y4, _ = _r4(orc, fmt, qa, qb, ta, tb, S, R)
    y, _ = orc.gemm_full(fmt, qa["q"], qa["scales"], ta, qb["q"], qb["scales"], tb, S, R)
    # W_deq[:, S] through an identity activation, as in the BF16 compensation pin
    ident = bf16_bits(np.eye(K, dtype=np.float32))
    qi = orc.quantize(fmt, ident)
    ti = float(qi["tscale"][0]) if fmt == 0 else 1.0
    wdeq, _ = orc.gemm_full(fmt, qi["q"], qi["scales"], ti, qb["q"], qb["scales"], tb, None, None)
    if fmt == 0:
        wdeq = wdeq / (2688.0 * ti)
    rv = np.abs(bf16_to_f32(R).astype(np.float64))
    amax_blk = np.repeat(rv.reshape(M, nS // BLK[fmt], BLK[fmt]).max(axis=2), BLK[fmt], axis=1)
    bound = (amax_blk / 4.0) @ np.abs(wdeq[S, :]) * (1 + 1e-9)
    diff = np.abs(y4 - y)
    assert np.all(diff <= bound + 1e-12)
    assert diff.max() > 0                       # a second pass that changed nothing would pass


@pytest.mark.parametrize("fmt", [0, 1])
def test_r4_points_match_full(orc, fmt):
    M, K, N, nS = 8, 128, 12, BLK[fmt]
    qa, qb, ta, tb, S = _operands(orc, fmt, M, K, N, nS, seed=71 + fmt)
    qr = orc.quantize_residual(fmt, qa["resid"])
    tr = float(qr["tscale"][0]) if fmt == 0 else 1.0
    yf, yaf = orc.gemm_full_r4(fmt, qa["q"], qa["scales"], ta, qb["q"], qb["scales"], tb, S,
                               qr["q"], qr["scales"], tr)
    pm = np.repeat(np.arange(M), N)
    pn = np.tile(np.arange(N), M)
    yp, yap = orc.gemm_points_r4(fmt, qa["q"], qa["scales"], ta, qb["q"], qb["scales"], tb, S,
                                 qr["q"], qr["scales"], tr, pm, pn)
    assert np.array_equal(yp, yf.ravel()) and np.array_equal(yap, yaf.ravel())


def test_r4_rejects_partial_blocks(orc):
    qa, qb, ta, tb, S = _operands(orc, 0, 4, 128, 8, 8, seed=81)
    with pytest.raises(ValueError):
        orc.gemm_full_r4(0, qa["q"], qa["scales"], ta, qb["q"], qb["scales"], tb, S,
                         np.zeros((4, 4), np.uint8), np.zeros((4, 1), np.uint8), 1.0)
