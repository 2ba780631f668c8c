"""Pins for the oracle GEMM (CPU only): the hand-derived 1x2 product, inputs
that quantize losslessly (then Y must equal the plain matmul of the inputs
themselves), the identity weight, compensation on every channel (an A16W4
product up to BF16 rounding of R), points == full, and grouped == per-group
dense."""
import json
import os

import numpy as np
import pytest

from workloads import bf16_bits, bf16_to_f32, dense_case

GOLD = os.path.join(os.path.dirname(__file__), "golden")
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _unpack(q):
    out = np.empty((q.shape[0], q.shape[1] * 2), np.uint8)
    out[:, 0::2], out[:, 1::2] = q & 15, q >> 4
    return out


def _quant(orc, fmt, x, S=None):
    return orc.quantize(fmt, x, chan_idx=S)


def _gemm_full(orc, fmt, qa, qb, S):
    ta = qa["tscale"][0] if fmt == 0 else 1.0
    tb = qb["tscale"][0] if fmt == 0 else 1.0
    return orc.gemm_full(fmt, qa["q"], qa["scales"], ta, qb["q"], qb["scales"], tb, S,
                         qa["resid"])


def test_golden_mxfp4_gemm(orc):
    g = json.load(open(os.path.join(GOLD, "mxfp4_gemm_1x2.json")))
    a = json.load(open(os.path.join(GOLD, g["activation_fixture"])))
    x = bf16_bits(np.array([a["x"]], np.float32))
    w = np.zeros((2, 64), np.float32)
    for r, ent in g["w_rows"].items():
        for k, v in ent.items():
            w[int(r), int(k)] = v
    S = np.array(a["chan_idx"], np.int32)
    qa = _quant(orc, orc.MXFP4, x, S)
    qb = _quant(orc, orc.MXFP4, bf16_bits(w))
    y, ya = _gemm_full(orc, orc.MXFP4, qa, qb, S)
    assert y[0].tolist() == g["y"]
    assert ya[0].tolist() == g["yabs"]


def _grid_exact(rng, rows, cols, blk, e_lo, e_hi):
    codes = rng.integers(0, 16, (rows, cols)).astype(np.uint8)
    codes[:, ::blk] = 7
    e = rng.integers(e_lo, e_hi, (rows, cols // blk))
    v = np.where(codes & 8, -1.0, 1.0) * GRID[codes & 7] * np.exp2(
        np.repeat(e, blk, axis=1).astype(np.float64))
    return v.astype(np.float32)


def test_mxfp4_lossless_inputs_give_plain_matmul(orc):
    rng = np.random.default_rng(21)
    M, K, N = 24, 256, 40
    xv = _grid_exact(rng, M, K, 32, -6, 4)
    wv = _grid_exact(rng, N, K, 32, -8, -2)
    S = np.array([1, 2, 100, 255], np.int32)
    qa = _quant(orc, orc.MXFP4, bf16_bits(xv), S)
    qb = _quant(orc, orc.MXFP4, bf16_bits(wv))
    y, ya = _gemm_full(orc, orc.MXFP4, qa, qb, S)
    ref = xv.astype(np.float64) @ wv.astype(np.float64).T      # the definition itself
    assert np.array_equal(y, ref)
    assert np.array_equal(ya, np.abs(xv.astype(np.float64)) @ np.abs(wv.astype(np.float64)).T)


def test_nvfp4_lossless_inputs_give_plain_matmul(orc):
    """t = 2^-8 exactly when the tensor amax is 10.5; with every block amax
    10.5 the block scale is 448 and d = 1.75, so grid*1.75 is lossless."""
    rng = np.random.default_rng(22)
    M, K, N = 20, 128, 36
    cx = rng.integers(0, 16, (M, K)).astype(np.uint8)
    cx[:, ::16] = 7
    cw = rng.integers(0, 16, (N, K)).astype(np.uint8)
    cw[:, ::16] = 7
    val = lambda c: np.where(c & 8, -1.0, 1.0) * GRID[c & 7] * 1.75
    xv, wv = val(cx).astype(np.float32), val(cw).astype(np.float32)
    S = np.array([0, 64, 127], np.int32)
    qa = _quant(orc, orc.NVFP4, bf16_bits(xv), S)
    qb = _quant(orc, orc.NVFP4, bf16_bits(wv))
    y, ya = _gemm_full(orc, orc.NVFP4, qa, qb, S)
    ref = xv.astype(np.float64) @ wv.astype(np.float64).T
    assert np.allclose(y, ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_identity_weight(orc):
    """W = I: each W^T row has one 1; its block gets scale 448 and code 7, so
    W_deq = 6*448*t_w*I with t_w = fl(1/2688) (1 up to one FP32 rounding):
    Y = (deq(Xq) + R on S) * 2688 * t_w."""
    K = 256
    d = dense_case(16, K, 8, x_dist="normal", n_out=4, out_mult=50.0, seed=1)
    x = d["x"]
    S = np.array([5, 17, 200], np.int32)
    qa = _quant(orc, orc.NVFP4, x, S)
    qb = _quant(orc, orc.NVFP4, bf16_bits(np.eye(K, dtype=np.float32)))
    tw = float(qb["tscale"][0])
    assert tw == float(np.float32(1.0) / np.float32(2688.0))
    y, _ = _gemm_full(orc, orc.NVFP4, qa, qb, S)
    codes = _unpack(qa["q"])
    e4 = lambda c: np.where((c >> 3) & 15 == 0, (c & 7) / 8 * 2.0 ** -6,
                            (1 + (c & 7) / 8) * 2.0 ** (((c >> 3) & 15).astype(float) - 7))
    sx = np.repeat(e4(qa["scales"].astype(np.int64)), 16, axis=1)
    deqx = np.where(codes & 8, -1.0, 1.0) * GRID[codes & 7] * sx * float(qa["tscale"][0])
    deqx[:, S] += bf16_to_f32(qa["resid"])
    assert np.allclose(y, deqx * 2688.0 * tw, rtol=1e-12, atol=0)
    # and that is the input up to FP4 error off S, BF16 rounding on S
    xs = bf16_to_f32(x)[:, S]
    assert np.allclose(y[:, S], xs, rtol=2 ** -8, atol=1e-6)


@pytest.mark.parametrize("fmt", [0, 1])
def test_all_channels_compensated_is_a16w4(orc, fmt):
    """S = every channel: X's FP4 error is replaced by R, so Y = X * W_deq^T
    up to the BF16 rounding of R (bounded by 2^-9 |R| per term)."""
    d = dense_case(12, 128, 20, seed=23)
    x, wt = d["x"], d["wt"]
    S = np.arange(128, dtype=np.int32)
    qa = _quant(orc, fmt, x, S)
    qb = _quant(orc, fmt, wt)
    y, _ = _gemm_full(orc, fmt, qa, qb, S)
    # W_deq through an identity activation: Y_I = I * W_deq^T
    ident = bf16_bits(np.eye(128, dtype=np.float32))
    qi = _quant(orc, fmt, ident)
    wdeq, _ = _gemm_full(orc, fmt, qi, qb, None)   # [128(k), N]: 2688*t_i*W_deq^T for NVFP4
    if fmt == 0:
        wdeq = wdeq / (2688.0 * float(qi["tscale"][0]))
    xv = bf16_to_f32(x).astype(np.float64)
    R = np.abs(bf16_to_f32(qa["resid"]).astype(np.float64))
    ref = xv @ wdeq
    bound = 2.0 ** -8 * (R @ np.abs(wdeq)) + 1e-9 * (np.abs(xv) @ np.abs(wdeq))
    assert np.all(np.abs(y - ref) <= bound)


@pytest.mark.parametrize("fmt", [0, 1])
def test_points_match_full_and_yabs(orc, fmt):
    d = dense_case(10, 256, 30, seed=24)
    S = np.array([3, 99, 250], np.int32)
    qa, qb = _quant(orc, fmt, d["x"], S), _quant(orc, fmt, d["wt"])
    y, ya = _gemm_full(orc, fmt, qa, qb, S)
    rng = np.random.default_rng(2)
    pm, pn = rng.integers(0, 10, 50), rng.integers(0, 30, 50)
    ta = qa["tscale"][0] if fmt == 0 else 1.0
    tb = qb["tscale"][0] if fmt == 0 else 1.0
    yp, yap = orc.gemm_points(fmt, qa["q"], qa["scales"], ta, qb["q"], qb["scales"], tb, S,
                              qa["resid"], pm, pn)
    assert np.array_equal(yp, y[pm, pn]) and np.array_equal(yap, ya[pm, pn])
    assert np.all(ya >= np.abs(y))
    # no compensation -> plain W4A4
    y0, _ = _gemm_full(orc, fmt, qa, qb, None)
    assert not np.array_equal(y0, y)


@pytest.mark.parametrize("fmt", [0, 1])
def test_grouped_points_equal_dense(orc, fmt):
    rng = np.random.default_rng(25)
    K, N, G = 128, 24, 3
    off = np.array([0, 5, 5, 17], np.int32)
    x = dense_case(17, K, 8, seed=26)["x"]
    W = np.stack([dense_case(1, K, N, seed=30 + g)["wt"] for g in range(G)])
    S = np.sort(np.stack([rng.choice(K, 4, replace=False) for _ in range(G)]), 1)
    S = S.astype(np.int32)
    qa = orc.quantize(fmt, x, offsets=off, chan_idx=S)
    qbs = [orc.quantize(fmt, W[g]) for g in range(G)]
    bq = np.stack([q["q"] for q in qbs])
    bs = np.stack([q["scales"] for q in qbs])
    bts = np.array([q["tscale"][0] for q in qbs], np.float32) if fmt == 0 else None
    pm = np.repeat(np.arange(17), N)
    pn = np.tile(np.arange(N), 17)
    y, ya = orc.grouped_gemm_points(fmt, off, qa["q"], qa["scales"], qa["tscale"], bq, bs, bts,
                                    S, qa["resid"], pm, pn)
    y = y.reshape(17, N)
    for g in range(G):
        a, b = off[g], off[g + 1]
        if a == b:
            continue
        ta = qa["tscale"][g] if fmt == 0 else 1.0
        tb = bts[g] if fmt == 0 else 1.0
        yd, _ = orc.gemm_full(fmt, qa["q"][a:b], qa["scales"][a:b], ta, bq[g], bs[g], tb, S[g],
                              qa["resid"][a:b])
        assert np.array_equal(y[a:b], yd)
