"""Pins for the oracle quantizer (CPU only): hand-derived worked blocks,
the amax/6 scale rules, equivariance and symmetry, residual bounds, grouped
= per-group dense, and lossless round trips of grid-exact inputs."""
import json
import os

import numpy as np
import pytest

from workloads import bf16_bits, bf16_to_f32, dense_case

GOLD = os.path.join(os.path.dirname(__file__), "golden")
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _x_from(values):
    return bf16_bits(np.array([[-0.0 if v == "-0.0" else v for v in values]], np.float32))


def _unpack(q):
    lo, hi = q & 15, q >> 4
    out = np.empty((q.shape[0], q.shape[1] * 2), np.uint8)
    out[:, 0::2], out[:, 1::2] = lo, hi
    return out


def _code_values(codes):
    return np.where(codes & 8, -1.0, 1.0) * GRID[codes & 7]


def _e4m3(code):
    code = np.asarray(code, np.int64)
    e, m = (code >> 3) & 15, code & 7
    return np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * 2.0 ** (e - 7.0))


def test_golden_nvfp4_two_blocks(orc):
    g = _load("nvfp4_two_blocks.json")
    x = _x_from(g["x"])
    out = orc.quantize(orc.NVFP4, x, chan_idx=np.array(g["chan_idx"], np.int32))
    assert out["q"][0].tolist() == g["packed"]
    assert _unpack(out["q"])[0].tolist() == g["codes"]
    assert out["scales"][0].tolist() == g["scales"]
    assert out["tscale"][0] == np.float32(g["tensor_scale"])
    assert out["resid"][0].tolist() == g["resid_bf16_bits"]


def test_golden_mxfp4_two_blocks(orc):
    g = _load("mxfp4_two_blocks.json")
    x = _x_from(g["x"])
    assert x[0, 8] == 0x3DCD
    out = orc.quantize(orc.MXFP4, x, chan_idx=np.array(g["chan_idx"], np.int32))
    assert _unpack(out["q"])[0].tolist() == g["codes"]
    assert out["q"][0].tolist() == g["packed"]
    assert out["scales"][0].tolist() == g["scales"]
    assert out["tscale"] is None
    assert out["resid"][0].tolist() == g["resid_bf16_bits"]


def _case(rows=48, cols=512, seed=11, dist="t4", n_out=5):
    return dense_case(rows, cols, 8, x_dist=dist, n_out=n_out, out_mult=30.0, seed=seed)["x"]


def test_nvfp4_amax_rules(orc):
    x = _case()
    out = orc.quantize(orc.NVFP4, x)
    xf = np.abs(bf16_to_f32(x)).reshape(x.shape[0], -1, 16)
    A = xf.max()
    assert out["tscale"][0] == np.float32(A) / np.float32(2688.0)
    sc = out["scales"]
    bam = xf.max(axis=2)
    # the block holding the tensor amax maps onto the largest E4M3 value 448
    assert np.all(sc[bam == A] == 0x7E)
    # in every block with a normal E4M3 scale (exponent field >= 1) the block
    # amax lands on the largest E2M1 level 6: amax/d lies in [5.65, 6.4]
    codes = _unpack(out["q"]).reshape(x.shape[0], -1, 16)
    normal = (sc >> 3) >= 1
    arg = xf.argmax(axis=2)
    amax_codes = np.take_along_axis(codes, arg[..., None], axis=2)[..., 0]
    assert np.all((amax_codes[normal] & 7) == 7)


def test_mxfp4_amax_rules(orc):
    x = _case(seed=12)
    out = orc.quantize(orc.MXFP4, x)
    xf = np.abs(bf16_to_f32(x)).reshape(x.shape[0], -1, 32)
    bam = xf.max(axis=2)
    e = out["scales"].astype(np.int64) - 127
    r = bam / np.exp2(e.astype(np.float64))
    nz = bam > 0
    assert np.all((r[nz] > 3.0) & (r[nz] <= 6.0))
    codes = _unpack(out["q"]).reshape(x.shape[0], -1, 32)
    amax_codes = np.take_along_axis(codes, xf.argmax(axis=2)[..., None], axis=2)[..., 0]
    assert np.all((amax_codes[nz] & 7) >= 5)   # amax/s in (3, 6] rounds to 3, 4 or 6


@pytest.mark.parametrize("fmt", [0, 1])
def test_power_of_two_equivariance(orc, fmt):
    x = _case(seed=13)
    xf = bf16_to_f32(x)
    base = orc.quantize(fmt, x)
    for k in (-3, 1, 4):
        xs = bf16_bits(xf * np.float32(2.0 ** k))   # exact: no overflow/underflow
        o = orc.quantize(fmt, xs)
        assert np.array_equal(o["q"], base["q"])
        if fmt == orc.NVFP4:
            assert np.array_equal(o["scales"], base["scales"])
            assert o["tscale"][0] == base["tscale"][0] * np.float32(2.0 ** k)
        else:
            assert np.array_equal(o["scales"].astype(int), base["scales"].astype(int) + k)


@pytest.mark.parametrize("fmt", [0, 1])
def test_sign_symmetry_and_row_permutation(orc, fmt):
    x = _case(seed=14)
    S = np.array([3, 40, 41, 300, 511], np.int32)
    base = orc.quantize(fmt, x, chan_idx=S)
    neg = orc.quantize(fmt, x ^ np.uint16(0x8000), chan_idx=S)
    assert np.array_equal(neg["q"], base["q"] ^ np.uint8(0x88))
    assert np.array_equal(neg["scales"], base["scales"])
    rb, rn = bf16_to_f32(base["resid"]), bf16_to_f32(neg["resid"])
    assert np.array_equal(rn, -rb)
    perm = np.random.default_rng(0).permutation(x.shape[0])
    p = orc.quantize(fmt, x[perm], chan_idx=S)
    assert np.array_equal(p["q"], base["q"][perm])
    assert np.array_equal(p["scales"], base["scales"][perm])
    assert np.array_equal(p["resid"], base["resid"][perm])
    if fmt == orc.NVFP4:
        assert p["tscale"][0] == base["tscale"][0]


def _dequant(fmt, out, cols):
    codes = _unpack(out["q"])
    vals = _code_values(codes)
    blk = 16 if fmt == 0 else 32
    sc = np.repeat(out["scales"], blk, axis=1)
    if fmt == 0:
        return vals * _e4m3(sc) * float(out["tscale"][0])
    return vals * np.exp2(sc.astype(np.float64) - 127)


@pytest.mark.parametrize("fmt", [0, 1])
def test_residual_reconstructs_channels(orc, fmt):
    x = _case(seed=15)
    S = np.arange(0, 512, 37, dtype=np.int32)
    out = orc.quantize(fmt, x, chan_idx=S)
    deq = _dequant(fmt, out, x.shape[1])[:, S]
    R = bf16_to_f32(out["resid"]).astype(np.float64)
    xs = bf16_to_f32(x)[:, S].astype(np.float64)
    # R is the BF16 rounding of (x - deq) (with deq rounded once in FP32):
    # the error of deq + R is within half a BF16 ulp of R plus FP32 slack
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(R), 1e-38))) - 7)
    err = np.abs(xs - (deq + R))
    assert np.all(err <= 0.5 * ulp + 1e-6 * np.abs(xs) + 1e-30)
    # compensation beats plain FP4 on these channels
    assert np.abs(xs - (deq + R)).sum() < 0.01 * np.abs(xs - deq).sum()


def test_mxfp4_grid_exact_roundtrip(orc):
    """X = grid value * 2^e per block with every block holding a 6 or a 4:
    quantization is lossless, codes/scales are the ones X was built from and
    the residual is identically zero."""
    rng = np.random.default_rng(16)
    rows, cols = 8, 256
    codes = rng.integers(0, 16, (rows, cols)).astype(np.uint8)
    codes[:, ::32] = 7  # magnitude 6 in every block
    e = rng.integers(-10, 10, (rows, cols // 32))
    xv = _code_values(codes) * np.exp2(np.repeat(e, 32, axis=1).astype(np.float64))
    x = bf16_bits(xv.astype(np.float32))
    out = orc.quantize(orc.MXFP4, x, chan_idx=np.arange(0, cols, 5, dtype=np.int32))
    # zero codes carry their sign; +0 vs -0 is the only freedom
    got = _unpack(out["q"])
    assert np.array_equal(got & 7, codes & 7)
    assert np.array_equal(got[(codes & 7) != 0], codes[(codes & 7) != 0])
    assert np.array_equal(out["scales"].astype(int), e + 127)
    assert not np.any(bf16_to_f32(out["resid"]))


def test_nvfp4_grid_exact_roundtrip(orc):
    """NVFP4 with tensor amax 10.5 (t = 2^-8 exactly) and block amax 6*1.75:
    every block scale is 448, d = 1.75, so X = grid*1.75 is lossless."""
    rng = np.random.default_rng(17)
    codes = rng.integers(0, 16, (6, 128)).astype(np.uint8)
    codes[:, ::16] = 7
    x = bf16_bits((_code_values(codes) * 1.75).astype(np.float32))
    out = orc.quantize(orc.NVFP4, x, chan_idx=np.array([0, 1, 77], np.int32))
    assert out["tscale"][0] == 2.0 ** -8
    assert np.all(out["scales"] == 0x7E)
    got = _unpack(out["q"])
    nz = (codes & 7) != 0
    assert np.array_equal(got[nz], codes[nz])
    assert not np.any(bf16_to_f32(out["resid"]))


@pytest.mark.parametrize("fmt", [0, 1])
def test_grouped_equals_per_group(orc, fmt):
    x = _case(rows=40, seed=18)
    off = np.array([0, 7, 7, 30, 40], np.int32)   # includes an empty group
    G = off.size - 1
    rng = np.random.default_rng(1)
    S = np.sort(np.stack([rng.choice(512, 6, replace=False) for _ in range(G)]), axis=1)
    S = S.astype(np.int32)
    grp = orc.quantize(fmt, x, offsets=off, chan_idx=S)
    for g in range(G):
        a, b = off[g], off[g + 1]
        if a == b:
            if fmt == orc.NVFP4:
                assert grp["tscale"][g] == 1.0
            continue
        d = orc.quantize(fmt, x[a:b], chan_idx=S[g])
        assert np.array_equal(grp["q"][a:b], d["q"])
        assert np.array_equal(grp["scales"][a:b], d["scales"])
        assert np.array_equal(grp["resid"][a:b], d["resid"])
        if fmt == orc.NVFP4:
            assert grp["tscale"][g] == d["tscale"][0]


def test_all_zero_and_tiny(orc):
    x = np.zeros((2, 64), np.uint16)
    x[1, 5] = 0x8000  # -0.0
    o = orc.quantize(orc.NVFP4, x)
    assert o["tscale"][0] == 1.0 and not np.any(o["scales"])
    assert _unpack(o["q"])[1, 5] == 8 and _unpack(o["q"]).sum() == 8
    o = orc.quantize(orc.MXFP4, x)
    assert np.all(o["scales"] == 0)   # e = -127
    # a block far below the tensor amax gets a zero E4M3 scale, so its codes
    # are all (signed) zero and its residual is x itself
    x = bf16_bits(np.array([[1000.0] + [0.0] * 15 + [1e-6, -2e-6] + [0.0] * 14], np.float32))
    o = orc.quantize(orc.NVFP4, x, chan_idx=np.array([16, 17], np.int32))
    assert o["scales"][0, 1] == 0
    assert _unpack(o["q"])[0, 16:18].tolist() == [0, 8]
    assert np.array_equal(o["resid"][0], x[0, 16:18])
