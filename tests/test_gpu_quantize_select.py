"""GPU parity of fp4q_quantize_select (quantization with the online channel
selection's scores taken in the same pass over x), through the C ABI,
against the oracle's quantize followed by its channel selection: codes,
block scales, tensor scale, chosen channels and the residual on them bit for
bit.  Both formats and layouts; tiles of 16, 32 and 64 rows (128-, 64- and
32-column row-major tensors); one band of row tiles and several; partial
maxima picked directly, reduced by the pick kernel and by a launch of their
own; more columns than the pick keeps in LDS; ragged rows; constructed ties;
a column count that takes the two-step path; no rows; k = 0, 1 and cols;
the workloads' full sizes; and equality with the two calls on the GPU."""
import numpy as np
import pytest
import torch

import fp4_w4a4_quantized_amd as fq
from gpu_helpers import assert_quant_equal, need_gpu, say, to_dev, to_host
from workloads import CONFIGS, bf16_bits, dense_case

pytestmark = pytest.mark.gpu


def _check(orc, fmt, x, k, layout):
    qx = orc.quantize(fmt, x)
    want_c, want_r = orc.select_channels(fmt, x, qx, k)
    a, chan, R = fq.quantize_select(fmt, to_dev(x), k, layout=layout)
    torch.cuda.synchronize()
    assert_quant_equal(dict(a, resid=None), qx, fmt)
    got_c, got_r = to_host(chan), to_host(R)
    assert np.array_equal(got_c, want_c), (got_c[:16], want_c[:16])
    bad = np.argwhere(got_r != want_r)
    assert bad.size == 0, f"resid: {len(bad)} mismatches, first {bad[:3].tolist()}"
    return got_c


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("layout", [fq.ROWMAJOR, fq.TILED])
@pytest.mark.parametrize("M,K,k", [(16, 256, 7),      # one row tile
                                   (40, 256, 64),     # three row tiles, ragged last
                                   (300, 512, 33),    # three bands, reduced while picking
                                   (64, 640, 1),      # five column tiles
                                   (129, 1024, 128),  # one row past a band
                                   (2050, 1024, 40),  # seventeen bands
                                   (20, 32768, 100),  # scores too many for LDS, one band
                                   (300, 32768, 50)])  # and three bands: the reduction launch
def test_quantize_select_matches_oracle(orc, fmt, layout, M, K, k):
    need_gpu()
    say(f"quantize_select fmt {fmt} layout {layout} M{M} K{K} k{k}")
    d = dense_case(M, K, 8, n_out=max(1, K // 64), seed=M * 5 + K + k + fmt)
    _check(orc, fmt, d["x"], k, layout)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("M,K,k", [(37, 32, 5),     # one unit per row: 64-row tiles
                                   (70, 64, 64),    # two units: 32-row tiles, all channels
                                   (100, 96, 10),   # three units in a four-unit tile
                                   (515, 160, 3)])  # five units, ragged column tile
def test_quantize_select_narrow_rowmajor(orc, fmt, M, K, k):
    need_gpu()
    say(f"quantize_select narrow fmt {fmt} M{M} K{K} k{k}")
    d = dense_case(M, K, 8, n_out=max(1, K // 32), seed=M + K * 3 + fmt)
    _check(orc, fmt, d["x"], k, fq.ROWMAJOR)


def test_quantize_select_two_step_columns(orc):
    """48 NVFP4 columns (not a multiple of 32): the two steps, same results."""
    need_gpu()
    say("quantize_select NVFP4 K48")
    d = dense_case(37, 48, 8, n_out=3, seed=21)
    _check(orc, 0, d["x"], 5, fq.ROWMAJOR)
    _check(orc, 0, d["x"], 48, fq.ROWMAJOR)


@pytest.mark.parametrize("fmt", [0, 1])
def test_quantize_select_ties_and_zero_columns(orc, fmt):
    """Four copies of one column tie; the top-k boundary falls inside the tie
    and in a run of all-zero columns: lower indices win."""
    need_gpu()
    say(f"quantize_select ties fmt {fmt}")
    rng = np.random.default_rng(9 + fmt)
    x = np.zeros((150, 1024), np.float32)
    col = rng.standard_normal(150).astype(np.float32) * 3.0
    for c in (5, 9, 300, 700):
        x[:, c] = col
    x[:, 900] = col * 8.0
    xb = bf16_bits(x)
    for k in (2, 3, 5, 6, 40):
        got = _check(orc, fmt, xb, k, fq.TILED)
        if k == 3:
            assert got.tolist() == [5, 9, 900]
        if k == 6:
            assert got.tolist() == [0, 5, 9, 300, 700, 900]


def test_quantize_select_no_rows_and_k0(orc):
    """No rows: the first k channels (every magnitude is 0); k = 0: codes only."""
    need_gpu()
    say("quantize_select rows 0 / k 0")
    for fmt in (0, 1):
        x = torch.empty((0, 256), dtype=torch.int16, device="cuda:0")
        a, chan, R = fq.quantize_select(fmt, x, 10)
        torch.cuda.synchronize()
        assert to_host(chan).tolist() == list(range(10)) and R.shape == (0, 10)
        d = dense_case(33, 256, 8, n_out=2, seed=3 + fmt)
        a, chan, R = fq.quantize_select(fmt, to_dev(d["x"]), 0)
        torch.cuda.synchronize()
        assert chan.numel() == 0
        assert_quant_equal(dict(a, resid=None), orc.quantize(fmt, d["x"]), fmt)


@pytest.mark.parametrize("name", ["decode_nvfp4", "prefill_nvfp4", "prefill_mxfp4"])
def test_quantize_select_full_size(orc, name):
    """The workloads' full activation shapes, k = the workload's channel
    count, tiled as the GEMM takes them."""
    need_gpu()
    cfg = CONFIGS[name]
    fmt = 0 if cfg["fmt"] == "nvfp4" else 1
    say(f"quantize_select full size {name}")
    d = dense_case(**{**cfg, "N": 8})
    _check(orc, fmt, d["x"], cfg["n_s"], fq.TILED)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("layout", [fq.ROWMAJOR, fq.TILED])
def test_quantize_select_equals_two_calls(fmt, layout):
    """Against fp4q_quantize then fp4q_select_channels on the GPU, at the
    prefill activation size, twice in a row (the workspace's state)."""
    need_gpu()
    say(f"quantize_select vs two calls fmt {fmt} layout {layout}")
    cfg = CONFIGS["prefill_nvfp4"]
    d = dense_case(**{**cfg, "N": 8})
    x = to_dev(d["x"])
    k = cfg["n_s"]
    a2 = fq.quantize(fmt, x, layout=layout)
    c2, r2 = fq.select_channels(fmt, x, a2, k)
    for _ in range(2):
        a1, c1, r1 = fq.quantize_select(fmt, x, k, layout=layout)
        torch.cuda.synchronize()
        assert torch.equal(a1["q"], a2["q"]) and torch.equal(a1["scales"], a2["scales"])
        if fmt == 0:
            assert torch.equal(a1["tscale"].view(torch.int32), a2["tscale"].view(torch.int32))
        assert torch.equal(c1, c2) and torch.equal(r1, r2)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("layout", [fq.ROWMAJOR, fq.TILED])
def test_quantize_select_strided_rows(orc, fmt, layout):
    """x as a column slice of a wider tensor (ldx = cols + 64): the scored
    pass reads rows by ldx; results as for the contiguous tensor."""
    need_gpu()
    say(f"quantize_select strided fmt {fmt} layout {layout}")
    M, K, k = 200, 512, 24
    d = dense_case(M, K, 8, n_out=8, seed=41 + fmt)
    wide = np.zeros((M, K + 64), np.uint16)
    wide[:, :K] = d["x"]
    wide[:, K:] = bf16_bits(np.full((M, 64), 1e4, np.float32))  # never part of x
    xw = to_dev(wide)[:, :K]
    qx = orc.quantize(fmt, d["x"])
    want_c, want_r = orc.select_channels(fmt, d["x"], qx, k)
    a, chan, R = fq.quantize_select(fmt, xw, k, layout=layout)
    torch.cuda.synchronize()
    assert_quant_equal(dict(a, resid=None), qx, fmt)
    assert np.array_equal(to_host(chan), want_c)
    assert np.array_equal(to_host(R), want_r)
