"""GPU parity of the online channel selection (fp4q_select_channels, through
the C ABI) against the oracle: the chosen channels and the residual on them
bit for bit, both formats and both packed layouts, at shapes that take one
score row block and several (reduced by the pick kernel or by a launch of
their own), more columns than the pick kernel keeps in LDS,
ragged rows and column counts that leave a score workgroup part-filled,
constructed ties, k = 1 and k = cols, no rows, and the workloads' full
sizes; then chained after the GPU quantizer and into the compensated GEMM."""
import numpy as np
import pytest
import torch

import fp4_w4a4_quantized_amd as fq
from gpu_helpers import assert_gemm_close, dev_quant, need_gpu, say, to_dev, to_host
from workloads import CONFIGS, bf16_bits, dense_case

pytestmark = pytest.mark.gpu


def _check(orc, fmt, x, k, layout):
    qx = orc.quantize(fmt, x)
    want_c, want_r = orc.select_channels(fmt, x, qx, k)
    a = dev_quant(qx, layout=layout, fmt=fmt)
    chan, R = fq.select_channels(fmt, to_dev(x), a, k)
    torch.cuda.synchronize()
    got_c, got_r = to_host(chan), to_host(R)
    assert np.array_equal(got_c, want_c), (got_c[:16], want_c[:16])
    bad = np.argwhere(got_r != want_r)
    assert bad.size == 0, f"resid: {len(bad)} mismatches, first {bad[:3].tolist()}"
    return got_c


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("layout", [fq.ROWMAJOR, fq.TILED])
@pytest.mark.parametrize("M,K,k", [(16, 256, 7),      # one row block
                                   (40, 256, 64),     # three row blocks, ragged last
                                   (300, 512, 33),    # many row blocks, reduced while picking
                                   (64, 640, 1),      # score workgroup part-filled
                                   (129, 1024, 128),
                                   (2050, 1024, 40),  # the reduction launch
                                   (20, 32768, 100)])  # scores too many for LDS
def test_select_matches_oracle(orc, fmt, layout, M, K, k):
    need_gpu()
    say(f"select fmt {fmt} layout {layout} M{M} K{K} k{k}")
    d = dense_case(M, K, 8, n_out=max(1, K // 64), seed=M * 7 + K + k + fmt)
    _check(orc, fmt, d["x"], k, layout)


@pytest.mark.parametrize("fmt", [0, 1])
def test_select_unaligned_columns_and_stride(orc, fmt):
    """Row-major only: 48 (NVFP4) / 96 (MXFP4) columns, not a multiple of the
    512-column score workgroup or of 128; all channels and one channel."""
    need_gpu()
    K = 48 if fmt == 0 else 96
    say(f"select fmt {fmt} K{K}")
    d = dense_case(37, K, 8, n_out=3, seed=11 + fmt)
    _check(orc, fmt, d["x"], K, fq.ROWMAJOR)
    _check(orc, fmt, d["x"], 1, fq.ROWMAJOR)


@pytest.mark.parametrize("fmt", [0, 1])
def test_select_ties_and_zero_columns(orc, fmt):
    """Four copies of one column tie; the top-2 boundary falls inside the tie
    and in a run of all-zero columns (zero residual): lower indices win."""
    need_gpu()
    say(f"select ties fmt {fmt}")
    rng = np.random.default_rng(5 + fmt)
    x = np.zeros((70, 1024), np.float32)
    col = rng.standard_normal(70).astype(np.float32) * 3.0
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


def test_select_no_rows_takes_the_lowest_indices():
    """Without rows every magnitude is 0, so the first k channels win."""
    need_gpu()
    say("select rows 0")
    for fmt in (0, 1):
        x = torch.empty((0, 256), dtype=torch.int16, device="cuda:0")
        a = {"q": torch.empty((0, 128), dtype=torch.uint8, device="cuda:0"),
             "scales": torch.empty((0, 256 // fq.BLOCK[fmt]), dtype=torch.uint8, device="cuda:0"),
             "tscale": torch.ones(1, dtype=torch.float32, device="cuda:0") if fmt == 0 else None,
             "layout": fq.ROWMAJOR}
        chan, R = fq.select_channels(fmt, x, a, 10)
        torch.cuda.synchronize()
        assert to_host(chan).tolist() == list(range(10)) and R.shape == (0, 10)


@pytest.mark.parametrize("name", ["decode_nvfp4", "prefill_nvfp4", "prefill_mxfp4"])
def test_select_full_size(orc, name):
    """The workloads' full activation shapes, k = the workload's channel
    count, tiled as the GEMM takes them: channels and residual bit for bit."""
    need_gpu()
    cfg = CONFIGS[name]
    fmt = 0 if cfg["fmt"] == "nvfp4" else 1
    M, K = cfg["M"], cfg["K"]
    k = cfg["n_s"]
    say(f"select full size {name} M{M} K{K} k{k}")
    d = dense_case(**{**cfg, "N": 8})
    _check(orc, fmt, d["x"], k, fq.TILED)


@pytest.mark.parametrize("fmt", [0, 1])
def test_select_chained_into_gemm(orc, fmt):
    """GPU quantize -> GPU select -> compensated GEMM on the chosen channels,
    against the oracle's quantize -> select -> GEMM."""
    need_gpu()
    say(f"select chained fmt {fmt}")
    M, K, N, k = 96, 512, 320, 32
    d = dense_case(M, K, N, n_out=6, seed=77 + fmt)
    qa = orc.quantize(fmt, d["x"])
    qb = orc.quantize(fmt, d["wt"])
    S, R = orc.select_channels(fmt, d["x"], qa, k)
    ta = float(qa["tscale"][0]) if fmt == 0 else 1.0
    tb = float(qb["tscale"][0]) if fmt == 0 else 1.0
    qa_s = dict(qa, resid=R)
    yo, ya = orc.gemm_full(fmt, qa_s["q"], qa_s["scales"], ta, qb["q"], qb["scales"], tb, S, R)

    x = to_dev(d["x"])
    ga = fq.quantize(fmt, x, layout=fq.TILED)
    chan, gR = fq.select_channels(fmt, x, ga, k)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(chan), S)
    assert np.array_equal(to_host(gR), R)
    b = dev_quant(qb, layout=fq.TILED, fmt=fmt)
    y = fq.gemm(fmt, dict(ga, resid=gR), b, chan_idx=chan)
    torch.cuda.synchronize()
    assert_gemm_close(to_host(y), yo, ya)


# ---- grouped (MoE) form: fp4q_select_channels_grouped ---------------------------

def _check_grouped(orc, fmt, x, off, k):
    qx = orc.quantize(fmt, x, offsets=off)
    want_c, want_r = orc.select_channels_grouped(fmt, x, qx, off, k)
    a = dev_quant(qx)
    chan, R = fq.select_channels_grouped(fmt, to_dev(x), to_dev(off), a, k)
    torch.cuda.synchronize()
    got_c, got_r = to_host(chan), to_host(R)
    assert np.array_equal(got_c, want_c), [(g, got_c[g][:8], want_c[g][:8])
                                           for g in range(want_c.shape[0])
                                           if not np.array_equal(got_c[g], want_c[g])][:3]
    bad = np.argwhere(got_r.view(np.uint16) != want_r)
    assert bad.size == 0, f"resid: {len(bad)} mismatches, first {bad[:3].tolist()}"
    return got_c


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("off,K,k", [([0, 0, 1, 40, 40, 57], 256, 16),      # empty, one row
                                     ([0, 300, 301, 900], 512, 33),         # several row blocks
                                     ([0, 5, 2055, 2060, 2061], 1024, 64),  # one big group
                                     ([0, 0, 0], 256, 8)])                  # no rows at all
def test_grouped_select_matches_oracle(orc, fmt, off, K, k):
    need_gpu()
    off = np.array(off, np.int32)
    say(f"grouped select fmt {fmt} rows {off[-1]} groups {off.size - 1} K{K} k{k}")
    d = dense_case(max(int(off[-1]), 1), K, 8, n_out=max(1, K // 64), seed=int(off[-1]) + K + k)
    _check_grouped(orc, fmt, d["x"][:int(off[-1])], off, k)


def test_grouped_select_moe_workload_and_gemm(orc):
    """The MoE gate_up input at full size (32,768 routed rows, 128 experts,
    k = 32 per expert): chosen channels and residual bit for bit, then the
    grouped GEMM on each expert's chosen channels against the oracle on
    sampled outputs."""
    need_gpu()
    say("grouped select, MoE gate_up workload, then the grouped GEMM")
    from gpu_helpers import workload
    m = workload("moe_nvfp4")
    off, x, wts = m["offsets"], m["x_perm"], m["wt_gate_up"]
    fmt, k = 0, CONFIGS["moe_nvfp4"]["n_s"]
    chan = _check_grouped(orc, fmt, x, off, k)
    doff = to_dev(off)
    ga = fq.quantize(fmt, to_dev(x), group_offsets=doff)
    dchan, R = fq.select_channels_grouped(fmt, to_dev(x), doff, ga, k)
    qbs = [fq.quantize(fmt, to_dev(wts[e])) for e in range(off.size - 1)]
    bq = torch.stack([q["q"] for q in qbs])
    bs = torch.stack([q["scales"] for q in qbs])
    bts = torch.cat([q["tscale"] for q in qbs])
    a = {"q": ga["q"], "scales": ga["scales"], "tscale": ga["tscale"], "resid": R}
    y = to_host(fq.grouped_gemm(fmt, doff, a, bq, bs, bts, chan_idx=dchan))
    qx = orc.quantize(fmt, x, offsets=off, chan_idx=chan)
    N = wts.shape[1]
    rng = np.random.default_rng(23)
    pm, pn = rng.integers(0, x.shape[0], 30000), rng.integers(0, N, 30000)
    yo, ya = orc.grouped_gemm_points(fmt, off, qx["q"], qx["scales"], qx["tscale"],
                                     to_host(bq), to_host(bs), to_host(bts), chan, qx["resid"],
                                     pm, pn)
    assert_gemm_close(y[pm, pn], yo, ya)
