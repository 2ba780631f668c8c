"""GPU parity of the exact launch sequence the benchmark times, at the full
workload sizes, against the oracle:

  * dense prefill (8192 x 4096 x 14336, |S| = 128) in NVFP4 and MXFP4:
    GPU quantization of X (with the residual) and of W^T, tiled layout,
    bit for bit; the prepared compensation weights; fp4q_gemm_prepared on
    the GPU's own codes, FP32 output, on 40000 sampled outputs plus a full
    row and a full column, |Y - Y_oracle| <= 1e-3 * Yabs;
  * the MoE layer (32768 routed rows, 128 experts, |S| = 32 per expert),
    gate_up and down: grouped GPU quantization bit for bit, each expert's
    weights quantized on the GPU, the grouped prepared compensation
    weights, fp4q_grouped_gemm_prepared on sampled outputs plus the first
    and last row of every non-empty expert; then the same with every
    expert's weights in the tiled layout (as benchmarked), bit for bit.
"""
import numpy as np
import pytest
import torch

import fp4_w4a4_quantized_amd as fq
from gpu_helpers import (assert_gemm_close, assert_quant_equal, need_gpu, say,
                         to_dev, to_host, workload)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["prefill_nvfp4", "prefill_mxfp4"])
def test_prefill_prepared_chain(orc, name):
    need_gpu()
    say(f"benchmarked prefill chain {name}: GPU quantize (tiled) -> fp4q_gemm_prepared")
    fmt = 0 if name == "prefill_nvfp4" else 1
    d = workload(name)
    chan = d["chan_idx"]
    ch = to_dev(chan)
    a = fq.quantize(fmt, to_dev(d["x"]), chan_idx=ch, layout=fq.TILED)
    b = fq.quantize(fmt, to_dev(d["wt"]), layout=fq.TILED)
    cw = fq.comp_weights(fmt, b, ch)
    y = fq.gemm_prepared(fmt, a, b, ch, cw)
    torch.cuda.synchronize()
    qa = orc.quantize(fmt, d["x"], chan_idx=chan)
    qb = orc.quantize(fmt, d["wt"])
    assert_quant_equal(a, qa, fmt)
    assert_quant_equal(b, qb, fmt)
    say("  codes, scales, tensor scales and residual bit-exact")
    y = to_host(y)
    M, N = y.shape
    rng = np.random.default_rng(2024)
    pm = np.concatenate([rng.integers(0, M, 40000), np.full(N, M - 1), np.arange(M)])
    pn = np.concatenate([rng.integers(0, N, 40000), np.arange(N), np.full(M, N - 1)])
    ta = float(qa["tscale"][0]) if fmt == 0 else 1.0
    tb = float(qb["tscale"][0]) if fmt == 0 else 1.0
    yo, ya = orc.gemm_points(fmt, qa["q"], qa["scales"], ta, qb["q"], qb["scales"], tb, chan,
                             qa["resid"], pm, pn)
    r = assert_gemm_close(y[pm, pn], yo, ya)
    say(f"  worst |dY|/Yabs = {r:.3e}")


@pytest.mark.parametrize("layer", ["gate_up", "down"])
def test_moe_prepared_chain(orc, layer):
    need_gpu()
    say(f"benchmarked MoE chain {layer}: grouped GPU quantize -> fp4q_grouped_gemm_prepared")
    m = workload("moe_nvfp4")
    off = m["offsets"]
    G = off.size - 1
    if layer == "gate_up":
        x, chan, wts = m["x_perm"], m["chan_gate_up"], m["wt_gate_up"]
    else:
        x, chan, wts = m["h_perm"], m["chan_down"], m["wt_down"]
    N = wts.shape[1]
    doff, dch = to_dev(off), to_dev(chan)
    a = fq.quantize(0, to_dev(x), group_offsets=doff, chan_idx=dch)
    qs = [fq.quantize(0, to_dev(wts[e])) for e in range(G)]
    bq = torch.stack([q["q"] for q in qs])
    bs = torch.stack([q["scales"] for q in qs])
    bts = torch.cat([q["tscale"] for q in qs])
    cw = fq.grouped_comp_weights(0, bq, bs, dch)
    y = fq.grouped_gemm_prepared(0, doff, a, bq, bs, bts, dch, cw)
    torch.cuda.synchronize()
    qa = orc.quantize(0, x, offsets=off, chan_idx=chan)
    assert_quant_equal(a, qa, 0)
    hq, hs, hts = to_host(bq), to_host(bs), to_host(bts)
    ref_b = [orc.quantize(0, wts[e]) for e in range(G)]
    for e in range(G):
        assert np.array_equal(hq[e], ref_b[e]["q"]), f"expert {e} weight codes"
        assert np.array_equal(hs[e], ref_b[e]["scales"]), f"expert {e} weight scales"
        assert hts[e].view(np.uint32) == ref_b[e]["tscale"][0].view(np.uint32), f"expert {e} t_w"
    say("  activation and weight quantization bit-exact")
    y = to_host(y)
    rng = np.random.default_rng(17)
    edge = np.concatenate([[off[g], off[g + 1] - 1] for g in range(G) if off[g + 1] > off[g]])
    pm = np.concatenate([rng.integers(0, x.shape[0], 30000), np.repeat(edge, 4)])
    pn = np.concatenate([rng.integers(0, N, 30000), rng.integers(0, N, edge.size * 4)])
    yo, ya = orc.grouped_gemm_points(0, off, qa["q"], qa["scales"], qa["tscale"], hq, hs, hts,
                                     chan, qa["resid"], pm, pn)
    r = assert_gemm_close(y[pm, pn], yo, ya)
    say(f"  worst |dY|/Yabs = {r:.3e}")
    # the benchmark keeps every expert's weights in the tiled layout: the
    # same kernel reads the same bytes into LDS, so Y is bit-identical
    qt = [fq.quantize(0, to_dev(wts[e]), layout=fq.TILED) for e in range(G)]
    tq = torch.stack([q["q"] for q in qt])
    ts = torch.stack([q["scales"] for q in qt])
    cwt = fq.grouped_comp_weights(0, tq, ts, dch, w_layout=fq.TILED, N=N, K=x.shape[1])
    assert torch.equal(cwt, cw), "grouped compensation weights from tiled weights"
    yt = fq.grouped_gemm_prepared(0, doff, a, tq, ts, bts, dch, cwt, w_layout=fq.TILED, N=N)
    torch.cuda.synchronize()
    yt = to_host(yt)
    bad = np.flatnonzero(yt.view(np.uint32) != y.view(np.uint32))
    assert bad.size == 0, f"tiled weights: {bad.size} outputs differ, first {bad[:4].tolist()}"
    say("  tiled expert weights: Y bit-identical")
