"""GPU parity of the expert-grouped GEMMs with every expert's weights in the
tiled layout (QUADS abstract: NVFP4 rollout for Mixture-of-Experts; the
layout is the library's own, fp4q.h), through the C ABI:

  * the grouped compensation weights from tiled weights equal those from
    row-major weights byte for byte;
  * fp4q_grouped_gemm_prepared and fp4q_grouped_gemm with tiled weights
    equal the row-major prepared product bit for bit (the same 128 x 512
    kernel with the same bytes in LDS), and the oracle's grouped GEMM on
    every output within 1e-3 * Yabs;
  * fp4q_grouped_gemm_residual_fp4 with tiled weights against the oracle,
    and bit for bit against row-major weights (same kernel, B_S gathered);
  * empty, single-row, 128-row-crossing and ragged experts; N with padded
    16-row code groups and 64-row scale groups; FP32 and BF16 outputs.
"""
import numpy as np
import pytest
import torch

import fp4_w4a4_quantized_amd as fq
from gpu_helpers import assert_gemm_close, dev_quant, need_gpu, say, to_dev, to_host
from workloads import dense_case

pytestmark = pytest.mark.gpu

OFF = np.array([0, 0, 1, 70, 70, 300, 333], np.int32)


def _weights(orc, K, N, G, seed):
    wts = [dense_case(1, K, N, seed=seed + g)["wt"] for g in range(G)]
    qbs = [orc.quantize(0, w) for w in wts]
    rq = torch.stack([to_dev(q["q"]) for q in qbs])
    rs = torch.stack([to_dev(q["scales"]) for q in qbs])
    tl = [dev_quant(q, layout=fq.TILED, fmt=0) for q in qbs]
    tq = torch.stack([t["q"] for t in tl])
    ts = torch.stack([t["scales"] for t in tl])
    bts = np.array([q["tscale"][0] for q in qbs], np.float32)
    return qbs, rq, rs, tq, ts, bts


def _bits_equal(a, b, what):
    a = a.contiguous().reshape(-1).view(torch.uint8)
    b = b.contiguous().reshape(-1).view(torch.uint8)
    assert a.numel() == b.numel(), what
    bad = torch.nonzero(a != b).flatten()
    assert bad.numel() == 0, f"{what}: {bad.numel()} bytes differ, first at {bad[:4].tolist()}"


@pytest.mark.parametrize("N,K,nS", [(512, 384, 32), (272, 256, 8), (1000, 384, 128),
                                    (640, 256, 0)])
def test_grouped_tiled_weights(orc, N, K, nS):
    need_gpu()
    say(f"grouped GEMM, tiled expert weights: N{N} K{K} nS{nS}")
    G = OFF.size - 1
    x = dense_case(int(OFF[-1]), K, 8, n_out=3, seed=N + K)["x"]
    rng = np.random.default_rng(N + nS)
    chan = (np.sort(np.stack([rng.choice(K, nS, replace=False) for _ in range(G)]), 1)
            .astype(np.int32) if nS else None)
    qa = orc.quantize(0, x, offsets=OFF, chan_idx=chan)
    qbs, rq, rs, tq, ts, bts = _weights(orc, K, N, G, seed=900 + N)
    doff, dch, dbts = to_dev(OFF), None if chan is None else to_dev(chan), to_dev(bts)
    a = {"q": to_dev(qa["q"]), "scales": to_dev(qa["scales"]), "tscale": to_dev(qa["tscale"]),
         "resid": None if qa["resid"] is None else to_dev(qa["resid"])}
    if nS:
        cw_r = fq.grouped_comp_weights(0, rq, rs, dch)
        cw_t = fq.grouped_comp_weights(0, tq, ts, dch, w_layout=fq.TILED, N=N, K=K)
        _bits_equal(cw_t, cw_r, "compensation weights")
        y_ref = fq.grouped_gemm_prepared(0, doff, a, rq, rs, dbts, dch, cw_r)
        y_pt = fq.grouped_gemm_prepared(0, doff, a, tq, ts, dbts, dch, cw_t, w_layout=fq.TILED,
                                        N=N)
        _bits_equal(y_pt, y_ref, "prepared, tiled weights")
        for dt in (fq.OUT_BF16,):
            yb_r = fq.grouped_gemm_prepared(0, doff, a, rq, rs, dbts, dch, cw_r, y_dtype=dt)
            yb_t = fq.grouped_gemm_prepared(0, doff, a, tq, ts, dbts, dch, cw_t, y_dtype=dt,
                                            w_layout=fq.TILED, N=N)
            _bits_equal(yb_t, yb_r, "prepared BF16 output, tiled weights")
    else:
        y_ref = fq.grouped_gemm(0, doff, a, rq, rs, dbts)
    # the per-call form: B_S gathered into the workspace from the tiled weights
    y_t = fq.grouped_gemm(0, doff, a, tq, ts, dbts, dch, w_layout=fq.TILED, N=N)
    torch.cuda.synchronize()
    _bits_equal(y_t, y_ref, "per-call form, tiled weights")
    rows = int(OFF[-1])
    pm = np.repeat(np.arange(rows), N)
    pn = np.tile(np.arange(N), rows)
    bq = np.stack([q["q"] for q in qbs])
    bs = np.stack([q["scales"] for q in qbs])
    yo, ya = orc.grouped_gemm_points(0, OFF, qa["q"], qa["scales"], qa["tscale"], bq, bs, bts,
                                     chan, qa["resid"], pm, pn)
    r = assert_gemm_close(to_host(y_t)[pm, pn], yo, ya)
    say(f"  worst |dY|/Yabs = {r:.3e}")


@pytest.mark.parametrize("N,nS", [(300, 32), (560, 128)])
def test_grouped_residual_fp4_tiled_weights(orc, N, nS):
    need_gpu()
    say(f"grouped second-pass residual, tiled expert weights: N{N} nS{nS}")
    off = np.array([0, 0, 1, 130, 130, 300, 555], np.int32)
    G, K = off.size - 1, 384
    x = dense_case(int(off[-1]), K, 8, n_out=3, seed=N + nS)["x"]
    rng = np.random.default_rng(nS)
    chan = np.sort(np.stack([rng.choice(K, nS, replace=False) for _ in range(G)]), 1)
    chan = chan.astype(np.int32)
    qa = orc.quantize(0, x, offsets=off, chan_idx=chan)
    qr = orc.quantize(0, qa["resid"], offsets=off)
    qbs, rq, rs, tq, ts, bts = _weights(orc, K, N, G, seed=700 + N)
    doff, dch, dbts = to_dev(off), to_dev(chan), to_dev(bts)
    a = {"q": to_dev(qa["q"]), "scales": to_dev(qa["scales"]), "tscale": to_dev(qa["tscale"])}
    r = {"q": to_dev(qr["q"]), "scales": to_dev(qr["scales"]), "tscale": to_dev(qr["tscale"])}
    y_t = fq.grouped_gemm_residual_fp4(0, doff, a, tq, ts, dbts, dch, r, w_layout=fq.TILED, N=N)
    y_r = fq.grouped_gemm_residual_fp4(0, doff, a, rq, rs, dbts, dch, r)
    _bits_equal(y_t, y_r, "second-pass residual, tiled weights")
    torch.cuda.synchronize()
    rows = int(off[-1])
    pm = np.repeat(np.arange(rows), N)
    pn = np.tile(np.arange(N), rows)
    bq = np.stack([q["q"] for q in qbs])
    bs = np.stack([q["scales"] for q in qbs])
    yo, ya = orc.grouped_gemm_points_r4(0, off, qa["q"], qa["scales"], qa["tscale"], bq, bs, bts,
                                        chan, qr["q"], qr["scales"], qr["tscale"], pm, pn)
    assert_gemm_close(to_host(y_t)[pm, pn], yo, ya)
