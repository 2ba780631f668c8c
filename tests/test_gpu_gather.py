"""GPU parity of the expert-grouped GEMM that gathers the token codes
(fp4q_grouped_gemm_gather; QUADS abstract: NVFP4 MoE rollout,
quantize-before-permute) and of the permute's residual-only mode:

  * the residual-only permute writes the same residual and tensor scales as
    the full permute, bit for bit;
  * the gathering GEMM equals the grouped GEMM on the permuted copy bit for
    bit (same kernel, same operand values, same order), and the oracle's
    quantize-before-permute product within 1e-3 * Yabs;
  * at the full MoE gate_up layer (32768 routed rows of 4096 tokens, 128
    experts) and on small cases with empty and single-row experts, both
    formats, with and without channels;
  * NVFP4 with every expert's weights in the tiled layout equals the
    row-major result bit for bit.
"""
import numpy as np
import pytest
import torch

import fp4_w4a4_quantized_amd as fq
from gpu_helpers import assert_gemm_close, need_gpu, say, to_dev, to_host, workload
from workloads import dense_case

pytestmark = pytest.mark.gpu


def _case(orc, fmt, x_tok, row_src, off, chan, wts, pm=None, pn=None):
    dev = need_gpu()
    T, K = x_tok.shape
    rows = row_src.size
    G = off.size - 1
    nS = 0 if chan is None else chan.shape[1]
    N = wts[0].shape[0]
    xt = to_dev(x_tok)
    src, doff = to_dev(row_src.astype(np.int32)), to_dev(off)
    dch = None if chan is None else to_dev(chan)
    tok = fq.quantize(fmt, xt)
    qs = [fq.quantize(fmt, to_dev(w)) for w in wts]
    bq = torch.stack([q["q"] for q in qs])
    bs = torch.stack([q["scales"] for q in qs])
    bts = torch.cat([q["tscale"] for q in qs]) if fmt == 0 else None
    cw = fq.grouped_comp_weights(fmt, bq, bs, dch) if nS else None
    # full permute (codes copied) and the residual-only permute
    full = fq.permute_quantized(fmt, xt, tok, src, doff, dch)
    r_only = torch.full((rows, nS), 7, dtype=torch.int16, device=dev) if nS else None
    ts_only = torch.full((G,), 3.0, dtype=torch.float32, device=dev) if fmt == 0 else None
    fq.permute_quantized_into(fmt, xt, tok["q"], tok["scales"], tok["tscale"], src, doff, G, dch,
                              nS, None, None, ts_only, r_only)
    y_gather = torch.empty((rows, N), dtype=torch.float32, device=dev)
    fq.grouped_gemm_gather_into(fmt, rows, N, K, doff, G, src, T, tok["q"], tok["scales"],
                                tok["tscale"], bq, bs, bts, dch, nS, r_only, cw, y_gather, 0)
    y_copy = (fq.grouped_gemm_prepared(fmt, doff, full, bq, bs, bts, dch, cw) if nS
              else fq.grouped_gemm(fmt, doff, full, bq, bs, bts))
    torch.cuda.synchronize()
    if nS:
        assert torch.equal(r_only, full["resid"]), "residual-only permute differs"
    if fmt == 0:
        assert torch.equal(ts_only, full["tscale"])
    assert torch.equal(y_gather, y_copy), "gathering GEMM differs from the permuted copy"
    if fmt == 0 and N >= 256 and nS % 8 == 0:
        # every expert's weights in the tiled layout: the same bytes reach the
        # kernel's LDS, so the gathering GEMM's Y is bit-identical
        qt_ = [fq.quantize(fmt, to_dev(w), layout=fq.TILED) for w in wts]
        tq = torch.stack([q["q"] for q in qt_])
        ts = torch.stack([q["scales"] for q in qt_])
        cwt = (fq.grouped_comp_weights(fmt, tq, ts, dch, w_layout=fq.TILED, N=N, K=K) if nS
               else None)
        y_t = torch.empty((rows, N), dtype=torch.float32, device=dev)
        fq.grouped_gemm_gather_into(fmt, rows, N, K, doff, G, src, T, tok["q"], tok["scales"],
                                    tok["tscale"], tq, ts, bts, dch, nS, r_only, cwt, y_t, 0,
                                    w_layout=fq.TILED)
        torch.cuda.synchronize()
        assert torch.equal(y_t, y_gather), "tiled expert weights: gathering GEMM differs"
    # the oracle: quantize-before-permute, then the grouped product
    qt = orc.quantize(fmt, x_tok)
    perm = orc.permute_quantized(fmt, x_tok, qt, row_src, off, chan)
    hq = to_host(bq)
    hs = to_host(bs)
    hts = None if fmt else to_host(bts)
    if pm is None:
        pm = np.repeat(np.arange(rows), N)
        pn = np.tile(np.arange(N), rows)
    yo, ya = orc.grouped_gemm_points(fmt, off, perm["q"], perm["scales"], perm["tscale"], hq, hs,
                                     hts, chan, perm["resid"], pm, pn)
    return assert_gemm_close(to_host(y_gather)[pm, pn], yo, ya)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("nS", [0, 8, 40])
def test_small(orc, fmt, nS):
    say(f"gathering grouped GEMM fmt {fmt} nS {nS}")
    K, N, T = 384, 300, 50
    off = np.array([0, 0, 1, 70, 70, 200, 233], np.int32)
    G = off.size - 1
    rng = np.random.default_rng(11 + nS)
    row_src = rng.integers(0, T, off[-1]).astype(np.int32)
    x_tok = dense_case(T, K, 8, n_out=3, seed=31)["x"]
    wts = [dense_case(1, K, N, seed=40 + g)["wt"] for g in range(G)]
    chan = (np.sort(np.stack([rng.choice(K, nS, replace=False) for _ in range(G)]), 1)
            .astype(np.int32) if nS else None)
    _case(orc, fmt, x_tok, row_src, off, chan, wts)


def test_moe_gate_up(orc):
    say("gathering grouped GEMM, MoE gate_up layer (32768 routed rows, 128 experts)")
    m = workload("moe_nvfp4")
    off = m["offsets"]
    rng = np.random.default_rng(5)
    rows = int(off[-1])
    N = m["wt_gate_up"].shape[1]
    edge = np.concatenate([[off[g], off[g + 1] - 1] for g in range(off.size - 1)
                           if off[g + 1] > off[g]])
    pm = np.concatenate([rng.integers(0, rows, 30000), np.repeat(edge, 4)])
    pn = np.concatenate([rng.integers(0, N, 30000), rng.integers(0, N, edge.size * 4)])
    r = _case(orc, 0, m["x_tok"], m["token_of_row"].astype(np.int32), off, m["chan_gate_up"],
              list(m["wt_gate_up"]), pm, pn)
    say(f"  worst |dY|/Yabs = {r:.3e}")
