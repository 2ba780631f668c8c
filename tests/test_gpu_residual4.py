"""GPU parity of the compensated GEMM with the second-pass FP4 residual
(fp4q_gemm_residual_fp4, through the C ABI) against the oracle, on every
GEMM path: the general kernel (small shapes), the decode kernel (M <= 64)
and the large-tile kernels (compensation weights gathered per call),
both formats and both operand layouts; and the GPU quantizer's second pass
on R bit-exact against the oracle's."""
import numpy as np
import pytest
import torch

import fp4_w4a4_quantized_amd as fq
from gpu_helpers import (assert_gemm_close, assert_quant_equal, dev_quant, need_gpu, say, to_dev,
                         to_host)
from workloads import dense_case

pytestmark = pytest.mark.gpu
BLK = {0: 16, 1: 32}


def _case(orc, fmt, M, K, N, nS, seed):
    d = dense_case(M, K, N, n_out=max(1, K // 128), seed=seed)
    S = np.sort(np.random.default_rng(seed + 1).choice(K, nS, replace=False)).astype(np.int32)
    qa = orc.quantize(fmt, d["x"], chan_idx=S)
    qb = orc.quantize(fmt, d["wt"])
    qr = orc.quantize_residual(fmt, qa["resid"])
    ta = float(qa["tscale"][0]) if fmt == 0 else 1.0
    tb = float(qb["tscale"][0]) if fmt == 0 else 1.0
    tr = float(qr["tscale"][0]) if fmt == 0 else 1.0
    yo, ya = orc.gemm_full_r4(fmt, qa["q"], qa["scales"], ta, qb["q"], qb["scales"], tb, S,
                              qr["q"], qr["scales"], tr)
    return S, qa, qb, qr, yo, ya


def _gpu(fmt, layout, S, qa, qb, qr, y_dtype=fq.OUT_F32):
    a = dev_quant(qa, layout=layout, fmt=fmt)
    b = dev_quant(qb, layout=layout, fmt=fmt)
    r = dev_quant(qr)                        # the residual operand is row-major
    y = fq.gemm_residual_fp4(fmt, a, b, to_dev(S), r, y_dtype=y_dtype)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("M,K,N,nS", [(16, 256, 256, 32),     # general kernel
                                      (64, 512, 640, 64),     # decode kernel
                                      (33, 384, 200, 32),     # general, ragged
                                      (300, 512, 520, 64),    # large-tile, gathered B_S
                                      (257, 512, 300, 128)])  # large-tile, four stages of B_S
def test_residual_fp4_matches_oracle(orc, fmt, M, K, N, nS):
    need_gpu()
    say(f"gemm fp4 residual fmt {fmt} M{M} K{K} N{N} nS{nS}")
    S, qa, qb, qr, yo, ya = _case(orc, fmt, M, K, N, nS, seed=M + K + N + nS)
    for layout in (fq.ROWMAJOR, fq.TILED):
        y = to_host(_gpu(fmt, layout, S, qa, qb, qr))
        assert_gemm_close(y, yo, ya)


@pytest.mark.parametrize("fmt", [0, 1])
def test_residual_fp4_bf16_out_and_quantizer(orc, fmt):
    """BF16 output (half an ulp more), and the GPU quantizer's second pass
    over the GPU residual reproduces the oracle's codes, scales and tensor
    scale bit for bit."""
    dev = need_gpu()
    say(f"gemm fp4 residual bf16 + GPU second pass fmt {fmt}")
    M, K, N, nS = 96, 512, 320, 2 * BLK[fmt]
    S, qa, qb, qr, yo, ya = _case(orc, fmt, M, K, N, nS, seed=123 + fmt)
    x = dense_case(M, K, N, n_out=max(1, K // 128), seed=123 + fmt)["x"]
    ga = fq.quantize(fmt, to_dev(x), chan_idx=to_dev(S))
    gr = fq.quantize(fmt, ga["resid"])
    torch.cuda.synchronize()
    assert_quant_equal(gr, qr, fmt)
    b = dev_quant(qb)
    y = fq.gemm_residual_fp4(fmt, ga, b, to_dev(S), gr, y_dtype=fq.OUT_BF16)
    torch.cuda.synchronize()
    from workloads import bf16_to_f32
    yb = bf16_to_f32(to_host(y.view(torch.int16))).astype(np.float64)
    assert np.all(np.abs(yb - yo) <= 1e-3 * ya + 2.0 ** -8 * np.abs(yo))


def test_residual_fp4_reduces_to_bf16_path_for_lossless_residual(orc):
    """MXFP4 residual values that are already on the grid: the second pass
    is exact, so the FP4-residual call and the BF16-residual call agree to
    FP32 accumulation order on the GPU."""
    need_gpu()
    M, K, N, nS = 64, 256, 192, 32
    d = dense_case(M, K, N, n_out=2, seed=9)
    S = np.arange(0, 256, 8, dtype=np.int32)
    qa = orc.quantize(1, d["x"], chan_idx=S)
    qb = orc.quantize(1, d["wt"])
    rng = np.random.default_rng(10)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    codes = rng.integers(0, 16, (M, nS))
    codes[:, 0] = 7
    rv = (np.where(codes & 8, -1.0, 1.0) * grid[codes & 7] * 2.0 ** -5).astype(np.float32)
    from workloads import bf16_bits
    qa["resid"] = bf16_bits(rv)
    qr = orc.quantize_residual(1, qa["resid"])
    a, b = dev_quant(qa), dev_quant(qb)
    y4 = to_host(fq.gemm_residual_fp4(1, a, b, to_dev(S), dev_quant(qr)))
    y2 = to_host(fq.gemm(1, a, b, chan_idx=to_dev(S)))
    torch.cuda.synchronize()
    yo, ya = orc.gemm_full(1, qa["q"], qa["scales"], 1.0, qb["q"], qb["scales"], 1.0, S,
                           qa["resid"])
    assert_gemm_close(y4, yo, ya)
    assert np.allclose(y4, y2, rtol=0, atol=1e-6 * ya.max())


# ---- grouped (MoE) form: fp4q_grouped_gemm_residual_fp4 -----------------------

def _grouped_case(orc, fmt, off, K, N, nS, seed):
    G = off.size - 1
    x = dense_case(int(off[-1]), K, 8, n_out=3, seed=seed)["x"]
    wts = [dense_case(1, K, N, seed=seed + 10 + g)["wt"] for g in range(G)]
    rng = np.random.default_rng(seed)
    chan = np.sort(np.stack([rng.choice(K, nS, replace=False) for _ in range(G)]), 1)
    chan = chan.astype(np.int32)
    qa = orc.quantize(fmt, x, offsets=off, chan_idx=chan)
    qr = orc.quantize(fmt, qa["resid"], offsets=off)
    qbs = [orc.quantize(fmt, w) for w in wts]
    bq = np.stack([q["q"] for q in qbs])
    bs = np.stack([q["scales"] for q in qbs])
    bts = np.array([q["tscale"][0] for q in qbs], np.float32) if fmt == 0 else None
    return x, chan, qa, qr, bq, bs, bts


def _grouped_gpu(fmt, off, chan, qa, qr, bq, bs, bts):
    a = {"q": to_dev(qa["q"]), "scales": to_dev(qa["scales"]),
         "tscale": None if fmt else to_dev(qa["tscale"])}
    r = {"q": to_dev(qr["q"]), "scales": to_dev(qr["scales"]),
         "tscale": None if fmt else to_dev(qr["tscale"])}
    y = fq.grouped_gemm_residual_fp4(fmt, to_dev(off), a, to_dev(bq), to_dev(bs),
                                     None if fmt else to_dev(bts), to_dev(chan), r)
    torch.cuda.synchronize()
    return to_host(y)


@pytest.mark.parametrize("fmt,N,nS", [(0, 300, 32),    # 128x512 NVFP4 kernel, gathered B_S
                                      (0, 560, 128),   # 128x512 NVFP4 kernel, gathered B_S
                                      (0, 200, 16),    # general grouped kernel
                                      (1, 300, 32), (1, 560, 128), (1, 200, 64)])
def test_grouped_residual_fp4_matches_oracle(orc, fmt, N, nS):
    """Empty, single-row and multi-tile experts; each expert's residual with
    its own tensor scale (NVFP4)."""
    need_gpu()
    say(f"grouped gemm fp4 residual fmt {fmt} N{N} nS{nS}")
    off = np.array([0, 0, 1, 130, 130, 300, 555], np.int32)
    K = 384
    x, chan, qa, qr, bq, bs, bts = _grouped_case(orc, fmt, off, K, N, nS, seed=N + nS + fmt)
    y = _grouped_gpu(fmt, off, chan, qa, qr, bq, bs, bts)
    pm = np.repeat(np.arange(int(off[-1])), N)
    pn = np.tile(np.arange(N), int(off[-1]))
    yo, ya = orc.grouped_gemm_points_r4(fmt, off, qa["q"], qa["scales"],
                                        None if fmt else qa["tscale"], bq, bs, bts, chan,
                                        qr["q"], qr["scales"], None if fmt else qr["tscale"],
                                        pm, pn)
    assert_gemm_close(y[pm, pn], yo, ya)


def test_grouped_residual_fp4_moe_workload(orc):
    """The MoE gate_up layer at full size (32,768 routed rows, 128 experts,
    32 channels each): the GPU's grouped second pass over the GPU residual
    bit-exact against the oracle's, and the GEMM on 30,000 sampled outputs
    plus each expert's first and last row."""
    need_gpu()
    say("grouped gemm fp4 residual, MoE gate_up workload")
    from gpu_helpers import workload
    m = workload("moe_nvfp4")
    off, x, chan, wts = m["offsets"], m["x_perm"], m["chan_gate_up"], m["wt_gate_up"]
    fmt, N = 0, wts.shape[1]
    qa = orc.quantize(fmt, x, offsets=off, chan_idx=chan)
    qr = orc.quantize(fmt, qa["resid"], offsets=off)
    doff = to_dev(off)
    ga = fq.quantize(fmt, to_dev(x), group_offsets=doff, chan_idx=to_dev(chan))
    gr = fq.quantize(fmt, ga["resid"], group_offsets=doff)
    torch.cuda.synchronize()
    assert_quant_equal(gr, qr, fmt)
    qbs = [fq.quantize(fmt, to_dev(wts[e])) for e in range(off.size - 1)]
    bq = torch.stack([q["q"] for q in qbs])
    bs = torch.stack([q["scales"] for q in qbs])
    bts = torch.cat([q["tscale"] for q in qbs])
    y = to_host(fq.grouped_gemm_residual_fp4(fmt, doff, ga, bq, bs, bts, to_dev(chan), gr))
    rng = np.random.default_rng(17)
    edge = np.concatenate([[off[g], off[g + 1] - 1] for g in range(off.size - 1)
                           if off[g + 1] > off[g]])
    pm = np.concatenate([rng.integers(0, x.shape[0], 30000), np.repeat(edge, 4)])
    pn = np.concatenate([rng.integers(0, N, 30000), rng.integers(0, N, edge.size * 4)])
    yo, ya = orc.grouped_gemm_points_r4(fmt, off, qa["q"], qa["scales"], qa["tscale"],
                                        to_host(bq), to_host(bs), to_host(bts), chan, qr["q"],
                                        qr["scales"], qr["tscale"], pm, pn)
    assert_gemm_close(y[pm, pn], yo, ya)
