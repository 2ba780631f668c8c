"""GPU parity of the compensated GEMM with the second-pass FP4 residual
(fp4q_gemm_residual_fp4, through the C ABI) against the oracle, on every
GEMM path: the general kernel (small shapes), the decode kernel (M <= 64)
and the 256x256-tile kernel (in-kernel and gathered compensation weights),
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
                                      (300, 512, 520, 64),    # 256-tile, in-kernel B_S
                                      (257, 512, 300, 128)])  # 256-tile, gathered B_S (|S| > 96)
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
