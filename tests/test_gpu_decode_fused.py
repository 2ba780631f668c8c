"""GPU parity of the fused decode datapath (fp4q_gemm_decode_fused: the
activations quantized inside the decode GEMM; FourSight abstract): the
quantized activations it reports (codes, block scales, tensor scale,
residual) bit for bit against the oracle's quantizer; Y against the FP64
oracle within 1e-3 * Yabs and bit for bit against the two-launch path
(fp4q_quantize, then fp4q_gemm_prepared), which multiplies in the same
order; at the decode workload size in both weight layouts, on ragged
shapes, and without the optional outputs."""
import numpy as np
import pytest
import torch

import fp4_w4a4_quantized_amd as fq
from gpu_helpers import assert_gemm_close, dev_quant, need_gpu, say, to_dev, to_host, workload
from workloads import dense_case

pytestmark = pytest.mark.gpu


def _run(orc, d, chan, layout, with_outputs=True, y_dtype=0):
    dev = need_gpu()
    x = d["x"]
    M, K = x.shape
    N = d["wt"].shape[0]
    nS = 0 if chan is None else chan.size
    ch = None if chan is None else to_dev(chan)
    qb = orc.quantize(0, d["wt"])
    b = dev_quant(qb, layout=layout, fmt=0)
    cw = fq.comp_weights(0, b, ch) if nS else None
    y = torch.full((M, N), 5.0, dtype=torch.float32 if y_dtype == 0 else torch.bfloat16, device=dev)
    outs = {}
    if with_outputs:
        outs = {"a_q_out": torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
                "a_s_out": torch.empty((M, K // 16), dtype=torch.uint8, device=dev),
                "a_ts_out": torch.empty(1, dtype=torch.float32, device=dev),
                "resid_out": torch.empty((M, nS), dtype=torch.int16, device=dev) if nS else None}
    xd = to_dev(x)
    fq.gemm_decode_fused_into(0, layout, xd, N, b["q"], b["scales"], b["tscale"], ch, nS, cw, y,
                              y_dtype, N, **outs)
    # the two-launch path on the same operands
    a = fq.quantize(0, xd, chan_idx=ch, layout=layout)
    y2 = (fq.gemm_prepared(0, a, b, ch, cw, y_dtype=y_dtype) if nS
          else fq.gemm(0, a, b, y_dtype=y_dtype))
    torch.cuda.synchronize()
    qa = orc.quantize(0, x, chan_idx=chan)
    if with_outputs:
        assert np.array_equal(to_host(outs["a_q_out"]), qa["q"]), "codes"
        assert np.array_equal(to_host(outs["a_s_out"]), qa["scales"]), "block scales"
        assert to_host(outs["a_ts_out"]).view(np.uint32)[0] == qa["tscale"].view(np.uint32)[0]
        if nS:
            assert np.array_equal(to_host(outs["resid_out"]), qa["resid"]), "residual"
    r = 0.0
    if y_dtype == 0:
        yo, ya = orc.gemm_full(0, qa["q"], qa["scales"], float(qa["tscale"][0]), qb["q"],
                               qb["scales"], float(qb["tscale"][0]), chan, qa["resid"])
        r = assert_gemm_close(to_host(y), yo, ya)
    # the two-launch path runs the same decode kernel (same order) when its
    # residual rows come in whole 16-byte pieces (M |S| a multiple of 8);
    # otherwise the general kernel, whose order differs
    if (M * nS) % 8 == 0:
        assert torch.equal(y, y2), "differs from the two-launch path"
    return r


@pytest.mark.parametrize("layout", [fq.ROWMAJOR, fq.TILED])
def test_decode_workload(orc, layout):
    say(f"fused decode datapath, decode workload 64 x 2048 x 11008, layout {layout}")
    d = workload("decode_nvfp4")
    r = _run(orc, d, d["chan_idx"], layout)
    say(f"  worst |dY|/Yabs = {r:.3e}")


@pytest.mark.parametrize("M,K,N,nS", [(1, 128, 1, 0), (5, 640, 47, 8), (33, 1024, 100, 24),
                                      (64, 2048, 1000, 64), (17, 256, 300, 33),
                                      (64, 1920, 96, 63), (48, 2048, 49, 1)])
def test_ragged(orc, M, K, N, nS):
    say(f"fused decode datapath M{M} K{K} N{N} nS{nS}")
    d = dense_case(M, K, N, n_out=max(1, K // 100), seed=7 * M + K + N + nS)
    chan = (np.sort(np.random.default_rng(M + K).choice(K, nS, replace=False)).astype(np.int32)
            if nS else None)
    for layout in (fq.ROWMAJOR, fq.TILED):
        _run(orc, d, chan, layout)


def test_without_outputs_and_bf16(orc):
    say("fused decode datapath without the optional outputs; BF16 output")
    d = workload("decode_nvfp4")
    _run(orc, d, d["chan_idx"], fq.TILED, with_outputs=False)
    _run(orc, d, d["chan_idx"], fq.TILED, with_outputs=False, y_dtype=1)
