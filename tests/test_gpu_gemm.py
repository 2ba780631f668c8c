"""GPU parity of fp4q_gemm against the FP64 oracle: every output of the
tiny and decode workloads, sampled outputs of the prefill workloads, ragged
tiles, channel counts that do not fill an MFMA step, BF16 output and an
output row stride.  Bound: |Y - Y_oracle| <= 1e-3 * Yabs per element."""
import numpy as np
import pytest
import torch

import fp4_w4a4_quantized_amd as fq
from gpu_helpers import workload, assert_gemm_close, dev_quant, need_gpu, say, to_dev, to_host
from workloads import CONFIGS, bf16_to_f32, dense_case

pytestmark = pytest.mark.gpu


def _prep(orc, fmt, d, chan):
    qa = orc.quantize(fmt, d["x"], chan_idx=chan)
    qb = orc.quantize(fmt, d["wt"])
    return qa, qb


def _gpu_gemm(fmt, qa, qb, chan, y_dtype=0, layout=fq.ROWMAJOR):
    a, b = dev_quant(qa, layout=layout, fmt=fmt), dev_quant(qb, layout=layout, fmt=fmt)
    y = fq.gemm(fmt, a, b, chan_idx=None if chan is None else to_dev(chan), y_dtype=y_dtype)
    torch.cuda.synchronize()
    return y


def _oracle_full(orc, fmt, qa, qb, chan):
    ta = qa["tscale"][0] if fmt == 0 else 1.0
    tb = qb["tscale"][0] if fmt == 0 else 1.0
    return orc.gemm_full(fmt, qa["q"], qa["scales"], ta, qb["q"], qb["scales"], tb, chan,
                         qa["resid"])


def _oracle_points(orc, fmt, qa, qb, chan, pm, pn):
    ta = qa["tscale"][0] if fmt == 0 else 1.0
    tb = qb["tscale"][0] if fmt == 0 else 1.0
    return orc.gemm_points(fmt, qa["q"], qa["scales"], ta, qb["q"], qb["scales"], tb, chan,
                           qa["resid"], pm, pn)


_PREP = {}


def _prep_cached(orc, fmt, name):
    """Oracle quantization of a named workload, shared by the layout variants."""
    key = (name, fmt)
    if key not in _PREP:
        d = workload(name)
        _PREP[key] = (d["chan_idx"],) + _prep(orc, fmt, d, d["chan_idx"])
    return _PREP[key]


@pytest.mark.parametrize("layout", [fq.ROWMAJOR, fq.TILED])
@pytest.mark.parametrize("name,fmt", [("tiny_nvfp4", 0), ("tiny_nvfp4", 1),
                                      ("decode_nvfp4", 0), ("decode_nvfp4", 1)])
def test_workload_all_outputs(orc, name, fmt, layout):
    need_gpu()
    say(f"gemm all outputs {name} fmt {fmt} layout {layout}")
    chan, qa, qb = _prep_cached(orc, fmt, name)
    y = to_host(_gpu_gemm(fmt, qa, qb, chan, layout=layout))
    yo, ya = _oracle_full(orc, fmt, qa, qb, chan)
    r = assert_gemm_close(y, yo, ya)
    say(f"  worst |dY|/Yabs = {r:.3e}")


@pytest.mark.parametrize("layout", [fq.ROWMAJOR, fq.TILED])
@pytest.mark.parametrize("name", ["prefill_nvfp4", "prefill_mxfp4"])
def test_prefill_sampled(orc, name, layout):
    """Full prefill shape (8192 x 4096 x 14336) in the benchmark's launch
    configuration; 40000 sampled outputs plus two full rows and columns."""
    need_gpu()
    say(f"gemm sampled {name} layout {layout}")
    cfg = CONFIGS[name]
    fmt = 0 if cfg["fmt"] == "nvfp4" else 1
    chan, qa, qb = _prep_cached(orc, fmt, name)
    y = to_host(_gpu_gemm(fmt, qa, qb, chan, layout=layout))
    M, N = y.shape
    rng = np.random.default_rng(123)
    pm = np.concatenate([rng.integers(0, M, 40000), np.full(N, M - 1), np.arange(M)])
    pn = np.concatenate([rng.integers(0, N, 40000), np.arange(N), np.full(M, N - 1)])
    yo, ya = _oracle_points(orc, fmt, qa, qb, chan, pm, pn)
    r = assert_gemm_close(y[pm, pn], yo, ya)
    say(f"  worst |dY|/Yabs = {r:.3e}")


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("M,N,K,nS", [(1, 1, 128, 0), (33, 17, 256, 5), (130, 200, 384, 37),
                                      (64, 96, 768, 32), (257, 129, 512, 128),
                                      (70, 300, 128, 128), (64, 100, 2048, 64),
                                      (1, 47, 1920, 63), (48, 49, 640, 64), (5, 50, 2048, 65)])
def test_ragged(orc, fmt, M, N, K, nS):
    need_gpu()
    say(f"gemm ragged fmt {fmt} M{M} N{N} K{K} nS{nS}")
    d = dense_case(M, K, N, n_out=max(1, K // 100), seed=M + 3 * N + K)
    chan = np.sort(np.random.default_rng(M).choice(K, nS, replace=False)).astype(np.int32)
    chan = chan if nS else None
    qa, qb = _prep(orc, fmt, d, chan)
    yo, ya = _oracle_full(orc, fmt, qa, qb, chan)
    for layout in (fq.ROWMAJOR, fq.TILED):
        y = to_host(_gpu_gemm(fmt, qa, qb, chan, layout=layout))
        assert_gemm_close(y, yo, ya)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("M,N,K,nS", [(300, 520, 512, 100), (256, 256, 256, 0), (513, 300, 768, 128),
                                      (260, 270, 256, 129), (1024, 768, 1024, 16)])
def test_large_tiles_ragged(orc, fmt, M, N, K, nS):
    """Shapes that take the 256x256-tile pipelined kernel (M, N >= 256,
    K % 256 == 0, |S| <= 128), with ragged edges, and the fallback past it."""
    need_gpu()
    say(f"gemm large-tile fmt {fmt} M{M} N{N} K{K} nS{nS}")
    d = dense_case(M, K, N, n_out=max(1, K // 100), seed=M + 7 * N + K + nS)
    chan = np.sort(np.random.default_rng(N).choice(K, nS, replace=False)).astype(np.int32)
    chan = chan if nS else None
    qa, qb = _prep(orc, fmt, d, chan)
    yo, ya = _oracle_full(orc, fmt, qa, qb, chan)
    for layout in (fq.ROWMAJOR, fq.TILED):
        y = to_host(_gpu_gemm(fmt, qa, qb, chan, layout=layout))
        assert_gemm_close(y, yo, ya)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("M,N,K,nS", [(256, 256, 128, 8), (512, 272, 384, 40), (300, 520, 640, 640),
                                      (768, 256, 256, 256), (257, 1000, 512, 96)])
def test_large_tiles_compensation_stages(orc, fmt, M, N, K, nS):
    """256x256-tile path with |S| % 32 != 0 (a partial compensation stage),
    N off the 16-row padding, |S| = K (every channel compensated)."""
    need_gpu()
    say(f"gemm large-tile comp stages fmt {fmt} M{M} N{N} K{K} nS{nS}")
    d = dense_case(M, K, N, n_out=max(1, K // 100), seed=M + 5 * N + K + nS)
    chan = np.sort(np.random.default_rng(N + nS).choice(K, nS, replace=False)).astype(np.int32)
    qa, qb = _prep(orc, fmt, d, chan)
    yo, ya = _oracle_full(orc, fmt, qa, qb, chan)
    for layout in (fq.ROWMAJOR, fq.TILED):
        y = to_host(_gpu_gemm(fmt, qa, qb, chan, layout=layout))
        assert_gemm_close(y, yo, ya)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("chan_kind", ["one_step", "edges"])
def test_large_tiles_clustered_channels(orc, fmt, chan_kind):
    """256x256-tile path with the compensated channels bunched into one
    128-column step (every channel of a compensation stage comes from the
    same B tile) or at the first and last columns of K."""
    need_gpu()
    M, N, K = 512, 512, 512
    if chan_kind == "one_step":
        chan = np.arange(256, 352, dtype=np.int32)                 # 96 channels, step 2
    else:
        chan = np.array([0, 1, 2, 127, 128, 383, 510, 511], np.int32)
    nS = len(chan)
    say(f"gemm large-tile clustered channels fmt {fmt} {chan_kind} nS{nS}")
    d = dense_case(M, K, N, n_out=4, seed=700 + nS)
    qa, qb = _prep(orc, fmt, d, chan)
    yo, ya = _oracle_full(orc, fmt, qa, qb, chan)
    for layout in (fq.ROWMAJOR, fq.TILED):
        y = to_host(_gpu_gemm(fmt, qa, qb, chan, layout=layout))
        assert_gemm_close(y, yo, ya)


@pytest.mark.parametrize("fmt", [0, 1])
def test_large_tiles_bf16_and_ldy(orc, fmt):
    """256x256-tile path: vector epilogue (FP32, BF16) and the element-wise
    one (row stride not a multiple of 8)."""
    dev = need_gpu()
    say(f"gemm large-tile bf16 + ldy fmt {fmt}")
    M, N, K, nS = 512, 384, 256, 64
    d = dense_case(M, K, N, n_out=3, seed=91)
    chan = np.sort(np.random.default_rng(3).choice(K, nS, replace=False)).astype(np.int32)
    qa, qb = _prep(orc, fmt, d, chan)
    yo, ya = _oracle_full(orc, fmt, qa, qb, chan)
    a = dev_quant(qa, layout=fq.TILED, fmt=fmt)
    b = dev_quant(qb, layout=fq.TILED, fmt=fmt)
    ws = torch.empty(fq.gemm_workspace_bytes(fmt, fq.TILED, M, N, K, nS), dtype=torch.uint8,
                     device=dev)
    for ldy in (400, 389):
        ybig = torch.full((M, ldy), 7.0, dtype=torch.float32, device=dev)
        fq.gemm_into(fmt, fq.TILED, M, N, K, a["q"], a["scales"], a["tscale"], b["q"],
                     b["scales"], b["tscale"], to_dev(chan), nS, a["resid"], ybig, 0, ldy, ws)
        torch.cuda.synchronize()
        yf = to_host(ybig)
        assert np.all(yf[:, N:] == 7.0)
        assert_gemm_close(yf[:, :N], yo, ya)
    yb = fq.gemm(fmt, a, b, chan_idx=to_dev(chan), y_dtype=1)
    torch.cuda.synchronize()
    ybf = bf16_to_f32(to_host(yb.view(torch.int16))).astype(np.float64)
    assert np.all(np.abs(ybf - yo) <= 1e-3 * ya + 2.0 ** -8 * np.abs(yo))


@pytest.mark.parametrize("fmt", [0, 1])
def test_bf16_output_and_ldy(orc, fmt):
    need_gpu()
    say(f"gemm bf16 out + ldy fmt {fmt}")
    d = dense_case(96, 256, 80, n_out=3, seed=77)
    chan = np.array([0, 5, 100, 255], np.int32)
    qa, qb = _prep(orc, fmt, d, chan)
    a, b = dev_quant(qa), dev_quant(qb)
    ybig = torch.full((96, 128), 7.0, dtype=torch.float32, device="cuda:0")
    fq.gemm_into(fmt, fq.ROWMAJOR, 96, 80, 256, a["q"], a["scales"], a["tscale"], b["q"],
                 b["scales"], b["tscale"], to_dev(chan), 4, a["resid"], ybig, 0, 128)
    yb = fq.gemm(fmt, a, b, chan_idx=to_dev(chan), y_dtype=1)
    torch.cuda.synchronize()
    yo, ya = _oracle_full(orc, fmt, qa, qb, chan)
    yf = to_host(ybig)
    assert np.all(yf[:, 80:] == 7.0)             # nothing written past N
    assert_gemm_close(yf[:, :80], yo, ya)
    # BF16 output: the FP32 result rounded once more (half a BF16 ulp)
    ybf = bf16_to_f32(to_host(yb.view(torch.int16))).astype(np.float64)
    assert np.all(np.abs(ybf - yo) <= 1e-3 * ya + 2.0 ** -8 * np.abs(yo))


def test_deterministic(orc):
    need_gpu()
    d = dense_case(200, 512, 300, n_out=5, seed=88)
    chan = np.array([1, 2, 3, 400], np.int32)
    qa, qb = _prep(orc, 0, d, chan)
    y1 = _gpu_gemm(0, qa, qb, chan)
    y2 = _gpu_gemm(0, qa, qb, chan)
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("layout", [fq.ROWMAJOR, fq.TILED])
def test_end_to_end_gpu_quantize_then_gemm(orc, layout):
    """GPU quantize feeding the GPU GEMM, against oracle quantize + oracle GEMM."""
    need_gpu()
    say(f"end-to-end decode workload on the GPU path, layout {layout}")
    d = workload("decode_nvfp4")
    chan = d["chan_idx"]
    a = fq.quantize(0, to_dev(d["x"]), chan_idx=to_dev(chan), layout=layout)
    b = fq.quantize(0, to_dev(d["wt"]), layout=layout)
    y = to_host(fq.gemm(0, a, b, chan_idx=to_dev(chan)))
    _, qa, qb = _prep_cached(orc, 0, "decode_nvfp4")
    rng = np.random.default_rng(4)
    pm, pn = rng.integers(0, 64, 20000), rng.integers(0, y.shape[1], 20000)
    yo, ya = _oracle_points(orc, 0, qa, qb, chan, pm, pn)
    assert_gemm_close(y[pm, pn], yo, ya)
