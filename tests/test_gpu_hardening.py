"""GPU tests of the boundary's failure handling and state rules (through the
C ABI):

  * the small-tensor NVFP4 quantizer keeps its exchange state in the
    caller's workspace: calls on two streams with two workspaces run
    concurrently and both stay exact;
  * when the exchange's bounded wait runs out (forced from the host by the
    test hooks: a low spin limit and one workgroup that skips its slot
    store, so every kernel still exits normally), the outputs are poisoned
    (NaN tensor scale, E4M3 NaN block scales, BF16 NaN residuals) and the
    workspace's status word reports it; the next normal call is exact again;
  * the injected launch failure returns FP4Q_ERR_HIP without touching the
    outputs, once;
  * the NVFP4 error decomposition flags a tensor whose amax is below 2^-89
    (where its exact sums are not guaranteed; the oracle rejects it).
"""
import numpy as np
import pytest
import torch

import fp4_w4a4_quantized_amd as fq
from gpu_helpers import assert_gemm_close, assert_quant_equal, need_gpu, say, to_dev, to_host, workload
from workloads import bf16_bits, dense_case

pytestmark = pytest.mark.gpu


def _bufs(rows, cols, nS, dev, layout=fq.ROWMAJOR):
    if layout == fq.ROWMAJOR:
        q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        s = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
    else:
        cb, sb = fq.packed_bytes(0, layout, rows, cols)
        q = torch.empty(cb, dtype=torch.uint8, device=dev)
        s = torch.empty(sb, dtype=torch.uint8, device=dev)
    return {"q": q, "scales": s, "tscale": torch.empty(1, dtype=torch.float32, device=dev),
            "resid": torch.empty((rows, nS), dtype=torch.int16, device=dev) if nS else None,
            "layout": layout, "rows": rows, "cols": cols,
            "ws": torch.zeros(fq.quantize_workspace_bytes(0, rows, cols, 1), dtype=torch.uint8,
                              device=dev)}


def _quant(b, x, chan, nS):
    fq.quantize_into(0, b["layout"], x, None, 1, chan, nS, b["q"], b["scales"], b["tscale"],
                     b["resid"], b["ws"])


def test_two_streams_two_workspaces(orc):
    """Small NVFP4 tensors quantized on two streams at once, each stream with
    its own workspace: every result bit-exact."""
    dev = need_gpu()
    say("small NVFP4 quantize on two concurrent streams")
    cases = [dense_case(64, 2048, 8, n_out=20, seed=700 + i) for i in range(2)]
    xs = [to_dev(c["x"]) for c in cases]
    refs = [orc.quantize(0, c["x"]) for c in cases]
    streams = [torch.cuda.Stream(dev), torch.cuda.Stream(dev)]
    reps = 40
    outs = [[_bufs(64, 2048, 0, dev) for _ in range(reps)] for _ in range(2)]
    for i in range(2):   # one workspace per stream, reused by all its calls
        for b in outs[i][1:]:
            b["ws"] = outs[i][0]["ws"]
    torch.cuda.synchronize(dev)
    for r in range(reps):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                _quant(outs[i][r], xs[i], None, 0)
    torch.cuda.synchronize(dev)
    for i in range(2):
        assert fq.quantize_status(outs[i][0]["ws"], streams[i]) == 0
        for r in range(reps):
            assert_quant_equal(outs[i][r], dict(refs[i], resid=None), 0)


@pytest.mark.parametrize("layout", [fq.ROWMAJOR, fq.TILED])
def test_grid_exchange_expiry_poisons_and_reports(orc, layout):
    dev = need_gpu()
    say(f"forced expiry of the small-tensor exchange, layout {layout}")
    d = workload("decode_nvfp4")
    M, K = d["x"].shape
    chan = d["chan_idx"]
    nS = chan.size
    x, dch = to_dev(d["x"]), to_dev(chan)
    ref = orc.quantize(0, d["x"], chan_idx=chan)
    b = _bufs(M, K, nS, dev, layout)
    _quant(b, x, dch, nS)          # a normal call first
    assert fq.quantize_status(b["ws"]) == 0
    assert_quant_equal(b, ref, 0)
    try:
        fq.test_hook(fq.binding.HOOK_GRID_SPIN_LIMIT, 256)
        fq.test_hook(fq.binding.HOOK_GRID_SKIP_SLOT, 3)
        _quant(b, x, dch, nS)
        torch.cuda.synchronize(dev)
    finally:
        fq.test_hook(fq.binding.HOOK_RESET)
    st = fq.quantize_status(b["ws"])
    assert st == fq.binding.QSTATUS_GRID_EXPIRED, st
    assert np.isnan(to_host(b["tscale"])[0])
    # every workgroup waited for the skipped slot: every block scale is the
    # E4M3 NaN code and every residual a BF16 NaN
    from gpu_helpers import host_packed
    _, hs = host_packed(b, 0)
    assert np.all(hs == 0x7F)
    assert np.all(to_host(b["resid"]) == 0x7FC0)
    # the GEMM on the poisoned operand is NaN, not a silent wrong value
    w = fq.quantize(0, to_dev(d["wt"]), layout=layout)
    y = to_host(fq.gemm(0, b, w, chan_idx=dch))
    assert np.all(np.isnan(y))
    # the status was cleared by the query; the next normal call is exact
    assert fq.quantize_status(b["ws"]) == 0
    _quant(b, x, dch, nS)
    assert fq.quantize_status(b["ws"]) == 0
    assert_quant_equal(b, ref, 0)


def test_injected_launch_failure_leaves_outputs(orc):
    dev = need_gpu()
    say("injected launch failure on the GPU")
    d = dense_case(16, 256, 8, n_out=2, seed=710)
    x = to_dev(d["x"])
    b = _bufs(16, 256, 0, dev)
    b["q"].fill_(0x5A)
    b["scales"].fill_(0x5A)
    torch.cuda.synchronize(dev)
    fq.test_hook(fq.binding.HOOK_FAIL_NEXT_LAUNCH, 719)
    with pytest.raises(fq.Fp4qError) as ei:
        _quant(b, x, None, 0)
    fq.test_hook(fq.binding.HOOK_RESET)
    assert ei.value.status == -4 and "hipError 719" in str(ei.value)
    torch.cuda.synchronize(dev)
    assert np.all(to_host(b["q"]) == 0x5A) and np.all(to_host(b["scales"]) == 0x5A)
    _quant(b, x, None, 0)             # the hook fired once
    assert_quant_equal(b, dict(orc.quantize(0, d["x"]), resid=None), 0)


def test_decomposition_flags_tiny_nvfp4_tensor(orc):
    need_gpu()
    say("NVFP4 decomposition of a tensor with amax below 2^-89")
    # amax 2^-120: the tensor scale is an FP32 subnormal and 6 Q_s(amax) is
    # not a multiple of 2^-136, so the oracle rejects the tensor
    rng = np.random.default_rng(12)
    tiny = bf16_bits((2.0 ** -120 * rng.choice([-1.0, 1.0, 0.5, 0.75], (8, 64))).astype(np.float32))
    with pytest.raises(ValueError):
        orc.error_decompose(tiny, fmt=0)
    assert fq.error_decompose(0, to_dev(tiny))["flags"] == fq.binding.DEC_INEXACT
    # amax 1e-30 (about 2^-99.7): below the 2^-89 guarantee, so flagged, but
    # these terms happen to fit the fixed point, the oracle accepts the
    # tensor, and the sums agree bit for bit
    small = bf16_bits((1e-30 * rng.choice([-1.0, 1.0, 0.5, 0.25], (8, 64))).astype(np.float32))
    g = fq.error_decompose(0, to_dev(small))
    assert g["flags"] == fq.binding.DEC_INEXACT
    assert g["exact"] == orc.error_decompose(small, fmt=0)["exact"]
    # a normal tensor, an all-zero tensor and MXFP4 carry no flag
    normal = dense_case(8, 64, 8, seed=13)["x"]
    assert fq.error_decompose(0, to_dev(normal))["flags"] == 0
    assert fq.error_decompose(0, to_dev(np.zeros((8, 64), np.uint16)))["flags"] == 0
    assert fq.error_decompose(1, to_dev(tiny))["flags"] == 0
    # at 2^-89 exactly the sums are exact and agree with the oracle
    edge = tiny.copy()
    edge[0, 0] = bf16_bits(np.array([2.0 ** -89], np.float32))[0]
    edge[0, 1:] = 0
    g = fq.error_decompose(0, to_dev(edge))
    o = orc.error_decompose(edge, fmt=0)
    assert g["flags"] == 0 and g["exact"] == o["exact"]
