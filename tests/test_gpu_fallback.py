"""GPU parity of fp4q_qdq_fallback (Outlier Fallback: quantize-dequantize
with the deadzone entries kept; MXFP4 error-decomposition abstract) against
the oracle: every output bit for bit (the NVFP4 values are one FP32
rounding of an exact product, the same operations on both sides) and the
fallback count, at the prefill activation size in both formats, on ragged
and special-valued tensors, with an output row stride, and the hand-worked
golden blocks."""
import json
import os

import numpy as np
import pytest
import torch

import fp4_w4a4_quantized_amd as fq
from gpu_helpers import need_gpu, say, to_dev, to_host, workload
from workloads import bf16_bits, dense_case

pytestmark = pytest.mark.gpu


def _check(orc, fmt, x, ldy_pad=0):
    dev = need_gpu()
    rows, cols = x.shape
    want, nwant = orc.qdq_fallback(fmt, x)
    xd = to_dev(x)
    y = torch.full((rows, cols + ldy_pad), 7.0, dtype=torch.float32, device=dev)
    n = torch.full((1,), -5, dtype=torch.int64, device=dev)
    wsb = fq.qdq_fallback_workspace_bytes(fmt, rows, cols)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    fq.qdq_fallback_into(fmt, xd, y, n, ws)
    got = to_host(y)
    assert np.all(got[:, cols:] == 7.0), "written past the row"
    bad = np.argwhere(got[:, :cols].view(np.uint32) != want.view(np.uint32))
    assert bad.size == 0, f"{len(bad)} outputs differ, first {bad[:3].tolist()}"
    assert int(to_host(n)[0]) == nwant
    return nwant


@pytest.mark.parametrize("fmt", [0, 1])
def test_prefill_activations(orc, fmt):
    say(f"outlier fallback, prefill activations 8192 x 4096, fmt {fmt}")
    d = workload("prefill_nvfp4")
    n = _check(orc, fmt, d["x"])
    say(f"  fallback entries {n} ({n / d['x'].size:.3%})")


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("rows,cols,pad", [(1, 32, 0), (3, 96, 4), (77, 640, 0), (130, 2048, 12),
                                           (64, 2048, 0), (9, 48, 4), (700, 64, 0), (900, 32, 8)])
def test_ragged(orc, fmt, rows, cols, pad):
    if fmt == 1 and cols % 32:
        pytest.skip("MXFP4 needs cols % 32")
    say(f"outlier fallback fmt {fmt} {rows}x{cols} ldy pad {pad}")
    d = dense_case(rows, cols, 8, n_out=max(1, cols // 100), seed=rows * 3 + cols + fmt)
    _check(orc, fmt, d["x"], pad)


@pytest.mark.parametrize("fmt", [0, 1])
def test_special_values(orc, fmt):
    say(f"outlier fallback special values fmt {fmt}")
    rng = np.random.default_rng(9)
    x = bf16_bits(rng.standard_normal((8, 256)).astype(np.float32))
    x[0] = 0
    x[1, :32] = 0x8000                                   # -0.0
    x[2, :] = np.arange(256, dtype=np.uint16) + 1        # positive subnormals
    x[3, :] = (np.arange(256, dtype=np.uint16) + 1) | 0x8000
    x[4, :16] = 0x7F7F                                   # largest finite bf16
    x[5, ::2] = bf16_bits(np.float32(0.25))
    _check(orc, fmt, x)
    # a tensor of tiny values: the NVFP4 tensor scale far below 2^-87
    tiny = bf16_bits((rng.standard_normal((40, 256)) * 1e-30).astype(np.float32))
    tiny[3, :] = (np.arange(256, dtype=np.uint16) + 1)   # subnormals beside them
    _check(orc, fmt, tiny)


def test_golden_blocks(orc):
    need_gpu()
    g = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                                    "fallback_blocks.json")))
    for fmt, key, cols in ((1, "mxfp4", 32), (0, "nvfp4", 16)):
        x = np.zeros((1, cols), np.uint16)
        want = np.zeros(cols, np.float32)
        for e in g[key]["elements"]:
            x[0, e["col"]] = int(e["bits"], 16)
            want[e["col"]] = np.float32(e["out"])
        y, n = fq.qdq_fallback(fmt, to_dev(x))
        assert np.array_equal(to_host(y)[0].view(np.uint32), want.view(np.uint32)), key
        assert int(to_host(n)[0]) == g[key]["n_fallback"]


def test_empty_tensor_count():
    dev = need_gpu()
    x = torch.empty((0, 64), dtype=torch.int16, device=dev)
    y = torch.empty((0, 64), dtype=torch.float32, device=dev)
    n = torch.full((1,), 9, dtype=torch.int64, device=dev)
    ws = torch.empty(fq.qdq_fallback_workspace_bytes(0, 0, 64), dtype=torch.uint8, device=dev)
    fq.qdq_fallback_into(0, x, y, n, ws)
    assert int(to_host(n)[0]) == 0
