"""fp4q_quantize_noalloc (the quantizer with the library's static per-GPU
scratch instead of a workspace) against fp4q_quantize with a caller
workspace, through the C ABI: codes, block scales, tensor scales and
residuals bit for bit, over calls in a row that take every NVFP4 path (the
two-pass large path, the single-launch small path whose exchange state lives
in the scratch, the grouped path) with the inputs shrinking, and MXFP4; plus
the host-side limit on the number of groups."""
import numpy as np
import pytest
import torch

import fp4_w4a4_quantized_amd as fq
from gpu_helpers import assert_quant_equal, need_gpu, say, to_dev
from workloads import dense_case

pytestmark = pytest.mark.gpu


def _outs(fmt, layout, rows, cols, nS, G, dev):
    blk = fq.BLOCK[fmt]
    if layout == fq.ROWMAJOR:
        q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        s = torch.empty((rows, cols // blk), dtype=torch.uint8, device=dev)
    else:
        cb, sb = fq.packed_bytes(fmt, layout, rows, cols)
        q = torch.empty(cb, dtype=torch.uint8, device=dev)
        s = torch.empty(sb, dtype=torch.uint8, device=dev)
    q.fill_(0xA5)
    s.fill_(0x5A)
    return {"q": q, "scales": s,
            "tscale": torch.full((G,), 7.0, dtype=torch.float32, device=dev) if fmt == 0 else None,
            "resid": torch.full((rows, nS), 3, dtype=torch.int16, device=dev) if nS else None,
            "layout": layout, "rows": rows, "cols": cols}


# (fmt, layout, rows, cols, nS, group offsets or None): shrinking inputs
CASES = [
    (0, fq.TILED, 1024, 4096, 64, None),        # large: partial maxima in the scratch
    (0, fq.ROWMAJOR, 64, 2048, 16, None),       # small: exchange state in the scratch
    (0, fq.ROWMAJOR, 333, 512, 8, [0, 40, 40, 41, 200, 333]),   # grouped amax words
    (0, fq.TILED, 48, 1024, 0, None),           # small again, fewer workgroups
    (1, fq.ROWMAJOR, 40, 256, 4, None),         # MXFP4: no scratch needed
]


def test_noalloc_matches_quantize(orc):
    dev = need_gpu()
    for i, (fmt, layout, rows, cols, nS, off) in enumerate(CASES):
        say(f"noalloc quantize call {i}: fmt {fmt} layout {layout} {rows}x{cols} nS {nS} "
            f"groups {1 if off is None else len(off) - 1}")
        d = dense_case(rows, cols, 8, n_out=max(1, cols // 100), seed=900 + i)
        G = 1 if off is None else len(off) - 1
        rng = np.random.default_rng(i)
        chan = (np.sort(np.stack([rng.choice(cols, nS, replace=False) for _ in range(G)]), 1)
                .astype(np.int32) if nS else None)
        x = to_dev(d["x"])
        doff = None if off is None else to_dev(np.array(off, np.int32))
        dch = None if chan is None else to_dev(chan)
        a = _outs(fmt, layout, rows, cols, nS, G, dev)
        b = _outs(fmt, layout, rows, cols, nS, G, dev)
        ws = torch.zeros(max(fq.quantize_workspace_bytes(fmt, rows, cols, G), 16),
                         dtype=torch.uint8, device=dev)
        fq.quantize_noalloc_into(fmt, layout, x, doff, G, dch, nS, a["q"], a["scales"],
                                 a["tscale"], a["resid"])
        fq.quantize_into(fmt, layout, x, doff, G, dch, nS, b["q"], b["scales"], b["tscale"],
                         b["resid"], ws)
        torch.cuda.synchronize(dev)
        for k in ("q", "scales", "tscale", "resid"):
            if a[k] is not None:
                assert torch.equal(a[k], b[k]), f"call {i}: {k} differs from fp4q_quantize"
        ref = orc.quantize(fmt, d["x"], offsets=None if off is None else np.array(off, np.int32),
                           chan_idx=chan)
        assert_quant_equal(a, ref, fmt)


def test_noalloc_rejects_too_many_groups():
    dev = need_gpu()
    say("noalloc quantize: group limit")
    x = torch.zeros((9000, 16), dtype=torch.int16, device=dev)
    off = torch.arange(9001, dtype=torch.int32, device=dev)
    q = torch.empty((9000, 8), dtype=torch.uint8, device=dev)
    s = torch.empty((9000, 1), dtype=torch.uint8, device=dev)
    t = torch.empty(9000, dtype=torch.float32, device=dev)
    with pytest.raises(fq.Fp4qError) as ei:
        fq.quantize_noalloc_into(0, fq.ROWMAJOR, x, off, 9000, None, 0, q, s, t, None)
    assert ei.value.status == -2
