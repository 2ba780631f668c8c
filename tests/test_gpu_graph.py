"""The hot path captured in a HIP graph (as the benchmark and a serving loop
run it): every replay must reproduce the eager result bit for bit, with
eager work and synchronisations between the replays.  Dense decode shape
(fused single-launch quantizer, skinny GEMM) and a grouped expert layer
(fill kernel, per-group amax, quantize, grouped GEMM).  The eager result
itself is checked against the oracle in the other GPU tests; here it is the
reference for the replays."""
import numpy as np
import pytest
import torch

import fp4_w4a4_quantized_amd as fq
from gpu_helpers import need_gpu, say, to_dev, workload
from workloads import dense_case

pytestmark = pytest.mark.gpu


def _bufs(fmt, rows, K, nS, G, dev, layout=fq.ROWMAJOR):
    cb, sb = fq.packed_bytes(fmt, layout, rows, K)
    return dict(
        q=torch.empty(cb, dtype=torch.uint8, device=dev),
        s=torch.empty(sb, dtype=torch.uint8, device=dev),
        t=torch.empty(G, dtype=torch.float32, device=dev) if fmt == fq.NVFP4 else None,
        r=torch.empty((rows, nS), dtype=torch.int16, device=dev) if nS else None,
        ws=torch.zeros(max(fq.quantize_workspace_bytes(fmt, rows, K, G), 16), dtype=torch.uint8,
                       device=dev))


def _check_replays(run, outputs, scramble):
    """run(): launches the sequence on the current stream.  outputs(): list of
    result tensors.  scramble(): eager work that overwrites the outputs."""
    run()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outputs()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(4):
        scramble()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outputs(), ref)):
            assert torch.equal(o, r), f"replay {rep}: output {i} differs from the eager result"
        run()  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("layout", [fq.ROWMAJOR, fq.TILED])
@pytest.mark.parametrize("fmt", [0, 1])
def test_graph_decode_step(fmt, layout):
    dev = need_gpu()
    say(f"graph replay: decode quantize + gemm, fmt {fmt} layout {layout}")
    d = workload("decode_nvfp4")
    M, K = d["x"].shape
    N = d["wt"].shape[0]
    nS = d["chan_idx"].size
    x, chan = to_dev(d["x"]), to_dev(d["chan_idx"])
    w = fq.quantize(fmt, to_dev(d["wt"]), layout=layout)
    b = _bufs(fmt, M, K, nS, 1, dev, layout)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)

    def run():
        fq.quantize_into(fmt, layout, x, None, 1, chan, nS, b["q"], b["s"], b["t"], b["r"],
                         b["ws"])
        fq.gemm_into(fmt, layout, M, N, K, b["q"], b["s"], b["t"], w["q"], w["scales"], w["tscale"], chan,
                     nS, b["r"], y, 0, N)

    def outputs():
        return [t for t in (b["q"], b["s"], b["t"], b["r"], y) if t is not None]

    def scramble():
        for t in outputs():
            t.fill_(3)

    _check_replays(run, outputs, scramble)


@pytest.mark.parametrize("N,nS", [(160, 8), (512, 8), (512, 104)])
def test_graph_grouped_layer(N, nS):
    """Staged grouped path with the compensation weights gathered into the
    workspace inside the captured graph (N >= 256), and the general grouped
    kernel (N < 256)."""
    dev = need_gpu()
    say(f"graph replay: grouped quantize + grouped gemm (NVFP4), N {N}, |S| {nS}")
    fmt = fq.NVFP4
    K = 256
    off_h = np.array([0, 40, 40, 41, 200, 333], np.int32)
    G = off_h.size - 1
    rows = int(off_h[-1])
    x = to_dev(dense_case(rows, K, 8, n_out=3, seed=91)["x"])
    off = to_dev(off_h)
    rng = np.random.default_rng(5)
    chan = to_dev(np.sort(np.stack([rng.choice(K, nS, replace=False) for _ in range(G)]), 1)
                  .astype(np.int32))
    ws = [fq.quantize(fmt, to_dev(dense_case(1, K, N, seed=70 + g)["wt"])) for g in range(G)]
    bq = torch.stack([q["q"] for q in ws])
    bs = torch.stack([q["scales"] for q in ws])
    bt = torch.cat([q["tscale"] for q in ws])
    b = _bufs(fmt, rows, K, nS, G, dev)
    y = torch.empty((rows, N), dtype=torch.float32, device=dev)
    gwsb = fq.grouped_gemm_workspace_bytes(fmt, rows, N, K, G, nS)
    gws = torch.empty(gwsb, dtype=torch.uint8, device=dev) if gwsb else None
    # NVFP4 on the 128 x 512 kernel gathers every group's B_S into the workspace
    assert (gwsb > 0) == (N >= 256 and nS > 0)

    def run():
        fq.quantize_into(fmt, fq.ROWMAJOR, x, off, G, chan, nS, b["q"], b["s"], b["t"], b["r"],
                         b["ws"])
        fq.grouped_gemm_into(fmt, rows, N, K, off, G, b["q"], b["s"], b["t"], bq, bs, bt, chan, nS,
                             b["r"], y, 0, gws)

    def outputs():
        return [b["q"], b["s"], b["t"], b["r"], y]

    def scramble():
        for t in outputs():
            t.fill_(5)

    _check_replays(run, outputs, scramble)
