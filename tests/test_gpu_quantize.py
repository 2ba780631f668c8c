"""GPU parity of fp4q_quantize against the oracle: codes, block scales,
tensor scales and residuals bit for bit, at the workload shapes (full
tensors), ragged shapes and the degenerate cases."""
import numpy as np
import pytest
import torch

import fp4_w4a4_quantized_amd as fq
from gpu_helpers import workload, assert_quant_equal, need_gpu, say, to_dev, to_host
from workloads import CONFIGS, bf16_bits, dense_case, moe_case

pytestmark = pytest.mark.gpu


_REF = {}


def _run(orc, fmt, x, chan=None, offsets=None, layout=fq.ROWMAJOR, key=None):
    dev = need_gpu()
    if key is None or key not in _REF:
        ref = orc.quantize(fmt, x, offsets=offsets, chan_idx=chan)
        if key is not None:
            _REF[key] = ref
    ref = _REF[key] if key is not None else ref
    got = fq.quantize(fmt, to_dev(x), group_offsets=None if offsets is None else to_dev(offsets),
                      chan_idx=None if chan is None else to_dev(np.ascontiguousarray(chan)),
                      layout=layout)
    torch.cuda.synchronize(dev)
    assert_quant_equal(got, ref, fmt)


@pytest.mark.parametrize("layout", [fq.ROWMAJOR, fq.TILED])
@pytest.mark.parametrize("name", ["tiny_nvfp4", "decode_nvfp4", "prefill_nvfp4", "prefill_mxfp4"])
def test_workload_activations(orc, name, layout):
    cfg = CONFIGS[name]
    say(f"quantize activations {name} layout {layout}")
    d = dense_case(**{**cfg, "N": 8})   # weights are not needed here
    _run(orc, 0 if cfg["fmt"] == "nvfp4" else 1, d["x"], d["chan_idx"], layout=layout,
         key=("act", name))


@pytest.mark.parametrize("layout", [fq.ROWMAJOR, fq.TILED])
@pytest.mark.parametrize("name", ["tiny_nvfp4", "decode_nvfp4"])
@pytest.mark.parametrize("fmt", [0, 1])
def test_workload_weights(orc, name, fmt, layout):
    say(f"quantize weights {name} fmt {fmt} layout {layout}")
    d = workload(name)
    _run(orc, fmt, d["wt"], layout=layout, key=("w", name, fmt))


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("rows,cols,nS", [(1, 256, 3), (37, 96 * 2, 11), (100, 64, 64),
                                          (300, 512, 0), (5, 2048, 2048), (3, 17408, 40),
                                          (600, 512, 37), (64, 4096, 64), (129, 2048, 64)])
def test_ragged_and_channel_counts(orc, fmt, rows, cols, nS):
    if fmt == 1 and cols % 32:
        pytest.skip("MXFP4 needs cols % 32")
    say(f"quantize ragged fmt {fmt} {rows}x{cols} nS {nS}")
    d = dense_case(rows, cols, 8, n_out=max(1, cols // 100), seed=rows * 7 + cols)
    chan = np.sort(np.random.default_rng(rows).choice(cols, nS, replace=False)).astype(np.int32)
    _run(orc, fmt, d["x"], chan if nS else None)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("rows,cols,nS", [(1, 128, 3), (17, 384, 11), (63, 256, 0),
                                          (65, 1024, 64), (3, 17408, 40), (600, 512, 37),
                                          (129, 2048, 64)])
def test_tiled_ragged(orc, fmt, rows, cols, nS):
    """Tiled packed layout: row counts off the 16- and 64-row padding, and
    nothing written past fp4q_packed_bytes()."""
    dev = need_gpu()
    say(f"quantize tiled fmt {fmt} {rows}x{cols} nS {nS}")
    d = dense_case(rows, cols, 8, n_out=max(1, cols // 100), seed=rows * 5 + cols)
    chan = np.sort(np.random.default_rng(rows).choice(cols, nS, replace=False)).astype(np.int32)
    ref = orc.quantize(fmt, d["x"], chan_idx=chan if nS else None)
    cb, sb = fq.packed_bytes(fmt, fq.TILED, rows, cols)
    tail = 512
    q = torch.full((cb + tail,), 0xA5, dtype=torch.uint8, device=dev)
    sc = torch.full((sb + tail,), 0x5A, dtype=torch.uint8, device=dev)
    ts = torch.empty(1, dtype=torch.float32, device=dev) if fmt == 0 else None
    R = torch.empty((rows, nS), dtype=torch.int16, device=dev) if nS else None
    wsb = fq.quantize_workspace_bytes(fmt, rows, cols, 1)
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=dev)
    fq.quantize_into(fmt, fq.TILED, to_dev(d["x"]), None, 1, to_dev(chan) if nS else None, nS,
                     q, sc, ts, R, ws)
    torch.cuda.synchronize(dev)
    qh, sh = to_host(q), to_host(sc)
    assert np.all(qh[cb:] == 0xA5) and np.all(sh[sb:] == 0x5A), "write past the packed size"
    got = {"q": q[:cb], "scales": sc[:sb], "tscale": ts, "resid": R, "layout": fq.TILED,
           "rows": rows, "cols": cols}
    assert_quant_equal(got, ref, fmt)


def test_workspace_reuse_across_paths(orc):
    """One NVFP4 workspace (zero-filled once, as the header asks) through the
    single-launch small-tensor path, the two-pass large path, the grouped
    path and the small path again: every result exact whatever the previous
    call left in the workspace, and no exchange reported expired."""
    dev = need_gpu()
    say("quantize workspace reuse across paths")
    wsb = max(fq.quantize_workspace_bytes(0, 4096, 4096, 1), fq.quantize_workspace_bytes(0, 600, 512, 5))
    ws = torch.zeros((wsb,), dtype=torch.uint8, device=dev)
    cases = [(64, 2048, None), (1, 256, None), (600, 4096, None),
             (333, 512, np.array([0, 40, 40, 41, 200, 333], np.int32)), (64, 2048, None),
             (300, 4096, None)]
    for i, (rows, cols, off) in enumerate(cases):
        d = dense_case(rows, cols, 8, n_out=3, seed=500 + i)
        G = 1 if off is None else off.size - 1
        ref = orc.quantize(0, d["x"], offsets=off)
        q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        sc = torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev)
        ts = torch.empty(G, dtype=torch.float32, device=dev)
        fq.quantize_into(0, fq.ROWMAJOR, to_dev(d["x"]), None if off is None else to_dev(off), G,
                         None, 0, q, sc, ts, None, ws)
        torch.cuda.synchronize(dev)
        assert_quant_equal({"q": q, "scales": sc, "tscale": ts, "resid": None}, ref, 0)
    assert fq.quantize_status(ws) == 0


@pytest.mark.parametrize("fmt", [0, 1])
def test_special_values(orc, fmt):
    say(f"quantize special values fmt {fmt}")
    rng = np.random.default_rng(5)
    x = bf16_bits(rng.standard_normal((16, 256)).astype(np.float32))
    x[0] = 0                        # all-zero row
    x[1, :32] = 0x8000              # -0.0
    x[2, :] = np.arange(256, dtype=np.uint16) + 1          # positive subnormals
    x[3, :] = (np.arange(256, dtype=np.uint16) + 1) | 0x8000
    x[4, :16] = 0x7F7F              # largest finite bf16
    x[4, 16:32] = 0xFF7F
    x[5, :] = bf16_bits(np.full(256, 1e-30, np.float32))
    x[6, ::2] = bf16_bits(np.float32(2.5))                 # exact ties
    x[7, :] = bf16_bits(np.linspace(-7, 7, 256).astype(np.float32))
    x[8, ::3] = 0x8000              # -0.0 inside blocks with a nonzero maximum
    x[9, 1::2] = 0x8000
    chan = np.arange(0, 256, 9, dtype=np.int32)
    _run(orc, fmt, x, chan)
    # tiny-magnitude tensor (tensor scale far below one)
    _run(orc, fmt, x[2:4].copy(), chan)


def _special_rows(cols, rng):
    """Ten rows of the special values of test_special_values, `cols` wide."""
    x = bf16_bits(rng.standard_normal((10, cols)).astype(np.float32))
    x[0] = 0
    x[1, :32] = 0x8000
    x[2, :] = (np.arange(cols) % 255 + 1).astype(np.uint16)
    x[3, :] = x[2, :] | 0x8000
    x[4, :16] = 0x7F7F
    x[4, 16:32] = 0xFF7F
    x[5, :] = bf16_bits(np.full(cols, 1e-30, np.float32))
    x[6, ::2] = bf16_bits(np.float32(2.5))
    x[7, :] = bf16_bits(np.linspace(-7, 7, cols).astype(np.float32))
    x[8, ::3] = 0x8000
    x[9, 1::2] = 0x8000
    return x


@pytest.mark.parametrize("layout", [fq.ROWMAJOR, fq.TILED])
@pytest.mark.parametrize("fmt", [0, 1])
def test_special_values_large(orc, fmt, layout):
    """The special values inside tensors large enough for the two-pass NVFP4
    path (the tile quantizer): special rows spread through 1,200 x 256
    random rows, and a tensor of subnormal and tiny values alone, whose
    NVFP4 tensor scale is far below 2^-87 (the IEEE-division form)."""
    say(f"quantize special values, large tensors, fmt {fmt} layout {layout}")
    rng = np.random.default_rng(15)
    x = bf16_bits(rng.standard_normal((1200, 256)).astype(np.float32))
    for i in range(0, 1200, 97):
        x[i:i + 10] = _special_rows(256, rng)
    chan = np.arange(3, 256, 9, dtype=np.int32)
    _run(orc, fmt, x, chan, layout=layout)
    tiny = np.tile(_special_rows(256, rng)[2:4], (600, 1))
    tiny[::7, 5] = bf16_bits(np.float32(3e-39))
    _run(orc, fmt, tiny, chan, layout=layout)
    # tensor scales on both sides of 2^-87: amax 2688 * 2^-87 * (1 +- 1/8)
    for f in (0.875, 1.125):
        xs = rng.standard_normal((1100, 128)).astype(np.float32)
        xs *= np.float32(2688 * 2.0 ** -87 * f) / np.abs(xs).max()
        _run(orc, fmt, bf16_bits(xs), chan[chan < 128], layout=layout)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("rows,cols,nS", [(5000, 32, 4), (4000, 64, 9), (3000, 96, 5),
                                          (1100, 160, 0), (70, 4224, 128), (33, 8192, 300),
                                          (2, 69632, 64), (1, 266240, 64), (130, 4096, 2500)])
def test_tile_widths(orc, fmt, rows, cols, nS):
    """Row-major shapes for every tile width of the tile quantizer (1, 2 and
    4 units across), partial column tiles, channel lists longer than a
    tile's share, rows wider than its LDS channel table and channel lists
    longer than it stages in LDS."""
    say(f"quantize tile widths fmt {fmt} {rows}x{cols} nS {nS}")
    d = dense_case(rows, cols, 8, n_out=max(1, cols // 100), seed=rows + 3 * cols)
    chan = np.sort(np.random.default_rng(cols).choice(cols, nS, replace=False)).astype(np.int32)
    _run(orc, fmt, d["x"], chan if nS else None)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("rows", [20, 600])
def test_ldx_larger_than_cols(orc, fmt, rows):
    """Row stride 640 over 512 used columns: the single-launch small-tensor
    path (20 rows) and the two-pass path (600 rows)."""
    need_gpu()
    say(f"quantize with row stride > cols, fmt {fmt}, {rows} rows")
    d = dense_case(rows, 640, 8, seed=9 + rows)
    chan = np.array([1, 255, 256, 511], np.int32)
    ref = orc.quantize(fmt, d["x"][:, :512].copy(), chan_idx=chan)
    xt = to_dev(d["x"])[:, :512]    # a strided view: ldx = 640
    got = fq.quantize(fmt, xt, chan_idx=to_dev(chan))
    torch.cuda.synchronize()
    assert_quant_equal(got, ref, fmt)


@pytest.mark.parametrize("fmt", [0, 1])
def test_grouped_small(orc, fmt):
    say(f"quantize grouped small fmt {fmt}")
    x = dense_case(90, 256, 8, n_out=3, seed=41)["x"]
    off = np.array([0, 0, 13, 13, 14, 60, 90, 90], np.int32)   # empty and 1-row groups
    G = off.size - 1
    rng = np.random.default_rng(2)
    chan = np.sort(np.stack([rng.choice(256, 7, replace=False) for _ in range(G)]), 1)
    _run(orc, fmt, x, chan.astype(np.int32), off)


@pytest.mark.parametrize("fmt", [0, 1])
def test_grouped_wide_rows(orc, fmt):
    """Rows wider than the workgroup's LDS channel table (17408 columns)."""
    say(f"quantize grouped wide rows fmt {fmt}")
    x = dense_case(40, 17408, 8, n_out=30, seed=43)["x"]
    off = np.array([0, 10, 10, 11, 40], np.int32)
    G = off.size - 1
    rng = np.random.default_rng(8)
    chan = np.sort(np.stack([rng.choice(17408, 5, replace=False) for _ in range(G)]), 1)
    _run(orc, fmt, x, chan.astype(np.int32), off)


@pytest.mark.parametrize("layout", [fq.ROWMAJOR, fq.TILED])
@pytest.mark.parametrize("fmt", [0, 1])
def test_grouped_tiles_across_groups(orc, fmt, layout):
    """Groups whose boundaries fall inside 16-row tiles (empty and one-row
    groups among them), a group of tiny values (its NVFP4 tensor scale far
    below 2^-87: the IEEE-division form for its waves), special values, and
    7 channels per group; both layouts."""
    say(f"quantize grouped tiles across groups fmt {fmt} layout {layout}")
    rng = np.random.default_rng(23)
    x = bf16_bits(rng.standard_normal((700, 384)).astype(np.float32))
    x[300:513] = bf16_bits((rng.standard_normal((213, 384)) * 1e-30).astype(np.float32))
    x[22:32] = _special_rows(384, rng)
    off = np.array([0, 0, 5, 21, 22, 300, 300, 513, 700], np.int32)
    G = off.size - 1
    chan = np.sort(np.stack([rng.choice(384, 7, replace=False) for _ in range(G)]), 1)
    _run(orc, fmt, x, chan.astype(np.int32), off, layout=layout)


def test_grouped_moe_workload(orc):
    """MoE layer at full size: 32768 routed rows x 2048, 128 experts with
    per-expert tensor scales and 32 channels each (and the down input)."""
    say("quantize grouped MoE workload")
    m = moe_case(**CONFIGS["moe_nvfp4"], with_weights=False)
    _run(orc, 0, m["x_perm"], m["chan_gate_up"], m["offsets"])
    _run(orc, 0, m["h_perm"], m["chan_down"], m["offsets"])


def test_deterministic(orc):
    dev = need_gpu()
    d = dense_case(64, 2048, 8, n_out=20, seed=2)
    x = to_dev(d["x"])
    a = fq.quantize(0, x, chan_idx=to_dev(d["chan_idx"]) if d["chan_idx"].size else None)
    b = fq.quantize(0, x)
    torch.cuda.synchronize(dev)
    assert torch.equal(a["q"], b["q"]) and torch.equal(a["scales"], b["scales"])


def test_small_nvfp4_many_launches_in_a_row(orc):
    """The one-launch NVFP4 path combines its workgroups' maxima through
    per-device state that alternates between launches.  Forty back-to-back
    launches of tensors whose maxima rise and fall (and one of 1, 16 and 32
    workgroups' size), with no synchronisation between them, each match the
    oracle; then the same sequence replayed three times from a HIP graph."""
    dev = need_gpu()
    say("small NVFP4 quantize, 40 launches in a row")
    rng = np.random.default_rng(17)
    shapes = [(32, 2048), (16, 256), (64, 2048), (7, 512)]   # 16, 1, 32, 1 workgroups
    xs, refs = [], []
    for i in range(40):
        r, c = shapes[i % len(shapes)]
        x = rng.standard_normal((r, c)).astype(np.float32) * np.float32(4.0 ** ((i * 7) % 5 - 2))
        xb = bf16_bits(x)
        xs.append(to_dev(xb))
        refs.append(orc.quantize(0, xb))
    outs = [fq.quantize(0, x) for x in xs]
    torch.cuda.synchronize(dev)
    for got, ref in zip(outs, refs):
        assert_quant_equal(got, ref, 0)

    bufs = []
    for x in xs:
        r, c = x.shape
        bufs.append(dict(q=torch.empty((r, c // 2), dtype=torch.uint8, device=dev),
                         s=torch.empty((r, c // 16), dtype=torch.uint8, device=dev),
                         t=torch.empty(1, dtype=torch.float32, device=dev)))
    ws = torch.zeros(max(fq.quantize_workspace_bytes(0, 128, 2048, 1), 16), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.Stream(dev)
    with torch.cuda.stream(stream):
        fq.quantize_into(0, fq.ROWMAJOR, xs[0], None, 1, None, 0, bufs[0]["q"], bufs[0]["s"],
                         bufs[0]["t"], None, ws)
        torch.cuda.synchronize(dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for x, b in zip(xs, bufs):
                fq.quantize_into(0, fq.ROWMAJOR, x, None, 1, None, 0, b["q"], b["s"], b["t"],
                                 None, ws)
    for _ in range(3):
        for b in bufs:
            b["q"].zero_()
            b["t"].zero_()
        torch.cuda.synchronize(dev)
        g.replay()
        torch.cuda.synchronize(dev)
        for b, ref in zip(bufs, refs):
            got = {"q": b["q"], "scales": b["s"], "tscale": b["t"], "resid": None}
            assert_quant_equal(got, dict(ref, resid=None), 0)
