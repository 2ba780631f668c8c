"""GPU parity of fp4q_grouped_gemm (MoE expert layer) against the oracle:
small cases with empty, single-row and ragged experts, and the full MoE
workload (128 experts, Zipf-skewed loads) on sampled outputs."""
import numpy as np
import pytest
import torch

import fp4_w4a4_quantized_amd as fq
from gpu_helpers import workload, assert_gemm_close, need_gpu, say, to_dev, to_host
from workloads import CONFIGS, dense_case, moe_case

pytestmark = pytest.mark.gpu


def _quant_experts(orc, fmt, wts):
    qs = [orc.quantize(fmt, w) for w in wts]
    bq = np.stack([q["q"] for q in qs])
    bs = np.stack([q["scales"] for q in qs])
    bts = np.array([q["tscale"][0] for q in qs], np.float32) if fmt == 0 else None
    return bq, bs, bts


def _run(orc, fmt, x, off, chan, wts, pm=None, pn=None):
    qa = orc.quantize(fmt, x, offsets=off, chan_idx=chan)
    bq, bs, bts = _quant_experts(orc, fmt, wts)
    G = off.size - 1
    a = {"q": to_dev(qa["q"]), "scales": to_dev(qa["scales"]),
         "tscale": None if fmt else to_dev(qa["tscale"]),
         "resid": None if chan is None else to_dev(qa["resid"])}
    y = fq.grouped_gemm(fmt, to_dev(off), a, to_dev(bq), to_dev(bs),
                        None if fmt else to_dev(bts),
                        chan_idx=None if chan is None else to_dev(chan))
    y = to_host(y)
    if pm is None:
        pm = np.repeat(np.arange(x.shape[0]), y.shape[1])
        pn = np.tile(np.arange(y.shape[1]), x.shape[0])
    yo, ya = orc.grouped_gemm_points(fmt, off, qa["q"], qa["scales"], qa["tscale"], bq, bs, bts,
                                     chan, qa["resid"], pm, pn)
    return assert_gemm_close(y[pm, pn], yo, ya)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("nS", [0, 7, 32])
def test_small_groups(orc, fmt, nS):
    need_gpu()
    say(f"grouped small fmt {fmt} nS {nS}")
    K, N = 256, 200
    off = np.array([0, 0, 1, 70, 70, 200, 333], np.int32)
    G = off.size - 1
    x = dense_case(333, K, 8, n_out=3, seed=51)["x"]
    wts = [dense_case(1, K, N, seed=60 + g)["wt"] for g in range(G)]
    rng = np.random.default_rng(3)
    chan = (np.sort(np.stack([rng.choice(K, nS, replace=False) for _ in range(G)]), 1)
            .astype(np.int32) if nS else None)
    _run(orc, fmt, x, off, chan, wts)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("nS", [0, 8, 40, 104])
def test_groups_large_tiles(orc, fmt, nS):
    """The staged 256x256-tile grouped path (N >= 256): empty, single-row,
    sub-tile and multi-tile experts, tiles ending mid-group and a partial
    last column tile; |S| off the 32-channel stage size."""
    need_gpu()
    say(f"grouped large-tile fmt {fmt} nS {nS}")
    K, N = 384, 300
    off = np.array([0, 0, 1, 257, 257, 300, 900, 1000], np.int32)
    G = off.size - 1
    x = dense_case(int(off[-1]), K, 8, n_out=3, seed=53)["x"]
    wts = [dense_case(1, K, N, seed=80 + g)["wt"] for g in range(G)]
    rng = np.random.default_rng(4)
    chan = (np.sort(np.stack([rng.choice(K, nS, replace=False) for _ in range(G)]), 1)
            .astype(np.int32) if nS else None)
    _run(orc, fmt, x, off, chan, wts)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("nS", [0, 104])
def test_groups_wide_tiles(orc, fmt, nS):
    """Groups of 127, 128, 129, 300 and 513 rows and N = 1088 (two full
    512-column tiles and a partial one): interior tiles of the 128 x 512
    NVFP4 grouped kernel (vector stores) beside edge tiles, with and without
    the compensation term (104 channels: weights gathered per call)."""
    need_gpu()
    say(f"grouped wide-tile fmt {fmt} nS {nS}")
    K, N = 256, 1088
    off = np.cumsum([0, 127, 0, 128, 129, 1, 300, 513]).astype(np.int32)
    G = off.size - 1
    x = dense_case(int(off[-1]), K, 8, n_out=3, seed=57)["x"]
    wts = [dense_case(1, K, N, seed=90 + g)["wt"] for g in range(G)]
    rng = np.random.default_rng(6)
    chan = (np.sort(np.stack([rng.choice(K, nS, replace=False) for _ in range(G)]), 1)
            .astype(np.int32) if nS else None)
    _run(orc, fmt, x, off, chan, wts)


def test_all_rows_in_one_group(orc):
    need_gpu()
    off = np.array([0, 0, 0, 150, 150], np.int32)
    x = dense_case(150, 384, 8, seed=52)["x"]
    wts = [dense_case(1, 384, 64, seed=70 + g)["wt"] for g in range(4)]
    _run(orc, 0, x, off, None, wts)


@pytest.mark.parametrize("layer", ["gate_up", "down"])
def test_moe_workload(orc, layer):
    """The MoE workload at full size: 32768 routed rows, 128 experts; 30000
    sampled outputs plus the first and last row of every non-empty expert."""
    need_gpu()
    say(f"grouped MoE workload {layer}")
    m = workload("moe_nvfp4")
    off = m["offsets"]
    if layer == "gate_up":
        x, chan, wts = m["x_perm"], m["chan_gate_up"], m["wt_gate_up"]
    else:
        x, chan, wts = m["h_perm"], m["chan_down"], m["wt_down"]
    N = wts.shape[1]
    rng = np.random.default_rng(9)
    edge = np.concatenate([[off[g], off[g + 1] - 1] for g in range(off.size - 1)
                           if off[g + 1] > off[g]])
    pm = np.concatenate([rng.integers(0, x.shape[0], 30000), np.repeat(edge, 4)])
    pn = np.concatenate([rng.integers(0, N, 30000), rng.integers(0, N, edge.size * 4)])
    r = _run(orc, 0, x, off, chan, wts, pm, pn)
    say(f"  loads max {m['loads'].max()} min {m['loads'].min()}; worst |dY|/Yabs = {r:.3e}")
