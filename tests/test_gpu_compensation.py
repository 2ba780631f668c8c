"""The compensation term alone, on the GPU, against the oracle.

The 1e-3 * Yabs bound of the GEMM parity tests is looser than one
compensated channel's contribution on these workloads, so it cannot catch a
dropped, duplicated or misplaced channel.  Here the kernel runs twice on the
same operands, once with the real residual R and once with R = 0; its main
sum is deterministic, so the difference isolates what the kernel added for
R[:, S] * B[:, S]^T (QUADS abstract: Residual Activation Compensation;
explainer section 2.2 B: the residual term added to the quantized output).
The expected term is the oracle's GEMM with every activation code zeroed
(same block scales, same R), whose main sum is then exactly 0:
t_w * sum_j R[m, j] * B[n, S_j] (t_w = 1 for MXFP4), and its Yabs is
t_w * sum_j |R[m, j] * B[n, S_j]|.

Bound, derived from the arithmetic: the BF16 x BF16 products are exact in
FP32, so the FP32 sum of the nS compensation products errs by at most
nS * 2^-24 * Yabs_c (taken as 2^-22 * nS * Yabs_c for margin), and the two
outputs differ from their exact values by the roundings where the term
meets the main sum: at most ceil(nS / 16) + 4 ulps of the larger output
(the MXFP4 256-tile kernel adds the term into the main accumulators one
16-deep MFMA step at a time).  A channel left out moves Y by about 1e-3 *
Yabs here, thousands of times this bound.
"""
import numpy as np
import pytest
import torch

import fp4_w4a4_quantized_amd as fq
from gpu_helpers import dev_quant, need_gpu, say, to_dev, to_host, workload
from workloads import dense_case

pytestmark = pytest.mark.gpu


def _check(y1, y0, yc, yca, nS):
    y1 = y1.astype(np.float64)
    y0 = y0.astype(np.float64)
    big = np.maximum(np.abs(y1), np.abs(y0)).astype(np.float32)
    ulp = np.spacing(big).astype(np.float64)
    bound = 2.0 ** -22 * nS * yca + (-(-nS // 16) + 4) * ulp
    err = np.abs((y1 - y0) - yc)
    bad = np.argwhere(~(err <= bound))
    worst = float(np.max(err / np.maximum(bound, 1e-300))) if err.size else 0.0
    assert bad.size == 0, (f"{len(bad)} compensation terms off; worst err/bound {worst:.3e}; "
                           f"first {bad[:3].tolist()}")
    # the check is not vacuous: the term is well above the bound where it is large
    assert np.max(np.abs(yc)) > 100 * np.max(bound)
    return worst


def _oracle_comp(orc, fmt, qa, qb, chan, pm=None, pn=None):
    """t_w * R B_S (and its absolute-value sum): the oracle GEMM with zero
    activation codes."""
    zq = np.zeros_like(qa["q"])
    ta = float(qa["tscale"][0]) if fmt == 0 else 1.0
    tb = float(qb["tscale"][0]) if fmt == 0 else 1.0
    if pm is None:
        return orc.gemm_full(fmt, zq, qa["scales"], ta, qb["q"], qb["scales"], tb, chan,
                             qa["resid"])
    return orc.gemm_points(fmt, zq, qa["scales"], ta, qb["q"], qb["scales"], tb, chan,
                           qa["resid"], pm, pn)


def _gpu_pair(fmt, qa, qb, chan, layout, prepared):
    a = dev_quant(qa, layout=layout, fmt=fmt)
    b = dev_quant(qb, layout=layout, fmt=fmt)
    ch = to_dev(chan)
    cw = fq.comp_weights(fmt, b, ch) if prepared else None

    def run(resid):
        a2 = dict(a, resid=resid)
        if prepared:
            return to_host(fq.gemm_prepared(fmt, a2, b, ch, cw))
        return to_host(fq.gemm(fmt, a2, b, chan_idx=ch))
    y1 = run(a["resid"])
    y0 = run(torch.zeros_like(a["resid"]))
    return y1, y0


@pytest.mark.parametrize("prepared", [False, True])
@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("name", ["tiny_nvfp4", "decode_nvfp4"])
def test_workload_term(orc, name, fmt, prepared):
    need_gpu()
    say(f"compensation term {name} fmt {fmt} prepared {prepared}")
    d = workload(name)
    chan = d["chan_idx"]
    qa = orc.quantize(fmt, d["x"], chan_idx=chan)
    qb = orc.quantize(fmt, d["wt"])
    yc, yca = _oracle_comp(orc, fmt, qa, qb, chan)
    for layout in (fq.ROWMAJOR, fq.TILED):
        y1, y0 = _gpu_pair(fmt, qa, qb, chan, layout, prepared)
        w = _check(y1, y0, yc, yca, chan.size)
        say(f"  layout {layout}: worst err/bound {w:.3e}")


@pytest.mark.parametrize("prepared", [False, True])
@pytest.mark.parametrize("name", ["prefill_nvfp4", "prefill_mxfp4"])
def test_prefill_term(orc, name, prepared):
    """Full prefill shape, tiled (the benchmark's layout), sampled outputs."""
    need_gpu()
    say(f"compensation term {name} prepared {prepared}")
    fmt = 0 if name == "prefill_nvfp4" else 1
    d = workload(name)
    chan = d["chan_idx"]
    qa = orc.quantize(fmt, d["x"], chan_idx=chan)
    qb = orc.quantize(fmt, d["wt"])
    y1, y0 = _gpu_pair(fmt, qa, qb, chan, fq.TILED, prepared)
    M, N = y1.shape
    rng = np.random.default_rng(31)
    pm = np.concatenate([rng.integers(0, M, 20000), np.full(N, M - 1)])
    pn = np.concatenate([rng.integers(0, N, 20000), np.arange(N)])
    yc, yca = _oracle_comp(orc, fmt, qa, qb, chan, pm, pn)
    w = _check(y1[pm, pn], y0[pm, pn], yc, yca, chan.size)
    say(f"  worst err/bound {w:.3e}")


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("M,N,K,nS", [(40, 100, 512, 40), (64, 300, 1024, 65),
                                      (300, 520, 512, 104), (513, 300, 768, 24),
                                      (257, 1000, 512, 96), (130, 200, 384, 37)])
def test_ragged_term(orc, fmt, M, N, K, nS):
    """Channel counts that leave a partial last compensation step, on the
    decode, large-tile (gathered per call and prepared) and general kernels."""
    need_gpu()
    say(f"compensation term fmt {fmt} M{M} N{N} K{K} nS{nS}")
    d = dense_case(M, K, N, n_out=max(1, K // 100), seed=5 * M + N + K + nS)
    chan = np.sort(np.random.default_rng(M * nS).choice(K, nS, replace=False)).astype(np.int32)
    qa = orc.quantize(fmt, d["x"], chan_idx=chan)
    qb = orc.quantize(fmt, d["wt"])
    yc, yca = _oracle_comp(orc, fmt, qa, qb, chan)
    for layout in (fq.ROWMAJOR, fq.TILED):
        for prepared in (False, True):
            y1, y0 = _gpu_pair(fmt, qa, qb, chan, layout, prepared)
            _check(y1, y0, yc, yca, nS)


@pytest.mark.parametrize("prepared", [False, True])
@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("N,nS", [(300, 40), (200, 8), (512, 32)])
def test_grouped_term(orc, fmt, N, nS, prepared):
    """Expert-grouped: empty, single-row and ragged experts; the 256-tile
    grouped kernel (N >= 256) and the general one."""
    need_gpu()
    say(f"grouped compensation term fmt {fmt} N{N} nS{nS} prepared {prepared}")
    K = 384
    off = np.array([0, 0, 1, 70, 70, 300, 333], np.int32)
    G = off.size - 1
    x = dense_case(333, K, 8, n_out=3, seed=91)["x"]
    wts = [dense_case(1, K, N, seed=100 + g)["wt"] for g in range(G)]
    rng = np.random.default_rng(N * nS)
    chan = np.sort(np.stack([rng.choice(K, nS, replace=False) for _ in range(G)]), 1).astype(np.int32)
    qa = orc.quantize(fmt, x, offsets=off, chan_idx=chan)
    qbs = [orc.quantize(fmt, w) for w in wts]
    bq = np.stack([q["q"] for q in qbs])
    bs = np.stack([q["scales"] for q in qbs])
    bts = np.array([q["tscale"][0] for q in qbs], np.float32) if fmt == 0 else None
    dbq, dbs, dch, doff = to_dev(bq), to_dev(bs), to_dev(chan), to_dev(off)
    dbts = None if fmt else to_dev(bts)
    a = {"q": to_dev(qa["q"]), "scales": to_dev(qa["scales"]),
         "tscale": None if fmt else to_dev(qa["tscale"]), "resid": to_dev(qa["resid"])}
    cw = fq.grouped_comp_weights(fmt, dbq, dbs, dch) if prepared else None

    def run(resid):
        a2 = dict(a, resid=resid)
        if prepared:
            return to_host(fq.grouped_gemm_prepared(fmt, doff, a2, dbq, dbs, dbts, dch, cw))
        return to_host(fq.grouped_gemm(fmt, doff, a2, dbq, dbs, dbts, chan_idx=dch))
    y1 = run(a["resid"])
    y0 = run(torch.zeros_like(a["resid"]))
    pm = np.repeat(np.arange(x.shape[0]), N)
    pn = np.tile(np.arange(N), x.shape[0])
    zq = np.zeros_like(qa["q"])
    yc, yca = orc.grouped_gemm_points(fmt, off, zq, qa["scales"], qa["tscale"], bq, bs, bts, chan,
                                      qa["resid"], pm, pn)
    _check(y1[pm, pn], y0[pm, pn], yc, yca, nS)
