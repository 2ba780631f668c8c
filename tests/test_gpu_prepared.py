"""GPU parity of the prepared compensation weights (fp4q_comp_weights and
fp4q_gemm_prepared, through the C ABI): the weights bit for bit against
values built from the oracle's quantization and its scalar codecs, and the
prepared GEMM against the oracle's GEMM on the decode, 256-tile and general
shapes, both formats and layouts."""
import numpy as np
import pytest
import torch

import fp4_w4a4_quantized_amd as fq
from gpu_helpers import assert_gemm_close, dev_quant, need_gpu, say, to_dev, to_host, workload
from workloads import dense_case

pytestmark = pytest.mark.gpu


def _expected_comp_weights(orc, fmt, qb, chan):
    """B[n, S_j] as BF16 bits from the oracle's codes and block scales, laid
    out as fp4q.h documents (1 KB per 16 columns and 32 channels)."""
    blk = 16 if fmt == 0 else 32
    codes = qb["q"]
    N = codes.shape[0]
    nS = chan.size
    byte = codes[:, chan >> 1].astype(np.uint32)
    code = np.where((chan & 1)[None, :] == 1, byte >> 4, byte & 15)
    sc = qb["scales"][:, chan // blk].astype(np.int64)
    e2 = np.array([orc.e2m1_value(c) for c in range(16)], np.float64)
    st = np.array([orc.e4m3_value(c) if fmt == 0 else orc.e8m0_value(c) for c in range(256)],
                  np.float64)
    v = (e2[code] * st[sc]).astype(np.float32)   # exact: at most 6 significant bits
    bits = (v.view(np.uint32) >> 16).astype(np.uint16)
    nc = (nS + 31) // 32
    ng = (N + 15) // 16
    out = np.zeros((ng, nc, 4, 16, 8), np.uint16)   # block (g, c), piece (u, r), entry e
    full = np.zeros((ng * 16, nc * 32), np.uint16)
    full[:N, :nS] = bits
    out[:] = full.reshape(ng, 16, nc, 4, 8).transpose(0, 2, 3, 1, 4)
    return out.reshape(-1)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("layout", [fq.ROWMAJOR, fq.TILED])
@pytest.mark.parametrize("N,K,nS", [(11008, 2048, 64), (37, 256, 5), (272, 384, 40),
                                    (100, 640, 129)])
def test_comp_weights_bit_exact(orc, fmt, layout, N, K, nS):
    need_gpu()
    say(f"comp weights fmt {fmt} layout {layout} N{N} K{K} nS{nS}")
    d = dense_case(4, K, N, n_out=2, seed=N + K + nS)
    chan = np.sort(np.random.default_rng(N + nS).choice(K, nS, replace=False)).astype(np.int32)
    qb = orc.quantize(fmt, d["wt"])
    b = dev_quant(qb, layout=layout, fmt=fmt)
    got = to_host(fq.comp_weights(fmt, b, to_dev(chan))).view(np.uint16)
    want = _expected_comp_weights(orc, fmt, qb, chan)
    assert got.size >= want.size
    bad = np.flatnonzero(got[:want.size] != want)
    assert bad.size == 0, f"{bad.size} mismatches, first at {bad[:4].tolist()}"


def _check_prepared(orc, fmt, layout, d, chan):
    qa = orc.quantize(fmt, d["x"], chan_idx=chan)
    qb = orc.quantize(fmt, d["wt"])
    a, b = dev_quant(qa, layout=layout, fmt=fmt), dev_quant(qb, layout=layout, fmt=fmt)
    ch = to_dev(chan)
    cw = fq.comp_weights(fmt, b, ch)
    y = to_host(fq.gemm_prepared(fmt, a, b, ch, cw))
    y_plain = to_host(fq.gemm(fmt, a, b, chan_idx=ch))
    ta = qa["tscale"][0] if fmt == 0 else 1.0
    tb = qb["tscale"][0] if fmt == 0 else 1.0
    yo, ya = orc.gemm_full(fmt, qa["q"], qa["scales"], ta, qb["q"], qb["scales"], tb, chan,
                           qa["resid"])
    r = assert_gemm_close(y, yo, ya)
    assert_gemm_close(y_plain, yo, ya)
    return r


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("layout", [fq.ROWMAJOR, fq.TILED])
def test_prepared_decode_workload(orc, fmt, layout):
    """64 x 2048 x 11008 with |S| = 64: the decode kernel staging the
    prepared weights instead of extracting them; every output."""
    need_gpu()
    say(f"prepared gemm decode fmt {fmt} layout {layout}")
    d = workload("decode_nvfp4")
    r = _check_prepared(orc, fmt, layout, d, d["chan_idx"])
    say(f"  worst |dY|/Yabs = {r:.3e}")


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("M,N,K,nS", [(1, 48, 128, 8), (37, 100, 384, 24), (64, 1000, 1024, 40),
                                      (300, 520, 512, 100), (512, 272, 384, 40),
                                      (257, 1000, 512, 96), (100, 200, 256, 12)])
def test_prepared_shapes(orc, fmt, M, N, K, nS):
    """Ragged decode shapes (columns past N, one or two channel stages), the
    large-tile kernels with the per-call gather replaced, and a
    general-kernel shape that takes the term from chan_idx."""
    need_gpu()
    say(f"prepared gemm fmt {fmt} M{M} N{N} K{K} nS{nS}")
    d = dense_case(M, K, N, n_out=max(1, K // 100), seed=3 * M + N + K + nS)
    chan = np.sort(np.random.default_rng(M + N).choice(K, nS, replace=False)).astype(np.int32)
    for layout in (fq.ROWMAJOR, fq.TILED):
        _check_prepared(orc, fmt, layout, d, chan)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("N,nS", [(512, 32), (300, 104), (200, 8)])
def test_grouped_prepared(orc, fmt, N, nS):
    """fp4q_grouped_comp_weights bit for bit per group, and
    fp4q_grouped_gemm_prepared against the oracle's grouped GEMM, with empty,
    single-row and ragged groups: the large-tile grouped kernels (the
    per-call gather replaced) and, at N < 256, the general grouped kernel
    taking the term from chan_idx."""
    need_gpu()
    say(f"grouped prepared fmt {fmt} N{N} nS{nS}")
    K = 384
    off = np.array([0, 0, 1, 70, 70, 300, 333], np.int32)
    G = off.size - 1
    x = dense_case(333, K, 8, n_out=3, seed=71)["x"]
    wts = [dense_case(1, K, N, seed=80 + g)["wt"] for g in range(G)]
    rng = np.random.default_rng(N + nS)
    chan = np.sort(np.stack([rng.choice(K, nS, replace=False) for _ in range(G)]), 1).astype(np.int32)
    qa = orc.quantize(fmt, x, offsets=off, chan_idx=chan)
    qbs = [orc.quantize(fmt, w) for w in wts]
    bq = np.stack([q["q"] for q in qbs])
    bs = np.stack([q["scales"] for q in qbs])
    bts = np.array([q["tscale"][0] for q in qbs], np.float32) if fmt == 0 else None
    cw = fq.grouped_comp_weights(fmt, to_dev(bq), to_dev(bs), to_dev(chan))
    got = to_host(cw).view(np.uint16)
    per = fq.comp_weights_bytes(fmt, fq.ROWMAJOR, N, K, nS) // 2
    for g in range(G):
        want = _expected_comp_weights(orc, fmt, qbs[g], chan[g])
        assert want.size == per
        bad = np.flatnonzero(got[g * per:(g + 1) * per] != want)
        assert bad.size == 0, f"group {g}: {bad.size} mismatches, first at {bad[:4].tolist()}"
    a = {"q": to_dev(qa["q"]), "scales": to_dev(qa["scales"]),
         "tscale": None if fmt else to_dev(qa["tscale"]), "resid": to_dev(qa["resid"])}
    y = to_host(fq.grouped_gemm_prepared(fmt, to_dev(off), a, to_dev(bq), to_dev(bs),
                                         None if fmt else to_dev(bts), to_dev(chan), cw))
    pm = np.repeat(np.arange(x.shape[0]), N)
    pn = np.tile(np.arange(N), x.shape[0])
    yo, ya = orc.grouped_gemm_points(fmt, off, qa["q"], qa["scales"], qa["tscale"], bq, bs, bts,
                                     chan, qa["resid"], pm, pn)
    assert_gemm_close(y[pm, pn], yo, ya)
