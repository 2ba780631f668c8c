"""GPU parity of quantize-before-permute (fp4q_permute_quantized, through the
C ABI) against the oracle: the expert-ordered codes, block scales, tensor
scales and per-expert residual bit for bit, both formats, with ragged row
counts, empty experts and no channels, at the MoE workload's full size, and
chained after the GPU quantizer into the grouped GEMM."""
import numpy as np
import pytest
import torch

import fp4_w4a4_quantized_amd as fq
from gpu_helpers import assert_gemm_close, need_gpu, say, to_dev, to_host
from workloads import CONFIGS, bf16_bits, moe_case

pytestmark = pytest.mark.gpu


def _dev_tok(qt):
    return {"q": to_dev(qt["q"]), "scales": to_dev(qt["scales"]),
            "tscale": None if qt["tscale"] is None else to_dev(qt["tscale"])}


def _check(orc, fmt, d, chan, gpu_quant=False):
    qt = orc.quantize(fmt, d["x_tok"])
    want = orc.permute_quantized(fmt, d["x_tok"], qt, d["token_of_row"], d["offsets"], chan)
    x = to_dev(d["x_tok"])
    a = fq.quantize(fmt, x) if gpu_quant else _dev_tok(qt)
    got = fq.permute_quantized(fmt, x, a, to_dev(d["token_of_row"].astype(np.int32)),
                               to_dev(d["offsets"]), None if chan is None else to_dev(chan))
    torch.cuda.synchronize()
    for key in ("q", "scales"):
        g = to_host(got[key])
        bad = np.argwhere(g != want[key])
        assert bad.size == 0, f"{key}: {len(bad)} mismatches, first {bad[:3].tolist()}"
    if fmt == 0:
        assert np.array_equal(to_host(got["tscale"]).view(np.uint32),
                              want["tscale"].view(np.uint32))
    if chan is None:
        assert got["resid"] is None
    else:
        g = to_host(got["resid"])
        bad = np.argwhere(g != want["resid"])
        assert bad.size == 0, f"resid: {len(bad)} mismatches, first {bad[:3].tolist()}"
    return got, want


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("tokens,hidden,experts,top_k,n_s", [(64, 256, 8, 2, 16),
                                                             (37, 512, 16, 3, 32),   # ragged rows
                                                             (64, 256, 32, 4, 16)])  # empty experts
def test_permute_matches_oracle(orc, fmt, tokens, hidden, experts, top_k, n_s):
    need_gpu()
    say(f"permute fmt {fmt} tokens {tokens} hidden {hidden} E{experts} top{top_k} nS{n_s}")
    d = moe_case(tokens=tokens, hidden=hidden, experts=experts, top_k=top_k, inter=64, n_s=n_s,
                 seed=tokens + experts + fmt, with_weights=False)
    _check(orc, fmt, d, d["chan_gate_up"])
    _check(orc, fmt, d, None)


@pytest.mark.parametrize("fmt,hidden", [(0, 48), (0, 80), (1, 96)])
def test_permute_narrow_rows(orc, fmt, hidden):
    """Rows whose code or scale bytes are not a multiple of 16 (or of 4): the
    narrower copy units."""
    need_gpu()
    say(f"permute narrow fmt {fmt} hidden {hidden}")
    d = moe_case(tokens=21, hidden=hidden, experts=4, top_k=2, inter=16, n_s=8, n_out=2,
                 h_out=1, seed=hidden + fmt, with_weights=False)
    _check(orc, fmt, d, d["chan_gate_up"])


@pytest.mark.parametrize("fmt", [0, 1])
def test_permute_full_moe_size(orc, fmt):
    """4096 tokens x 2048, 128 experts, top-8, 32 channels per expert, the
    token quantization itself on the GPU as the benchmark runs it."""
    need_gpu()
    cfg = CONFIGS["moe_nvfp4"]
    say(f"permute full size fmt {fmt}")
    d = moe_case(**{**cfg, "with_weights": False})
    _check(orc, fmt, d, d["chan_gate_up"], gpu_quant=True)


@pytest.mark.parametrize("fmt", [0, 1])
def test_permute_chained_into_grouped_gemm(orc, fmt):
    """GPU token quantize -> GPU permute -> grouped GEMM, against the oracle's
    grouped GEMM over the oracle's permuted operand (sampled outputs)."""
    need_gpu()
    say(f"permute chained fmt {fmt}")
    E, H, N, ns = 8, 512, 256, 32
    d = moe_case(tokens=96, hidden=H, experts=E, top_k=2, inter=64, n_s=ns, seed=21 + fmt,
                 with_weights=False)
    rng = np.random.default_rng(3)
    wt = [bf16_bits(rng.standard_normal((N, H)).astype(np.float32) * 0.02) for _ in range(E)]
    qw = [orc.quantize(fmt, w) for w in wt]
    bq = np.stack([q["q"] for q in qw])
    bs = np.stack([q["scales"] for q in qw])
    bts = np.array([q["tscale"][0] for q in qw], np.float32) if fmt == 0 else None
    S = d["chan_gate_up"]
    got, want = _check(orc, fmt, d, S, gpu_quant=True)
    y = fq.grouped_gemm(fmt, to_dev(d["offsets"]), got, to_dev(bq), to_dev(bs),
                        None if bts is None else to_dev(bts), chan_idx=to_dev(S))
    torch.cuda.synchronize()
    rows = d["token_of_row"].size
    pm = rng.integers(0, rows, 4000)
    pn = rng.integers(0, N, 4000)
    ats = want["tscale"] if fmt == 0 else np.ones(E, np.float32)
    yo, ya = orc.grouped_gemm_points(fmt, d["offsets"], want["q"], want["scales"], ats, bq, bs,
                                     bts if fmt == 0 else np.ones(E, np.float32), S,
                                     want["resid"], pm, pn)
    assert_gemm_close(to_host(y)[pm, pn], yo, ya)
