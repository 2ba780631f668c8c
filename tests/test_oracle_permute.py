"""Pins for the oracle's quantize-before-permute (CPU only): the token
matrix quantized once and its codes, block scales and per-expert residual
carried to the expert-ordered rows.  Checked against the already-pinned
quantizer run on the permuted BF16 rows (every token is routed, so both
see the same tensor amax), against the dense GEMM of the token matrix, and
at the edges (empty experts, no channels, bad token indices)."""
import numpy as np
import pytest

from workloads import moe_case

BLK = {0: 16, 1: 32}


def _case(seed, tokens=64, hidden=256, experts=8, top_k=2, n_s=16):
    d = moe_case(tokens=tokens, hidden=hidden, experts=experts, top_k=top_k, inter=64,
                 n_s=n_s, seed=seed, with_weights=False)
    return d


@pytest.mark.parametrize("fmt", [0, 1])
def test_codes_equal_quantizing_the_permuted_rows(orc, fmt):
    d = _case(1 + fmt)
    qt = orc.quantize(fmt, d["x_tok"])
    pq = orc.permute_quantized(fmt, d["x_tok"], qt, d["token_of_row"], d["offsets"],
                               d["chan_gate_up"])
    ref = orc.quantize(fmt, d["x_perm"])          # one group over the permuted rows
    assert np.array_equal(pq["q"], ref["q"])
    assert np.array_equal(pq["scales"], ref["scales"])
    if fmt == 0:
        assert np.all(pq["tscale"] == ref["tscale"][0])


@pytest.mark.parametrize("fmt", [0, 1])
def test_residual_is_the_quantizer_residual_of_each_expert(orc, fmt):
    d = _case(3 + fmt)
    qt = orc.quantize(fmt, d["x_tok"])
    S, off = d["chan_gate_up"], d["offsets"]
    pq = orc.permute_quantized(fmt, d["x_tok"], qt, d["token_of_row"], off, S)
    for g in range(S.shape[0]):
        ref = orc.quantize(fmt, d["x_perm"], chan_idx=S[g])["resid"]
        assert np.array_equal(pq["resid"][off[g]:off[g + 1]], ref[off[g]:off[g + 1]]), g


@pytest.mark.parametrize("fmt", [0, 1])
def test_grouped_gemm_on_permuted_rows_is_the_token_gemm(orc, fmt):
    """Expert e's rows of the grouped product over the permuted operand equal
    the dense product of the token matrix with expert e's weights, at the
    tokens routed to e, bit for bit (same terms, same order)."""
    d = _case(5 + fmt)
    rng = np.random.default_rng(9)
    E, H, N = 8, 256, 48
    from workloads import bf16_bits
    w = [bf16_bits(rng.standard_normal((N, H)).astype(np.float32) * 0.02) for _ in range(E)]
    qw = [orc.quantize(fmt, wi) for wi in w]
    qt = orc.quantize(fmt, d["x_tok"])
    S, off, src = d["chan_gate_up"], d["offsets"], d["token_of_row"]
    pq = orc.permute_quantized(fmt, d["x_tok"], qt, src, off, S)
    ta = float(qt["tscale"][0]) if fmt == 0 else 1.0
    rows = src.size
    pm = np.arange(rows)
    pn = rng.integers(0, N, rows)
    bq = np.stack([q["q"] for q in qw])
    bs = np.stack([q["scales"] for q in qw])
    bts = np.array([q["tscale"][0] if fmt == 0 else 1.0 for q in qw], np.float32)
    ats = pq["tscale"] if fmt == 0 else np.ones(E, np.float32)
    yg = orc.grouped_gemm_points(fmt, off, pq["q"], pq["scales"], ats, bq, bs, bts, S,
                                 pq["resid"], pm, pn)[0]
    for e in range(E):
        Rt = orc.quantize(fmt, d["x_tok"], chan_idx=S[e])["resid"]
        tb = float(bts[e])
        for m in range(off[e], off[e + 1]):
            y, _ = orc.gemm_points(fmt, qt["q"], qt["scales"], ta, qw[e]["q"], qw[e]["scales"],
                                   tb, S[e], Rt, np.array([src[m]]), np.array([pn[m]]))
            assert yg[m] == y[0], (e, m)


def test_token_copies_share_codes_and_empty_experts(orc):
    """A token routed to several experts has the same code row in each copy;
    experts with no rows contribute nothing; no channels gives no residual."""
    x = _case(7, experts=32, top_k=4)   # 64 tokens over 32 experts: some get none
    qt = orc.quantize(0, x["x_tok"])
    off = x["offsets"]
    assert np.any(np.diff(off) == 0)
    pq = orc.permute_quantized(0, x["x_tok"], qt, x["token_of_row"], off, x["chan_gate_up"])
    src = x["token_of_row"]
    for tok in np.unique(src)[:10]:
        rows = np.nonzero(src == tok)[0]
        assert rows.size == 4
        for r in rows[1:]:
            assert np.array_equal(pq["q"][r], pq["q"][rows[0]])
            assert np.array_equal(pq["scales"][r], pq["scales"][rows[0]])
    p0 = orc.permute_quantized(0, x["x_tok"], qt, src, off, None)
    assert p0["resid"] is None and np.array_equal(p0["q"], pq["q"])


def test_rejects_bad_tokens_and_offsets(orc):
    d = _case(11)
    qt = orc.quantize(1, d["x_tok"])
    src = d["token_of_row"].copy()
    src[3] = d["x_tok"].shape[0]
    with pytest.raises(ValueError):
        orc.permute_quantized(1, d["x_tok"], qt, src, d["offsets"])
    off = d["offsets"].copy()
    off[-1] -= 1
    with pytest.raises(ValueError):
        orc.permute_quantized(1, d["x_tok"], qt, d["token_of_row"], off)
