"""Seeded synthetic workloads.

The pages report that FP4 activation error concentrates in a few high-variance
activation channels (FourSight abstract) and that activations are recomputed
online (QUADS abstract).  The inputs below stand in for real rollout
activations and weights with that structure: heavy-tailed activations
(Student-t, 4 degrees of freedom) with a seeded 1% of channels scaled up as
outlier channels, Gaussian weights, and, for the MoE layer, Zipf-skewed expert
loads from top-8 routing.  Nothing here comes from a dataset or a trained
model.

Recipe (all draws from numpy's PCG64 generator seeded per workload):
  * N(0, s): standard normal times s (s is the standard deviation).
  * t(4): numpy's standard_t with 4 degrees of freedom.
  * outlier channels: the first n_out entries of a seeded permutation of the
    columns, multiplied by the outlier factor before rounding.
  * every tensor is drawn in float32 and rounded to BF16 (nearest, ties to
    even) by torch's float32 -> bfloat16 conversion.
  * the compensated channel set S is the n_s columns with the largest
    population variance (FP64) over the rows, ties to the lower index,
    returned in ascending order.
  * weights are drawn as W [K, N] and returned transposed, W^T [N, K], the
    layout the GEMM takes.
"""
from __future__ import annotations

import numpy as np
import torch

# name -> parameters of the five workloads
CONFIGS = {
    "tiny_nvfp4": dict(fmt="nvfp4", M=16, K=256, N=256, x_dist="normal", n_out=4, out_mult=50.0,
                       w_std=0.02, n_s=8, seed=1),
    "decode_nvfp4": dict(fmt="nvfp4", M=64, K=2048, N=11008, x_dist="t4", n_out=20,
                         out_mult=30.0, w_std=0.02, n_s=64, seed=2),
    "prefill_nvfp4": dict(fmt="nvfp4", M=8192, K=4096, N=14336, x_dist="t4", n_out=41,
                          out_mult=30.0, w_std=0.015, n_s=128, seed=3),
    "moe_nvfp4": dict(fmt="nvfp4", tokens=4096, hidden=2048, experts=128, top_k=8,
                      inter=768, zipf=1.1, n_out=20, out_mult=30.0, h_out=8, w_std=0.02,
                      n_s=32, seed=4),
    "prefill_mxfp4": dict(fmt="mxfp4", M=8192, K=4096, N=14336, x_dist="t4", n_out=41,
                          out_mult=30.0, w_std=0.015, n_s=128, seed=3),
}


def bf16_bits(a) -> np.ndarray:
    """float array -> uint16 BF16 bit patterns (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _activations(rng, rows, cols, dist, n_out, mult):
    if dist == "normal":
        x = rng.standard_normal((rows, cols), dtype=np.float32)
    elif dist == "t4":
        x = rng.standard_t(4.0, size=(rows, cols)).astype(np.float32)
    else:
        raise ValueError(dist)
    if n_out:
        out_cols = rng.permutation(cols)[:n_out]
        x[:, out_cols] *= np.float32(mult)
    return x


def top_variance_channels(x_bits: np.ndarray, n_s: int) -> np.ndarray:
    """Indices of the n_s highest-variance columns (FP64 population variance
    over rows; ties to the lower index), ascending, int32."""
    if n_s == 0:
        return np.zeros(0, np.int32)
    x = bf16_to_f32(x_bits).astype(np.float64)
    if x.shape[0] == 0:
        var = np.zeros(x.shape[1])
    else:
        var = x.var(axis=0)
    order = np.lexsort((np.arange(var.size), -var))  # by -var, then index
    return np.sort(order[:n_s]).astype(np.int32)


def dense_case(M, K, N, x_dist="t4", n_out=0, out_mult=30.0, w_std=0.02, n_s=0, seed=0,
               **_):
    """Returns dict(x [M,K] u16, wt [N,K] u16, chan_idx [n_s] i32)."""
    rng = np.random.default_rng(seed)
    x = bf16_bits(_activations(rng, M, K, x_dist, n_out, out_mult))
    w = rng.standard_normal((K, N), dtype=np.float32) * np.float32(w_std)
    wt = bf16_bits(np.ascontiguousarray(w.T))
    return {"x": x, "wt": wt, "chan_idx": top_variance_channels(x, n_s)}


def moe_routing(rng, tokens, experts, top_k, zipf):
    """Top-k expert choice per token from logits log(p_e) + Gumbel noise, with
    a Zipf prior p_e ~ rank_e^-zipf over a seeded ranking of the experts
    (Gumbel-top-k: sampling without replacement proportional to p).
    Returns (expert ids [tokens, top_k], per-expert loads [experts])."""
    ranks = rng.permutation(experts) + 1
    p = ranks.astype(np.float64) ** (-zipf)
    p /= p.sum()
    logits = np.log(p)[None, :] + rng.gumbel(size=(tokens, experts))
    choice = np.argsort(-logits, axis=1, kind="stable")[:, :top_k]
    loads = np.bincount(choice.ravel(), minlength=experts)
    return choice, loads


def moe_case(tokens=4096, hidden=2048, experts=128, top_k=8, inter=768, zipf=1.1, n_out=20,
             out_mult=30.0, h_out=8, w_std=0.02, n_s=32, seed=4, with_weights=True, **_):
    """Expert-grouped workload: gate_up (hidden -> 2*inter) and down
    (inter -> hidden) layers, inputs permuted into expert order.

    Returns dict with
      offsets [E+1] i32, loads [E],
      token_of_row [rows] (the token of each expert-ordered row),
      x_tok [tokens, hidden] u16 (the token activations),
      x_perm [rows, hidden] u16 (routed token copies in expert order),
      h_perm [rows, inter] u16 (independent down-projection input),
      wt_gate_up [E, 2*inter, hidden] u16, wt_down [E, hidden, inter] u16,
      chan_gate_up [E, n_s] i32, chan_down [E, n_s] i32.
    """
    rng = np.random.default_rng(seed)
    x_tok = _activations(rng, tokens, hidden, "t4", n_out, out_mult)
    choice, loads = moe_routing(rng, tokens, experts, top_k, zipf)
    loads = np.minimum(loads, tokens)
    offsets = np.zeros(experts + 1, np.int64)
    offsets[1:] = np.cumsum(loads)
    rows = int(offsets[-1])
    # token ids routed to each expert, ascending
    tok_of = [np.nonzero((choice == e).any(axis=1))[0][:tokens] for e in range(experts)]
    perm = np.concatenate(tok_of) if rows else np.zeros(0, np.int64)
    x_perm = bf16_bits(x_tok[perm])
    h_perm = bf16_bits(_activations(rng, rows, inter, "t4", h_out, out_mult))
    out = {"offsets": offsets.astype(np.int32), "loads": loads, "token_of_row": perm,
           "x_tok": bf16_bits(x_tok), "x_perm": x_perm, "h_perm": h_perm}
    chan_gu = np.zeros((experts, n_s), np.int32)
    chan_dn = np.zeros((experts, n_s), np.int32)
    for e in range(experts):
        a, b = offsets[e], offsets[e + 1]
        chan_gu[e] = top_variance_channels(x_perm[a:b], n_s)
        chan_dn[e] = top_variance_channels(h_perm[a:b], n_s)
    out["chan_gate_up"], out["chan_down"] = chan_gu, chan_dn
    if with_weights:
        gu = np.empty((experts, 2 * inter, hidden), np.uint16)
        dn = np.empty((experts, hidden, inter), np.uint16)
        for e in range(experts):
            w = rng.standard_normal((hidden, 2 * inter), dtype=np.float32) * np.float32(w_std)
            gu[e] = bf16_bits(np.ascontiguousarray(w.T))
            w = rng.standard_normal((inter, hidden), dtype=np.float32) * np.float32(w_std)
            dn[e] = bf16_bits(np.ascontiguousarray(w.T))
        out["wt_gate_up"], out["wt_down"] = gu, dn
    return out
