"""Python face of the CPU oracle (``fp4q_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU
baseline leg of the benchmark import this module; the product library never
does.  It marshals numpy arrays into the plain C oracle and shares no code
with the HIP path.

Formats (readings of the pages, stated in ``fp4q_oracle.c``):
  * NVFP4: 16-element blocks, E4M3 block scale, FP32 tensor scale.
  * MXFP4: 32-element blocks, E8M0 power-of-two block scale.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

NVFP4 = 0
MXFP4 = 1
BLOCK = {NVFP4: 16, MXFP4: 32}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp4q_oracle.c")
_LIB = os.path.join(_HERE, "liborc_fp4q.so")
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
          "-std=gnu11", "-Wall"]

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/liborc_fp4q.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


class ErrStats(ctypes.Structure):
    _fields_ = [
        ("exact", (ctypes.c_int64 * 5) * 4),
        ("sum", ctypes.c_double * 4),
        ("sumsq", ctypes.c_double * 4),
        ("cross_sb_gn", ctypes.c_double),
        ("n_elems", ctypes.c_int64),
        ("n_deadzone", ctypes.c_int64),
        ("n_clipped", ctypes.c_int64),
    ]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32, f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        L.orc_set_num_threads.restype = None
        L.orc_set_num_threads.argtypes = [ctypes.c_int]
        L.orc_max_threads.restype = ctypes.c_int
        L.orc_max_threads.argtypes = []
        L.orc_e2m1_value.restype = ctypes.c_double
        L.orc_e2m1_value.argtypes = [ctypes.c_uint8]
        L.orc_e2m1_encode_mag.restype = ctypes.c_uint8
        L.orc_e2m1_encode_mag.argtypes = [f32]
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_e4m3_encode.argtypes = [f32]
        L.orc_e8m0_value.restype = ctypes.c_double
        L.orc_e8m0_value.argtypes = [ctypes.c_uint8]
        L.orc_bf16_value.restype = f32
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]
        L.orc_bf16_from_f32.restype = ctypes.c_uint16
        L.orc_bf16_from_f32.argtypes = [f32]
        L.orc_mx_exponent.restype = ctypes.c_int
        L.orc_mx_exponent.argtypes = [f32]
        L.orc_nv_tensor_scale.restype = f32
        L.orc_nv_tensor_scale.argtypes = [f32]
        L.orc_quantize.restype = ctypes.c_int
        L.orc_quantize.argtypes = [ctypes.c_int, P, i64, i64, i64, P, i32, P, i32, P, P, P, P]
        L.orc_gemm_points.restype = ctypes.c_int
        L.orc_gemm_points.argtypes = [ctypes.c_int, i64, i64, i64, P, P, f32, P, P, f32, P, i32,
                                      P, P, P, i64, P, P]
        L.orc_gemm_full.restype = ctypes.c_int
        L.orc_gemm_full.argtypes = [ctypes.c_int, i64, i64, i64, P, P, f32, P, P, f32, P, i32,
                                    P, P, P]
        L.orc_select_channels.restype = ctypes.c_int
        L.orc_select_channels.argtypes = [ctypes.c_int, P, i64, i64, i64, P, P, f32, i32, P, P]
        L.orc_permute_quantized.argtypes = [ctypes.c_int, P, i64, i64, i64, P, P, f32, P, i64, P,
                                            i32, P, i32, P, P, P]
        L.orc_gemm_points_r4.restype = ctypes.c_int
        L.orc_gemm_points_r4.argtypes = [ctypes.c_int, i64, i64, i64, P, P, f32, P, P, f32, P, i32,
                                         P, P, f32, P, P, i64, P, P]
        L.orc_gemm_full_r4.restype = ctypes.c_int
        L.orc_gemm_full_r4.argtypes = [ctypes.c_int, i64, i64, i64, P, P, f32, P, P, f32, P, i32,
                                       P, P, f32, P, P]
        L.orc_grouped_gemm_points.restype = ctypes.c_int
        L.orc_grouped_gemm_points.argtypes = [ctypes.c_int, i64, i64, i64, P, i32, P, P, P, P, P,
                                              P, P, i32, P, P, P, i64, P, P]
        L.orc_error_components.restype = ctypes.c_int
        L.orc_error_components.argtypes = [P, i64, i64, i64, P]
        L.orc_error_decompose.restype = ctypes.c_int
        L.orc_error_decompose.argtypes = [P, i64, i64, i64, ctypes.POINTER(ErrStats)]
        L.orc_error_components_nv.restype = ctypes.c_int
        L.orc_error_components_nv.argtypes = [P, i64, i64, i64, P]
        L.orc_qdq_fallback.restype = ctypes.c_int
        L.orc_qdq_fallback.argtypes = [ctypes.c_int, P, i64, i64, i64, P,
                                       ctypes.POINTER(ctypes.c_int64)]
        L.orc_error_decompose_nv.restype = ctypes.c_int
        L.orc_error_decompose_nv.argtypes = [P, i64, i64, i64, ctypes.POINTER(ErrStats)]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


# ---- threads (timing only: no result depends on the count) ----------------

def set_num_threads(n: int) -> None:
    lib().orc_set_num_threads(int(n))


def max_threads() -> int:
    return int(lib().orc_max_threads())


# ---- scalar codecs (exposed for the pins) --------------------------------

def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(code)


def e2m1_encode_mag(q: float) -> int:
    return lib().orc_e2m1_encode_mag(q)


def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(code)


def e4m3_encode(v: float) -> int:
    return lib().orc_e4m3_encode(v)


def e8m0_value(code: int) -> float:
    return lib().orc_e8m0_value(code)


def bf16_value(h: int) -> float:
    return lib().orc_bf16_value(h)


def bf16_from_f32(f: float) -> int:
    return lib().orc_bf16_from_f32(f)


def mx_exponent(amax: float) -> int:
    return lib().orc_mx_exponent(amax)


def nv_tensor_scale(amax: float) -> float:
    return lib().orc_nv_tensor_scale(amax)


# ---- quantizer -----------------------------------------------------------

def quantize(fmt: int, x: np.ndarray, offsets=None, chan_idx=None):
    """x: uint16 bf16 bit patterns [rows, cols].  offsets: int32 [G+1] or None.
    chan_idx: int32 [G, nS] (or [nS] for one group) or None.
    Returns dict(q [rows, cols/2] u8, scales [rows, cols/blk] u8,
    tscale [G] f32 (NVFP4) or None, resid [rows, nS] u16 or None)."""
    x = _c(x, np.uint16)
    rows, cols = x.shape
    blk = BLOCK[fmt]
    G = 1 if offsets is None else len(offsets) - 1
    off = _c(offsets, np.int32)
    if chan_idx is not None:
        ci = _c(chan_idx, np.int32).reshape(G, -1)
        nS = ci.shape[1]
    else:
        ci, nS = None, 0
    q = np.zeros((rows, cols // 2), np.uint8)
    sc = np.zeros((rows, cols // blk), np.uint8)
    ts = np.zeros(G, np.float32) if fmt == NVFP4 else None
    R = np.zeros((rows, nS), np.uint16) if nS else None
    rc = lib().orc_quantize(fmt, _p(x), rows, cols, cols, _p(off), G, _p(ci), nS, _p(q), _p(sc),
                            _p(ts), _p(R))
    if rc != 0:
        raise ValueError(f"oracle quantize rejected the shape (rc={rc})")
    return {"q": q, "scales": sc, "tscale": ts, "resid": R}


# ---- GEMM ----------------------------------------------------------------

def gemm_points(fmt, aq, as_, ats, bq, bs, bts, chan_idx, resid, pm, pn):
    """Y and Yabs at points (pm[i], pn[i]); A = [M, K/2] codes, B = W^T codes."""
    aq, as_, bq, bs = (_c(a, np.uint8) for a in (aq, as_, bq, bs))
    M, K2 = aq.shape
    N = bq.shape[0]
    ci = _c(chan_idx, np.int32)
    nS = 0 if ci is None else ci.size
    R = _c(resid, np.uint16)
    pm, pn = _c(pm, np.int64), _c(pn, np.int64)
    y = np.zeros(pm.size, np.float64)
    ya = np.zeros(pm.size, np.float64)
    lib().orc_gemm_points(fmt, M, N, 2 * K2, _p(aq), _p(as_), float(ats), _p(bq), _p(bs),
                          float(bts), _p(ci), nS, _p(R), _p(pm), _p(pn), pm.size, _p(y), _p(ya))
    return y, ya


def gemm_full(fmt, aq, as_, ats, bq, bs, bts, chan_idx, resid):
    aq, as_, bq, bs = (_c(a, np.uint8) for a in (aq, as_, bq, bs))
    M, K2 = aq.shape
    N = bq.shape[0]
    ci = _c(chan_idx, np.int32)
    nS = 0 if ci is None else ci.size
    R = _c(resid, np.uint16)
    y = np.zeros((M, N), np.float64)
    ya = np.zeros((M, N), np.float64)
    lib().orc_gemm_full(fmt, M, N, 2 * K2, _p(aq), _p(as_), float(ats), _p(bq), _p(bs),
                        float(bts), _p(ci), nS, _p(R), _p(y), _p(ya))
    return y, ya


def select_channels(fmt: int, x: np.ndarray, qx: dict, k: int):
    """The k channels of largest residual magnitude (max over rows of the BF16
    residual) of x given its quantize() result qx (one group); ties to the
    lower index.  Returns (chan int32 [k] ascending, resid uint16 [rows, k])."""
    x = _c(x, np.uint16)
    rows, cols = x.shape
    t = float(qx["tscale"][0]) if fmt == NVFP4 else 1.0
    chan = np.zeros(k, np.int32)
    R = np.zeros((rows, k), np.uint16)
    rc = lib().orc_select_channels(fmt, _p(x), rows, cols, cols, _p(_c(qx["q"], np.uint8)),
                                   _p(_c(qx["scales"], np.uint8)), t, k, _p(chan), _p(R))
    if rc != 0:
        raise ValueError("oracle select_channels: k must lie in [0, cols]")
    return chan, R


def select_channels_grouped(fmt: int, x: np.ndarray, qx: dict, offsets, k: int):
    """The MoE form of select_channels (QUADS abstract: MoE rollout;
    explainer section 2.2 B): each group g (rows offsets[g] .. offsets[g+1])
    chooses its k channels from its own rows with its own tensor scale, by
    the single-group definition.  qx = quantize(fmt, x, offsets).  Returns
    (chan int32 [G, k], resid uint16 [rows, k])."""
    x = _c(x, np.uint16)
    off = np.asarray(offsets, np.int64)
    G = off.size - 1
    rows = x.shape[0]
    chan = np.zeros((G, k), np.int32)
    R = np.zeros((rows, k), np.uint16)
    for g in range(G):
        r0, r1 = int(off[g]), int(off[g + 1])
        sub = {"q": qx["q"][r0:r1], "scales": qx["scales"][r0:r1],
               "tscale": None if fmt == MXFP4 else qx["tscale"][g:g + 1]}
        chan[g], R[r0:r1] = select_channels(fmt, x[r0:r1], sub, k)
    return chan, R


def permute_quantized(fmt: int, x_tok: np.ndarray, qx: dict, row_src, offsets, chan_idx=None):
    """Quantize-before-permute: qx = quantize(fmt, x_tok) (one group).  Row m
    of the expert-ordered result is token row_src[m]; group g holds rows
    offsets[g] .. offsets[g+1]-1 and has channels chan_idx[g] ([G, nS]).
    Returns dict(q, scales, tscale [G] (all the token tensor scale; NVFP4),
    resid [rows, nS] or None)."""
    x_tok = _c(x_tok, np.uint16)
    tokens, cols = x_tok.shape
    blk = 16 if fmt == NVFP4 else 32
    src = _c(row_src, np.int32)
    off = _c(offsets, np.int32)
    G = off.size - 1
    rows = src.size
    ci = None if chan_idx is None else _c(np.asarray(chan_idx).reshape(G, -1), np.int32)
    nS = 0 if ci is None else ci.shape[1]
    q = np.zeros((rows, cols // 2), np.uint8)
    sc = np.zeros((rows, cols // blk), np.uint8)
    R = np.zeros((rows, nS), np.uint16) if nS else None
    t = float(qx["tscale"][0]) if fmt == NVFP4 else 1.0
    rc = lib().orc_permute_quantized(fmt, _p(x_tok), tokens, cols, cols,
                                     _p(_c(qx["q"], np.uint8)), _p(_c(qx["scales"], np.uint8)),
                                     t, _p(src), rows, _p(off), G, _p(ci), nS, _p(q), _p(sc),
                                     _p(R))
    if rc != 0:
        raise ValueError("oracle permute_quantized: token index or offsets out of range")
    ts = np.full(G, qx["tscale"][0], np.float32) if fmt == NVFP4 else None
    return {"q": q, "scales": sc, "tscale": ts, "resid": R}


def quantize_residual(fmt: int, resid: np.ndarray):
    """Second pass: the BF16 residual R [M, nS] quantized by the same rule as
    an M x nS tensor (blocks along the selected-channel index; NVFP4 with
    its own tensor scale).  Returns the quantize() dict of R."""
    return quantize(fmt, resid)


def gemm_points_r4(fmt, aq, as_, ats, bq, bs, bts, chan_idx, rq, rs, rts, pm, pn):
    """gemm_points with the compensation term deq(Q(R)) B_S^T: rq [M, nS/2],
    rs [M, nS/blk], rts the residual's tensor scale (NVFP4)."""
    aq, as_, bq, bs = (_c(a, np.uint8) for a in (aq, as_, bq, bs))
    M, K2 = aq.shape
    N = bq.shape[0]
    ci = _c(chan_idx, np.int32)
    nS = 0 if ci is None else ci.size
    rq, rs = _c(rq, np.uint8), _c(rs, np.uint8)
    pm, pn = _c(pm, np.int64), _c(pn, np.int64)
    y = np.zeros(pm.size, np.float64)
    ya = np.zeros(pm.size, np.float64)
    rc = lib().orc_gemm_points_r4(fmt, M, N, 2 * K2, _p(aq), _p(as_), float(ats), _p(bq), _p(bs),
                                  float(bts), _p(ci), nS, _p(rq), _p(rs), float(rts), _p(pm),
                                  _p(pn), pm.size, _p(y), _p(ya))
    if rc != 0:
        raise ValueError("oracle: |S| must be a multiple of the block size")
    return y, ya


def gemm_full_r4(fmt, aq, as_, ats, bq, bs, bts, chan_idx, rq, rs, rts):
    aq, as_, bq, bs = (_c(a, np.uint8) for a in (aq, as_, bq, bs))
    M, K2 = aq.shape
    N = bq.shape[0]
    ci = _c(chan_idx, np.int32)
    nS = 0 if ci is None else ci.size
    rq, rs = _c(rq, np.uint8), _c(rs, np.uint8)
    y = np.zeros((M, N), np.float64)
    ya = np.zeros((M, N), np.float64)
    rc = lib().orc_gemm_full_r4(fmt, M, N, 2 * K2, _p(aq), _p(as_), float(ats), _p(bq), _p(bs),
                                float(bts), _p(ci), nS, _p(rq), _p(rs), float(rts), _p(y), _p(ya))
    if rc != 0:
        raise ValueError("oracle: |S| must be a multiple of the block size")
    return y, ya


def grouped_gemm_points_r4(fmt, offsets, aq, as_, ats, bq, bs, bts, chan_idx, rq, rs, rts, pm,
                           pn):
    """Grouped form of gemm_points_r4 (QUADS abstract: MoE rollout; explainer
    section 2.2 B): each expert g's rows offsets[g] .. offsets[g+1] are the
    dense second-pass-residual GEMM with its own weights bq[g], bs[g], tensor
    scales ats[g], bts[g], channel list chan_idx[g] and residual tensor scale
    rts[g]; rq, rs [rows, ...] are indexed by global row.  Points pm, pn."""
    off = np.asarray(offsets, np.int64)
    G = off.size - 1
    ci = None if chan_idx is None else np.asarray(chan_idx, np.int32).reshape(G, -1)
    pm, pn = np.asarray(pm, np.int64), np.asarray(pn, np.int64)
    y = np.zeros(pm.size, np.float64)
    ya = np.zeros(pm.size, np.float64)
    grp = np.searchsorted(off, pm, side="right") - 1
    for g in range(G):
        sel = np.nonzero(grp == g)[0]
        if sel.size == 0:
            continue
        r0, r1 = int(off[g]), int(off[g + 1])
        yg, yag = gemm_points_r4(fmt, aq[r0:r1], as_[r0:r1],
                                 1.0 if ats is None else float(ats[g]), bq[g], bs[g],
                                 1.0 if bts is None else float(bts[g]),
                                 None if ci is None else ci[g], rq[r0:r1], rs[r0:r1],
                                 1.0 if rts is None else float(rts[g]), pm[sel] - r0, pn[sel])
        y[sel], ya[sel] = yg, yag
    return y, ya


def grouped_gemm_points(fmt, offsets, aq, as_, ats, bq, bs, bts, chan_idx, resid, pm, pn):
    """Grouped GEMM at points; bq [G, N, K/2], bs [G, N, K/blk], ats/bts [G],
    chan_idx [G, nS], resid [rows, nS] indexed by global row."""
    aq, as_, bq, bs = (_c(a, np.uint8) for a in (aq, as_, bq, bs))
    off = _c(offsets, np.int32)
    G = off.size - 1
    rows, K2 = aq.shape
    N = bq.shape[1]
    ats = _c(ats if ats is not None else np.ones(G), np.float32)
    bts = _c(bts if bts is not None else np.ones(G), np.float32)
    ci = _c(chan_idx, np.int32)
    nS = 0 if ci is None else ci.reshape(G, -1).shape[1]
    R = _c(resid, np.uint16)
    pm, pn = _c(pm, np.int64), _c(pn, np.int64)
    y = np.zeros(pm.size, np.float64)
    ya = np.zeros(pm.size, np.float64)
    lib().orc_grouped_gemm_points(fmt, rows, N, 2 * K2, _p(off), G, _p(aq), _p(as_), _p(ats),
                                  _p(bq), _p(bs), _p(bts), _p(ci), nS, _p(R), _p(pm), _p(pn),
                                  pm.size, _p(y), _p(ya))
    return y, ya


# ---- error decomposition -------------------------------------------------

COMPONENTS = ("total", "scale_bias", "deadzone", "grid_noise")


def error_components6(x: np.ndarray, fmt: int = MXFP4) -> np.ndarray:
    """Per-element components times 6: float64 [4, rows, cols] (total,
    scale_bias, deadzone, grid_noise) under the MXFP4 or NVFP4 quantizer."""
    x = _c(x, np.uint16)
    rows, cols = x.shape
    out = np.zeros((4, rows, cols), np.float64)
    f = lib().orc_error_components if fmt == MXFP4 else lib().orc_error_components_nv
    rc = f(_p(x), rows, cols, cols, _p(out))
    if rc != 0:
        raise ValueError("cols must be a multiple of the block size")
    return out


def fixed_to_int(limbs) -> int:
    """320-bit two's complement (5 little-endian int64 limbs) -> Python int."""
    v = 0
    for i, l in enumerate(limbs):
        v |= (int(l) & 0xFFFFFFFFFFFFFFFF) << (64 * i)
    if v >> 319:
        v -= 1 << 320
    return v


def error_decompose(x: np.ndarray, fmt: int = MXFP4) -> dict:
    """Exact component sums (and FP64 statistics) of the three-way split under
    the MXFP4 or NVFP4 quantizer."""
    x = _c(x, np.uint16)
    rows, cols = x.shape
    st = ErrStats()
    f = lib().orc_error_decompose if fmt == MXFP4 else lib().orc_error_decompose_nv
    rc = f(_p(x), rows, cols, cols, ctypes.byref(st))
    if rc == -2:
        raise ValueError("NVFP4 decomposition: tensor amax below 2^-89 (terms below 2^-136)")
    if rc != 0:
        raise ValueError("cols must be a multiple of the block size")
    return {
        "exact": [[int(st.exact[c][i]) for i in range(5)] for c in range(4)],
        "exact_int": [fixed_to_int(st.exact[c]) for c in range(4)],
        "sum": [st.sum[c] for c in range(4)],
        "sumsq": [st.sumsq[c] for c in range(4)],
        "cross_sb_gn": st.cross_sb_gn,
        "n_elems": st.n_elems,
        "n_deadzone": st.n_deadzone,
        "n_clipped": st.n_clipped,
    }


# ---- Outlier Fallback ------------------------------------------------------

def qdq_fallback(fmt: int, x: np.ndarray):
    """Quantize-dequantize with Outlier Fallback: entries whose code magnitude
    is 0 keep their own value, the rest are dequantized.  Returns
    (out float32 [rows, cols], number of non-zero entries that fell back)."""
    x = _c(x, np.uint16)
    rows, cols = x.shape
    out = np.zeros((rows, cols), np.float32)
    n = ctypes.c_int64(0)
    rc = lib().orc_qdq_fallback(fmt, _p(x), rows, cols, cols, _p(out), ctypes.byref(n))
    if rc != 0:
        raise ValueError(f"oracle qdq_fallback rejected the shape (rc={rc})")
    return out, int(n.value)
