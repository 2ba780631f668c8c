"""ctypes binding of libfp4q (include/fp4q.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
libfp4q.so.  Tensors are torch tensors on the GPU (torch supplies device
memory and the current HIP stream); each function has the name of the C
entry point it calls, minus the ``fp4q_`` prefix.  The library must be built
(``python -m fp4_w4a4_quantized_amd.build``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

NVFP4 = 0
MXFP4 = 1
OUT_F32 = 0
OUT_BF16 = 1
ROWMAJOR = 0
TILED = 1
BLOCK = {NVFP4: 16, MXFP4: 32}

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp4q.so")
_lib = None


class Fp4qError(RuntimeError):
    def __init__(self, fn, status, hip_error=0):
        self.status = status
        msg = f"{fn} failed: {lib().fp4q_status_str(status).decode()} ({status})"
        if hip_error:
            msg += f", hipError {hip_error}"
        super().__init__(msg)


class ErrStats(ctypes.Structure):
    _fields_ = [
        ("exact", (ctypes.c_int64 * 5) * 4),
        ("sum", ctypes.c_double * 4),
        ("sumsq", ctypes.c_double * 4),
        ("cross_sb_gn", ctypes.c_double),
        ("n_elems", ctypes.c_int64),
        ("n_deadzone", ctypes.c_int64),
        ("n_clipped", ctypes.c_int64),
        ("flags", ctypes.c_int64),
    ]


ERR_STATS_BYTES = ctypes.sizeof(ErrStats)


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """Load libfp4q.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: build it with "
                              "`python -m fp4_w4a4_quantized_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        P, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        L.fp4q_status_str.restype = ctypes.c_char_p
        L.fp4q_status_str.argtypes = [ctypes.c_int]
        L.fp4q_last_hip_error.restype = ctypes.c_int
        L.fp4q_last_hip_error.argtypes = []
        L.fp4q_packed_bytes.restype = ctypes.c_int
        L.fp4q_packed_bytes.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64,
                                        ctypes.POINTER(sz), ctypes.POINTER(sz)]
        L.fp4q_quantize_workspace_bytes.restype = sz
        L.fp4q_quantize_workspace_bytes.argtypes = [ctypes.c_int, i64, i64, i32]
        L.fp4q_quantize.restype = ctypes.c_int
        L.fp4q_quantize.argtypes = [ctypes.c_int, ctypes.c_int, P, i64, i64, i64, P, i32, P, i32,
                                    P, P, P, P, P, sz, P]
        L.fp4q_gemm_workspace_bytes.restype = sz
        L.fp4q_gemm_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, i32]
        L.fp4q_gemm.restype = ctypes.c_int
        L.fp4q_gemm.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, P, P, P, P, P, P, P,
                                i32, P, P, ctypes.c_int, i64, P, sz, P]
        L.fp4q_comp_weights_bytes.restype = sz
        L.fp4q_comp_weights_bytes.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i32]
        L.fp4q_comp_weights.restype = ctypes.c_int
        L.fp4q_comp_weights.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, P, P, P, i32, P, sz,
                                        P]
        L.fp4q_gemm_prepared.restype = ctypes.c_int
        L.fp4q_gemm_prepared.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, P, P, P, P, P,
                                         P, P, i32, P, P, sz, P, ctypes.c_int, i64, P]
        L.fp4q_grouped_comp_weights_bytes.restype = sz
        L.fp4q_grouped_comp_weights_bytes.argtypes = [ctypes.c_int, i64, i64, i32, i32]
        L.fp4q_grouped_comp_weights.restype = ctypes.c_int
        L.fp4q_grouped_comp_weights.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i32, P, P, P,
                                                i32, P, sz, P]
        L.fp4q_grouped_gemm_prepared.restype = ctypes.c_int
        L.fp4q_grouped_gemm_prepared.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, P, i32,
                                                 P, P, P, P, P, P, P, i32, P, P, sz, P,
                                                 ctypes.c_int, P]
        L.fp4q_grouped_gemm_workspace_bytes.restype = sz
        L.fp4q_grouped_gemm_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64,
                                                        i32, i32]
        L.fp4q_gemm_residual_fp4_workspace_bytes.restype = sz
        L.fp4q_gemm_residual_fp4_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64,
                                                             i64, i32]
        L.fp4q_gemm_residual_fp4.restype = ctypes.c_int
        L.fp4q_gemm_residual_fp4.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, P, P, P, P,
                                             P, P, P, i32, P, P, P, P, ctypes.c_int, i64, P, sz,
                                             P]
        L.fp4q_grouped_gemm_residual_fp4_workspace_bytes.restype = sz
        L.fp4q_grouped_gemm_residual_fp4_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int,
                                                                     i64, i64, i64, i32, i32]
        L.fp4q_grouped_gemm_residual_fp4.restype = ctypes.c_int
        L.fp4q_grouped_gemm_residual_fp4.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, P,
                                                     i32, P, P, P, P, P, P, P, i32, P, P, P, P,
                                                     ctypes.c_int, P, sz, P]
        L.fp4q_grouped_gemm.restype = ctypes.c_int
        L.fp4q_grouped_gemm.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, P, i32, P, P, P,
                                        P, P, P, P, i32, P, P, ctypes.c_int, P, sz, P]
        L.fp4q_select_channels_workspace_bytes.restype = sz
        L.fp4q_select_channels_workspace_bytes.argtypes = [i64, i64]
        L.fp4q_select_channels.restype = ctypes.c_int
        L.fp4q_select_channels.argtypes = [ctypes.c_int, ctypes.c_int, P, i64, i64, i64, P, P, P,
                                           i32, P, P, P, sz, P]
        L.fp4q_quantize_select_workspace_bytes.restype = sz
        L.fp4q_quantize_select_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64]
        L.fp4q_quantize_select.restype = ctypes.c_int
        L.fp4q_quantize_select.argtypes = [ctypes.c_int, ctypes.c_int, P, i64, i64, i64, i32, P, P,
                                           P, P, P, P, sz, P]
        L.fp4q_select_channels_grouped_workspace_bytes.restype = sz
        L.fp4q_select_channels_grouped_workspace_bytes.argtypes = [i64, i64, i32]
        L.fp4q_select_channels_grouped.restype = ctypes.c_int
        L.fp4q_select_channels_grouped.argtypes = [ctypes.c_int, P, i64, i64, i64, P, i32, P, P, P,
                                                   i32, P, P, P, sz, P]
        L.fp4q_permute_quantized.restype = ctypes.c_int
        L.fp4q_permute_quantized.argtypes = [ctypes.c_int, P, i64, i64, i64, P, P, P, P, i64, P,
                                             i32, P, i32, P, P, P, P, P]
        L.fp4q_qdq_fallback_workspace_bytes.restype = sz
        L.fp4q_qdq_fallback_workspace_bytes.argtypes = [ctypes.c_int, i64, i64]
        L.fp4q_qdq_fallback.restype = ctypes.c_int
        L.fp4q_qdq_fallback.argtypes = [ctypes.c_int, P, i64, i64, i64, P, i64, P, P, sz, P]
        L.fp4q_grouped_gemm_gather.restype = ctypes.c_int
        L.fp4q_grouped_gemm_gather.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, P, i32, P,
                                               i64, P, P, P, P, P, P, P, i32, P, P, sz, P,
                                               ctypes.c_int, P]
        L.fp4q_gemm_decode_fused.restype = ctypes.c_int
        L.fp4q_gemm_decode_fused.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, P, i64,
                                             P, P, P, P, i32, P, sz, P, ctypes.c_int, i64, P, P,
                                             P, P, P]
        L.fp4q_quantize_noalloc.restype = ctypes.c_int
        L.fp4q_quantize_noalloc.argtypes = [ctypes.c_int, ctypes.c_int, P, i64, i64, i64, P, i32,
                                            P, i32, P, P, P, P, P]
        L.fp4q_quantize_status.restype = ctypes.c_int
        L.fp4q_quantize_status.argtypes = [P, sz, ctypes.POINTER(i32), P]
        L.fp4q_test_hook.restype = ctypes.c_int
        L.fp4q_test_hook.argtypes = [i32, i64]
        L.fp4q_error_decompose_workspace_bytes.restype = sz
        L.fp4q_error_decompose_workspace_bytes.argtypes = [i64, i64]
        L.fp4q_error_decompose.restype = ctypes.c_int
        L.fp4q_error_decompose.argtypes = [ctypes.c_int, P, i64, i64, i64, P, P, sz, P]
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn, rc):
    if rc != 0:
        raise Fp4qError(fn, rc, lib().fp4q_last_hip_error() if rc == -4 else 0)


# ---- raw entry points (same names and argument order as the C ABI) --------

def packed_bytes(fmt, layout, rows, cols):
    """(code_bytes, scale_bytes) of one packed operand."""
    cb, sb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check("fp4q_packed_bytes",
           lib().fp4q_packed_bytes(fmt, layout, rows, cols, ctypes.byref(cb), ctypes.byref(sb)))
    return cb.value, sb.value


def quantize_workspace_bytes(fmt, rows, cols, num_groups=1) -> int:
    return lib().fp4q_quantize_workspace_bytes(fmt, rows, cols, num_groups)


def gemm_workspace_bytes(fmt, layout, M, N, K, n_chan) -> int:
    return lib().fp4q_gemm_workspace_bytes(fmt, layout, M, N, K, n_chan)


def comp_weights_bytes(fmt, layout, N, K, n_chan) -> int:
    return lib().fp4q_comp_weights_bytes(fmt, layout, N, K, n_chan)


def comp_weights_into(fmt, layout, N, K, b_q, b_s, chan_idx, n_chan, out, stream=None):
    nb = 0 if out is None else out.numel() * out.element_size()
    rc = lib().fp4q_comp_weights(fmt, layout, N, K, _ptr(b_q), _ptr(b_s), _ptr(chan_idx), n_chan,
                                 _ptr(out), nb, _stream(stream))
    _check("fp4q_comp_weights", rc)


def gemm_prepared_into(fmt, layout, M, N, K, a_q, a_s, a_ts, b_q, b_s, b_ts, chan_idx, n_chan,
                       resid, comp_w, y, y_dtype=OUT_F32, ldy=None, stream=None):
    nb = 0 if comp_w is None else comp_w.numel() * comp_w.element_size()
    rc = lib().fp4q_gemm_prepared(fmt, layout, M, N, K, _ptr(a_q), _ptr(a_s), _ptr(a_ts), _ptr(b_q),
                                  _ptr(b_s), _ptr(b_ts), _ptr(chan_idx), n_chan, _ptr(resid),
                                  _ptr(comp_w), nb, _ptr(y), y_dtype, N if ldy is None else ldy,
                                  _stream(stream))
    _check("fp4q_gemm_prepared", rc)


def grouped_comp_weights_bytes(fmt, N, K, num_groups, n_chan) -> int:
    return lib().fp4q_grouped_comp_weights_bytes(fmt, N, K, num_groups, n_chan)


def grouped_comp_weights(fmt, bq, bs, chan_idx, stream=None, w_layout=ROWMAJOR, N=None, K=None):
    """Every group's compensation weights: bq [G, N, K/2], bs [G, N, K/blk]
    (row-major), or each group's tiled bytes [G, ...] with w_layout=TILED
    and N, K given; chan_idx [G, n_chan]; a uint8 tensor in the grouped
    layout."""
    G = bq.shape[0]
    if w_layout == ROWMAJOR:
        N, K = bq.shape[1], 2 * bq.shape[2]
    elif N is None or K is None:
        raise ValueError("tiled weights: N and K must be given")
    nS = chan_idx.numel() // G
    nb = grouped_comp_weights_bytes(fmt, N, K, G, nS)
    out = torch.empty(max(nb, 16), dtype=torch.uint8, device=bq.device)
    rc = lib().fp4q_grouped_comp_weights(fmt, w_layout, N, K, G, _ptr(bq), _ptr(bs),
                                         _ptr(chan_idx), nS, _ptr(out), out.numel(),
                                         _stream(stream))
    _check("fp4q_grouped_comp_weights", rc)
    return out


def grouped_gemm_prepared_into(fmt, total_rows, N, K, group_offsets, num_groups, a_q, a_s, a_ts,
                               b_q, b_s, b_ts, chan_idx, n_chan, resid, comp_w, y,
                               y_dtype=OUT_F32, stream=None, w_layout=ROWMAJOR):
    nb = 0 if comp_w is None else comp_w.numel() * comp_w.element_size()
    rc = lib().fp4q_grouped_gemm_prepared(fmt, w_layout, total_rows, N, K, _ptr(group_offsets),
                                          num_groups,
                                          _ptr(a_q), _ptr(a_s), _ptr(a_ts), _ptr(b_q), _ptr(b_s),
                                          _ptr(b_ts), _ptr(chan_idx), n_chan, _ptr(resid),
                                          _ptr(comp_w), nb, _ptr(y), y_dtype, _stream(stream))
    _check("fp4q_grouped_gemm_prepared", rc)


def gemm_residual_fp4_workspace_bytes(fmt, layout, M, N, K, n_chan) -> int:
    return lib().fp4q_gemm_residual_fp4_workspace_bytes(fmt, layout, M, N, K, n_chan)


def grouped_gemm_residual_fp4_workspace_bytes(fmt, total_rows, N, K, num_groups, n_chan,
                                              w_layout=ROWMAJOR) -> int:
    return lib().fp4q_grouped_gemm_residual_fp4_workspace_bytes(fmt, w_layout, total_rows, N, K,
                                                                num_groups, n_chan)


def grouped_gemm_workspace_bytes(fmt, total_rows, N, K, num_groups, n_chan,
                                 w_layout=ROWMAJOR) -> int:
    return lib().fp4q_grouped_gemm_workspace_bytes(fmt, w_layout, total_rows, N, K, num_groups,
                                                   n_chan)


def select_channels_workspace_bytes(rows, cols) -> int:
    return lib().fp4q_select_channels_workspace_bytes(rows, cols)


def error_decompose_workspace_bytes(rows, cols) -> int:
    return lib().fp4q_error_decompose_workspace_bytes(rows, cols)


def quantize_into(fmt, layout, x, group_offsets, num_groups, chan_idx, n_chan, q, scales,
                  tensor_scale, resid, workspace, stream=None):
    rows, cols = x.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().fp4q_quantize(fmt, layout, _ptr(x), rows, cols, x.stride(0), _ptr(group_offsets),
                             num_groups, _ptr(chan_idx), n_chan, _ptr(q), _ptr(scales),
                             _ptr(tensor_scale), _ptr(resid), _ptr(workspace), ws_bytes,
                             _stream(stream))
    _check("fp4q_quantize", rc)


def gemm_into(fmt, layout, M, N, K, a_q, a_s, a_ts, b_q, b_s, b_ts, chan_idx, n_chan, resid, y,
              y_dtype=OUT_F32, ldy=None, workspace=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().fp4q_gemm(fmt, layout, M, N, K, _ptr(a_q), _ptr(a_s), _ptr(a_ts), _ptr(b_q), _ptr(b_s),
                         _ptr(b_ts), _ptr(chan_idx), n_chan, _ptr(resid), _ptr(y), y_dtype,
                         N if ldy is None else ldy, _ptr(workspace), ws_bytes, _stream(stream))
    _check("fp4q_gemm", rc)


def gemm_residual_fp4_into(fmt, layout, M, N, K, a_q, a_s, a_ts, b_q, b_s, b_ts, chan_idx, n_chan,
                           r_q, r_s, r_ts, y, y_dtype=OUT_F32, ldy=None, workspace=None,
                           stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().fp4q_gemm_residual_fp4(fmt, layout, M, N, K, _ptr(a_q), _ptr(a_s), _ptr(a_ts),
                                      _ptr(b_q), _ptr(b_s), _ptr(b_ts), _ptr(chan_idx), n_chan,
                                      _ptr(r_q), _ptr(r_s), _ptr(r_ts), _ptr(y), y_dtype,
                                      N if ldy is None else ldy, _ptr(workspace), ws_bytes,
                                      _stream(stream))
    _check("fp4q_gemm_residual_fp4", rc)


def grouped_gemm_residual_fp4_into(fmt, total_rows, N, K, group_offsets, num_groups, a_q, a_s,
                                   a_ts, b_q, b_s, b_ts, chan_idx, n_chan, r_q, r_s, r_ts, y,
                                   y_dtype=OUT_F32, workspace=None, stream=None,
                                   w_layout=ROWMAJOR):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().fp4q_grouped_gemm_residual_fp4(fmt, w_layout, total_rows, N, K, _ptr(group_offsets),
                                              num_groups, _ptr(a_q), _ptr(a_s), _ptr(a_ts),
                                              _ptr(b_q), _ptr(b_s), _ptr(b_ts), _ptr(chan_idx),
                                              n_chan, _ptr(r_q), _ptr(r_s), _ptr(r_ts), _ptr(y),
                                              y_dtype, _ptr(workspace), ws_bytes, _stream(stream))
    _check("fp4q_grouped_gemm_residual_fp4", rc)


def grouped_gemm_into(fmt, total_rows, N, K, group_offsets, num_groups, a_q, a_s, a_ts, b_q,
                      b_s, b_ts, chan_idx, n_chan, resid, y, y_dtype=OUT_F32, workspace=None,
                      stream=None, w_layout=ROWMAJOR):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().fp4q_grouped_gemm(fmt, w_layout, total_rows, N, K, _ptr(group_offsets), num_groups,
                                 _ptr(a_q), _ptr(a_s), _ptr(a_ts), _ptr(b_q), _ptr(b_s),
                                 _ptr(b_ts), _ptr(chan_idx), n_chan, _ptr(resid), _ptr(y),
                                 y_dtype, _ptr(workspace), ws_bytes, _stream(stream))
    _check("fp4q_grouped_gemm", rc)


def select_channels_into(fmt, layout, x, q, scales, tensor_scale, k, chan_out, resid_out,
                         workspace, stream=None):
    rows, cols = x.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().fp4q_select_channels(fmt, layout, _ptr(x), rows, cols, x.stride(0), _ptr(q),
                                    _ptr(scales), _ptr(tensor_scale), k, _ptr(chan_out),
                                    _ptr(resid_out), _ptr(workspace), ws_bytes, _stream(stream))
    _check("fp4q_select_channels", rc)


def quantize_select_workspace_bytes(fmt, layout, rows, cols) -> int:
    return lib().fp4q_quantize_select_workspace_bytes(fmt, layout, rows, cols)


def quantize_select_into(fmt, layout, x, k, q, scales, tensor_scale, chan_out, resid_out,
                         workspace, stream=None):
    rows, cols = x.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().fp4q_quantize_select(fmt, layout, _ptr(x), rows, cols, x.stride(0), k, _ptr(q),
                                    _ptr(scales), _ptr(tensor_scale), _ptr(chan_out),
                                    _ptr(resid_out), _ptr(workspace), ws_bytes, _stream(stream))
    _check("fp4q_quantize_select", rc)


def permute_quantized_into(fmt, x, q, scales, tensor_scale, row_src, group_offsets, num_groups,
                           chan_idx, n_chan, q_out, scales_out, tensor_scale_out, resid_out,
                           stream=None):
    tokens, cols = (x.shape if x is not None else (q.shape[0], q.shape[1] * 2))
    ldx = x.stride(0) if x is not None else cols
    rows = row_src.numel()
    rc = lib().fp4q_permute_quantized(fmt, _ptr(x), tokens, cols, ldx, _ptr(q), _ptr(scales),
                                      _ptr(tensor_scale), _ptr(row_src), rows,
                                      _ptr(group_offsets), num_groups, _ptr(chan_idx), n_chan,
                                      _ptr(q_out), _ptr(scales_out), _ptr(tensor_scale_out),
                                      _ptr(resid_out), _stream(stream))
    _check("fp4q_permute_quantized", rc)


def error_decompose_into(fmt, x, out, workspace, stream=None):
    rows, cols = x.shape
    ws_bytes = workspace.numel() * workspace.element_size()
    rc = lib().fp4q_error_decompose(fmt, _ptr(x), rows, cols, x.stride(0), _ptr(out),
                                    _ptr(workspace), ws_bytes, _stream(stream))
    _check("fp4q_error_decompose", rc)


QSTATUS_GRID_EXPIRED = 1
HOOK_RESET = 0
HOOK_FAIL_NEXT_LAUNCH = 1
HOOK_GRID_SPIN_LIMIT = 2
HOOK_GRID_SKIP_SLOT = 3
DEC_INEXACT = 1


def qdq_fallback_workspace_bytes(fmt, rows, cols) -> int:
    return lib().fp4q_qdq_fallback_workspace_bytes(fmt, rows, cols)


def qdq_fallback_into(fmt, x, y, n_fallback, workspace, stream=None):
    """fp4q_qdq_fallback: y (f32 [rows, >= cols]) = the dequantized x with the
    deadzone entries kept; n_fallback: int64 [1] on the GPU or None."""
    rows, cols = x.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("fp4q_qdq_fallback",
           lib().fp4q_qdq_fallback(fmt, _ptr(x), rows, cols, x.stride(0), _ptr(y), y.stride(0),
                                   _ptr(n_fallback), _ptr(workspace), ws_bytes, _stream(stream)))


def qdq_fallback(fmt, x, stream=None):
    """Returns (y f32 [rows, cols], n_fallback int64 [1]) on the GPU."""
    rows, cols = x.shape
    y = torch.empty((rows, cols), dtype=torch.float32, device=x.device)
    n = torch.empty(1, dtype=torch.int64, device=x.device)
    wsb = qdq_fallback_workspace_bytes(fmt, rows, cols)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=x.device) if wsb else None
    qdq_fallback_into(fmt, x, y, n, ws, stream)
    return y, n


def grouped_gemm_gather_into(fmt, total_rows, N, K, group_offsets, num_groups, row_src, tokens,
                             a_q, a_s, a_ts, b_q, b_s, b_ts, chan_idx, n_chan, resid, comp_w, y,
                             y_dtype, stream=None, w_layout=ROWMAJOR):
    """fp4q_grouped_gemm_gather: the grouped GEMM reading each routed row's
    codes from the token matrix (row_src)."""
    cw_bytes = 0 if comp_w is None else comp_w.numel() * comp_w.element_size()
    _check("fp4q_grouped_gemm_gather",
           lib().fp4q_grouped_gemm_gather(fmt, w_layout, total_rows, N, K, _ptr(group_offsets),
                                          num_groups,
                                          _ptr(row_src), tokens, _ptr(a_q), _ptr(a_s),
                                          _ptr(a_ts), _ptr(b_q), _ptr(b_s), _ptr(b_ts),
                                          _ptr(chan_idx), n_chan, _ptr(resid), _ptr(comp_w),
                                          cw_bytes, _ptr(y), y_dtype, _stream(stream)))


def gemm_decode_fused_into(fmt, layout, x, N, b_q, b_s, b_ts, chan_idx, n_chan, comp_w, y,
                           y_dtype, ldy, a_q_out=None, a_s_out=None, a_ts_out=None,
                           resid_out=None, stream=None):
    """fp4q_gemm_decode_fused: Y from BF16 activations x [M, K] (quantized
    inside the GEMM) and packed weights; optional outputs of the quantized
    activations."""
    M, K = x.shape
    cw_bytes = 0 if comp_w is None else comp_w.numel() * comp_w.element_size()
    _check("fp4q_gemm_decode_fused",
           lib().fp4q_gemm_decode_fused(fmt, layout, M, N, K, _ptr(x), x.stride(0), _ptr(b_q),
                                        _ptr(b_s), _ptr(b_ts), _ptr(chan_idx), n_chan,
                                        _ptr(comp_w), cw_bytes, _ptr(y), y_dtype, ldy,
                                        _ptr(a_q_out), _ptr(a_s_out), _ptr(a_ts_out),
                                        _ptr(resid_out), _stream(stream)))


def quantize_noalloc_into(fmt, layout, x, group_offsets, num_groups, chan_idx, n_chan, q, scales,
                          tensor_scale, resid, stream=None):
    """fp4q_quantize_noalloc: quantize_into without a workspace (the library's
    static per-GPU scratch stands in for it)."""
    rows, cols = x.shape
    _check("fp4q_quantize_noalloc",
           lib().fp4q_quantize_noalloc(fmt, layout, _ptr(x), rows, cols, x.stride(0),
                                       _ptr(group_offsets), num_groups, _ptr(chan_idx), n_chan,
                                       _ptr(q), _ptr(scales), _ptr(tensor_scale), _ptr(resid),
                                       _stream(stream)))


def quantize_status(workspace, stream=None) -> int:
    """Status word of an NVFP4 quantize workspace (waits for the stream,
    then reads and clears it); 0 = every call found its tensor maximum."""
    st = ctypes.c_int32(0)
    _check("fp4q_quantize_status",
           lib().fp4q_quantize_status(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                      ctypes.byref(st), _stream(stream)))
    return st.value


def test_hook(hook: int, value: int = 0) -> None:
    """Failure-injection hooks for tests (fp4q_test_hook)."""
    _check("fp4q_test_hook", lib().fp4q_test_hook(hook, value))


# ---- allocating conveniences ---------------------------------------------

def quantize(fmt, x, group_offsets=None, chan_idx=None, layout=ROWMAJOR, stream=None):
    """x: bf16 (or int16/uint16 bit patterns) [rows, cols] on the GPU.
    group_offsets: int32 [G+1] on the GPU or None.  chan_idx: int32 [G, nS]
    (or [nS]) on the GPU or None.  Returns dict(q, scales, tscale, resid,
    layout, rows, cols); q and scales are [rows, cols/2] and [rows, cols/blk]
    when row-major, flat byte buffers of packed_bytes() when tiled."""
    dev = x.device
    rows, cols = x.shape
    blk = BLOCK[fmt]
    G = 1 if group_offsets is None else group_offsets.numel() - 1
    nS = 0 if chan_idx is None else chan_idx.numel() // G
    if layout == ROWMAJOR:
        q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        sc = torch.empty((rows, cols // blk), dtype=torch.uint8, device=dev)
    else:
        cb, sb = packed_bytes(fmt, layout, rows, cols)
        q = torch.empty(cb, dtype=torch.uint8, device=dev)
        sc = torch.empty(sb, dtype=torch.uint8, device=dev)
    ts = torch.empty(G, dtype=torch.float32, device=dev) if fmt == NVFP4 else None
    R = torch.empty((rows, nS), dtype=torch.int16, device=dev) if nS else None
    wsb = quantize_workspace_bytes(fmt, rows, cols, G)
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=dev) if wsb else None
    quantize_into(fmt, layout, x, group_offsets, G, chan_idx, nS, q, sc, ts, R, ws, stream)
    return {"q": q, "scales": sc, "tscale": ts, "resid": R, "layout": layout, "rows": rows,
            "cols": cols}


def _shape(t):
    """(rows, cols, layout) of a quantize() result (or a row-major dict of
    q [rows, cols/2] and scales without those keys)."""
    if "rows" in t:
        return t["rows"], t["cols"], t["layout"]
    return t["q"].shape[0], t["q"].shape[1] * 2, ROWMAJOR


def gemm(fmt, a, b, chan_idx=None, y_dtype=OUT_F32, stream=None):
    """a, b: quantize() results in one layout (b from W^T [N, K]).
    Returns Y [M, N]."""
    M, K, layout = _shape(a)
    N, Kb, layout_b = _shape(b)
    if Kb != K or layout_b != layout:
        raise ValueError("operands differ in K or layout")
    nS = 0 if chan_idx is None else chan_idx.numel()
    dev = a["q"].device
    y = torch.empty((M, N), dtype=torch.float32 if y_dtype == OUT_F32 else torch.bfloat16,
                    device=dev)
    wsb = gemm_workspace_bytes(fmt, layout, M, N, K, nS)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None
    gemm_into(fmt, layout, M, N, K, a["q"], a["scales"], a["tscale"], b["q"], b["scales"],
              b["tscale"], chan_idx, nS, a["resid"] if nS else None, y, y_dtype, N, ws, stream)
    return y


def comp_weights(fmt, b, chan_idx, stream=None):
    """The compensation weights B[n, S_j] of a quantize() result b (W^T),
    in the tiled BF16 layout fp4q_gemm_prepared streams (uint8 tensor)."""
    N, K, layout = _shape(b)
    nS = chan_idx.numel()
    out = torch.empty(max(comp_weights_bytes(fmt, layout, N, K, nS), 16), dtype=torch.uint8,
                      device=b["q"].device)
    comp_weights_into(fmt, layout, N, K, b["q"], b["scales"], chan_idx, nS, out, stream)
    return out


def gemm_prepared(fmt, a, b, chan_idx, comp_w, y_dtype=OUT_F32, stream=None):
    """gemm() with the compensation weights from comp_weights(fmt, b, chan_idx)."""
    M, K, layout = _shape(a)
    N, Kb, layout_b = _shape(b)
    if Kb != K or layout_b != layout:
        raise ValueError("operands differ in K or layout")
    nS = chan_idx.numel()
    y = torch.empty((M, N), dtype=torch.float32 if y_dtype == OUT_F32 else torch.bfloat16,
                    device=a["q"].device)
    gemm_prepared_into(fmt, layout, M, N, K, a["q"], a["scales"], a["tscale"], b["q"], b["scales"],
                       b["tscale"], chan_idx, nS, a["resid"], comp_w, y, y_dtype, N, stream)
    return y


def gemm_residual_fp4(fmt, a, b, chan_idx, r, y_dtype=OUT_F32, stream=None):
    """The compensated GEMM with the second-pass residual: a, b as for gemm();
    r = quantize(fmt, a["resid"]) (row-major, the residual as an M x n_chan
    tensor).  Returns Y [M, N]."""
    M, K, layout = _shape(a)
    N, Kb, layout_b = _shape(b)
    if Kb != K or layout_b != layout:
        raise ValueError("operands differ in K or layout")
    nS = chan_idx.numel()
    dev = a["q"].device
    y = torch.empty((M, N), dtype=torch.float32 if y_dtype == OUT_F32 else torch.bfloat16,
                    device=dev)
    wsb = gemm_residual_fp4_workspace_bytes(fmt, layout, M, N, K, nS)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None
    gemm_residual_fp4_into(fmt, layout, M, N, K, a["q"], a["scales"], a["tscale"], b["q"],
                           b["scales"], b["tscale"], chan_idx, nS, r["q"], r["scales"],
                           r["tscale"], y, y_dtype, N, ws, stream)
    return y


def grouped_gemm_residual_fp4(fmt, group_offsets, a, bq, bs, bts, chan_idx, r, y_dtype=OUT_F32,
                              stream=None, w_layout=ROWMAJOR, N=None):
    """grouped_gemm() with the second-pass residual: r = quantize(fmt,
    a["resid"], group_offsets) (row-major, one tensor scale per group)."""
    total, K = a["q"].shape[0], a["q"].shape[1] * 2
    G = group_offsets.numel() - 1
    if w_layout == ROWMAJOR:
        N = bq.shape[1]
    elif N is None:
        raise ValueError("tiled weights: N must be given")
    nS = chan_idx.numel() // G
    dev = a["q"].device
    y = torch.empty((total, N), dtype=torch.float32 if y_dtype == OUT_F32 else torch.bfloat16,
                    device=dev)
    wsb = grouped_gemm_residual_fp4_workspace_bytes(fmt, total, N, K, G, nS, w_layout)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None
    grouped_gemm_residual_fp4_into(fmt, total, N, K, group_offsets, G, a["q"], a["scales"],
                                   a["tscale"], bq, bs, bts, chan_idx, nS, r["q"], r["scales"],
                                   r["tscale"], y, y_dtype, ws, stream, w_layout)
    return y


def select_channels_grouped_workspace_bytes(rows, cols, num_groups) -> int:
    return lib().fp4q_select_channels_grouped_workspace_bytes(rows, cols, num_groups)


def select_channels_grouped_into(fmt, x, group_offsets, num_groups, q, scales, tensor_scale, k,
                                 chan_out, resid_out, workspace, stream=None):
    rows, cols = x.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().fp4q_select_channels_grouped(fmt, _ptr(x), rows, cols, x.stride(0),
                                            _ptr(group_offsets), num_groups, _ptr(q),
                                            _ptr(scales), _ptr(tensor_scale), k, _ptr(chan_out),
                                            _ptr(resid_out), _ptr(workspace), ws_bytes,
                                            _stream(stream))
    _check("fp4q_select_channels_grouped", rc)


def select_channels_grouped(fmt, x, group_offsets, a, k, stream=None):
    """a = quantize(fmt, x, group_offsets) (row-major).  Returns (chan int32
    [G, k], ascending per group; resid bf16 bits as int16 [rows, k]): each
    group's k channels of largest residual magnitude and the residual."""
    rows, cols = x.shape
    G = group_offsets.numel() - 1
    dev = x.device
    chan = torch.empty((G, k), dtype=torch.int32, device=dev)
    resid = torch.empty((rows, k), dtype=torch.int16, device=dev)
    wsb = select_channels_grouped_workspace_bytes(rows, cols, G)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    select_channels_grouped_into(fmt, x, group_offsets, G, a["q"], a["scales"], a["tscale"], k,
                                 chan, resid, ws, stream)
    return chan, resid


def select_channels(fmt, x, a, k, stream=None):
    """a = quantize(fmt, x) (one group, any layout).  Returns (chan int32
    [k] ascending, resid bf16 bits as int16 [rows, k]): the k channels of
    largest residual magnitude and the residual on them."""
    rows, cols = x.shape
    dev = x.device
    chan = torch.empty(k, dtype=torch.int32, device=dev)
    R = torch.empty((rows, k), dtype=torch.int16, device=dev)
    wsb = select_channels_workspace_bytes(rows, cols)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None
    select_channels_into(fmt, a["layout"], x, a["q"], a["scales"], a["tscale"], k, chan, R, ws,
                         stream)
    return chan, R


def quantize_select(fmt, x, k, layout=ROWMAJOR, stream=None):
    """Quantize x (one group) and choose its k channels of largest residual
    magnitude in one call.  Returns (a, chan, resid): a as quantize(fmt, x,
    layout=layout) with a["resid"] the residual on chan (int16 bits
    [rows, k]), chan int32 [k] ascending."""
    dev = x.device
    rows, cols = x.shape
    blk = BLOCK[fmt]
    if layout == ROWMAJOR:
        q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
        sc = torch.empty((rows, cols // blk), dtype=torch.uint8, device=dev)
    else:
        cb, sb = packed_bytes(fmt, layout, rows, cols)
        q = torch.empty(cb, dtype=torch.uint8, device=dev)
        sc = torch.empty(sb, dtype=torch.uint8, device=dev)
    ts = torch.empty(1, dtype=torch.float32, device=dev) if fmt == NVFP4 else None
    chan = torch.empty(max(k, 1), dtype=torch.int32, device=dev)[:k]
    R = torch.empty((rows, k), dtype=torch.int16, device=dev)
    wsb = quantize_select_workspace_bytes(fmt, layout, rows, cols)
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=dev)
    quantize_select_into(fmt, layout, x, k, q, sc, ts, chan, R, ws, stream)
    a = {"q": q, "scales": sc, "tscale": ts, "resid": R, "layout": layout, "rows": rows,
         "cols": cols}
    return a, chan, R


def permute_quantized(fmt, x, a, row_src, group_offsets, chan_idx=None, stream=None):
    """a = quantize(fmt, x) of the token activations (one group, row-major).
    Returns a grouped quantize()-style dict (q, scales, tscale [G], resid)
    of the expert-ordered rows row_src, ready for grouped_gemm()."""
    dev = a["q"].device
    rows = row_src.numel()
    cols = a["q"].shape[1] * 2
    blk = BLOCK[fmt]
    G = group_offsets.numel() - 1
    nS = 0 if chan_idx is None else chan_idx.numel() // G
    q = torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    sc = torch.empty((rows, cols // blk), dtype=torch.uint8, device=dev)
    ts = torch.empty(G, dtype=torch.float32, device=dev) if fmt == NVFP4 else None
    R = torch.empty((rows, nS), dtype=torch.int16, device=dev) if nS else None
    permute_quantized_into(fmt, x, a["q"], a["scales"], a["tscale"], row_src, group_offsets, G,
                           chan_idx, nS, q, sc, ts, R, stream)
    return {"q": q, "scales": sc, "tscale": ts, "resid": R, "layout": ROWMAJOR, "rows": rows,
            "cols": cols}


def grouped_gemm(fmt, group_offsets, a, bq, bs, bts, chan_idx=None, y_dtype=OUT_F32,
                 stream=None, w_layout=ROWMAJOR, N=None):
    """a: grouped quantize() result; bq [G, N, K/2], bs [G, N, K/blk], bts [G]
    (w_layout=TILED: each group's tiled bytes [G, ...], N given)."""
    total, K = a["q"].shape[0], a["q"].shape[1] * 2
    G = group_offsets.numel() - 1
    if w_layout == ROWMAJOR:
        N = bq.shape[1]
    elif N is None:
        raise ValueError("tiled weights: N must be given")
    nS = 0 if chan_idx is None else chan_idx.numel() // G
    dev = a["q"].device
    y = torch.empty((total, N), dtype=torch.float32 if y_dtype == OUT_F32 else torch.bfloat16,
                    device=dev)
    wsb = grouped_gemm_workspace_bytes(fmt, total, N, K, G, nS, w_layout)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None
    grouped_gemm_into(fmt, total, N, K, group_offsets, G, a["q"], a["scales"], a["tscale"], bq,
                      bs, bts, chan_idx, nS, a["resid"] if nS else None, y, y_dtype, ws, stream,
                      w_layout)
    return y


def grouped_gemm_prepared(fmt, group_offsets, a, bq, bs, bts, chan_idx, comp_w, y_dtype=OUT_F32,
                          stream=None, w_layout=ROWMAJOR, N=None):
    """grouped_gemm() with comp_w = grouped_comp_weights(fmt, bq, bs, chan_idx)."""
    total, K = a["q"].shape[0], a["q"].shape[1] * 2
    G = group_offsets.numel() - 1
    if w_layout == ROWMAJOR:
        N = bq.shape[1]
    elif N is None:
        raise ValueError("tiled weights: N must be given")
    nS = chan_idx.numel() // G
    y = torch.empty((total, N), dtype=torch.float32 if y_dtype == OUT_F32 else torch.bfloat16,
                    device=a["q"].device)
    grouped_gemm_prepared_into(fmt, total, N, K, group_offsets, G, a["q"], a["scales"],
                               a["tscale"], bq, bs, bts, chan_idx, nS, a["resid"], comp_w, y,
                               y_dtype, stream, w_layout)
    return y


def error_decompose(fmt, x, stream=None):
    """Returns a dict like the fp4q_err_stats_t struct (copied to the host)."""
    rows, cols = x.shape
    out = torch.zeros(ERR_STATS_BYTES, dtype=torch.uint8, device=x.device)
    wsb = error_decompose_workspace_bytes(rows, cols)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=x.device)
    error_decompose_into(fmt, x, out, ws, stream)
    host = out.cpu().numpy().tobytes()
    st = ErrStats.from_buffer_copy(host)
    return {
        "exact": [[int(st.exact[c][i]) for i in range(5)] for c in range(4)],
        "sum": [st.sum[c] for c in range(4)],
        "sumsq": [st.sumsq[c] for c in range(4)],
        "cross_sb_gn": st.cross_sb_gn,
        "n_elems": st.n_elems,
        "n_deadzone": st.n_deadzone,
        "n_clipped": st.n_clipped,
        "flags": st.flags,
    }
