"""Helpers for the GPU parity tests: move seeded numpy inputs to the device,
run the HIP path through the C ABI (ctypes binding), and compare with the
oracle.  Inputs come from the shared seeded generators; expected values come
only from the oracle."""
import sys

import numpy as np
import torch

# tolerance of the FP32-accumulated GEMM against the exact FP64 oracle,
# relative to the sum of absolute terms (Yabs)
GEMM_RTOL = 1e-3


def need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X (torch.cuda unavailable)"
    return torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, device="cuda:0"):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def to_host(t) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    return a


# ---- the tiled packed layout, written from its definition in include/fp4q.h:
# codes in 1 KB blocks per (16-row group, 128-column step), the 16 bytes of
# row r and step chunk c at (c*16 + r)*16; scales in blocks per (64-row
# group, step), NVFP4 byte 4d + e of a row's step at (d*64 + r)*4 + e,
# MXFP4 byte e at r*4 + e.  Rows are padded to 16 (codes) and 64 (scales).

def _pad_rows(a: np.ndarray, mult: int) -> np.ndarray:
    rows = a.shape[0]
    rp = -(-rows // mult) * mult
    out = np.zeros((rp,) + a.shape[1:], a.dtype)
    out[:rows] = a
    return out


def tile_codes(q: np.ndarray) -> np.ndarray:
    """Row-major codes [rows, K/2] -> tiled byte buffer."""
    rows, kh = q.shape
    assert kh % 64 == 0
    p = _pad_rows(q, 16)
    t = p.reshape(p.shape[0] // 16, 16, kh // 64, 4, 16)      # [G, r, k, c, byte]
    return np.ascontiguousarray(t.transpose(0, 2, 3, 1, 4)).reshape(-1)


def untile_codes(buf: np.ndarray, rows: int, K: int) -> np.ndarray:
    rp = -(-rows // 16) * 16
    t = buf[:rp * K // 2].reshape(rp // 16, K // 128, 4, 16, 16)  # [G, k, c, r, byte]
    return np.ascontiguousarray(t.transpose(0, 3, 1, 2, 4)).reshape(rp, K // 2)[:rows]


def tile_scales(s: np.ndarray, fmt: int) -> np.ndarray:
    """Row-major block scales [rows, K/blk] -> tiled byte buffer."""
    rows, ks = s.shape
    p = _pad_rows(s, 64)
    H = p.shape[0] // 64
    if fmt == 0:
        t = p.reshape(H, 64, ks // 8, 2, 4).transpose(0, 2, 3, 1, 4)   # [H, k, d, r, e]
    else:
        t = p.reshape(H, 64, ks // 4, 4).transpose(0, 2, 1, 3)         # [H, k, r, e]
    return np.ascontiguousarray(t).reshape(-1)


def untile_scales(buf: np.ndarray, rows: int, K: int, fmt: int) -> np.ndarray:
    rp = -(-rows // 64) * 64
    H = rp // 64
    if fmt == 0:
        t = buf[:rp * K // 16].reshape(H, K // 128, 2, 64, 4).transpose(0, 3, 1, 2, 4)
        return np.ascontiguousarray(t).reshape(rp, K // 16)[:rows]
    t = buf[:rp * K // 32].reshape(H, K // 128, 64, 4).transpose(0, 2, 1, 3)
    return np.ascontiguousarray(t).reshape(rp, K // 32)[:rows]


def host_packed(gpu: dict, fmt: int):
    """(codes, scales) of a quantize() result as row-major host arrays."""
    q, s = to_host(gpu["q"]), to_host(gpu["scales"])
    if gpu.get("layout", 0) == 1:
        rows, K = gpu["rows"], gpu["cols"]
        return untile_codes(q, rows, K), untile_scales(s, rows, K, fmt)
    return q, s


def assert_quant_equal(gpu: dict, ref: dict, fmt: int):
    hq, hs = host_packed(gpu, fmt)
    for k, g in (("q", hq), ("scales", hs)):
        r = ref[k]
        assert g.shape == r.shape, (k, g.shape, r.shape)
        bad = np.argwhere(g != r)
        assert bad.size == 0, f"{k}: {len(bad)} mismatches, first {bad[:3].tolist()}"
    if fmt == 0:
        g = to_host(gpu["tscale"])
        assert np.array_equal(g.view(np.uint32), ref["tscale"].view(np.uint32)), (g, ref["tscale"])
    if ref["resid"] is not None:
        g = to_host(gpu["resid"])
        bad = np.argwhere(g != ref["resid"])
        assert bad.size == 0, f"resid: {len(bad)} mismatches, first {bad[:3].tolist()}"


def assert_gemm_close(y_gpu: np.ndarray, y: np.ndarray, yabs: np.ndarray, rtol=GEMM_RTOL):
    y_gpu = y_gpu.astype(np.float64)
    err = np.abs(y_gpu - y)
    bound = rtol * yabs
    bad = np.argwhere(~(err <= bound))
    ratio = float(np.max(err / np.maximum(yabs, 1e-300))) if err.size else 0.0
    assert bad.size == 0, (f"{len(bad)} outputs outside {rtol}*Yabs; worst ratio {ratio:.3e}; "
                           f"first {bad[:3].tolist()}")
    return ratio


def oracle_quant(orc, fmt, x, chan=None, offsets=None):
    return orc.quantize(fmt, x, offsets=offsets, chan_idx=chan)


def dev_quant(ref: dict, device="cuda:0", layout=0, fmt=None):
    """Upload an oracle-quantized tensor set for the GEMM (tiled on the host
    when layout == 1; fmt is then needed for the scale arrangement)."""
    q, s = ref["q"], ref["scales"]
    rows, K = q.shape[0], q.shape[1] * 2
    if layout == 1:
        q, s = tile_codes(q), tile_scales(s, fmt)
    out = {"q": to_dev(q, device), "scales": to_dev(s, device),
           "tscale": None if ref["tscale"] is None else to_dev(ref["tscale"], device),
           "resid": None if ref["resid"] is None else to_dev(ref["resid"], device),
           "layout": layout, "rows": rows, "cols": K}
    return out


_CACHE = {}


def workload(name: str, **over):
    """Seeded workload from the shared generators, cached for the session."""
    from workloads import CONFIGS, dense_case, moe_case
    key = (name, tuple(sorted(over.items())))
    if key not in _CACHE:
        cfg = {**CONFIGS[name], **over}
        _CACHE[key] = moe_case(**cfg) if name.startswith("moe") else dense_case(**cfg)
    return _CACHE[key]
