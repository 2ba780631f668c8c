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


def assert_quant_equal(gpu: dict, ref: dict, fmt: int):
    for k in ("q", "scales"):
        g, r = to_host(gpu[k]), ref[k]
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


def dev_quant(ref: dict, device="cuda:0"):
    """Upload an oracle-quantized tensor set for the GEMM."""
    out = {"q": to_dev(ref["q"], device), "scales": to_dev(ref["scales"], device),
           "tscale": None if ref["tscale"] is None else to_dev(ref["tscale"], device),
           "resid": None if ref["resid"] is None else to_dev(ref["resid"], device)}
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
