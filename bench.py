#!/usr/bin/env python3
"""Benchmark of the FP4 W4A4 hot path on one MI355X.

One step = one pass of the hot path over one batch of seeded synthetic
input, inputs resident in HBM: online activation quantization (tensor amax,
block scales, E2M1 codes, BF16 residual on the compensated channels) and the
compensated W4A4 GEMM.  Weights are quantized once before timing (they are
re-quantized only at weight sync).  Enough distinct weight and output copies
rotate to defeat the 256 MB last-level cache on the memory-bound workloads.

The timed steps run as one captured HIP graph (host launch cost out of the
measurement); per-kernel times come from HIP events on the launch stream
around a graph of repeated launches of that kernel.

Default line: the largest single-GPU workload, dense prefill NVFP4
(X [8192 x 4096], W [4096 x 14336], |S| = 128).  The same line carries the
other workloads (prefill MXFP4 on the same tensors, dense decode NVFP4, the
MoE layer) under "extra_workloads", and the chip's attainable matrix-core
and HBM peaks measured by microbenchmarks under "attainable".  Prints ONE
JSON line.  --workload alone measures one workload (with its variants) for
profiling.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "compensated W4A4 GEMM effective TFLOP/s + quantize GB/s, % of roofline"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "fp4": 10100.0}
LLC_BYTES = 256 << 20
HEADLINE = "prefill_nvfp4"
EXTRAS = ("prefill_mxfp4", "decode_nvfp4", "moe_nvfp4")
WORKLOADS = ("prefill_nvfp4", "prefill_mxfp4", "decode_nvfp4", "moe_nvfp4", "tiny_nvfp4")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default=None, choices=WORKLOADS,
                   help="measure this workload only (default: the prefill NVFP4 line with the "
                        "other workloads as extra keys)")
    p.add_argument("--layout", choices=("tiled", "rowmajor"), default="tiled",
                   help="packed operand layout of the dense workloads, and of the experts' "
                        "weights in the MoE workload (its routed activations are row-major)")
    p.add_argument("--out-dtype", choices=("f32", "bf16"), default="f32",
                   help="GEMM output type of the dense workloads")
    p.add_argument("--residual", choices=("bf16", "fp4"), default="bf16",
                   help="compensation residual of the dense workloads: BF16, or quantized a "
                        "second time to the workload's FP4 format (fp4q_gemm_residual_fp4)")
    p.add_argument("--channels", choices=("fixed", "online", "online-2step"), default="fixed",
                   help="compensated channels: the workload's fixed list, or chosen each step "
                        "by residual magnitude, k = the workload's channel count (dense: "
                        "fp4q_quantize_select, the scores taken in the quantizer's pass; "
                        "online-2step: fp4q_quantize then fp4q_select_channels; MoE: "
                        "fp4q_select_channels_grouped either way)")
    p.add_argument("--comp-weights", choices=("prepared", "inkernel"), default="prepared",
                   help="fixed channels and the BF16 residual (dense and MoE): stream the "
                        "compensation weights B[n, S_j] made once per weight copy "
                        "(fp4q_comp_weights, fp4q_gemm_prepared), or extract them from the "
                        "packed weights in every call (fp4q_gemm)")
    p.add_argument("--moe-quant", choices=("expert", "token", "token-gather"), default="expert",
                   help="MoE gate_up input: quantize the routed copies per expert; or quantize "
                        "the token matrix once and permute its FP4 codes "
                        "(fp4q_permute_quantized, one tensor scale for all tokens); or quantize "
                        "it once and let the grouped GEMM gather each routed row's codes "
                        "(fp4q_grouped_gemm_gather; the permute writes only the residual)")
    p.add_argument("--decode-datapath", choices=("separate", "fused"), default="separate",
                   help="decode workload: quantize then GEMM (two launches), or the fused "
                        "decode datapath (fp4q_gemm_decode_fused: the activations quantized "
                        "inside the GEMM)")
    p.add_argument("--no-extras", action="store_true",
                   help="default line without the extra workloads")
    p.add_argument("--no-peaks", action="store_true",
                   help="skip the attainable-peak microbenchmarks")
    p.add_argument("--peaks-only", action="store_true",
                   help="run only the attainable-peak microbenchmarks and print them")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target CPU time of the oracle baseline sample")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a device-to-device copy of 256 MiB, 5 times (the known-size "
                        "reference for the FETCH_SIZE / WRITE_SIZE counter scale)")
    p.add_argument("--record-traffic", default=None, metavar="PMC_DIR",
                   help="no GPU: read rocprofv3 --pmc CSV output under PMC_DIR "
                        "(<workload>_FETCH_SIZE, <workload>_WRITE_SIZE, copy_FETCH_SIZE, "
                        "copy_WRITE_SIZE) and write each workload's entry of "
                        "profiles/traffic.json")
    p.add_argument("--decompose-only", default=None, choices=("nvfp4", "mxfp4"),
                   help="run only the error decomposition of the prefill activations, 5 calls "
                        "(the command behind its counter profile)")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def copy_calibration():
    """A plain copy kernel of known size: 256 MiB read and 256 MiB written per
    launch.  Run under rocprofv3 --pmc, its FETCH_SIZE and WRITE_SIZE give the
    factor that turns those counters into HBM bytes."""
    import torch
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}), flush=True)


def src_hash(files=None) -> str:
    """Hash of the named kernel sources (all of csrc/ when None)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp4_w4a4_quantized_amd", "csrc")
    for f in (sorted(os.listdir(csrc)) if files is None else files):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# dominant kernel of each workload's default variant: a substring of its
# demangled name, the sources that define it, and its dispatches per launch
DOMINANT = {
    "prefill_nvfp4": ("k_gemm_nv4<true>", ["gemm_big.hip", "fp4q_device.h"], 1),
    "prefill_mxfp4": ("k_gemm_big<1, true, 0>", ["gemm_big.hip", "fp4q_device.h"], 1),
    "decode_nvfp4": ("k_gemm_skinny<0, true, true>", ["gemm_skinny.hip", "fp4q_device.h"], 1),
    "moe_nvfp4": ("k_gemm_nv4g<false, true>", ["gemm_big.hip", "fp4q_device.h"], 2),
}


def _pmc_per_dispatch(run_dir, counter, kernel=None):
    """Mean value of `counter` per dispatch (and the dispatch count) over the
    rocprofv3 *counter_collection.csv files under run_dir, for dispatches whose
    kernel name contains `kernel` (for None: the most frequent kernel)."""
    import csv
    import glob
    per = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") != counter:
                    continue
                key = (f, row.get("Dispatch_Id"))
                name, v = row.get("Kernel_Name", ""), float(row["Counter_Value"])
                per[key] = (name, per.get(key, (name, 0.0))[1] + v)
    if kernel is None:
        names = [n for n, _ in per.values()]
        if not names:
            raise SystemExit(f"no {counter} rows under {run_dir}")
        kernel = max(set(names), key=names.count)
    vals = [v for n, v in per.values() if kernel in n]
    if not vals:
        raise SystemExit(f"no {counter} rows for {kernel} under {run_dir}")
    return sum(vals) / len(vals), len(vals)


def record_traffic(pmc_dir):
    """Turn FETCH_SIZE / WRITE_SIZE (KiB per dispatch) into HBM bytes per launch
    with the copy calibration (256 MiB read and written per copy), for every
    workload whose two counter runs are under pmc_dir."""
    copy_bytes = 256 << 20
    cf, _ = _pmc_per_dispatch(os.path.join(pmc_dir, "copy_FETCH_SIZE"), "FETCH_SIZE", "copyBuffer")
    cw, _ = _pmc_per_dispatch(os.path.join(pmc_dir, "copy_WRITE_SIZE"), "WRITE_SIZE", "copyBuffer")
    ff, wf = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path) as f:
        t = json.load(f)
    for wl, (kern, sources, per_launch) in DOMINANT.items():
        fd = os.path.join(pmc_dir, f"{wl}_FETCH_SIZE")
        wd = os.path.join(pmc_dir, f"{wl}_WRITE_SIZE")
        if not (os.path.isdir(fd) and os.path.isdir(wd)):
            continue
        fk, nf = _pmc_per_dispatch(fd, "FETCH_SIZE", kern)
        wk, nw = _pmc_per_dispatch(wd, "WRITE_SIZE", kern)
        t[wl] = {"kernel": kern, "sources": sources, "src_hash": src_hash(sources),
                 "fetch_kib_per_dispatch": round(fk, 1), "write_kib_per_dispatch": round(wk, 1),
                 "dispatches": [nf, nw], "dispatches_per_launch": per_launch,
                 "fetch_factor": round(ff, 4), "write_factor": round(wf, 4),
                 "bytes_per_launch": int(round(per_launch * 1024 * (fk * ff + wk * wf)))}
        print(f"{wl}: {json.dumps(t[wl])}")
    with open(path, "w") as f:
        json.dump(t, f, indent=2)
        f.write("\n")


def load_traffic(workload: str, default_variant: bool):
    """HBM traffic per launch of the workload's dominant kernel, measured with
    rocprofv3 --pmc (FETCH_SIZE and WRITE_SIZE, scaled by a copy-kernel
    calibration) on the default variant of the workload; used only if the
    sources that define that kernel are unchanged since."""
    if not default_variant:
        return None
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
        ent = t.get(workload)
        if ent and ent.get("src_hash") == src_hash(ent.get("sources")):
            return ent["bytes_per_launch"]
    except (OSError, ValueError):
        pass
    return None


# ---- attainable peaks ---------------------------------------------------------

def measure_peaks(stream):
    """Matrix-core and HBM throughput the chip delivers to simple kernels
    (libfp4q_peaks.so): f16 and FP4 MFMA chains with no memory traffic, a
    streaming read and a streaming copy of 4 GiB (far above the 256 MB
    last-level cache).  Best of a few launches each."""
    import torch
    path = os.path.join(ROOT, "fp4_w4a4_quantized_amd", "libfp4q_peaks.so")
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m fp4_w4a4_quantized_amd.build`")
    L = ctypes.CDLL(path)
    P, i32, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64
    L.fp4q_peak_mfma.argtypes = [i32, i32, i32, P, ctypes.POINTER(ctypes.c_double), P]
    L.fp4q_peak_mfma_out_floats.restype = ctypes.c_int64
    L.fp4q_peak_mfma_out_floats.argtypes = [i32]
    L.fp4q_peak_read.argtypes = [P, u64, i32, P, P]
    L.fp4q_peak_copy.argtypes = [P, P, u64, i32, P]
    sp = ctypes.c_void_p(stream.cuda_stream)

    def best_time(launch, reps=5):
        best = None
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            launch()
            b.record(stream)
            torch.cuda.synchronize()
            t = a.elapsed_time(b) * 1e-3
            best = t if best is None else min(best, t)
        return best

    out = {}
    blocks = 256 * 2                     # two 4-wave workgroups per CU: 2 waves per SIMD
    buf = torch.empty(L.fp4q_peak_mfma_out_floats(blocks), dtype=torch.float32,
                      device=stream.device)
    for kind, key, iters in ((0, "mfma_f16_tflops", 20000), (1, "mfma_fp4_tflops", 10000)):
        fl = ctypes.c_double(0.0)

        def run():
            rc = L.fp4q_peak_mfma(kind, blocks, iters, ctypes.c_void_p(buf.data_ptr()),
                                  ctypes.byref(fl), sp)
            assert rc == 0, f"fp4q_peak_mfma rc {rc}"
        t = best_time(run)
        out[key] = round(fl.value / t / 1e12, 1)
    nbytes = 4 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=stream.device)
    src.fill_(3)
    sink = torch.empty(2048 * 256, dtype=torch.int32, device=stream.device)

    def read():
        assert L.fp4q_peak_read(ctypes.c_void_p(src.data_ptr()), nbytes, 2048,
                                ctypes.c_void_p(sink.data_ptr()), sp) == 0
    out["hbm_read_gbs"] = round(nbytes / best_time(read) / 1e9, 1)
    half = nbytes // 2

    def copy():
        assert L.fp4q_peak_copy(ctypes.c_void_p(src.data_ptr()),
                                ctypes.c_void_p(src.data_ptr() + half), half, 2048, sp) == 0
    out["hbm_copy_gbs"] = round(2 * half / best_time(copy) / 1e9, 1)
    del src, sink, buf
    torch.cuda.empty_cache()
    out["about"] = ("best of 5 launches: 512 workgroups x 4 waves of 8 independent MFMA chains "
                    "(f16 32x32x16; FP4 32x32x64 scaled, random codes); streaming read and "
                    "copy over 4 GiB, 16 B per lane per load (copy counts read + write bytes)")
    return out


# ---- workloads ----------------------------------------------------------------

_DATA = {}


def workload_data(name, cfg):
    """Seeded inputs; the two prefill workloads share their tensors."""
    from workloads import dense_case, moe_case
    key = tuple(sorted((k, v) for k, v in cfg.items() if k != "fmt"))
    if key not in _DATA:
        t0 = time.time()
        log(f"generating {name} inputs")
        _DATA[key] = moe_case(**cfg) if name == "moe_nvfp4" else dense_case(**cfg)
        log(f"inputs ready in {time.time() - t0:.1f}s")
    return _DATA[key]


def input_sha256(name, data) -> str:
    h = hashlib.sha256()
    keys = (("x_perm", "h_perm", "offsets", "chan_gate_up", "chan_down") if name == "moe_nvfp4"
            else ("x", "wt", "chan_idx"))
    for k in keys:
        h.update(memoryview(data[k]).cast("B"))
    return h.hexdigest()


class Step:
    """The pieces of one workload's step: quant(), gemm(i), optional select(),
    the algorithmic work and the configuration record."""


def build_dense(name, cfg, data, args, dev):
    import numpy as np
    import torch

    import fp4_w4a4_quantized_amd as fq
    s = Step()
    fmt = fq.NVFP4 if cfg["fmt"] == "nvfp4" else fq.MXFP4
    blk = fq.BLOCK[fmt]

    def up(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    M, K, N = cfg["M"], cfg["K"], cfg["N"]
    nS = int(data["chan_idx"].size)
    x = up(data["x"])
    chan = up(data["chan_idx"]) if nS else None
    layout = fq.TILED if args.layout == "tiled" else fq.ROWMAJOR
    wq = fq.quantize(fmt, up(data["wt"]), layout=layout)  # offline weight quantization
    torch.cuda.synchronize()
    w_bytes = N * (K // 2) + N * (K // blk)
    y_bytes = M * N * (2 if args.out_dtype == "bf16" else 4)
    prepared = (args.comp_weights == "prepared" and nS > 0 and args.channels == "fixed" and
                args.residual == "bf16")
    cw_bytes = fq.comp_weights_bytes(fmt, layout, N, K, nS) if prepared else 0
    n_rot = max(1, math.ceil(1.2 * LLC_BYTES / (w_bytes + y_bytes + cw_bytes)))
    n_rot = min(n_rot, 64)
    wcopies = [wq] + [{k: (v.clone() if isinstance(v, torch.Tensor) else v)
                       for k, v in wq.items()} for _ in range(n_rot - 1)]
    if prepared:  # made once per weight copy, like the weight quantization itself
        for w in wcopies:
            w["comp_w"] = fq.comp_weights(fmt, w, chan)
    ydt = fq.OUT_BF16 if args.out_dtype == "bf16" else fq.OUT_F32
    ys = [torch.empty((M, N), dtype=torch.bfloat16 if ydt == fq.OUT_BF16 else torch.float32,
                      device=dev) for _ in range(n_rot)]
    gwsb = fq.gemm_workspace_bytes(fmt, layout, M, N, K, nS)
    gws = torch.empty(gwsb, dtype=torch.uint8, device=dev) if gwsb else None
    qws = torch.zeros(max(fq.quantize_workspace_bytes(fmt, M, K, 1), 16), dtype=torch.uint8,
                      device=dev)
    cb, sb = fq.packed_bytes(fmt, layout, M, K)
    aq = torch.empty(cb, dtype=torch.uint8, device=dev)
    asc = torch.empty(sb, dtype=torch.uint8, device=dev)
    ats = torch.empty(1, dtype=torch.float32, device=dev) if fmt == fq.NVFP4 else None
    ar = torch.empty((M, nS), dtype=torch.int16, device=dev) if nS else None

    online = args.channels != "fixed"
    fused_sel = args.channels == "online"
    s.select = None
    if online:
        if nS == 0:
            sys.exit("--channels online needs a workload with compensated channels")
        chan = torch.empty(nS, dtype=torch.int32, device=dev)
        if fused_sel:
            qsws = torch.zeros(max(fq.quantize_select_workspace_bytes(fmt, layout, M, K), 16),
                               dtype=torch.uint8, device=dev)
        else:
            sws = torch.empty(fq.select_channels_workspace_bytes(M, K), dtype=torch.uint8,
                              device=dev)

            def select():
                fq.select_channels_into(fmt, layout, x, aq, asc, ats, nS, chan, ar, sws)
            s.select = select

    r4 = args.residual == "fp4"
    if r4:
        if nS == 0 or nS % blk:
            sys.exit(f"--residual fp4 needs |S| a multiple of {blk} (this workload: {nS})")
        # second pass: R [M, nS] quantized row-major, then the FP4-residual GEMM
        rq = torch.empty((M, nS // 2), dtype=torch.uint8, device=dev)
        rsc = torch.empty((M, nS // blk), dtype=torch.uint8, device=dev)
        rts = torch.empty(1, dtype=torch.float32, device=dev) if fmt == fq.NVFP4 else None
        rqws = torch.zeros(max(fq.quantize_workspace_bytes(fmt, M, nS, 1), 16),
                           dtype=torch.uint8, device=dev)
        gwsb = fq.gemm_residual_fp4_workspace_bytes(fmt, layout, M, N, K, nS)
        gws = torch.empty(gwsb, dtype=torch.uint8, device=dev)

    def quant():
        if fused_sel:
            fq.quantize_select_into(fmt, layout, x, nS, aq, asc, ats, chan, ar, qsws)
        elif online:
            fq.quantize_into(fmt, layout, x, None, 1, None, 0, aq, asc, ats, None, qws)
            select()
        else:
            fq.quantize_into(fmt, layout, x, None, 1, chan, nS, aq, asc, ats, ar, qws)
        if r4:
            fq.quantize_into(fmt, fq.ROWMAJOR, ar, None, 1, None, 0, rq, rsc, rts, None, rqws)

    def gemm(i):
        w = wcopies[i % n_rot]
        if r4:
            fq.gemm_residual_fp4_into(fmt, layout, M, N, K, aq, asc, ats, w["q"], w["scales"],
                                      w["tscale"], chan, nS, rq, rsc, rts, ys[i % n_rot], ydt,
                                      N, gws)
        elif prepared:
            fq.gemm_prepared_into(fmt, layout, M, N, K, aq, asc, ats, w["q"], w["scales"],
                                  w["tscale"], chan, nS, ar, w["comp_w"], ys[i % n_rot], ydt, N)
        else:
            fq.gemm_into(fmt, layout, M, N, K, aq, asc, ats, w["q"], w["scales"],
                         w["tscale"], chan, nS, ar, ys[i % n_rot], ydt, N, gws)

    s.quant, s.gemm = quant, gemm
    s.fmt, s.M, s.K, s.x = fmt, M, K, x
    # the fused decode datapath: BF16 activations in, the quantization inside
    # the GEMM (NVFP4, M <= 64, K <= 2048, prepared compensation weights)
    s.fused = None
    if (fmt == fq.NVFP4 and M <= 64 and K <= 2048 and K % 128 == 0 and nS <= 64 and
            (prepared or nS == 0) and not r4 and not online):
        def fused(i):
            w = wcopies[i % n_rot]
            fq.gemm_decode_fused_into(fmt, layout, x, N, w["q"], w["scales"], w["tscale"], chan,
                                      nS, w.get("comp_w"), ys[i % n_rot], ydt, N)
        s.fused = fused
    s.flops = 2.0 * M * N * K
    r_bytes = (M * nS // 2 + M * nS // blk + (4 if fmt == fq.NVFP4 else 0)) if r4 else M * nS * 2
    # algorithmic bytes of the compensated GEMM: Xq + sx + R + S + Wq + sw + Y
    # (+ the two tensor scales); the prepared compensation weights are the
    # implementation's choice and are reported apart as extra bytes
    s.gemm_bytes = (M * K // 2 + M * K // blk + r_bytes + nS * 4 + w_bytes + y_bytes +
                    (8 if fmt == fq.NVFP4 else 0))
    s.extra_bytes = cw_bytes
    s.quant_bytes = M * K * 2 + M * K // 2 + M * K // blk + M * nS * 2 + (4 if fmt == fq.NVFP4
                                                                           else 0)
    if r4:
        s.quant_bytes += M * nS * 2 + r_bytes
    s.select_bytes = None
    if fused_sel:
        s.quant_bytes += nS * 4  # and S; x is read once for codes and scores
    elif online:
        # the selection reads x, codes and scales again, writes R and S
        s.select_bytes = (M * K * 2 + M * K // 2 + M * K // blk + M * nS * 2 + nS * 4 +
                          (4 if fmt == fq.NVFP4 else 0))
        s.quant_bytes += s.select_bytes
    s.mfma = name in ("prefill_nvfp4", "prefill_mxfp4")
    s.wl = {"workload": name, "format": cfg["fmt"], "M": M, "K": K, "N": N, "n_s": nS,
            "layout": args.layout, "out_dtype": args.out_dtype, "weight_copies_rotated": n_rot,
            "residual": args.residual, "channels": args.channels,
            "comp_weights": "prepared" if prepared else "inkernel"}
    s.keep = (wcopies, ys, gws, qws, aq, asc, ats, ar, x, chan)
    if args.decode_datapath == "fused":
        if s.fused is None:
            sys.exit("--decode-datapath fused needs an NVFP4 workload with M <= 64, K <= 2048, "
                     "|S| <= 64 and the default variant")
        s.quant = lambda: None
        s.gemm = s.fused
        s.wl["datapath"] = "fused"
    return s


def build_moe(name, cfg, data, args, dev):
    import numpy as np
    import torch

    import fp4_w4a4_quantized_amd as fq
    online = args.channels != "fixed"  # each expert chooses its channels every step
    r4 = args.residual == "fp4"   # each expert's residual quantized again, own tensor scale
    s = Step()
    s.select = None
    fmt = fq.NVFP4
    blk = fq.BLOCK[fmt]

    def up(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    moe_tok = args.moe_quant in ("token", "token-gather")
    gather = args.moe_quant == "token-gather"
    if gather and not (args.comp_weights == "prepared" or cfg["n_s"] == 0):
        sys.exit("--moe-quant token-gather streams the prepared compensation weights")
    if (r4 or online) and moe_tok:
        sys.exit("--residual fp4 / --channels online on moe_nvfp4 take the per-expert "
                 "quantization")
    off = up(data["offsets"])
    G = int(data["offsets"].size - 1)
    rows = int(data["offsets"][-1])
    H, I2 = cfg["hidden"], 2 * cfg["inter"]
    I = cfg["inter"]
    nS = cfg["n_s"]
    xg, xd = up(data["x_perm"]), up(data["h_perm"])
    cg, cd = up(data["chan_gate_up"]), up(data["chan_down"])

    wl = fq.TILED if args.layout == "tiled" else fq.ROWMAJOR  # the experts' weights

    def qexperts(wt):
        qs = [fq.quantize(fmt, up(wt[e]), layout=wl) for e in range(G)]
        return (torch.stack([q["q"] for q in qs]), torch.stack([q["scales"] for q in qs]),
                torch.cat([q["tscale"] for q in qs]))

    wgu = qexperts(data["wt_gate_up"])
    wdn = qexperts(data["wt_down"])
    # the second-pass residual GEMM and channels chosen per step take B_S from
    # the packed weights
    prepared = args.comp_weights == "prepared" and nS > 0 and not r4 and not online
    if prepared:  # made once per expert weight set, like its quantization
        wgu = wgu + (fq.grouped_comp_weights(fmt, wgu[0], wgu[1], cg, w_layout=wl, N=I2, K=H),)
        wdn = wdn + (fq.grouped_comp_weights(fmt, wdn[0], wdn[1], cd, w_layout=wl, N=H, K=I),)
    torch.cuda.synchronize()
    bufs = {}
    for tag, (r, k) in {"gu": (rows, H), "dn": (rows, I)}.items():
        bufs[tag] = dict(
            q=torch.empty((r, k // 2), dtype=torch.uint8, device=dev),
            s=torch.empty((r, k // blk), dtype=torch.uint8, device=dev),
            t=torch.empty(G, dtype=torch.float32, device=dev),
            r=torch.empty((r, nS), dtype=torch.int16, device=dev),
            ws=torch.zeros(max(fq.quantize_workspace_bytes(fmt, r, k, G), 16),
                           dtype=torch.uint8, device=dev))
        if online:
            bufs[tag].update(
                ch=torch.empty((G, nS), dtype=torch.int32, device=dev),
                sws=torch.empty(max(fq.select_channels_grouped_workspace_bytes(r, k, G), 16),
                                dtype=torch.uint8, device=dev))
        if r4:
            bufs[tag].update(
                rq=torch.empty((r, nS // 2), dtype=torch.uint8, device=dev),
                rs=torch.empty((r, nS // blk), dtype=torch.uint8, device=dev),
                rt=torch.empty(G, dtype=torch.float32, device=dev),
                rws=torch.zeros(max(fq.quantize_workspace_bytes(fmt, r, nS, G), 16),
                                dtype=torch.uint8, device=dev))
    ygu = torch.empty((rows, I2), dtype=torch.float32, device=dev)
    ydn = torch.empty((rows, H), dtype=torch.float32, device=dev)

    if moe_tok:
        T = cfg["tokens"]
        xt = up(data["x_tok"])
        src = up(data["token_of_row"].astype(np.int32))
        tq = torch.empty((T, H // 2), dtype=torch.uint8, device=dev)
        tsc = torch.empty((T, H // blk), dtype=torch.uint8, device=dev)
        tts = torch.empty(1, dtype=torch.float32, device=dev)
        tws = torch.zeros(max(fq.quantize_workspace_bytes(fmt, T, H, 1), 16),
                          dtype=torch.uint8, device=dev)

    def quant():
        if moe_tok:
            b = bufs["gu"]
            fq.quantize_into(fmt, fq.ROWMAJOR, xt, None, 1, None, 0, tq, tsc, tts, None, tws)
            fq.permute_quantized_into(fmt, xt, tq, tsc, tts, src, off, G, cg, nS,
                                      None if gather else b["q"], None if gather else b["s"],
                                      b["t"], b["r"])
        for tag, xin, ch in ((("dn", xd, cd),) if moe_tok else
                             (("gu", xg, cg), ("dn", xd, cd))):
            b = bufs[tag]
            if online:
                fq.quantize_into(fmt, fq.ROWMAJOR, xin, off, G, None, 0, b["q"], b["s"], b["t"],
                                 None, b["ws"])
                fq.select_channels_grouped_into(fmt, xin, off, G, b["q"], b["s"], b["t"], nS,
                                                b["ch"], b["r"], b["sws"])
                continue
            fq.quantize_into(fmt, fq.ROWMAJOR, xin, off, G, ch, nS, b["q"], b["s"], b["t"],
                             b["r"], b["ws"])
            if r4:
                fq.quantize_into(fmt, fq.ROWMAJOR, b["r"], off, G, None, 0, b["rq"], b["rs"],
                                 b["rt"], None, b["rws"])

    gws_bytes = max(fq.grouped_gemm_workspace_bytes(fmt, rows, I2, H, G, nS, wl),
                    fq.grouped_gemm_workspace_bytes(fmt, rows, H, I, G, nS, wl))
    if r4:
        gws_bytes = max(fq.grouped_gemm_residual_fp4_workspace_bytes(fmt, rows, I2, H, G, nS, wl),
                        fq.grouped_gemm_residual_fp4_workspace_bytes(fmt, rows, H, I, G, nS, wl))
    gws = torch.empty(gws_bytes, dtype=torch.uint8, device=dev) if gws_bytes else None

    def gemm(i):
        for tag, w, y, n, k, ch in (("gu", wgu, ygu, I2, H, cg), ("dn", wdn, ydn, H, I, cd)):
            b = bufs[tag]
            if online:
                ch = b["ch"]
            if r4:
                fq.grouped_gemm_residual_fp4_into(fmt, rows, n, k, off, G, b["q"], b["s"], b["t"],
                                                  w[0], w[1], w[2], ch, nS, b["rq"], b["rs"],
                                                  b["rt"], y, 0, gws, w_layout=wl)
            elif gather and tag == "gu":
                fq.grouped_gemm_gather_into(fmt, rows, n, k, off, G, src, cfg["tokens"], tq, tsc,
                                            tts, w[0], w[1], w[2], ch, nS, b["r"],
                                            w[3] if prepared else None, y, 0, w_layout=wl)
            elif prepared:
                fq.grouped_gemm_prepared_into(fmt, rows, n, k, off, G, b["q"], b["s"], b["t"],
                                              w[0], w[1], w[2], ch, nS, b["r"], w[3], y, 0,
                                              w_layout=wl)
            else:
                fq.grouped_gemm_into(fmt, rows, n, k, off, G, b["q"], b["s"], b["t"], w[0],
                                     w[1], w[2], ch, nS, b["r"], y, 0, gws, w_layout=wl)

    loads = data["loads"]
    active = int((loads > 0).sum())
    s.quant, s.gemm = quant, gemm
    s.fmt, s.x = fmt, None
    s.flops = 2.0 * rows * (H * I2 + I * H)
    # algorithmic bytes: activations (codes, scales, residual, channel lists),
    # the active experts' packed weights, FP32 outputs, offsets and tensor scales
    wb = active * (I2 * H // 2 + I2 * H // blk + H * I // 2 + H * I // blk)
    # the residual: BF16, or (second pass) its FP4 codes, scales and tensor scales
    rbytes = (2 * (rows * nS // 2 + rows * nS // blk) + 2 * G * 4) if r4 else 2 * rows * nS * 2
    s.gemm_bytes = (rows * (H + I) // 2 + rows * (H + I) // blk + rbytes +
                    2 * G * nS * 4 + wb + rows * (I2 + H) * 4 + 2 * (G + 1) * 4 + 4 * G * 4)
    s.extra_bytes = (active * (fq.comp_weights_bytes(fmt, fq.ROWMAJOR, I2, H, nS) +
                               fq.comp_weights_bytes(fmt, fq.ROWMAJOR, H, I, nS))
                     if prepared else 0)
    dn_bytes = rows * I * 2 + rows * I // 2 + rows * I // blk + rows * nS * 2 + G * 4
    if moe_tok:
        # tokens read and quantized once; codes read once and written per routed row
        # (not with the gathering GEMM); the residual gathers x and writes R
        T = cfg["tokens"]
        gu_bytes = (T * H * 2 + 2 * T * (H // 2 + H // blk) +
                    (0 if gather else rows * (H // 2 + H // blk)) + rows * nS * 4 + G * 4 + 4)
    else:
        gu_bytes = rows * H * 2 + rows * H // 2 + rows * H // blk + rows * nS * 2 + G * 4
    s.quant_bytes = gu_bytes + dn_bytes
    if online:  # the selection reads x, codes and scales again, writes R and S
        s.quant_bytes += sum(rows * k * 2 + rows * k // 2 + rows * k // blk + rows * nS * 2 +
                             G * nS * 4 + G * 4 for k in (H, I))
    if r4:  # the second pass reads R and writes its codes and scales, per layer
        s.quant_bytes += 2 * (rows * nS * 2 + rows * nS // 2 + rows * nS // blk + G * 4)
    s.select_bytes = None
    s.mfma = False
    s.wl = {"workload": name, "format": "nvfp4", "tokens": cfg["tokens"], "experts": G,
            "top_k": cfg["top_k"], "hidden": H, "inter": I, "routed_rows": rows,
            "n_s_per_expert": nS, "max_expert_rows": int(loads.max()),
            "moe_quant": args.moe_quant, "residual": args.residual, "channels": args.channels,
            "comp_weights": "prepared" if prepared else "inkernel",
            "weight_layout": args.layout, "empty_experts": int((loads == 0).sum())}
    s.keep = (wgu, wdn, bufs, ygu, ydn, gws, xg, xd, cg, cd, off)
    return s


def measure(name, args, stream, dev, variant_args=None):
    """Build, warm up and time one workload; returns its record."""
    import torch

    import fp4_w4a4_quantized_amd as fq
    from workloads import CONFIGS
    a = variant_args or args
    cfg = CONFIGS[name]
    data = workload_data(name, cfg)
    s = (build_moe if name == "moe_nvfp4" else build_dense)(name, cfg, data, a, dev)

    def step(i):
        s.quant()
        s.gemm(i)

    # warmup (eager), then the K timed steps as one HIP graph: launching each
    # kernel from Python costs more host time than the decode kernels take on
    # the GPU, so the timed steps are captured once and replayed back to back
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    def capture(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)
        torch.cuda.synchronize()
        g.replay()  # untimed first replay
        torch.cuda.synchronize()
        return g

    g_steps = capture(step, args.steps)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    g_steps.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    step_ms = ev0.elapsed_time(ev1) / args.steps
    log(f"{name}: {args.steps} steps, {step_ms * 1e3:.2f} us/step")
    del g_steps

    # per-kernel averages: HIP events on the launch stream around a graph of
    # `reps` launches of one kernel sequence
    def timed(fn, reps):
        g = capture(fn, reps)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3  # seconds

    reps = max(args.steps, 20)
    t_gemm = timed(s.gemm, reps)
    t_quant = timed(lambda i: s.quant(), reps)
    log(f"{name}: gemm {t_gemm * 1e6:.2f} us, quantize {t_quant * 1e6:.2f} us per launch")
    t_sel = timed(lambda i: s.select(), reps) if s.select else None
    t_fused = None
    if getattr(s, "fused", None) is not None and a.decode_datapath == "separate":
        t_fused = timed(s.fused, reps)
        log(f"{name}: fused decode datapath {t_fused * 1e6:.2f} us per launch "
            f"(quantize + GEMM in one)")
    t_dec = None
    if s.x is not None:
        dec_out = torch.zeros(fq.binding.ERR_STATS_BYTES, dtype=torch.uint8, device=dev)
        dec_ws = torch.empty(max(fq.error_decompose_workspace_bytes(s.M, s.K), 16),
                             dtype=torch.uint8, device=dev)
        t_dec = timed(lambda i: fq.error_decompose_into(s.fmt, s.x, dec_out, dec_ws), reps)
        log(f"{name}: error decomposition {t_dec * 1e6:.2f} us per call")
        # Outlier Fallback: the activations quantized and dequantized with the
        # deadzone entries kept (FP32 out), and the fallback count
        fb_y = torch.empty((s.M, s.K), dtype=torch.float32, device=dev)
        fb_n = torch.empty(1, dtype=torch.int64, device=dev)
        fb_ws = torch.empty(max(fq.qdq_fallback_workspace_bytes(s.fmt, s.M, s.K), 16),
                            dtype=torch.uint8, device=dev)
        t_fb = timed(lambda i: fq.qdq_fallback_into(s.fmt, s.x, fb_y, fb_n, fb_ws), reps)
        fb_count = int(fb_n.item())
        del fb_y, fb_ws
        log(f"{name}: outlier fallback {t_fb * 1e6:.2f} us per call, {fb_count} entries")

    default_variant = (a.layout == "tiled" and a.out_dtype == "f32" and a.residual == "bf16" and
                       a.channels == "fixed" and a.comp_weights == "prepared" and
                       a.moe_quant == "expert")
    traffic = load_traffic(name, default_variant)
    if s.mfma:
        mfma_dtype = "f16" if s.fmt == fq.NVFP4 else "fp4"
        peak = MFMA_PEAK_TFLOPS[mfma_dtype]
        ach = s.flops / t_gemm / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4), "traffic": traffic, "mfma_dtype": mfma_dtype,
                "peak_fp4": MFMA_PEAK_TFLOPS["fp4"],
                "frac_fp4": round(ach / MFMA_PEAK_TFLOPS["fp4"], 4),
                "algorithmic_bytes": s.gemm_bytes, "extra_bytes": s.extra_bytes}
    else:
        ach = s.gemm_bytes / t_gemm / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
                "algorithmic_bytes": s.gemm_bytes, "extra_bytes": s.extra_bytes}
    quant_gbs = s.quant_bytes / t_quant / 1e9
    rec = {
        "value": round(s.flops / (step_ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "ms_per_step": round(step_ms, 5),
        "dtype": "f16" if s.fmt == fq.NVFP4 else "fp4",
        "config": s.wl,
        "gemm_us": round(t_gemm * 1e6, 3),
        "gemm_tflops": round(s.flops / t_gemm / 1e12, 2),
        "quantize_us": round(t_quant * 1e6, 3),
        "quantize_gbps": round(quant_gbs, 1),
        "quantize_frac_hbm": round(quant_gbs / HBM_PEAK_GBS, 4),
        "quantize_bytes": s.quant_bytes,
        "roofline": roof,
    }
    if t_dec is not None:
        dec_bytes = s.M * s.K * 2
        rec["decompose_us"] = round(t_dec * 1e6, 3)
        rec["decompose_gbps"] = round(dec_bytes / t_dec / 1e9, 1)
        rec["decompose_frac_hbm"] = round(dec_bytes / t_dec / 1e9 / HBM_PEAK_GBS, 4)
        fb_bytes = s.M * s.K * (2 + 4)          # read X (BF16), write the FP32 result
        rec["fallback_us"] = round(t_fb * 1e6, 3)
        rec["fallback_gbps"] = round(fb_bytes / t_fb / 1e9, 1)
        rec["fallback_frac_hbm"] = round(fb_bytes / t_fb / 1e9 / HBM_PEAK_GBS, 4)
        rec["fallback_entries"] = fb_count
    if t_fused is not None:
        rec["fused_decode_us"] = round(t_fused * 1e6, 3)
        rec["fused_decode_tflops"] = round(s.flops / t_fused / 1e12, 2)
    if t_sel is not None:
        rec["select_us"] = round(t_sel * 1e6, 3)
        rec["select_gbps"] = round(s.select_bytes / t_sel / 1e9, 1)
    rec["_data"] = data
    rec["_fmt"] = s.fmt
    del s
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def add_attainable(rec, peaks):
    """Fractions of the measured attainable peaks next to the published ones."""
    if not peaks:
        return
    r = rec["roofline"]
    if r["bound"] == "mfma":
        key = "mfma_f16_tflops" if r["mfma_dtype"] == "f16" else "mfma_fp4_tflops"
    else:
        key = "hbm_read_gbs"
    r["attainable_peak"] = peaks[key]
    r["frac_attainable"] = round(r["achieved"] / peaks[key], 4)
    if "quantize_gbps" in rec:
        rec["quantize_frac_attainable"] = round(rec["quantize_gbps"] / peaks["hbm_copy_gbs"], 4)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.record_traffic:
        record_traffic(args.record_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path is "
              "single-GPU by design and multi-GPU sharding is not built.", file=sys.stderr)
        sys.exit(2)

    import torch

    import fp4_w4a4_quantized_amd as fq

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    fq.lib()   # fails loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    # an explicit stream (default priority) for all work and for the timing
    # events.  Library calls take the current stream (no explicit argument):
    # under graph capture that is the capture stream.
    stream = torch.cuda.Stream(dev)
    torch.cuda.set_stream(stream)

    if args.decompose_only:
        decompose_only(args, stream, dev)
        return
    peaks = None
    if args.peaks_only or not args.no_peaks:
        peaks = measure_peaks(stream)
        log(f"attainable: {peaks}")
        if args.peaks_only:
            print(json.dumps({"attainable": peaks}), flush=True)
            return

    name = args.workload or HEADLINE
    rec = measure(name, args, stream, dev)
    add_attainable(rec, peaks)
    extras = {}
    if args.workload is None and not args.no_extras:
        dflt = argparse.Namespace(**{**vars(args), "layout": "tiled", "out_dtype": "f32",
                                     "residual": "bf16", "channels": "fixed",
                                     "comp_weights": "prepared", "moe_quant": "expert",
                                     "decode_datapath": "separate"})
        for n in EXTRAS:
            e = measure(n, args, stream, dev, variant_args=dflt)
            add_attainable(e, peaks)
            e.pop("_data")
            e.pop("_fmt")
            extras[n] = e
            if n == "moe_nvfp4":
                _DATA.clear()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(name, rec["_data"], rec["_fmt"], args.cpu_seconds,
                           r4=name != "moe_nvfp4" and args.residual == "fp4",
                           online=args.channels != "fixed" and name != "moe_nvfp4",
                           moe_tok=name == "moe_nvfp4" and args.moe_quant == "token")
    rec.pop("_data")
    rec.pop("_fmt")
    out = {
        "metric": METRIC,
        "value": rec.pop("value"),
        "unit": rec.pop("unit"),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": rec.pop("dtype"),
        "data": "synthetic (seeded; no dataset or trained weights)",
        "config": rec.pop("config"),
    }
    out.update(rec)
    out["cpu_baseline"] = cpu
    if peaks:
        out["attainable"] = peaks
    if extras:
        out["extra_workloads"] = extras
    out["kernel_src_hash"] = src_hash()
    print(json.dumps(out), flush=True)


def decompose_only(args, stream, dev):
    """Five calls of the error decomposition of the prefill activations
    (8192 x 4096) in one format: the command the decomposition's counter
    profile is taken with."""
    import numpy as np
    import torch

    import fp4_w4a4_quantized_amd as fq
    from workloads import CONFIGS
    name = "prefill_nvfp4" if args.decompose_only == "nvfp4" else "prefill_mxfp4"
    cfg = CONFIGS[name]
    data = workload_data(name, cfg)
    x = torch.from_numpy(np.ascontiguousarray(data["x"]).view(np.int16)).to(dev)
    fmt = fq.NVFP4 if args.decompose_only == "nvfp4" else fq.MXFP4
    M, K = x.shape
    out = torch.zeros(fq.binding.ERR_STATS_BYTES, dtype=torch.uint8, device=dev)
    ws = torch.empty(max(fq.error_decompose_workspace_bytes(M, K), 16), dtype=torch.uint8,
                     device=dev)
    for _ in range(5):
        fq.error_decompose_into(fmt, x, out, ws)
    torch.cuda.synchronize()
    print(json.dumps({"decompose": name, "calls": 5}), flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(name, data, fmt, target_s, r4=False, online=False, moe_tok=False):
    """Time the oracle (as it is) on the host: quantize the activations (with
    online channels, then choose them; with the FP4 residual, quantize the
    residual a second time), then the FP64 GEMM on a bounded sample of
    outputs, scaled to TFLOP/s.  Also the quantizer on one thread over the
    first rows, the CPU model and the inputs' SHA-256."""
    import numpy as np

    from oracle import oracle as orc
    from workloads import CONFIGS

    cfg = CONFIGS[name]
    cores = orc.max_threads()
    if name == "moe_nvfp4":
        x, chan, off = data["x_perm"], data["chan_gate_up"], data["offsets"]
        K = cfg["hidden"]
    else:
        x, chan, off = data["x"], data["chan_idx"], None
        K = cfg["K"]
    t0 = time.perf_counter()
    if online:
        qa = orc.quantize(fmt, x)
        chan, qa["resid"] = orc.select_channels(fmt, x, qa, int(chan.size))
    elif moe_tok:
        qt = orc.quantize(fmt, data["x_tok"])
        qa = orc.permute_quantized(fmt, data["x_tok"], qt, data["token_of_row"], off, chan)
    else:
        qa = orc.quantize(fmt, x, offsets=off, chan_idx=chan if chan.size else None)
    t_q = time.perf_counter() - t0
    # the quantizer on one thread, over at most 1024 rows (one group)
    rows1 = min(x.shape[0], 1024)
    orc.set_num_threads(1)
    try:
        t0 = time.perf_counter()
        orc.quantize(fmt, x[:rows1],
                     chan_idx=(chan if off is None else chan[0]) if chan.size else None)
        t_q1 = time.perf_counter() - t0
    finally:
        orc.set_num_threads(cores)
    # weights for the sample: the first rows of W^T (first expert for MoE)
    wt = data["wt_gate_up"][0] if name == "moe_nvfp4" else data["wt"]
    n_cols = min(wt.shape[0], 256)
    qb = orc.quantize(fmt, wt[:n_cols])
    M = x.shape[0] if off is None else int(off[1] - off[0])
    ch0 = chan if off is None else chan[0]
    if M == 0:
        return None
    # calibrate the sample size to about target_s seconds of oracle GEMM
    rng = np.random.default_rng(0)
    npts = 2048
    ta = float(qa["tscale"][0]) if fmt == 0 else 1.0
    tb = float(qb["tscale"][0]) if fmt == 0 else 1.0
    R = qa["resid"][:M] if qa["resid"] is not None else None
    if r4:
        t0 = time.perf_counter()
        qr = orc.quantize_residual(fmt, R)
        t_q += time.perf_counter() - t0
        tr = float(qr["tscale"][0]) if fmt == 0 else 1.0
    while True:
        pm, pn = rng.integers(0, M, npts), rng.integers(0, n_cols, npts)
        t0 = time.perf_counter()
        if r4:
            orc.gemm_points_r4(fmt, qa["q"][:M], qa["scales"][:M], ta, qb["q"], qb["scales"], tb,
                               ch0, qr["q"], qr["scales"], tr, pm, pn)
        else:
            orc.gemm_points(fmt, qa["q"][:M], qa["scales"][:M], ta, qb["q"], qb["scales"], tb,
                            ch0 if ch0.size else None, R, pm, pn)
        t_g = time.perf_counter() - t0
        if t_g > 0.2 * target_s or npts >= 1 << 24:
            break
        npts *= 4
    if moe_tok:
        prep = "oracle quantization of the token matrix and the permutation of its codes"
    elif online:
        prep = "oracle quantization and channel selection of the full activation tensor"
    else:
        prep = "oracle quantization of the full activation tensor"
    sample_flops = 2.0 * npts * K
    q_bytes = x.shape[0] * x.shape[1] * 2
    return {"value": round(sample_flops / t_g / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"oracle FP64 GEMM on {npts} sampled outputs of the {name} workload "
                      f"(K={K}, {t_g:.1f}s) after {prep} ({t_q:.2f}s)",
            "quantize_s": round(t_q, 4),
            "quantize_gbps": round(q_bytes / t_q / 1e9, 3),
            "quantize_1thread_s": round(t_q1, 4),
            "quantize_1thread_sample": f"first {rows1} rows x {x.shape[1]} columns, one group",
            "cpu_model": cpu_model(),
            "input_sha256": input_sha256(name, data)}


if __name__ == "__main__":
    main()
