#!/usr/bin/env python3
"""Benchmark of the FP4 W4A4 hot path on one MI355X.

One step = one pass of the hot path over one batch of seeded synthetic
input, inputs resident in HBM: online activation quantization (tensor amax,
block scales, E2M1 codes, BF16 residual on the compensated channels) and the
compensated W4A4 GEMM.  Weights are quantized once before timing (they are
re-quantized only at weight sync).  Enough distinct weight and output copies
rotate to defeat the 256 MB last-level cache on the memory-bound workloads.

The timed steps run as one captured HIP graph (host launch cost out of the
measurement); per-kernel times come from HIP events around a graph of
repeated launches of that kernel on the same stream.

Default workload: dense decode NVFP4, X [64 x 2048], W [2048 x 11008],
|S| = 64.  Prints ONE JSON line.  --workload selects another configuration
(prefill_nvfp4, prefill_mxfp4, moe_nvfp4, tiny_nvfp4) for profiling.
"""
from __future__ import annotations

import argparse
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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="decode_nvfp4",
                   choices=["decode_nvfp4", "prefill_nvfp4", "prefill_mxfp4", "moe_nvfp4",
                            "tiny_nvfp4"])
    p.add_argument("--layout", choices=("tiled", "rowmajor"), default="tiled",
                   help="packed operand layout of the dense workloads (MoE is row-major)")
    p.add_argument("--out-dtype", choices=("f32", "bf16"), default="f32",
                   help="GEMM output type of the dense workloads")
    p.add_argument("--residual", choices=("bf16", "fp4"), default="bf16",
                   help="compensation residual of the dense workloads: BF16, or quantized a "
                        "second time to the workload's FP4 format (fp4q_gemm_residual_fp4)")
    p.add_argument("--channels", choices=("fixed", "online"), default="fixed",
                   help="compensated channels of the dense workloads: the workload's fixed "
                        "list, or chosen each step by residual magnitude "
                        "(fp4q_select_channels, k = the workload's channel count)")
    p.add_argument("--comp-weights", choices=("prepared", "inkernel"), default="prepared",
                   help="fixed channels and the BF16 residual (dense and MoE): stream the "
                        "compensation weights B[n, S_j] made once per weight copy "
                        "(fp4q_comp_weights, fp4q_gemm_prepared), or extract them from the "
                        "packed weights in every call (fp4q_gemm)")
    p.add_argument("--moe-quant", choices=("expert", "token"), default="expert",
                   help="MoE gate_up input: quantize the routed copies per expert, or quantize "
                        "the token matrix once and permute its FP4 codes "
                        "(fp4q_permute_quantized, one tensor scale for all tokens)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target CPU time of the oracle baseline sample")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a device-to-device copy of 256 MiB, 5 times (the known-size "
                        "reference for the FETCH_SIZE / WRITE_SIZE counter scale)")
    return p.parse_args()


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


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path is "
              "single-GPU by design and multi-GPU sharding is not built.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fp4_w4a4_quantized_amd as fq
    from workloads import CONFIGS, dense_case, moe_case

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    dev = torch.device("cuda:0")
    # an explicit stream (default priority) for all work and for the timing
    # events.  Library calls take the current stream (no explicit argument):
    # under graph capture that is the capture stream.
    stream = torch.cuda.Stream(dev)
    torch.cuda.set_stream(stream)
    name = args.workload
    cfg = CONFIGS[name]
    fmt = fq.NVFP4 if cfg["fmt"] == "nvfp4" else fq.MXFP4
    blk = fq.BLOCK[fmt]

    def up(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    t0 = time.time()
    print(f"[bench] generating {name} inputs", file=sys.stderr, flush=True)
    if name == "moe_nvfp4":
        data = moe_case(**cfg)
    else:
        data = dense_case(**cfg)
    print(f"[bench] inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    # ---- build the step ------------------------------------------------------
    if name != "moe_nvfp4":
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
        G = 1
        qws = torch.zeros(max(fq.quantize_workspace_bytes(fmt, M, K, 1), 16), dtype=torch.uint8,
                          device=dev)
        cb, sb = fq.packed_bytes(fmt, layout, M, K)
        aq = torch.empty(cb, dtype=torch.uint8, device=dev)
        asc = torch.empty(sb, dtype=torch.uint8, device=dev)
        ats = torch.empty(1, dtype=torch.float32, device=dev) if fmt == fq.NVFP4 else None
        ar = torch.empty((M, nS), dtype=torch.int16, device=dev) if nS else None

        online = args.channels == "online"
        if online:
            if nS == 0:
                sys.exit("--channels online needs a workload with compensated channels")
            chan = torch.empty(nS, dtype=torch.int32, device=dev)
            sws = torch.empty(fq.select_channels_workspace_bytes(M, K), dtype=torch.uint8,
                              device=dev)

            def select():
                fq.select_channels_into(fmt, layout, x, aq, asc, ats, nS, chan, ar, sws)

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
            if online:
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
                                      w["tscale"], chan, nS, ar, w["comp_w"], ys[i % n_rot], ydt,
                                      N)
            else:
                fq.gemm_into(fmt, layout, M, N, K, aq, asc, ats, w["q"], w["scales"],
                             w["tscale"], chan, nS, ar, ys[i % n_rot], ydt, N, gws)

        flops = 2.0 * M * N * K
        r_bytes = (M * nS // 2 + M * nS // blk + (4 if fmt == fq.NVFP4 else 0)) if r4 else M * nS * 2
        gemm_bytes = (M * K // 2 + M * K // blk + r_bytes + nS * 4 + w_bytes + y_bytes +
                      cw_bytes + (8 if fmt == fq.NVFP4 else 0))
        quant_bytes = M * K * 2 + M * K // 2 + M * K // blk + M * nS * 2 + (4 if fmt == fq.NVFP4
                                                                             else 0)
        if r4:
            quant_bytes += M * nS * 2 + r_bytes
        if online:
            # the selection reads x, codes and scales again, writes R and S
            select_bytes = (M * K * 2 + M * K // 2 + M * K // blk + M * nS * 2 + nS * 4 +
                            (4 if fmt == fq.NVFP4 else 0))
            quant_bytes += select_bytes
        wl = {"workload": name, "format": cfg["fmt"], "M": M, "K": K, "N": N, "n_s": nS,
              "layout": args.layout, "out_dtype": args.out_dtype, "weight_copies_rotated": n_rot,
              "residual": args.residual, "channels": args.channels,
              "comp_weights": "prepared" if prepared else "inkernel"}
    else:
        if args.channels != "fixed" or args.residual != "bf16":
            sys.exit("moe_nvfp4 takes the fixed per-expert channel lists and the BF16 residual")
        moe_tok = args.moe_quant == "token"
        online = False
        # MoE layer: gate_up then down, per-expert NVFP4, grouped GEMMs
        off = up(data["offsets"])
        G = int(data["offsets"].size - 1)
        rows = int(data["offsets"][-1])
        H, I2 = cfg["hidden"], 2 * cfg["inter"]
        I = cfg["inter"]
        nS = cfg["n_s"]
        xg, xd = up(data["x_perm"]), up(data["h_perm"])
        cg, cd = up(data["chan_gate_up"]), up(data["chan_down"])

        def qexperts(wt):
            qs = [fq.quantize(fmt, up(wt[e])) for e in range(G)]
            return (torch.stack([q["q"] for q in qs]), torch.stack([q["scales"] for q in qs]),
                    torch.cat([q["tscale"] for q in qs]))

        wgu = qexperts(data["wt_gate_up"])
        wdn = qexperts(data["wt_down"])
        prepared = args.comp_weights == "prepared" and nS > 0
        if prepared:  # made once per expert weight set, like its quantization
            wgu = wgu + (fq.grouped_comp_weights(fmt, wgu[0], wgu[1], cg),)
            wdn = wdn + (fq.grouped_comp_weights(fmt, wdn[0], wdn[1], cd),)
        torch.cuda.synchronize()
        n_rot = 1   # 128 experts' weights already exceed the last-level cache
        bufs = {}
        for tag, (r, k) in {"gu": (rows, H), "dn": (rows, I)}.items():
            bufs[tag] = dict(
                q=torch.empty((r, k // 2), dtype=torch.uint8, device=dev),
                s=torch.empty((r, k // blk), dtype=torch.uint8, device=dev),
                t=torch.empty(G, dtype=torch.float32, device=dev),
                r=torch.empty((r, nS), dtype=torch.int16, device=dev),
                ws=torch.zeros(max(fq.quantize_workspace_bytes(fmt, r, k, G), 16),
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
                fq.permute_quantized_into(fmt, xt, tq, tsc, tts, src, off, G, cg, nS, b["q"],
                                          b["s"], b["t"], b["r"])
            for tag, xin, ch in ((("dn", xd, cd),) if moe_tok else
                                 (("gu", xg, cg), ("dn", xd, cd))):
                b = bufs[tag]
                fq.quantize_into(fmt, fq.ROWMAJOR, xin, off, G, ch, nS, b["q"], b["s"], b["t"], b["r"],
                                 b["ws"])

        gws_bytes = max(fq.grouped_gemm_workspace_bytes(fmt, rows, I2, H, G, nS),
                        fq.grouped_gemm_workspace_bytes(fmt, rows, H, I, G, nS))
        gws = torch.empty(gws_bytes, dtype=torch.uint8, device=dev) if gws_bytes else None

        def gemm(i):
            for tag, w, y, n, k, ch in (("gu", wgu, ygu, I2, H, cg), ("dn", wdn, ydn, H, I, cd)):
                b = bufs[tag]
                if prepared:
                    fq.grouped_gemm_prepared_into(fmt, rows, n, k, off, G, b["q"], b["s"], b["t"],
                                                  w[0], w[1], w[2], ch, nS, b["r"], w[3], y, 0)
                else:
                    fq.grouped_gemm_into(fmt, rows, n, k, off, G, b["q"], b["s"], b["t"], w[0],
                                         w[1], w[2], ch, nS, b["r"], y, 0, gws)

        loads = data["loads"]
        active = int((loads > 0).sum())
        flops = 2.0 * rows * (H * I2 + I * H)
        wb = active * (I2 * H // 2 + I2 * H // blk + H * I // 2 + H * I // blk)
        if prepared:  # each active expert's compensation weights, both layers
            wb += active * (fq.comp_weights_bytes(fmt, fq.ROWMAJOR, I2, H, nS) +
                            fq.comp_weights_bytes(fmt, fq.ROWMAJOR, H, I, nS))
        gemm_bytes = (rows * (H + I) // 2 + rows * (H + I) // blk + 2 * rows * nS * 2 +
                      2 * G * nS * 4 + wb + rows * (I2 + H) * 4 + 2 * (G + 1) * 4 + 4 * G * 4)
        dn_bytes = rows * I * 2 + rows * I // 2 + rows * I // blk + rows * nS * 2 + G * 4
        if moe_tok:
            # tokens read and quantized once; codes read once and written per routed row;
            # the residual gathers x and writes R
            T = cfg["tokens"]
            gu_bytes = (T * H * 2 + 2 * T * (H // 2 + H // blk) + rows * (H // 2 + H // blk) +
                        rows * nS * 4 + G * 4 + 4)
        else:
            gu_bytes = rows * H * 2 + rows * H // 2 + rows * H // blk + rows * nS * 2 + G * 4
        quant_bytes = gu_bytes + dn_bytes
        M, K, N = rows, H, I2
        wl = {"workload": name, "format": "nvfp4", "tokens": cfg["tokens"], "experts": G,
              "top_k": cfg["top_k"], "hidden": H, "inter": I, "routed_rows": rows,
              "n_s_per_expert": nS, "max_expert_rows": int(loads.max()),
              "moe_quant": args.moe_quant,
              "comp_weights": "prepared" if prepared else "inkernel",
              "empty_experts": int((loads == 0).sum())}

    def step(i):
        quant()
        gemm(i)

    # ---- warmup (eager), then the K timed steps as one HIP graph ----------------
    # Launching each kernel from Python costs more host time than the decode
    # kernels take on the GPU, so the timed steps are captured once and
    # replayed: the GPU then runs them back to back, as a serving loop does.
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
    t_start = time.perf_counter()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    g_steps.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    step_ms = ev0.elapsed_time(ev1) / args.steps
    print(f"[bench] {args.steps} steps: {step_ms * 1e3:.2f} us/step (wall {wall:.3f}s)",
          file=sys.stderr, flush=True)
    del g_steps

    # ---- per-kernel averages: HIP events on the launch stream around a graph of
    # `reps` launches of one kernel sequence
    def timed(fn, reps):
        g = capture(fn, reps)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e-3  # seconds

    reps = max(args.steps, 20)
    t_gemm = timed(gemm, reps)
    t_quant = timed(lambda i: quant(), reps)
    print(f"[bench] gemm {t_gemm * 1e6:.2f} us, quantize {t_quant * 1e6:.2f} us per launch",
          file=sys.stderr, flush=True)
    t_sel = timed(lambda i: select(), reps) if online else None
    # the exact three-way error decomposition of the activations
    t_dec = None
    if name != "moe_nvfp4":
        dec_out = torch.zeros(fq.binding.ERR_STATS_BYTES, dtype=torch.uint8, device=dev)
        dec_ws = torch.empty(max(fq.error_decompose_workspace_bytes(M, K), 16), dtype=torch.uint8,
                             device=dev)
        t_dec = timed(lambda i: fq.error_decompose_into(fmt, x, dec_out, dec_ws), reps)
        dec_bytes = M * K * 2
        print(f"[bench] error decomposition {t_dec * 1e6:.2f} us per call", file=sys.stderr,
              flush=True)
    if online:
        print(f"[bench] channel selection {t_sel * 1e6:.2f} us per call", file=sys.stderr,
              flush=True)

    kh = src_hash()
    default_variant = (args.layout == "tiled" and args.out_dtype == "f32" and
                       args.residual == "bf16" and args.channels == "fixed" and
                       args.comp_weights == "prepared" and args.moe_quant == "expert")
    if name in ("prefill_nvfp4", "prefill_mxfp4"):
        mfma_dtype = "f16" if fmt == fq.NVFP4 else "fp4"
        peak = MFMA_PEAK_TFLOPS[mfma_dtype]
        ach = flops / t_gemm / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4), "traffic": load_traffic(name, default_variant),
                "mfma_dtype": mfma_dtype}
    else:
        ach = gemm_bytes / t_gemm / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": load_traffic(name, default_variant),
                "algorithmic_bytes": gemm_bytes}
    quant_gbs = quant_bytes / t_quant / 1e9

    # ---- CPU baseline: the oracle on this host --------------------------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(name, cfg, data, fmt, args.cpu_seconds,
                           r4=name != "moe_nvfp4" and args.residual == "fp4", online=online,
                           moe_tok=name == "moe_nvfp4" and args.moe_quant == "token")

    value = flops / (step_ms * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if fmt == fq.NVFP4 else "fp4",
        "data": "synthetic (seeded; no dataset or trained weights)",
        "config": wl,
        "quantize_gbps": round(quant_gbs, 1),
        "quantize_frac_hbm": round(quant_gbs / HBM_PEAK_GBS, 4),
        "quantize_bytes": quant_bytes,
        "gemm_us": round(t_gemm * 1e6, 3),
        "quantize_us": round(t_quant * 1e6, 3),
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernel_src_hash": kh,
    }
    if t_dec is not None:
        out["decompose_us"] = round(t_dec * 1e6, 3)
        out["decompose_gbps"] = round(dec_bytes / t_dec / 1e9, 1)
        out["decompose_frac_hbm"] = round(dec_bytes / t_dec / 1e9 / HBM_PEAK_GBS, 4)
    if online:
        out["select_us"] = round(t_sel * 1e6, 3)
        out["select_gbps"] = round(select_bytes / t_sel / 1e9, 1)
    print(json.dumps(out), flush=True)


def cpu_baseline(name, cfg, data, fmt, target_s, r4=False, online=False, moe_tok=False):
    """Time the oracle (as it is) on the host: quantize the activations (with
    online channels, then choose them; with the FP4 residual, quantize the
    residual a second time), then the FP64 GEMM on
    a bounded sample of outputs, scaled to TFLOP/s."""
    import numpy as np

    from oracle import oracle as orc

    cores = int(os.environ.get("OMP_NUM_THREADS") or len(os.sched_getaffinity(0)))
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
    gflops_rate = sample_flops / t_g
    return {"value": round(gflops_rate / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"oracle FP64 GEMM on {npts} sampled outputs of the {name} workload "
                      f"(K={K}, {t_g:.1f}s) after {prep} ({t_q:.2f}s)",
            "quantize_s": round(t_q, 4)}


if __name__ == "__main__":
    main()
