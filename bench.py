#!/usr/bin/env python3
"""Throughput of the quantized-linear hot path on one MI355X.

One step runs every step of the path once, at the DiT projection shapes of the
BFL schemes (M = 4608 tokens = 4096 image + 512 text):

* fp8r   4608 x 3072 x 12288: row-wise E4M3 activation quantize + FP8 GEMM;
* nvfp4  4608 x 3072 x 12288: NVFP4 activation quantize (calibrated input_scale)
         + block-scaled GEMM;
* svdq   4608 x 3072 x 3072 + rank 32: NVFP4 quantize, x L1, GEMM with the
         low-rank up-projection in the epilogue.

value = total GEMM FLOPs (2 M N K per linear, low-rank FLOPs not counted) / step
time, with every input resident in HBM.  Weights are quantized once before
timing by the library's own quantizers, as a pre-quantized checkpoint would
arrive.  Inputs are seeded synthetic data (see synthetic/workloads.py).

The roofline object covers the dominant kernel (the nvfp4 GEMM at 4608 x 3072 x
12288): after the timed region, a pass of the same steps times every launch with
HIP events on the launch stream (the library's event timing), and the roofline
takes that kernel's average over all of them (`kernels` lists every kind).  `parts`
comes from another pass with one event pair around each linear and none inside it.  The
cpu_baseline object times the CPU oracle on a bounded sample of the same workload
(rank 0, one GPU only).  `cold` times the same step with its tensors rotated over three
copies (working set above the 256 MB last-level cache).  `extras` times what lies beyond the step: the svdq linear
with SVDQuant smoothing factors, the INT4 variant of svdq_w4a4 at the DiT shapes,
the weight-only 4-bit (awq_w4a16) GEMV at the FLUX modulation shapes, and the
model-specific epilogues: GELU on the nvfp4 linear, the GELU MLP against the same
layers with a separate GELU pass, and the fused QKV scatter.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "fp4": 10100.0}
HBM_GBS = 8000.0
METRIC = "qlinear TFLOP/s (act-quant+GEMM) and % of FP8/FP4 MFMA peak, M=4608"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_nvfp4_4608x3072x12288.md")
# sources of the kernel the traffic counters were taken on; a changed source voids them
TRAFFIC_SOURCES = ("precision_quantized_linear_amd/csrc/gemm_kernels.hip", "precision_quantized_linear_amd/csrc/qpl_dma.h",
                   "precision_quantized_linear_amd/csrc/qpl_device.h", "precision_quantized_linear_amd/csrc/qpl_nvfp4.h")
COPY_PROBE_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # about 26 ms of the step: the clocks ramp over the first milliseconds of MFMA load
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle timing")
    ap.add_argument("--cpu-rows", type=int, default=4608, help="activation rows per linear in the CPU sample")
    ap.add_argument("--no-extras", action="store_true", help="skip the measurements beyond the step (extras)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain 256 MiB device copy (the reference kernel for HBM counter scaling)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the library has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import precision_quantized_linear_amd as qpl
    from synthetic import calibration_batches, make, smooth_factors

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def global_scale_of(tensors):
        amax = torch.zeros((1,), dtype=torch.float32, device=dev)
        for t in tensors:
            qpl.amax_bf16(t, amax=amax)
        return qpl.nvfp4_global_scale(float(amax.item()))

    # ---------------------------------------------------------------- inputs
    t0 = time.time()
    lin = {}
    d = make("fp8r_dit_n12288")
    w = bf16(d["w"])
    wq, ws = qpl.quant_act_fp8_row(w)
    lin["fp8r"] = dict(M=d["M"], K=d["K"], N=d["N"], R=0, x=bf16(d["x"]), wq=wq, ws=ws, host=d)
    del w
    for key, name in (("nvfp4", "nvfp4_dit"), ("svdq", "svdq_w4a4")):
        d = make(name)
        w = bf16(d["w"])
        g_w = global_scale_of([w])
        g_in = global_scale_of(bf16(b) for b in calibration_batches(name))
        wq, wbs = qpl.quant_act_nvfp4(w, g_w)
        e = dict(M=d["M"], K=d["K"], N=d["N"], R=d.get("R", 0), x=bf16(d["x"]), wq=wq, wbs=wbs, g_w=g_w, g_in=g_in,
                 host=d)
        if e["R"]:
            e["l1"], e["l2"] = bf16(d["l1"]), bf16(d["l2"])
        lin[key] = e
        del w
    for key, e in lin.items():
        scheme = qpl.QPL_FP8R if key == "fp8r" else qpl.QPL_NVFP4
        e["y"] = torch.empty((e["M"], e["N"]), dtype=torch.bfloat16, device=dev)
        e["ws_buf"] = torch.empty((qpl.qlinear_workspace_bytes(scheme, e["M"], e["K"], e["N"], e["R"]),),
                                  dtype=torch.uint8, device=dev)
        e["flops"] = 2.0 * e["M"] * e["N"] * e["K"]
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f}s")
    if args.copy_probe:
        src = torch.empty((COPY_PROBE_BYTES,), dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy probe: {COPY_PROBE_BYTES} bytes read and written")

    def run(key):
        e = lin[key]
        if key == "fp8r":
            qpl.qlinear_fp8r(e["x"], e["wq"], e["ws"], y=e["y"], workspace=e["ws_buf"])
        else:
            kw = dict(lora_down=e["l1"], lora_up=e["l2"]) if e["R"] else {}
            qpl.qlinear_nvfp4(e["x"], e["wq"], e["wbs"], e["g_w"], e["g_in"], y=e["y"], workspace=e["ws_buf"], **kw)

    order = ("fp8r", "nvfp4", "svdq")
    for _ in range(args.warmup):
        for k in order:
            run(k)
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed region
    # No events here (an event pair holds the stream for a few microseconds on each
    # side of a launch); the per-linear and per-kernel figures come from two passes
    # below, one with events around each linear, one around each launch.
    qpl.timing_collect()  # drop anything recorded so far
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        for k in order:
            run(k)
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    log(f"timed {args.steps} steps in {t_total * 1e3:.1f} ms")

    ms_step = t_total * 1e3 / args.steps
    total_flops = sum(lin[k]["flops"] for k in order)
    value = total_flops / (ms_step * 1e-3) / 1e12

    # ---------------------------------------------------------------- breakdown passes
    # per linear: an event pair around each call, nothing inside it
    ev = {k: [] for k in order}
    for _ in range(args.steps):
        for k in order:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            run(k)
            b.record()
            ev[k].append((a, b))
    torch.cuda.synchronize()
    # per kernel: the library's events around each of its launches (a pass of its own,
    # since those events lengthen the linear they sit in)
    qpl.timing_enable(True)
    for _ in range(args.steps):
        for k in order:
            run(k)
    torch.cuda.synchronize()
    qpl.timing_enable(False)
    kern = qpl.timing_collect()

    parts = {}
    for k in order:
        per_step = sorted(a.elapsed_time(b) for a, b in ev[k])
        ms = sum(per_step) / len(per_step)
        e = lin[k]
        tf = e["flops"] / (ms * 1e-3) / 1e12
        peak = "fp8" if k == "fp8r" else "fp4"
        parts[k] = {"shape": [e["M"], e["K"], e["N"]] + ([e["R"]] if e["R"] else []), "ms": round(ms, 4),
                    "ms_median": round(per_step[len(per_step) // 2], 4), "ms_min": round(per_step[0], 4),
                    "tflops": round(tf, 1), f"pct_{peak}_peak": round(100 * tf / PEAK_TFLOPS[peak], 2)}
        if k != "fp8r":
            parts[k]["pct_bf16_peak"] = round(100 * tf / PEAK_TFLOPS["bf16"], 2)
        if e["R"]:
            lr_flops = 2.0 * e["M"] * e["R"] * (e["K"] + e["N"])
            parts[k]["tflops_incl_lowrank"] = round((e["flops"] + lr_flops) / (ms * 1e-3) / 1e12, 1)
    kernels = {k: {"launches": n, "avg_us": round(1e3 * t / n, 2)} for k, (n, t) in kern.items() if n}

    # ---------------------------------------------------------------- roofline (dominant kernel)
    # every launch of the per-kernel pass (clocks ramped by the warm-up and the timed region)
    n_g, t_g = kern["gemm_nvfp4"]
    avg_s = t_g / n_g * 1e-3
    e = lin["nvfp4"]
    achieved = e["flops"] / avg_s / 1e12
    traffic = measured_traffic()
    roofline = {"kernel": "gemm_nvfp4 (packed E2M1 + E4M3 operands expanded to f16, f16 MFMA, 4608x3072x12288)",
                "bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_TFLOPS["bf16"], 4), "traffic": traffic,
                "avg_us": round(avg_s * 1e6, 2), "event_samples": n_g,
                "frac_of_fp4_peak": round(achieved / PEAK_TFLOPS["fp4"], 4)}
    # the quantizers against HBM on their algorithmic bytes: fp8r 2 B in + 1 B out per
    # element (+ 4 B per row); nvfp4 2 B in + 0.5 B codes + 1/16 B scales per element
    # (+ the weight's block scales read and written again in the GEMM's layout, which
    # the linear quantizer's launch also does; + T out for the fused low-rank quantizer)
    def gbs(kind, nbytes):
        n, t = kern[kind]
        return round(nbytes / (t / n * 1e-3) / 1e9, 1) if n else None
    mk = lin["fp8r"]["M"] * lin["fp8r"]["K"]
    quant_gbs = {"quant_fp8_row": gbs("quant_fp8_row", 3.0 * mk + 4.0 * lin["fp8r"]["M"]),
                 "quant_nvfp4_linear": gbs("quant_nvfp4_linear", 2.5625 * lin["nvfp4"]["M"] * lin["nvfp4"]["K"] +
                                           2.0 * lin["nvfp4"]["N"] * lin["nvfp4"]["K"] / 16),
                 "quant_nvfp4_lowrank": gbs("quant_nvfp4_lowrank", 2.5625 * lin["svdq"]["M"] * lin["svdq"]["K"] +
                                            4.0 * lin["svdq"]["M"] * 32 * ((lin["svdq"]["R"] + 31) // 32))}
    # reference: a plain device copy of the same activation tensor (read once, written
    # once), timed like the quantizers with events around each launch, so that the
    # figures above can be read against what a copy of that size reaches
    src_x = lin["fp8r"]["x"]
    dst_x = torch.empty_like(src_x)
    copy_ev = []
    for _ in range(args.steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst_x.copy_(src_x)
        b.record()
        copy_ev.append((a, b))
    torch.cuda.synchronize()
    copy_ms = sum(a.elapsed_time(b) for a, b in copy_ev) / len(copy_ev)
    quant_gbs["copy_reference"] = round(2.0 * src_x.numel() * src_x.element_size() / (copy_ms * 1e-3) / 1e9, 1)
    del dst_x

    cold = measure_cold(args, qpl, torch, lin, order, total_flops)
    extras = None if args.no_extras else measure_extras(args, qpl, torch, dev, bf16, lin, kern, make, smooth_factors)

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(lin, args.cpu_rows)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "e4m3/e2m1 operands, fp32 accumulate, bf16 out", "data": "synthetic",
        "config": {"workload": "dit_linear_m4608: fp8r 4608x3072x12288 + nvfp4 4608x3072x12288 + "
                               "svdq nvfp4 4608x3072x3072 r32",
                   "global_batch": 4608, "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "parts": parts,
        "kernels": kernels,
        "quant_gbs": quant_gbs,
        "cold": cold,
        "extras": extras,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def measure_cold(args, qpl, torch, lin, order, total_flops, sets=3):
    """The step with its inputs, weights, workspaces and outputs rotated over `sets`
    copies, so that the working set exceeds the 256 MB MALL and each step finds its
    operands in HBM rather than in the last-level cache."""
    keys = ("x", "wq", "ws", "wbs", "l1", "l2", "y", "ws_buf")
    copies = [{k: e for k, e in lin.items()}]
    for _ in range(sets - 1):
        copies.append({k: {f: (v.clone() if f in keys and torch.is_tensor(v) else v) for f, v in e.items()}
                       for k, e in lin.items()})
    nbytes = sum(v.numel() * v.element_size() for e in copies[0].values() for f, v in e.items()
                 if f in keys and torch.is_tensor(v))

    def run(e, key):
        if key == "fp8r":
            qpl.qlinear_fp8r(e["x"], e["wq"], e["ws"], y=e["y"], workspace=e["ws_buf"])
        else:
            kw = dict(lora_down=e["l1"], lora_up=e["l2"]) if e["R"] else {}
            qpl.qlinear_nvfp4(e["x"], e["wq"], e["wbs"], e["g_w"], e["g_in"], y=e["y"], workspace=e["ws_buf"], **kw)

    for i in range(args.warmup):
        for k in order:
            run(copies[i % sets][k], k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        for k in order:
            run(copies[i % sets][k], k)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    del copies
    return {"ms_per_step": round(ms, 4), "value": round(total_flops / (ms * 1e-3) / 1e12, 2), "sets": sets,
            "working_set_mb": round(sets * nbytes / 1e6, 1)}


def measure_extras(args, qpl, torch, dev, bf16, lin, kern, make, smooth_factors):
    """Timings of what lies beyond the step (the other rows of the method), each on its own."""
    # ---------------------------------------------------------------- SVDQuant smoothing
    # The svdq linear again with per-channel smoothing factors (quantize fused with
    # x L1 now divides x by them first); same shapes, timed on its own.
    e = lin["svdq"]
    lam = torch.from_numpy(smooth_factors("svdq_w4a4")).to(dev)

    def run_smooth():
        qpl.qlinear_nvfp4(e["x"], e["wq"], e["wbs"], e["g_w"], e["g_in"], y=e["y"], workspace=e["ws_buf"],
                          lora_down=e["l1"], lora_up=e["l2"], smooth=lam)

    for _ in range(args.warmup):
        run_smooth()
    torch.cuda.synchronize()
    qpl.timing_collect()
    qpl.timing_select(["quant_nvfp4_lowrank"])
    evs = []
    for _ in range(args.steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        run_smooth()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    qpl.timing_select([])
    ns, ts = qpl.timing_collect()["quant_nvfp4_lowrank"]
    ms = sum(a.elapsed_time(b) for a, b in evs) / len(evs)
    kl = 2 * 32 * ((e["R"] + 31) // 32)
    # x in, packed codes and scales out, T out (hi | lo bf16), smoothing factors
    qlr_bytes = 2.5625 * e["M"] * e["K"] + 2.0 * e["M"] * kl + 4.0 * e["K"]
    extras = {"svdq_smooth": {"shape": [e["M"], e["K"], e["N"], e["R"]], "ms": round(ms, 4),
                              "tflops": round(e["flops"] / (ms * 1e-3) / 1e12, 1),
                              "quant_nvfp4_lowrank_smooth_us": round(1e3 * ts / ns, 2),
                              "quant_nvfp4_lowrank_smooth_gbs": round(qlr_bytes / (ts / ns * 1e-3) / 1e9, 1)}}
    nl, tl = kern["quant_nvfp4_lowrank"]
    extras["quant_nvfp4_lowrank_gbs"] = round((qlr_bytes - 4.0 * e["K"]) / (tl / nl * 1e-3) / 1e9, 1)

    # ---------------------------------------------------------------- beyond the step: INT4 W4A4
    # The INT4 variant of svdq_w4a4 at the DiT shapes: weights quantized by the
    # library's quantizer (one rule for weights and activations), timed per linear
    # with HIP events and per kernel with the library's events.
    for key, name, smooth in (("int4_dit", "nvfp4_dit", False), ("svdq_int4", "svdq_w4a4", False),
                              ("svdq_int4_smooth", "svdq_w4a4", True)):
        d = make(name)
        xa = bf16(d["x"])
        wa = bf16(d["w"])
        wq4, ws4 = qpl.quant_act_int4(wa)
        del wa
        R = d.get("R", 0)
        kw = dict(lora_down=bf16(d["l1"]), lora_up=bf16(d["l2"])) if R else {}
        if smooth:
            kw["smooth"] = torch.from_numpy(smooth_factors(name)).to(dev)
        ya = torch.empty((d["M"], d["N"]), dtype=torch.bfloat16, device=dev)
        wsb = torch.empty((qpl.qlinear_workspace_bytes(qpl.QPL_INT4, d["M"], d["K"], d["N"], R),), dtype=torch.uint8,
                          device=dev)
        for _ in range(args.warmup):
            qpl.qlinear_int4(xa, wq4, ws4, y=ya, workspace=wsb, **kw)
        torch.cuda.synchronize()
        qpl.timing_collect()
        qpl.timing_select(["gemm_int4"])
        evs = []
        for _ in range(args.steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            qpl.qlinear_int4(xa, wq4, ws4, y=ya, workspace=wsb, **kw)
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        qpl.timing_select([])
        ng_, tg_ = qpl.timing_collect()["gemm_int4"]
        ms = sum(a.elapsed_time(b) for a, b in evs) / len(evs)
        fl = 2.0 * d["M"] * d["N"] * d["K"]
        extras[key] = {"shape": [d["M"], d["K"], d["N"]] + ([R] if R else []), "ms": round(ms, 4),
                       "tflops": round(fl / (ms * 1e-3) / 1e12, 1), "gemm_int4_us": round(1e3 * tg_ / ng_, 2),
                       "gemm_int4_tflops": round(fl / (tg_ / ng_ * 1e-3) / 1e12, 1)}
        del xa, wq4, ws4, ya, wsb

    # ---------------------------------------------------------------- beyond the step: weight-only 4-bit
    # FLUX modulation projections (awq_w4a16) at one and two conditioning rows,
    # weights quantized by the library's quantizer; HBM-bound, so bytes per launch
    # (codes + scales + zero points + x + y) over the kernel's event time.
    for name, M in (("awq_adanorm_zero", 1), ("awq_adanorm_zero", 2), ("awq_adanorm_single", 1)):
        d = make(name, M=M)
        G, K, N = d["spec"]["G"], d["K"], d["N"]
        xa = bf16(d["x"])
        wa = bf16(d["w"])
        wq, wsc, wz = qpl.quant_weight_awq(wa, G)
        del wa
        ya = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        for _ in range(args.warmup):
            qpl.qlinear_awq_w4a16(xa, wq, wsc, wz, G, y=ya)
        torch.cuda.synchronize()
        qpl.timing_collect()
        qpl.timing_select(["gemv_w4a16"])
        for _ in range(4 * args.steps):
            qpl.qlinear_awq_w4a16(xa, wq, wsc, wz, G, y=ya)
        torch.cuda.synchronize()
        qpl.timing_select([])
        na, ta = qpl.timing_collect()["gemv_w4a16"]
        nbytes = N * K / 2 + 3.0 * N * (K // G) + 2.0 * M * K + 2.0 * M * N
        gbs = nbytes / (ta / na * 1e-3) / 1e9
        extras[f"{name}_m{M}"] = {"shape": [M, K, N, G], "us": round(1e3 * ta / na, 2), "gbs": round(gbs, 1),
                                  "frac_hbm": round(gbs / HBM_GBS, 4)}
    extras.update(measure_epilogues(args, qpl, torch, dev, bf16, lin, kern, make, smooth_factors))
    return extras


def measure_epilogues(args, qpl, torch, dev, bf16, lin, kern, make, smooth_factors):
    """The model-specific epilogues: GELU on the nvfp4 linear, the GELU MLP against
    the same layers with a separate GELU pass, and the fused QKV scatter."""
    from synthetic import calibration_batches

    def timed(fn, kinds=()):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        qpl.timing_collect()
        qpl.timing_select(list(kinds))
        evs = []
        for _ in range(args.steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        qpl.timing_select([])
        got = qpl.timing_collect()
        us = {k: round(1e3 * got[k][1] / got[k][0], 2) for k in kinds if got[k][0]}
        return sum(a.elapsed_time(b) for a, b in evs) / len(evs), us

    def gscale(t):
        amax = torch.zeros((1,), dtype=torch.float32, device=dev)
        qpl.amax_bf16(t.contiguous(), amax=amax)
        return qpl.nvfp4_global_scale(float(amax.item()))

    out = {}
    # GELU on the nvfp4 linear 4608 x 3072 x 12288 (the step's dominant GEMM)
    e = lin["nvfp4"]
    ms, us = timed(lambda: qpl.qlinear_nvfp4(e["x"], e["wq"], e["wbs"], e["g_w"], e["g_in"], y=e["y"],
                                             workspace=e["ws_buf"], act="gelu_tanh"), ["gemm_epilogue"])
    ng, tg = kern["gemm_nvfp4"]
    out["gelu_nvfp4"] = {"shape": [e["M"], e["K"], e["N"]], "ms": round(ms, 4), "gemm_us": us.get("gemm_epilogue"),
                         "gemm_plain_us": round(1e3 * tg / ng, 2)}

    # FLUX feed-forward 4608 x 3072 -> 12288 -> 3072 as SVDQuant layers (rank 32 and
    # smoothing on both); fc2's input_scale calibrated on this batch's hidden activation
    d = make("svdq_mlp")
    M, K, H, N = d["M"], d["K"], d["N"], d["N2"]
    x = bf16(d["x"])
    w1, w2 = bf16(d["w"]), bf16(d["w2"])
    g_w1, g_w2 = gscale(w1), gscale(w2)
    w1q, w1b = qpl.quant_act_nvfp4(w1, g_w1)
    w2q, w2b = qpl.quant_act_nvfp4(w2, g_w2)
    del w1, w2
    lam1 = torch.from_numpy(smooth_factors("svdq_mlp")).to(dev)
    lam2 = torch.from_numpy(smooth_factors("svdq_mlp", K=H)).to(dev)
    g1 = max(gscale(bf16(b)) for b in calibration_batches("svdq_mlp"))
    lr1 = dict(lora_down=bf16(d["l1"]), lora_up=bf16(d["l2"]))
    lr2 = dict(lora_down=bf16(d["l1_2"]), lora_up=bf16(d["l2_2"]))
    h = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    ws1 = torch.empty((qpl.qlinear_workspace_bytes(qpl.QPL_NVFP4, M, K, H, 32),), dtype=torch.uint8, device=dev)
    ws2 = torch.empty((qpl.qlinear_workspace_bytes(qpl.QPL_NVFP4, M, H, N, 32),), dtype=torch.uint8, device=dev)
    qpl.qlinear_nvfp4(x, w1q, w1b, g_w1, g1, y=h, act="gelu_tanh", smooth=lam1, workspace=ws1, **lr1)
    g2 = gscale((h.float() / lam2).to(torch.bfloat16))
    y2 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    fc1 = dict(weight=w1q, weight_scale=w1b, weight_scale_2=g_w1, input_scale=g1, smooth=lam1, **lr1)
    fc2 = dict(weight=w2q, weight_scale=w2b, weight_scale_2=g_w2, input_scale=g2, smooth=lam2, **lr2)
    wsm = torch.empty((qpl.qlinear_mlp_nvfp4_workspace_bytes(M, K, H, N, 32, 32),), dtype=torch.uint8, device=dev)

    def unfused():
        qpl.qlinear_nvfp4(x, w1q, w1b, g_w1, g1, y=h, smooth=lam1, workspace=ws1, **lr1)
        torch.nn.functional.gelu(h, approximate="tanh")
        qpl.qlinear_nvfp4(h, w2q, w2b, g_w2, g2, y=y2, smooth=lam2, workspace=ws2, **lr2)

    ms_f, us_f = timed(lambda: qpl.qlinear_mlp_nvfp4(x, fc1, fc2, y=y2, workspace=wsm),
                       ["gemm_epilogue", "gemm_nvfp4_lowrank", "quant_nvfp4_lowrank"])
    ms_u, us_u = timed(unfused, ["gemm_nvfp4_lowrank"])
    fl = 2.0 * M * K * H + 2.0 * M * H * N
    out["mlp_nvfp4"] = {"shape": [M, K, H, N, 32], "ms": round(ms_f, 4), "tflops": round(fl / (ms_f * 1e-3) / 1e12, 1),
                        "unfused_torch_gelu_ms": round(ms_u, 4),
                        "fc1_gemm_gelu_us": us_f.get("gemm_epilogue"),
                        "fc1_gemm_plain_us": us_u.get("gemm_nvfp4_lowrank"),
                        "gemm_lowrank_us": us_f.get("gemm_nvfp4_lowrank"),
                        "quant_lowrank_us": us_f.get("quant_nvfp4_lowrank")}
    del x, w1q, w1b, w2q, w2b, h, ws1, ws2, y2, wsm

    # FLUX attention input projection over the 4096 image tokens into q, k, v
    # [24, 4608, 128] after the 512 text tokens
    d = make("qkv_dit")
    s = d["spec"]
    x = bf16(d["x"])
    w = bf16(d["w"])
    g_w = gscale(w)
    wq, wb = qpl.quant_act_nvfp4(w, g_w)
    del w
    g_in = max(gscale(bf16(b)) for b in calibration_batches("qkv_dit"))
    q, k, v = (torch.empty((s["heads"], s["tokens"], s["head_dim"]), dtype=torch.bfloat16, device=dev)
               for _ in range(3))
    wsq = torch.empty((qpl.qlinear_workspace_bytes(qpl.QPL_NVFP4, d["M"], d["K"], d["N"], 0),), dtype=torch.uint8,
                      device=dev)

    ms_q, us_q = timed(lambda: qpl.qlinear_nvfp4(x, wq, wb, g_w, g_in, workspace=wsq, qkv=(q, k, v, s["offset"])),
                       ["gemm_epilogue"])
    out["qkv_nvfp4"] = {"shape": [d["M"], d["K"], d["N"]], "heads": s["heads"], "head_dim": s["head_dim"],
                        "fused_ms": round(ms_q, 4), "gemm_us": us_q.get("gemm_epilogue")}
    return out


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the nvfp4 GEMM from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel factors), or None when the
    summary is missing or the kernel sources changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    fields = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].strip().split(": ", 1)
                fields[k.strip("`")] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(lin, rows, min_seconds=10.0, max_passes=4):
    """The oracle, as written, on `rows` activation rows of each linear (all of them by
    default: one whole step): activation quantize, dequantize both operands, float64
    matmul (plus the low-rank term).  Passes repeat until min_seconds of work."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle.quant import amax_bf16, calibrate_input_scale, global_scale, quant_fp8_row, quant_nvfp4
    from oracle.reference import dequant_fp8r, dequant_nvfp4, lowrank_ref
    from synthetic import calibration_batches

    prep = {}
    for k, e in lin.items():
        h = e["host"]
        if k == "fp8r":
            prep[k] = quant_fp8_row(h["w"])
        else:
            g_w = global_scale(amax_bf16(h["w"]))
            name = "nvfp4_dit" if k == "nvfp4" else "svdq_w4a4"
            g_in = calibrate_input_scale(calibration_batches(name))
            prep[k] = quant_nvfp4(h["w"], g_w) + (g_w, g_in)
    flops = 0.0
    passes = 0
    t0 = time.perf_counter()
    while passes < max_passes and (passes == 0 or time.perf_counter() - t0 < min_seconds):
        for k, e in lin.items():
            h = e["host"]
            r = min(rows, e["M"])
            x = h["x"][:r]
            if k == "fp8r":
                wq, ws = prep[k]
                xq, xs = quant_fp8_row(x)
                y = dequant_fp8r(xq, xs) @ dequant_fp8r(wq, ws).T
            else:
                wq, wbs, g_w, g_in = prep[k]
                xq, xbs = quant_nvfp4(x, g_in)
                y = dequant_nvfp4(xq, xbs, g_in) @ dequant_nvfp4(wq, wbs, g_w).T
                if e["R"]:
                    y = y + lowrank_ref(x, h["l1"], h["l2"])
            flops += 2.0 * r * e["N"] * e["K"]
            del y
        passes += 1
    dt = time.perf_counter() - t0
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = max([p.get("num_threads", 1) for p in blas] or [1])
    r = min(rows, min(e["M"] for e in lin.values()))
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{passes} pass(es) over {r} activation rows of each of the 3 linears (full weights), "
                      f"{dt:.1f} s", "seconds": round(dt, 2), "nproc": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
            "blas": ", ".join(sorted({f"{p.get('internal_api')} {p.get('version')}" for p in blas}))}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
