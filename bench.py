#!/usr/bin/env python3
"""Throughput of the modulated deformable conv2d forward on one MI355X.

One step = the whole forward over one batch of synthetic input already
resident in HBM: dcn_forward = weight-pack kernel + fused sample-and-contract
kernel, both launched through the C ABI on torch's current stream.

Prints ONE JSON line: output pixels/s (``value``), effective TFLOP/s
(2 * P * O * K * C per step), the fused kernel's roofline fraction against the
dense fp32 (or bf16) MFMA peak, and the CPU oracle timed on this host on a
bounded sample of the same workload.

Default workload: the BiRefNet-decoder-like 7x7, 64-channel deformable conv at
1024 input (256x256 map, fp32).  ``--workload`` picks another; ``--gpus`` > 1
is refused (this path runs on one GPU).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "deform-conv output pixels/s + effective TFLOP/s and % roofline, 256^2x64ch 7x7"
MFMA_PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6}   # MI355X dense matrix peaks
HBM_PEAK_GBS = 8000.0
# vector L1 return bandwidth: 64 B per clock per CU x 256 CUs x 2.4 GHz
L1_PEAK_GBS = 64 * 256 * 2.4
KERNEL_DIR = os.path.join(ROOT, "modulated_deformable_convolution_dcn_amd", "csrc")


# The sources each workload's forward kernel is built from (the kernel, its
# device helpers and argument structs, and the host code that sizes and
# launches it); a traffic record counts only while these are unchanged.
_QUAD = ("dcn_quad.hip", "dcn_device.h", "dcn_launch.h", "dcn_api.cpp")
KERNEL_SOURCES = {
    "birefnet512_fp32": _QUAD,
    "birefnet1024_fp32": _QUAD,
    "detection_bf16": ("dcn_bf16.hip", "dcn_device.h", "dcn_launch.h", "dcn_api.cpp"),
    "edge_stress_fp32": ("dcn_wsk.hip", "dcn_device.h", "dcn_launch.h", "dcn_api.cpp"),
}


def kernel_source_hash(workload: str = None) -> str:
    """sha256 over the workload's kernel sources (every kernel source and
    internal header when the workload has no entry), sorted by name."""
    names = KERNEL_SOURCES.get(workload)
    if names is None:
        names = [n for n in os.listdir(KERNEL_DIR) if n.endswith((".hip", ".h", ".cpp"))]
    h = hashlib.sha256()
    for name in sorted(names):
        h.update(name.encode())
        with open(os.path.join(KERNEL_DIR, name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per fused launch from the committed PMC summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "fused_kernel_%s_traffic.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_sha256") != kernel_source_hash(workload):
        return None
    return rec.get("traffic_bytes_per_launch")


def summarize_traffic(pmc_dir: str, workload: str, copy_mib: int) -> dict:
    """Per-launch HBM bytes of the fused kernel from four rocprofv3 --pmc runs
    under pmc_dir: <workload>_FETCH_SIZE, <workload>_WRITE_SIZE (this script on
    the workload) and copy_FETCH_SIZE, copy_WRITE_SIZE (this script with
    --copy-calibration-mib copy_mib).  Each counter is scaled by the bytes a
    plain device copy of known size moves per unit of the same counter."""
    import csv

    def mean(run, pick):
        vals = []
        with open(os.path.join(pmc_dir, run, "p_counter_collection.csv")) as fh:
            for r in csv.DictReader(fh):
                if pick(r["Kernel_Name"]):
                    vals.append(float(r["Counter_Value"]))
        if not vals:
            raise SystemExit("no matching dispatch in %s" % run)
        return sum(vals) / len(vals), len(vals)

    fused = lambda k: "fused" in k
    copy = lambda k: "copyBuffer" in k
    fk, n = mean("%s_FETCH_SIZE" % workload, fused)
    wk, _ = mean("%s_WRITE_SIZE" % workload, fused)
    cf, _ = mean("copy_FETCH_SIZE", copy)
    cw, _ = mean("copy_WRITE_SIZE", copy)
    copy_bytes = copy_mib * (1 << 20)
    fs, ws = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    cmd = ("rocprofv3 --pmc %s --output-format csv -d " + pmc_dir + "/%s -o p -- python bench.py ")
    return {
        "workload": workload,
        "commands": [cmd % (c, "%s_%s" % (workload, c)) +
                     "--steps 5 --warmup 2 --no-cpu-baseline --workload " + workload
                     for c in ("FETCH_SIZE", "WRITE_SIZE")] +
                    [cmd % (c, "copy_" + c) + "--copy-calibration-mib %d --steps 3" % copy_mib
                     for c in ("FETCH_SIZE", "WRITE_SIZE")],
        "dispatches": n,
        "fused_fetch_kib_per_dispatch": round(fk, 1),
        "fused_write_kib_per_dispatch": round(wk, 1),
        "copy_bytes": copy_bytes,
        "copy_fetch_kib": round(cf, 1),
        "copy_write_kib": round(cw, 1),
        "fetch_scale": round(fs, 4),
        "write_scale": round(ws, 4),
        "traffic_read_bytes_per_launch": round(fk * 1024 * fs),
        "traffic_write_bytes_per_launch": round(wk * 1024 * ws),
        "traffic_bytes_per_launch": round(fk * 1024 * fs + wk * 1024 * ws),
        "kernel_source_sha256": kernel_source_hash(workload),
    }


def bench_msda(args, torch, synth) -> int:
    """Multi-scale deformable attention sampling: one launch per step."""
    from modulated_deformable_convolution_dcn_amd import MsdaPlan
    spec = synth.MSDA_WORKLOADS[args.msda]
    d = synth.make_msda_inputs(spec)
    if spec.dtype == "f32":
        dev = {k: torch.from_numpy(d[k]).cuda() for k in ("value", "locations", "weights")}
    else:
        dev = {k: torch.from_numpy(d["bits"][k].astype("int16")).cuda().view(torch.bfloat16)
               for k in ("value", "locations", "weights")}
    plan = MsdaPlan(spec.B, spec.Q, spec.G, spec.D, spec.shapes, spec.K, spec.softmax, spec.dtype)
    out = torch.empty((spec.B, spec.Q, spec.G * spec.D), device="cuda")
    for _ in range(args.warmup):
        plan.forward(dev["value"], dev["locations"], dev["weights"], out)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record()
        plan.forward(dev["value"], dev["locations"], dev["weights"], out)
        ev[i][1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ks = [e[0].elapsed_time(e[1]) for e in ev]
    kern_ms = sum(ks) / len(ks)
    ms = elapsed * 1e3 / args.steps
    pairs = spec.B * spec.Q * spec.G
    points = pairs * spec.L * spec.K
    # compulsory bytes: value read once, locations, weights, fp32 output
    e = 2 if spec.dtype == "bf16" else 4
    compulsory = e * (spec.B * spec.S * spec.G * spec.D + points * 2 + points) + 4 * pairs * spec.D
    gathered = points * 4 * spec.D * e  # four corner vectors per point
    hbm = compulsory / (kern_ms * 1e-3) / 1e9
    gather_gbs = gathered / (kern_ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "msda sampling points/s", "value": points / (ms * 1e-3), "unit": "points/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": spec.dtype,
        "data": "synthetic",
        "config": {"workload": spec.name, "B": spec.B, "Q": spec.Q, "G": spec.G, "D": spec.D,
                   "levels": [list(x) for x in spec.shapes], "K": spec.K,
                   "softmax": spec.softmax},
        # the bound is the corner gather through the vector L1: 4 corner
        # vectors per point at the L1's 64 B/clk per CU (256 CUs, 2.4 GHz);
        # the compulsory HBM bytes are reported beside it
        "roofline": {"bound": "l1_gather", "achieved": gather_gbs, "peak": L1_PEAK_GBS,
                     "unit": "GB/s", "frac": gather_gbs / L1_PEAK_GBS, "traffic": None},
        "hbm": {"achieved": hbm, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": hbm / HBM_PEAK_GBS, "compulsory_bytes": compulsory},
        "kernels_us": {"msda": kern_ms * 1e3},
        "fused_us_percentiles": {k: v * 1e3 for k, v in percentiles(ks).items()},
    }), flush=True)
    return 0


def bench_dsample(args, torch, synth) -> int:
    """Single-scale deformable sampling (page 5, DCNv3 form): one launch per step."""
    import numpy as np
    from modulated_deformable_convolution_dcn_amd import DsamplePlan
    spec = synth.DS_WORKLOADS[args.dsample]
    d = synth.make_ds_inputs(spec)
    dev = {k: (torch.from_numpy(d[k]).cuda() if spec.dtype == "f32" else
               torch.from_numpy(d["bits"][k].astype(np.int16)).cuda().view(torch.bfloat16))
           for k in ("x", "offset", "weights")}
    plan = DsamplePlan(spec.B, spec.G, spec.D, spec.H, spec.W, spec.kh, spec.kw, spec.ph,
                       spec.pw, spec.dtype, spec.softmax, args.layout)
    out = torch.empty(plan.out_shape(), device="cuda")
    for _ in range(args.warmup):
        plan.forward(dev["x"], dev["offset"], dev["weights"], out)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record()
        plan.forward(dev["x"], dev["offset"], dev["weights"], out)
        ev[i][1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ks = [e[0].elapsed_time(e[1]) for e in ev]
    kern_ms = sum(ks) / len(ks)
    ms = elapsed * 1e3 / args.steps
    e = 2 if spec.dtype == "bf16" else 4
    P = spec.pixels
    # compulsory: x once, offsets, weights, fp32 output; gathered: 4 corner
    # slices of D channels per (pixel, group, tap)
    compulsory = (spec.B * spec.H * spec.W * spec.C * e + P * spec.G * spec.K * 3 * e +
                  P * spec.C * 4)
    gathered = P * spec.G * spec.K * 4 * spec.D * e
    hbm = compulsory / (kern_ms * 1e-3) / 1e9
    gather_gbs = gathered / (kern_ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "deformable sampling output pixels/s", "value": P / (ms * 1e-3),
        "unit": "px/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": spec.dtype, "data": "synthetic",
        "config": {"workload": spec.name, "B": spec.B, "G": spec.G, "D": spec.D, "H": spec.H,
                   "W": spec.W, "kernel": "%dx%d" % (spec.kh, spec.kw),
                   "pad": [spec.ph, spec.pw], "softmax": spec.softmax,
                   "out_layout": args.layout},
        "roofline": {"bound": "l1_gather", "achieved": gather_gbs, "peak": L1_PEAK_GBS,
                     "unit": "GB/s", "frac": gather_gbs / L1_PEAK_GBS, "traffic": None},
        "hbm": {"achieved": hbm, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": hbm / HBM_PEAK_GBS, "compulsory_bytes": compulsory},
        "kernels_us": {"dsample": kern_ms * 1e3},
        "fused_us_percentiles": {k: v * 1e3 for k, v in percentiles(ks).items()},
    }), flush=True)
    return 0


def percentiles(xs):
    ys = sorted(xs)
    pick = lambda f: ys[min(len(ys) - 1, int(round(f * (len(ys) - 1))))]
    return {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9)}


def cpu_baseline(spec, d, seconds: float):
    """The oracle (as it stands) on evenly spaced output pixels of the workload."""
    import numpy as np
    import oracle
    s = oracle.Shape(spec.B, spec.C, spec.H, spec.W, spec.O, spec.kh, spec.kw, spec.ph, spec.pw)
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = max(1, min(cores, 16))
    P = spec.pixels
    args = (d["x"], d["offset"], d["mask"], d["weight"], d["bias"])
    probe = np.linspace(0, P - 1, num=min(P, 512)).astype(np.int64)
    t = time.perf_counter()
    oracle.forward(s, *args, pixels=probe, nthreads=cores, with_norm=False)
    rate = probe.size / max(time.perf_counter() - t, 1e-6)
    n = int(min(P, max(probe.size, rate * seconds)))
    pix = np.linspace(0, P - 1, num=n).astype(np.int64)
    t = time.perf_counter()
    oracle.forward(s, *args, pixels=pix, nthreads=cores, with_norm=False)
    dt = time.perf_counter() - t
    # the same oracle on one thread, over a short evenly spaced sample
    n1 = int(min(P, max(64, rate / cores * min(seconds, 5.0))))
    pix1 = np.linspace(0, P - 1, num=n1).astype(np.int64)
    t = time.perf_counter()
    oracle.forward(s, *args, pixels=pix1, nthreads=1, with_norm=False)
    dt1 = time.perf_counter() - t
    return {"value": n / dt, "unit": "px/s", "cores": cores, "kind": "oracle",
            "sample": "%d of %d output pixels (evenly spaced, all %d output channels), %.1f s"
                      % (n, P, spec.O, dt),
            "one_thread": {"value": n1 / dt1, "unit": "px/s",
                           "sample": "%d output pixels, %.1f s" % (n1, dt1)}}


def copy_calibration(mib: int, reps: int) -> None:
    """A plain device-to-device copy of known size, for scaling PMC byte counters."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.randn(n, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4,
                      "reps": reps}))


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="birefnet1024_fp32")
    ap.add_argument("--layout", default="nchw", choices=["nchw", "nhwc"],
                    help="output layout")
    ap.add_argument("--input-layout", default="nhwc", choices=["nhwc", "nchw"],
                    help="nchw: x is held NCHW and every step first runs the library's "
                         "NCHW->NHWC transpose (the torchvision-order entry)")
    ap.add_argument("--branches", type=int, default=1,
                    help="run this many branches of the workload (own offsets/mask/weight/"
                         "bias, shared input) per step with one multi-branch call")
    ap.add_argument("--sequential", action="store_true",
                    help="with --branches: one forward call per branch instead")
    ap.add_argument("--backward", action="store_true",
                    help="time the fp32 backward (all five gradients) instead of the forward")
    ap.add_argument("--msda", metavar="WORKLOAD", default=None,
                    help="time multi-scale deformable attention sampling on this workload "
                         "(msda_encoder_fp32, msda_decoder_fp32, msda_encoder_bf16) instead")
    ap.add_argument("--dsample", metavar="WORKLOAD", default=None,
                    help="time single-scale deformable sampling on this workload "
                         "(dcnv3_page5_fp32, dcnv3_map256_fp32, dcnv3_map256_bf16) instead")
    ap.add_argument("--bands", type=int, default=1,
                    help="run the forward as this many output-row bands (row0 calls), "
                         "back to back on one stream")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0)
    ap.add_argument("--cold", action="store_true",
                    help="write a 512 MiB scratch buffer before every timed step "
                         "(inputs no longer cache-resident); not the default")
    ap.add_argument("--summarize-traffic", metavar="PMC_DIR",
                    help="write profiles/fused_kernel_<workload>_traffic.json from "
                         "rocprofv3 --pmc runs under PMC_DIR and exit")
    args = ap.parse_args()

    if args.summarize_traffic:
        rec = summarize_traffic(args.summarize_traffic, args.workload, 256)
        path = os.path.join(ROOT, "profiles", "fused_kernel_%s_traffic.json" % args.workload)
        with open(path, "w") as fh:
            json.dump(rec, fh, indent=1)
        print(json.dumps(rec))
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs the deformable-conv forward on one GPU only; "
              "--gpus %d (WORLD_SIZE %d) is not supported" % (args.gpus, world), file=sys.stderr)
        return 2

    import torch
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib, max(1, args.steps))
        return 0

    from modulated_deformable_convolution_dcn_amd import Desc, Plan, synth
    if args.msda:
        return bench_msda(args, torch, synth)
    if args.dsample:
        return bench_dsample(args, torch, synth)

    spec = synth.WORKLOADS[args.workload]
    d = synth.make_inputs(spec)
    dev = {}
    for k in ("x", "offset", "mask", "weight", "bias"):
        v = d[k]
        if v is None:
            dev[k] = None
        elif spec.dtype == "f32":
            dev[k] = torch.from_numpy(v).cuda()
        else:
            dev[k] = torch.from_numpy(d["bits"][k].astype("int16")).cuda().view(torch.bfloat16)
    plan = Plan(Desc(spec.B, spec.C, spec.H, spec.W, spec.O, spec.kh, spec.kw, spec.ph, spec.pw,
                     spec.dtype, args.layout))
    ws = plan.new_workspace()
    out = plan.new_output()
    from modulated_deformable_convolution_dcn_amd import nchw_to_nhwc
    x_nchw = dev["x"].permute(0, 3, 1, 2).contiguous() if args.input_layout == "nchw" else None
    x_nhwc = torch.empty_like(dev["x"]) if x_nchw is not None else dev["x"]
    nb = max(1, min(args.bands, plan.Ho))
    cuts = [plan.Ho * i // nb for i in range(nb + 1)]
    def band_out(rows):
        shape = ((spec.B, spec.O, rows, plan.Wo) if args.layout == "nchw"
                 else (spec.B, rows, plan.Wo, spec.O))
        return torch.empty(shape, dtype=torch.float32, device="cuda")

    bands = [(r0, dev["offset"][:, :, r0:r1].contiguous(),
              None if dev["mask"] is None else dev["mask"][:, :, r0:r1].contiguous(),
              band_out(r1 - r0))
             for r0, r1 in zip(cuts[:-1], cuts[1:])]

    from modulated_deformable_convolution_dcn_amd import forward_multi
    nbr = max(1, args.branches)
    extra = []  # branches 1.. : own offsets/mask/weight/bias (seeds spec.seed + i), shared x
    for i in range(1, nbr):
        di = synth.make_inputs(spec.scaled(seed=spec.seed + 1000 * i))
        e = {}
        for k in ("offset", "mask", "weight", "bias"):
            v = di[k]
            e[k] = (None if v is None else torch.from_numpy(v).cuda() if spec.dtype == "f32"
                    else torch.from_numpy(di["bits"][k].astype("int16")).cuda().view(torch.bfloat16))
        e["ws"] = plan.new_workspace()
        e["out"] = plan.new_output()
        extra.append(e)

    def step(ev=None):
        # events: [0] start, [1] after transpose + pack, [2] after the fused forward
        if ev is not None:
            ev[0].record()
        if x_nchw is not None:
            nchw_to_nhwc(x_nchw, x_nhwc)
        plan.pack_weight(dev["weight"], ws)
        for e in extra:
            plan.pack_weight(e["weight"], e["ws"])
        if ev is not None:
            ev[1].record()
        if extra and not args.sequential:
            forward_multi([plan] * nbr, x_nhwc, [dev["offset"]] + [e["offset"] for e in extra],
                          [dev["mask"]] + [e["mask"] for e in extra],
                          [ws] + [e["ws"] for e in extra], [dev["bias"]] + [e["bias"] for e in extra],
                          [out] + [e["out"] for e in extra])
        elif extra:
            plan.forward_packed(x_nhwc, dev["offset"], dev["mask"], ws, dev["bias"], out)
            for e in extra:
                plan.forward_packed(x_nhwc, e["offset"], e["mask"], e["ws"], e["bias"], e["out"])
        elif nb == 1:
            plan.forward_packed(x_nhwc, dev["offset"], dev["mask"], ws, dev["bias"], out)
        else:
            for r0, off, msk, bo in bands:
                plan.forward_rows(r0, x_nhwc, off, msk, ws, dev["bias"], bo)
        if ev is not None:
            ev[2].record()

    if args.backward:
        gout = torch.randn(plan.out_shape(), device="cuda")
        bws = torch.empty(plan.backward_workspace_bytes(), dtype=torch.uint8, device="cuda")
        grads = plan.backward(x_nhwc, dev["offset"], dev["mask"], dev["weight"], gout,
                              workspace=bws)

        def step(ev=None):  # noqa: F811 -- the backward step replaces the forward one
            if ev is not None:
                ev[0].record()
                ev[1].record()
            plan.backward(x_nhwc, dev["offset"], dev["mask"], dev["weight"], gout, grads=grads,
                          workspace=bws)
            if ev is not None:
                ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    scratch = torch.empty(512 << 18, device="cuda") if args.cold else None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if scratch is not None:
            scratch.fill_(float(i))
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    pack_list = [e[0].elapsed_time(e[1]) for e in events]
    fused_list = [e[1].elapsed_time(e[2]) for e in events]
    pack_ms = sum(pack_list) / args.steps
    fused_ms = sum(fused_list) / args.steps
    # with --cold the scratch writes sit inside the wall-clock window: the
    # step time then comes from the events alone
    ms_per_step = (sum(e[0].elapsed_time(e[2]) for e in events) / args.steps if args.cold
                   else elapsed * 1e3 / args.steps)
    P = spec.pixels * nbr
    # runs of the split tap sum (1: none) and tap groups per workgroup (the
    # forward runs with the full workspace; multi-branch launches never split)
    one_launch = bool(extra) and not args.sequential
    tap_split = plan.tap_runs if not one_launch and not args.backward else 1
    tap_groups = plan.tap_groups if not one_launch and not args.backward else 1
    # the backward runs two contractions of the forward's size (dL/dsample and dL/dW)
    flops = spec.gemm_flops * nbr * (2 if args.backward else 1)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    # the backward runs fp32 MFMAs for every operand dtype (bf16 operands are
    # widened first)
    peak = MFMA_PEAK_TFLOPS["f32" if args.backward else spec.dtype]
    fused_tflops = flops / (fused_ms * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": P / (ms_per_step * 1e-3),
        "unit": "px/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic",
        "config": {"workload": spec.name, "B": spec.B, "C": spec.C, "O": spec.O, "H": spec.H,
                   "W": spec.W, "kernel": "%dx%d" % (spec.kh, spec.kw),
                   "pad": [spec.ph, spec.pw], "out_layout": args.layout,
                   "input_layout": args.input_layout, "row_bands": nb,
                   "pass": "backward" if args.backward else "forward",
                   "tap_split": tap_split, "tap_groups": tap_groups,
                   "branches": nbr, "branch_launch": ("one per branch" if args.sequential
                                                      else "one for all") if nbr > 1 else None},
        "tflops": tflops,
        "pct_roofline": 100.0 * tflops / peak,
        "roofline": {"bound": "mfma", "achieved": fused_tflops, "peak": peak,
                     "unit": "TFLOP/s", "frac": fused_tflops / peak,
                     # the counter record covers the forward kernel only
                     "traffic": None if args.backward else measured_traffic(spec.name)},
        # "fused" spans the whole forward call: with a tap split, the fused
        # kernel and the reduce that adds the runs
        "kernels_us": {"fused": fused_ms * 1e3,
                       ("transpose+pack" if x_nchw is not None else "pack"): pack_ms * 1e3},
        "fused_us_percentiles": {k: v * 1e3 for k, v in percentiles(fused_list).items()},
        "inputs": "cold (512 MiB written before each step)" if args.cold else "warm (resident)",
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(spec, d, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
