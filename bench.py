#!/usr/bin/env python3
"""ConvTranspose throughput on one MI355X.

Metric: TFLOP/s counted as 2 x useful MACs (the (input sample, tap) pairs whose target
lies inside Y, times N x C/group x M) per second of wall time for whole calls with the
inputs already resident in device memory, plus the roofline fraction of the call's
dominant kernel and the fp64 oracle timed on the host cores as a reference point.

Default workload: the dense fp16 decoder upsampling ConvTranspose
X[8,512,64,64], W[512,256,4,4], bias[256], stride 2, pads 1 -> Y[8,256,128,128] (NCHW),
float32 accumulation.  Other workloads (--workload) print the same JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c4]

One timed step is one convtranspose_nd call (shape resolution, weight re-layout,
the MFMA / bandwidth / direct kernel), enqueued through a prepared plan.  The K steps
are bracketed by torch.cuda.synchronize(); the dominant kernel's device time comes from
HIP events the library records around that kernel on the call's stream.

--pmc-summary DIR turns two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this
script with --calibrate-copy into profiles/<workload>_<kernel>_traffic.json.
"""
from __future__ import annotations

import argparse
import ctypes
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ConvTranspose TFLOP/s (2*useful MACs) and % of MFMA/HBM roofline on 1 MI355X"
PEAK_TFLOPS = {"f16": 2500.0, "f32": 157.3}   # dense MFMA peaks of MI355X
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = {"igemm": ["ct_igemm.hip", "ct_mphase.hip", "ct_tapsplit.hip"], "grouped": ["ct_grouped.hip", "ct_depthwise.hip", "ct_dwcl.hip"],
                  "direct": ["ct_direct.hip"]}
COPY_BYTES = 256 << 20  # calibration copy: 256 MiB read + 256 MiB written
CALIBRATE_COPY = [False]  # --calibrate-copy: one plain copy before the timed steps
FORCE = ["auto", None]     # --kernel, --igemm-tile
OPERANDS = ["random"]      # --operands


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def workloads():
    import workloads as W
    return {"c1": W.C1, "c2": W.C2, "c3": W.C3, "c3_nhwc": W.C3_NHWC, "c4": W.C4, "c4_nhwc": W.C4_NHWC,
            "c5_s1": W.C5_S1, "c5_s1_p1": W.C5_S1_P1, "c5_s2": W.C5_S2,
            "f2_k2s2": W.F2_K2S2, "f2_1x1": W.F2_1X1, "g3_dw": W.G3_DW, "g2_nchw": W.G2_NCHW, "g2_nhwc": W.G2_NHWC,
            # the forward convolution with the same W (the adjoint) of a configuration
            "adj_c5_s1": W.C5_S1, "adj_c4": W.C4,
            # the quantized (QLinear scheme) decoder shapes
            "f4_int8": W.F4_C4, "f4_int8_nchw": W.F4_C4.with_(name="f4_2d_int8_decoder_s2", channels_last=False)}


def source_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES.get(kernel, []):
        path = os.path.join(ROOT, "transposed_convolution_amd", "csrc", name)
        if not os.path.isfile(path):
            return ""
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def traffic_file(wl_key: str, kernel: str) -> str:
    return os.path.join(ROOT, "profiles", f"{wl_key}_{kernel}_traffic.json")


def algorithmic_bytes(wl, y_shape) -> int:
    esz = 2 if wl.dtype == "f16" else 4
    n = math.prod(wl.x_shape) + math.prod(wl.w_shape) + math.prod(y_shape)
    if wl.has_bias:
        n += y_shape[1]
    return n * esz


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, x, w, b, images: int, repeats: int = 3):
    """The fp64 oracle on the first `images` images of the workload (all channels): the
    median of `repeats` runs (one run when a run takes longer than 60 s)."""
    from oracle import oracle as O
    xs = x[:images]
    macs = O.useful_macs(xs.shape, w.shape, **wl.attrs)
    times = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        O.convtranspose(xs, w, b, **wl.attrs)
        times.append(time.perf_counter() - t0)
        if times[-1] > 60.0:
            break
    dt = float(sorted(times)[len(times) // 2])
    return {"value": 2.0 * macs / dt / 1e12, "unit": "TFLOP/s", "cores": O.threads(), "kind": "oracle",
            "cpu_model": cpu_model(), "runs": len(times), "run_s": [round(t, 2) for t in times],
            "sample": f"first {images} of {wl.x_shape[0]} images, every channel and output "
                      f"({macs / 1e9:.2f} GMAC; median of {len(times)} run(s), {dt:.1f} s)"}


class KernelEvents:
    """HIP timing events created without the system-scope fence on record
    (hipEventDisableSystemFence), so the event pair around a kernel costs less than a
    default event pair; the library records them around the dominant kernel of each call."""
    FLAGS = 0x20000000  # hipEventDisableSystemFence

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pairs = [(self._make(), self._make()) for _ in range(n)]

    def _make(self):
        e = ctypes.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.FLAGS)
        if rc != 0:
            raise SystemExit(f"hipEventCreateWithFlags failed ({rc})")
        return e

    def arm(self, lib, i):
        a, c = self.pairs[i]
        lib.convtranspose_profile_events(a, c)

    def milliseconds(self):
        out = []
        for a, c in self.pairs:
            f = ctypes.c_float()
            rc = self.hip.hipEventElapsedTime(ctypes.byref(f), a, c)
            if rc != 0:
                raise SystemExit(f"hipEventElapsedTime failed ({rc})")
            out.append(f.value)
        for a, c in self.pairs:
            self.hip.hipEventDestroy(a)
            self.hip.hipEventDestroy(c)
        return out


def summarize_pmc(args):
    """Per-launch FETCH_SIZE / WRITE_SIZE of the dominant kernel, scaled by the same
    counters' reading for a plain device copy of known size."""
    def rows(pattern):
        out = []
        for f in glob.glob(os.path.join(args.pmc_summary, "**", pattern), recursive=True):
            with open(f) as fh:
                out += list(csv.DictReader(fh))
        return out

    res = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        vals, copy = [], []
        for r in rows("*counter_collection.csv"):
            if r.get("Counter_Name") != counter:
                continue
            name = r.get("Kernel_Name", "")
            v = float(r["Counter_Value"])
            if args.kernel_match in name:
                vals.append(v)
            elif "copybuffer" in name.lower():  # the runtime's device-to-device copy
                copy.append(v)
        if not vals or not copy:
            raise SystemExit(f"no {counter} rows for the kernel or the calibration copy in {args.pmc_summary}")
        # counters are KiB per dispatch; the largest runtime copy is the calibration
        # copy, which moves COPY_BYTES each way
        scale = COPY_BYTES / (max(copy) * 1024.0)
        res[counter] = {"kib_per_launch": sum(vals) / len(vals), "copy_kib": max(copy),
                        "bytes_per_launch": sum(vals) / len(vals) * 1024.0 * scale, "scale": scale}
    out = {"workload": args.workload, "kernel": args.kernel, "source_sha": source_digest(args.kernel),
           "fetch": res["FETCH_SIZE"], "write": res["WRITE_SIZE"],
           "bytes_per_launch": res["FETCH_SIZE"]["bytes_per_launch"] + res["WRITE_SIZE"]["bytes_per_launch"]}
    path = traffic_file(args.workload, args.kernel)
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


def bench_adjoint(args):
    """The forward convolution with a configuration's W, strides, dilations, begin pads and
    end pads e - output_padding: it maps a Y-shaped tensor back to X's shape (the adjoint).
    Useful MACs are the configuration's (the same (input, tap) pairs)."""
    import numpy as np
    import torch

    import transposed_convolution_amd as T
    import workloads as W
    from oracle import oracle as O

    base = workloads()[args.workload]
    if int(base.attrs.get("group", 1)) != 1:
        raise SystemExit("the adjoint bench samples one output channel at a time: group 1 only")
    dev = torch.device("cuda:0")
    _, w, _ = W.make_inputs(base)
    ys, pads = T.convtranspose_output_shape(base.x_shape, base.w_shape, **base.attrs)
    nsp = len(base.x_shape) - 2
    op = base.attrs.get("output_padding") or [0] * nsp
    attrs = dict(strides=base.attrs.get("strides"), dilations=base.attrs.get("dilations"),
                 group=base.attrs.get("group", 1),
                 pads=list(pads[:nsp]) + [pads[nsp + a] - op[a] for a in range(nsp)])
    rng = np.random.default_rng(base.seed + 200)
    a = rng.normal(size=ys).astype(np.float16)
    b = rng.normal(size=base.w_shape[0]).astype(np.float16)
    ta, tw, tb = (torch.from_numpy(v).to(dev) for v in (a, w, b))
    macs = T.convtranspose_useful_macs(base.x_shape, base.w_shape, **base.attrs)
    flops = 2.0 * macs
    # the MFMA path (stride 1 directly, strided through the input phases); a call it
    # cannot serve fails here
    out = T.convolution_nd(ta, tw, tb, kernel="igemm", **attrs)
    torch.cuda.synchronize()
    assert tuple(out.shape) == tuple(base.x_shape)
    lib = T.load_library()
    kernel = "igemm"
    got = out.double().cpu().numpy()
    pts = W.make_points(got.shape, 16, seed=base.seed + 12)
    err = 0.0
    for p in pts:
        n, m = int(p[0]), int(p[1])
        ref = O.conv(a[n:n + 1], w[m:m + 1], b[m:m + 1], **attrs)[(0, 0) + tuple(p[2:])]
        err = max(err, abs(got[tuple(p)] - ref) / (1 + abs(ref)))
    if not err <= 2e-3:
        raise SystemExit(f"adjoint output disagrees with the oracle: max rel err {err:.3e}")
    log(f"adjoint of {base.name}: y{ys} -> x{base.x_shape}, {attrs}, {macs / 1e9:.2f} GMAC, parity {err:.2e}")
    call = T.PreparedCall(T.convolution_nd, ta, tw, tb, out=out, kernel="igemm", **attrs)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    evs = KernelEvents(args.steps)
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs.arm(lib, i)
        call()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    lib.convtranspose_profile_events(None, None)
    k_avg = float(np.mean(evs.milliseconds()))
    peak = PEAK_TFLOPS["f16"]
    achieved = flops / (k_avg * 1e-3) / 1e12
    log(f"{args.steps} steps: {wall * 1e6 / args.steps:.1f} us/step wall, {kernel} kernel {k_avg * 1e3:.1f} us avg, "
        f"{achieved:.1f} TFLOP/s = {achieved / peak * 100:.1f}% of {peak}")
    print(json.dumps({
        "metric": METRIC, "value": round(flops * args.steps / wall / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"adjoint (forward convolution) of {base.name}: X{list(ys)} W{list(base.w_shape)} "
                               f"{attrs} -> Y{list(base.x_shape)}", "kernel": kernel, "useful_macs": macs,
                   "parity_max_rel_err": err},
        "roofline": {"bound": "mfma" if kernel == "igemm" else "alu", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None,
                     "kernel_us": round(k_avg * 1e3, 2)},
        "cpu_baseline": None}), flush=True)


def bench_quant(args):
    """The quantized transposed convolution (QLinear scheme) on the C4 decoder shapes:
    uint8 x, int8 per-channel w, uint8 y, int32 bias.  Checked code for code against the
    oracle on whole planes of the first image and channels before timing."""
    import numpy as np
    import torch

    import transposed_convolution_amd as T
    from oracle import oracle as O

    qw = workloads()[args.workload]
    q = __import__("workloads").make_qinputs(qw)
    dev = torch.device("cuda:0")
    tq = {"uint8": torch.uint8, "int8": torch.int8}
    tx = torch.from_numpy(q["x"]).to(dev)
    if qw.channels_last:
        tx = T.to_channels_last(tx)
    kernel = "igemm"  # forced: a call the kernel cannot serve fails
    tw = torch.from_numpy(q["w"]).to(dev)
    ws = torch.from_numpy(q["w_scale"]).to(dev)
    wz = torch.from_numpy(q["w_zero_point"]).to(dev)
    tb = torch.from_numpy(q["bias"]).to(dev)
    call = dict(x=tx, x_scale=float(q["x_scale"]), x_zero_point=int(q["x_zero_point"]), w=tw, w_scale=ws,
                w_zero_point=wz, y_scale=float(q["y_scale"]), y_zero_point=int(q["y_zero_point"]),
                y_dtype=tq[qw.y_type], bias=tb, channels_last=qw.channels_last, kernel=kernel, **qw.attrs)
    y = T.qlinear_convtranspose_nd(**call)
    torch.cuda.synchronize()
    got = y[:1, :8].contiguous().cpu().numpy().astype(np.int64)
    sub = dict(q, x=q["x"][:1], w=q["w"][:, :8], w_scale=q["w_scale"][:8], w_zero_point=q["w_zero_point"][:8],
               bias=q["bias"][:8])
    ref = O.qconvtranspose(**sub, **qw.attrs)
    if not np.array_equal(got, ref):
        raise SystemExit(f"quantized output disagrees with the oracle in {int((got != ref).sum())} codes")
    macs = T.convtranspose_useful_macs(qw.x_shape, qw.w_shape, **qw.attrs)
    # the oracle timed on the whole first image (every channel)
    cpu = None
    if not args.no_cpu_baseline:
        sub = dict(q, x=q["x"][:1])
        sub_macs = T.convtranspose_useful_macs((1,) + qw.x_shape[1:], qw.w_shape, **qw.attrs)
        t0 = time.perf_counter()
        O.qconvtranspose(**sub, **qw.attrs)
        cpu_dt = time.perf_counter() - t0
        cpu = {"value": round(2.0 * sub_macs / cpu_dt / 1e12, 6), "unit": "TOP/s", "cores": O.threads(),
               "kind": "oracle", "sample": f"image 0 of {qw.x_shape[0]}, every channel ({sub_macs / 1e9:.2f} GMAC, "
                                           f"{cpu_dt:.1f} s)"}
    lib = T.load_library()
    prepared = T.PreparedCall(T.qlinear_convtranspose_nd, **call, out=y)
    for _ in range(args.warmup):
        prepared()
    torch.cuda.synchronize()
    evs = KernelEvents(args.steps)
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs.arm(lib, i)
        prepared()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    lib.convtranspose_profile_events(None, None)
    k_avg = float(np.mean(evs.milliseconds()))
    ops = 2.0 * macs
    achieved = ops / (k_avg * 1e-3) / 1e12
    # int8 MFMA: 5.0 POP/s dense; the gather kernel: the vector ALU, 157.3 Tops/s
    peak = 5000.0 if kernel == "igemm" else 157.3
    log(f"{args.workload}: {macs / 1e9:.2f} GMAC, {args.steps} steps: {wall * 1e6 / args.steps:.1f} us/step wall, "
        f"{kernel} kernel {k_avg * 1e3:.1f} us avg, {achieved:.2f} TOP/s = {achieved / peak * 100:.1f}% of {peak}")
    print(json.dumps({
        "metric": METRIC, "value": round(ops * args.steps / wall / 1e12, 3), "unit": "TOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8/i8 -> i32", "data": "synthetic",
        "config": {"workload": f"{qw.name}: X{list(qw.x_shape)} {qw.x_type} W{list(qw.w_shape)} {qw.w_type} "
                               f"per-channel -> Y {qw.y_type}, {qw.attrs}, channels_last={qw.channels_last}",
                   "kernel": kernel, "useful_macs": macs},
        "roofline": {"bound": "mfma" if kernel == "igemm" else "alu", "achieved": round(achieved, 3), "peak": peak,
                     "unit": "TOP/s",
                     "frac": round(achieved / peak, 5), "traffic": None, "kernel_us": round(k_avg * 1e3, 2)},
        "cpu_baseline": cpu}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c4", choices=sorted(workloads()))
    ap.add_argument("--rotate", type=int, default=0,
                    help="independent (X, Y) buffer sets cycled per step (0: 1 for MFMA-bound, 4 otherwise)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only --workload (the default c4 run also times C4 channels-last, C3 and C5)")
    ap.add_argument("--cpu-images", type=int, default=0, help="images in the oracle sample (0: all)")
    ap.add_argument("--family", default="auto", choices=["auto", "direct", "grouped", "igemm"],
                    help="kernel family to force (default: the dispatcher's choice)")
    ap.add_argument("--igemm-tile", default=None, help="force one block shape of the float16 MFMA family")
    ap.add_argument("--operands", default="random", choices=["random", "zero-x"],
                    help="zero-x: X all zeros, the same work on operands with no bit activity (separates the "
                         "kernel's own limits from the clock the chip sustains under random operands)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain device copy of 256 MiB (counter calibration)")
    ap.add_argument("--pmc-summary", default="", help="rocprofv3 output dir to summarise (no GPU use)")
    ap.add_argument("--kernel", default="igemm", help="with --pmc-summary: kernel family")
    ap.add_argument("--kernel-match", default="igemm_kernel", help="with --pmc-summary: kernel name part")
    args = ap.parse_args()

    if args.pmc_summary:
        return summarize_pmc(args)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this ConvTranspose build has no multi-GPU path; "
              "run it with --gpus 1", flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import transposed_convolution_amd as T
    import workloads as W

    if args.workload.startswith("adj_"):
        return bench_adjoint(args)
    if args.workload.startswith("f4_int8"):
        return bench_quant(args)
    CALIBRATE_COPY[0] = args.calibrate_copy
    OPERANDS[0] = args.operands
    FORCE[0], FORCE[1] = args.family, args.igemm_tile
    if args.igemm_tile:
        T.set_igemm_tile(args.igemm_tile)
    head = time_workload(args.workload, args.steps, args.warmup, args.rotate)
    wl = head.pop("_wl")
    inputs = head.pop("_inputs")
    extras = []
    if args.workload == "c4" and not args.no_extras:
        # the other benchmark configurations, each timed the same way in its own
        # dispatcher-chosen launch configuration (C3 with rotated buffer sets)
        FORCE[0], FORCE[1] = "auto", None
        T.set_igemm_tile(None)
        for key in EXTRA_CONFIGS:
            r = time_workload(key, args.steps, args.warmup, 0)
            r.pop("_wl")
            r.pop("_inputs")
            extras.append({"workload": r["config"]["workload"], "kernel": r["config"]["kernel"],
                           "value": r["value"], "unit": r["unit"], "ms_per_step": r["ms_per_step"],
                           "buffer_sets": r["config"]["buffer_sets"],
                           "parity_max_rel_err": r["config"]["parity_max_rel_err"], "roofline": r["roofline"]})

    base = None
    if not args.no_cpu_baseline:
        x, w, b = inputs
        images = args.cpu_images or wl.x_shape[0]
        log(f"timing the fp64 oracle on {images} image(s), median of 3 ...")
        base = cpu_baseline(wl, x, w, b, images)
        log(f"oracle: {base['value'] * 1e3:.3f} GFLOP/s on {base['cores']} threads ({base['cpu_model']})")
    head["cpu_baseline"] = base
    if extras:
        head["extra_configs"] = extras
    print(json.dumps(head), flush=True)


# Configurations timed after the headline one in the default run.
EXTRA_CONFIGS = ("c4_nhwc", "c3", "c3_nhwc", "c5_s1", "c5_s1_p1", "c5_s2", "g3_dw", "g2_nchw", "g2_nhwc")


def time_workload(key, steps, warmup, rotate_arg):
    """Times one float workload: `steps` whole calls after `warmup`, checked against the
    oracle on 2000 sampled outputs first.  Returns the JSON fields of its line (without
    the CPU baseline) plus the workload and its inputs under private keys."""
    import numpy as np
    import torch

    import transposed_convolution_amd as T
    import workloads as W
    from oracle import oracle as O

    torch.cuda.empty_cache()
    wl = workloads()[key]
    dev = torch.device("cuda:0")
    x, w, b = W.make_inputs(wl)
    if OPERANDS[0] == "zero-x":  # the same work on an input with no bit activity
        x = np.zeros_like(x)
    yshape, _ = T.convtranspose_output_shape(wl.x_shape, wl.w_shape, **wl.attrs)
    macs = T.convtranspose_useful_macs(wl.x_shape, wl.w_shape, **wl.attrs)
    flops = 2.0 * macs

    def to_dev(a):
        t = torch.from_numpy(a).to(dev)
        return T.to_channels_last(t) if wl.channels_last else t

    tx = to_dev(x)
    tw = torch.from_numpy(w).to(dev)
    tb = None if b is None else torch.from_numpy(b).to(dev)
    kernel = T.convtranspose_select_kernel(tx, tw, tb, channels_last=wl.channels_last, **wl.attrs) \
        if FORCE[0] == "auto" else FORCE[0]
    bound = "mfma" if kernel == "igemm" else "hbm"
    rotate = rotate_arg or (1 if bound == "mfma" else 4)
    plans = []
    for r in range(rotate):
        xr = tx if r == 0 else tx.clone()
        plans.append(T.ConvTransposePlan(xr, tw, tb, channels_last=wl.channels_last, kernel=FORCE[0], **wl.attrs))
    log(f"workload {wl.name}: x{wl.x_shape} w{wl.w_shape} -> y{yshape}, kernel {kernel}, "
        f"{macs / 1e9:.2f} GMAC, {rotate} buffer set(s)")

    # correctness gate on the first buffer set: sampled outputs against the oracle
    y = plans[0]()
    torch.cuda.synchronize()
    pts = W.make_points(yshape, 2000, seed=wl.seed + 11)
    ref = O.convtranspose_at(x, w, b, pts, **wl.attrs)
    got = y.double().cpu().numpy()[tuple(pts.T)]
    tol = 2e-3 if wl.dtype == "f16" else 1e-5
    err = float(np.max(np.abs(got - ref) / (1.0 + np.abs(ref))))
    if not err <= tol:
        raise SystemExit(f"bench output disagrees with the oracle: max rel err {err:.3e} > {tol}")
    log(f"parity vs oracle on {len(pts)} sampled outputs: max rel err {err:.2e}")

    if CALIBRATE_COPY[0]:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for i in range(warmup):
        plans[i % rotate]()
    torch.cuda.synchronize()

    lib = T.load_library()
    evs = KernelEvents(steps)  # created outside the timed region
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        evs.arm(lib, i)
        plans[i % rotate]()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    lib.convtranspose_profile_events(None, None)
    kms = np.array(evs.milliseconds())  # milliseconds
    k_avg = float(kms.mean())

    ms_per_step = wall * 1e3 / steps
    value = flops * steps / wall / 1e12
    alg_bytes = algorithmic_bytes(wl, yshape)
    if bound == "mfma":
        achieved = flops / (k_avg * 1e-3) / 1e12
        peak, unit = PEAK_TFLOPS[wl.dtype], "TFLOP/s"
    else:
        achieved = alg_bytes / (k_avg * 1e-3) / 1e9
        peak, unit = PEAK_HBM_GBS, "GB/s"
    traffic = None
    tf = traffic_file(key, kernel)
    if os.path.isfile(tf):
        rec = json.load(open(tf))
        if rec.get("source_sha") == source_digest(kernel):
            traffic = rec["bytes_per_launch"]
    log(f"{wl.name}: {steps} steps: {ms_per_step * 1e3:.1f} us/step wall, {kernel} kernel {k_avg * 1e3:.1f} us avg "
        f"(min {kms.min() * 1e3:.1f}), {achieved:.1f} {unit} = {achieved / peak * 100:.1f}% of {peak} {unit}")

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: X{list(wl.x_shape)} W{list(wl.w_shape)} "
                               f"{'bias ' if wl.has_bias else ''}{wl.attrs} -> Y{list(yshape)} "
                               f"{'channels-last' if wl.channels_last else 'NCHW'}",
                   "kernel": kernel, "igemm_tile": FORCE[1], "useful_macs": macs, "accumulate": "f32",
                   "buffer_sets": rotate, "operands": OPERANDS[0],
                   "parity_max_rel_err": err},
        "roofline": {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel_us": round(k_avg * 1e3, 2), "algorithmic_bytes": alg_bytes},
        "_wl": wl, "_inputs": (x, w, b),
    }
    del plans, y
    return out


if __name__ == "__main__":
    main()
