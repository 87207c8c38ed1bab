#!/usr/bin/env python3
"""FusedConv throughput on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-per-config]
                [--no-cpu-baseline] [--only-headline-kernel]

One step = one FusedConv call (every kernel of the planned route) over one
batch of the workload's seeded synthetic inputs, already resident in HBM.
Steps rotate over several input/output sets whose total footprint exceeds
the 256 MB MALL, so a step cannot be served from the last-level cache of
the previous one.  Prints one JSON line.

FLOP = 2 * n * M * OS * K (multiply-add = 2), OS = output pixels per image,
K = (C/group) * taps.  Algorithmic bytes = X + W + B + Z + Y, each once.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from workloads import HEADLINE, WORKLOADS, make_inputs  # noqa: E402

METRIC = "conv TFLOP/s and % MFMA/HBM roofline at 1 GPU per config; oracle max error"
# MI355X published peaks (dense).
PEAK_TFLOPS = {"f16": 2500.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
TAU = {"f16": 2e-2, "f32": 1e-4}
MALL_BYTES = 256 << 20


def log(msg):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def work(wl, y_shape):
    n, M = wl["x"][0], wl["w"][0]
    os_ = int(np.prod(y_shape[2:]))
    K = int(np.prod(wl["w"][1:]))
    flop = 2.0 * n * M * os_ * K
    if wl["attrs"].get("transposed"):
        # every X element times M/group outputs and every tap: 2*|X|*(M/group)*prod(k)
        flop = 2.0 * float(np.prod(wl["x"])) * wl["w"][1] * float(np.prod(wl["w"][2:]))
    esz = 2 if wl["dtype"] == "f16" else 4
    elems = np.prod(wl["x"]) + np.prod(wl["w"]) + np.prod(y_shape)
    if wl["b"]:
        elems += np.prod(wl["b"])
    if wl["z"]:
        elems += np.prod(wl["z"])
    return flop, float(elems * esz)


def bound_of(wl, flop, nbytes):
    peak = PEAK_TFLOPS[wl["dtype"]]
    t_compute = flop / (peak * 1e12)
    t_mem = nbytes / (PEAK_HBM_GBS * 1e9)
    return ("mfma" if t_compute >= t_mem else "hbm"), t_compute, t_mem


# source files each measured kernel is built from
KERNEL_SOURCES = {"halo_kernel": "kernels_halo.hip", "dw_fast_kernel": "kernels_depthwise.hip",
                  "depthwise_kernel": "kernels_depthwise.hip", "igemm_kernel": "kernels_igemm.hip",
                  "direct_kernel": "kernels_direct.hip", "smallc_kernel": "kernels_smallc.hip",
                  "dwm_kernel": "kernels_dwmfma.hip", "pw_kernel": "kernels_pointwise.hip",
                  "im2col_kernel": "kernels_im2col.hip", "halo32_kernel": "kernels_halo32.hip"}


def sources_hash(kernel_pat):
    csrc = os.path.join(ROOT, "convolution_implicit_gemm_amd", "csrc")
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES[kernel_pat], "epilogue.h", "conv_params.h"):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_for(name):
    """HBM bytes per launch from committed rocprofv3 counter runs; None when the
    kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("sources_hash") != sources_hash(rec["kernel_pattern"]):
        return None
    return rec.get("bytes_per_launch")


class Runner:
    def __init__(self, name, seed_sets=None, route=None):
        import torch
        import convolution_implicit_gemm_amd as fc
        self.torch = torch
        self.name = name
        wl = WORKLOADS[name]
        self.wl = wl
        attrs = dict(wl["attrs"])
        if attrs.get("activation_params") is not None:
            attrs["activation_params"] = [float(np.float32(v)) for v in attrs["activation_params"]]
        if route:
            attrs["route"] = route
        self.attrs = attrs
        self.op = fc.FusedConv(wl["x"], wl["w"], wl["dtype"], wl["b"] is not None,
                               wl["z"] is not None, **attrs)
        self.kernel = self.op.handle.kernel_name
        self.flop, self.nbytes = work(wl, self.op.y_shape)
        inp = make_inputs(name)
        self.inp = inp
        foot = self.nbytes
        nsets = seed_sets or max(2, min(8, int(math.ceil(2 * MALL_BYTES / foot)) + 1))
        self.sets = []
        for _ in range(nsets):
            s = {k: (torch.from_numpy(v).cuda() if v is not None else None) for k, v in inp.items()}
            s["y"] = torch.empty(self.op.y_shape, dtype=s["x"].dtype, device="cuda")
            self.sets.append(s)
        self.ws = (torch.empty(self.op.workspace_bytes, dtype=torch.uint8, device="cuda")
                   if self.op.workspace_bytes else None)
        torch.cuda.synchronize()

    def step(self, i, events=None):
        """One full pass: weight preparation (a no-op on the routes without a
        weight layout of their own), then the convolution kernels.  events: a
        (start, stop) pair that the convolution kernels' dispatches record."""
        s = self.sets[i % len(self.sets)]
        self.op.prepare_weights(s["w"], self.ws)
        return self.op(s["x"], s["w"], s["b"], s["z"], out=s["y"], workspace=self.ws,
                       weights_prepared=True, events=events)

    def time(self, steps, warmup):
        """Wall time per step over exactly `steps` steps (synchronized on both
        sides), and within those same steps each step's convolution-kernel
        duration, from events that the kernel dispatches record themselves
        (fusedconv_run_timed: start at the first convolution kernel's begin,
        stop at the last one's end; no marker packet in the stream).  Then,
        outside the timed steps, one event pair around `steps` weight
        preparations."""
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for a, b in evs:  # torch creates an event on its first record
            a.record()
            b.record()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(i, events=evs[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        kern = np.array([a.elapsed_time(b) for a, b in evs]) * 1e-3
        stream = torch.cuda.current_stream()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for i in range(steps):
            self.op.prepare_weights(self.sets[i % len(self.sets)]["w"], self.ws)
        ev[1].record(stream)
        torch.cuda.synchronize()
        self.prep_ms = ev[0].elapsed_time(ev[1]) / steps
        self.kern_all = kern
        return wall / steps, float(kern.mean())

    def max_err(self, n_points=4000):
        from oracle import oracle
        torch = self.torch
        y = self.step(0)
        torch.cuda.synchronize()
        yh = y.cpu().numpy().ravel()
        rng = np.random.default_rng(123)
        if self.attrs.get("transposed"):
            # the transposed oracle on the first image, all its outputs
            kw = {k: v for k, v in self.attrs_oracle().items() if k != "transposed"}
            z0 = self.inp["z"][:1] if self.inp["z"] is not None else None
            ref = oracle.conv_transpose(self.inp["x"][:1], self.inp["w"], self.inp["b"], z0,
                                        **kw).ravel()
            got = yh[:ref.size].astype(np.float64)
            return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))
        idx = rng.integers(0, yh.size, n_points)
        ref = oracle.fusedconv_at(self.inp["x"], self.inp["w"], self.inp["b"], self.inp["z"],
                                  idx=idx, **self.attrs_oracle())
        return float(np.max(np.abs(yh[idx].astype(np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-30))

    def attrs_oracle(self):
        return {k: v for k, v in self.attrs.items() if k not in ("route", "split_k")}

    def summary(self, steps, warmup):
        per_step, k_mean = self.time(steps, warmup)
        bound, t_c, t_m = bound_of(self.wl, self.flop, self.nbytes)
        tflops = self.flop / k_mean / 1e12
        gbs = self.nbytes / k_mean / 1e9
        return dict(workload=self.name, kernel=self.kernel, route=self.op.handle.route,
                    split_k=self.op.handle.split_k, dtype=self.wl["dtype"],
                    wall_ms_per_step=per_step * 1e3, kernel_ms_mean=k_mean * 1e3,
                    kernel_ms_median=float(np.median(self.kern_all)) * 1e3,
                    kernel_ms_min=float(self.kern_all.min()) * 1e3,
                    weight_prep_ms_mean=self.prep_ms,
                    tflops=tflops, gbs=gbs,
                    mfma_frac=tflops / PEAK_TFLOPS[self.wl["dtype"]], hbm_frac=gbs / PEAK_HBM_GBS,
                    bound=bound, bound_frac=max(t_c, t_m) / k_mean, rotating_sets=len(self.sets))

    def free(self):
        self.sets = []
        self.ws = None


def backward_timing(name, steps, warmup):
    """The backward of a workload's convolution, each entry point timed over
    `steps` calls between two events on the stream (so the weight flip and
    the column matrix are inside): the input gradient with the QuickGelu
    derivative of the layer below and a residual gradient, and the weight
    gradient with the bias gradient.  FLOPs as the forward (2 n M P K)."""
    import torch
    import convolution_implicit_gemm_amd as fc
    wl = WORKLOADS[name]
    xs, ws, dt = wl["x"], wl["w"], wl["dtype"]
    attrs = {k: v for k, v in wl["attrs"].items() if k not in ("activation", "activation_params")}
    tdt = torch.float16 if dt == "f16" else torch.float32
    gen = torch.Generator(device="cuda").manual_seed(5)
    rnd = lambda shape, s=1.0: (torch.randn(shape, generator=gen, device="cuda") * s).to(tdt)
    x, w = rnd(xs), rnd(ws, 1.0 / math.sqrt(float(np.prod(ws[1:]))))
    g, pre, r = rnd(wl["y"], 0.1), rnd(xs, 2.0), rnd(xs, 0.1)
    opd = fc.ConvBackwardData(xs, ws, dt, True, "QuickGelu", [1.702], **attrs)
    opw = fc.ConvBackwardWeight(xs, ws, dt, True, **attrs)
    dx = torch.empty(xs, dtype=tdt, device="cuda")
    dw = torch.empty(ws, dtype=torch.float32, device="cuda")
    db = torch.empty([ws[0]], dtype=torch.float32, device="cuda")
    wsd = torch.empty(max(opd.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    wsw = torch.empty(max(opw.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    flop = work(wl, wl["y"])[0]
    esz = 2 if dt == "f16" else 4
    ny, nx, nw = float(np.prod(wl["y"])), float(np.prod(xs)), float(np.prod(ws))
    out = []
    for label, call, nbytes, op in [
            ("backward_data", lambda: opd(g, w, pre, r, out=dx, workspace=wsd),
             (ny + nw + 3 * nx) * esz, opd),
            ("backward_weight", lambda: opw(x, g, dw, db, workspace=wsw),
             (nx + ny) * esz + (nw + ws[0]) * 4, opw)]:
        for _ in range(warmup):
            call()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(steps):
            call()
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / steps
        tf = flop / (ms * 1e-3) / 1e12
        out.append(dict(workload=name, op=label, route=op.handle.route,
                        kernel=op.handle.kernel_name, ms_per_call=ms, tflops=tf,
                        mfma_frac=tf / PEAK_TFLOPS[dt], gbs=nbytes / (ms * 1e-3) / 1e9,
                        workspace_bytes=op.workspace_bytes,
                        time_source="events around the calls on the stream"))
    return out


def cpu_baseline(name, target_s=20.0):
    """The oracle, as it stands, on a bounded sample of the workload's images."""
    from oracle import oracle
    wl = WORKLOADS[name]
    inp = make_inputs(name)
    attrs = dict(wl["attrs"])
    n = wl["x"][0]
    flop_all, _ = work(wl, wl["y"])
    per_img = flop_all / n
    # warm the thread pool, then calibrate on a few images
    oracle.fusedconv(inp["x"], inp["w"], inp["b"], inp["z"], batches=(0, 1), **attrs)
    cal = min(4, n)
    t0 = time.perf_counter()
    oracle.fusedconv(inp["x"], inp["w"], inp["b"], inp["z"], batches=(0, cal), **attrs)
    t1 = (time.perf_counter() - t0) / cal
    k = int(max(1, min(n, target_s / max(t1, 1e-4))))
    t0 = time.perf_counter()
    oracle.fusedconv(inp["x"], inp["w"], inp["b"], inp["z"], batches=(0, k), **attrs)
    dt = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", 0)) or os.cpu_count()
    return dict(value=per_img * k / dt / 1e12, unit="TFLOP/s", cores=cores, kind="oracle",
                sample=f"{k} of {n} images (all {wl['w'][0]} output channels), {dt:.1f} s",
                seconds=dt)


def pmc_summary(name, kernel_pat, fetch_csv, write_csv, copy_bytes):
    """HBM bytes per launch of the kernel matching kernel_pat, from a FETCH_SIZE
    run and a WRITE_SIZE run (rocprofv3 --pmc, csv).  Each counter is scaled by
    the ratio it reads for the plain copy kernel of copy_bytes in the same run."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
        return vals

    out = {}
    for key, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        vals = per_kernel(path, counter)
        copy = [v for k, vs in vals.items() if "copy" in k.lower() for v in vs]
        kern = [v for k, vs in vals.items() if kernel_pat in k for v in vs]
        if not copy or not kern:
            raise SystemExit(f"no copy or no '{kernel_pat}' dispatch with {counter} in {path}")
        scale = copy_bytes / max(copy)  # the largest copy dispatch is the calibration copy
        out[key] = dict(measured=float(np.median(kern)), scale=scale,
                        bytes=float(np.median(kern)) * scale)
    wl = WORKLOADS[name]
    algo = work(wl, wl["y"])[1]
    rec = dict(workload=name, kernel_pattern=kernel_pat, sources_hash=sources_hash(kernel_pat),
               fetch_bytes=out["fetch"]["bytes"], write_bytes=out["write"]["bytes"],
               bytes_per_launch=out["fetch"]["bytes"] + out["write"]["bytes"],
               algorithmic_bytes=algo, fetch_scale=out["fetch"]["scale"],
               write_scale=out["write"]["scale"], copy_bytes=copy_bytes,
               commands=[f"cd /tmp && timeout -s KILL 240 rocprofv3 --pmc {c} --output-format csv "
                         f"-d <out>/pmc_{name}_{c} -o run -- python3 /root/repo/bench.py "
                         f"--workload {name} --steps 3 --warmup 1 --no-per-config "
                         f"--no-cpu-baseline --no-route-comparison --no-backward "
                         f"--calib-copy-mb {copy_bytes >> 20}"
                         for c in ("FETCH_SIZE", "WRITE_SIZE")],
               note="FETCH_SIZE/WRITE_SIZE in KiB per dispatch, median over the kernel's "
                    "dispatches, times the factor that maps the copy kernel's reading to its "
                    "known size")
    return rec


def peaks():
    """Reference rates of this GPU, for reading the roofline fractions: HBM
    bandwidth of a plain 1 GiB device-to-device copy, and the fp16 matrix-core
    rate a tuned library GEMM (torch.matmul, 8192^3) reaches on random U(-1, 1)
    data and on zeros.  Measurement context only: the convolutions never call
    the library."""
    import torch
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e-3

    src = torch.rand(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    t = timed(lambda: dst.copy_(src), 20)
    copy_tbs = 2 * src.numel() * 4 / t / 1e12
    del src, dst
    n = 8192
    out = dict(copy_1gib_tb_s=copy_tbs)
    for tag, make in (("random", lambda: torch.rand(n, n, dtype=torch.float16, device="cuda") * 2 - 1),
                      ("zeros", lambda: torch.zeros(n, n, dtype=torch.float16, device="cuda"))):
        a, b = make(), make()
        c = torch.empty(n, n, dtype=torch.float16, device="cuda")
        t = timed(lambda: torch.matmul(a, b, out=c), 30)
        out[f"gemm_fp16_{tag}_tflops"] = 2 * n ** 3 / t / 1e12
        del a, b, c
    out["published_hbm_tb_s"] = PEAK_HBM_GBS / 1e3
    out["published_fp16_tflops"] = PEAK_TFLOPS["f16"]
    out["device"] = torch.cuda.get_device_properties(0).gcnArchName
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE, choices=list(WORKLOADS))
    ap.add_argument("--no-per-config", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--per-config-steps", type=int, default=20)
    ap.add_argument("--no-route-comparison", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="run a plain device copy of this many MiB first (counter calibration)")
    ap.add_argument("--peaks", action="store_true",
                    help="print this GPU's copy bandwidth and library fp16 GEMM rate and exit")
    ap.add_argument("--pmc-summary", nargs=3, metavar=("KERNEL_PATTERN", "FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_<workload>.json from two counter runs and exit")
    args = ap.parse_args()
    if args.peaks:
        print(json.dumps(peaks()))
        return
    if args.pmc_summary:
        rec = pmc_summary(args.workload, *args.pmc_summary, copy_bytes=args.calib_copy_mb << 20)
        path = os.path.join(ROOT, "profiles", f"traffic_{args.workload}.json")
        json.dump(rec, open(path, "w"), indent=1)
        print(json.dumps(rec))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this FusedConv build runs on one GPU only; "
                          "bench.py measures --gpus 1"}))
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    if args.calib_copy_mb:
        src = torch.ones(args.calib_copy_mb << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log(f"bench: workload {args.workload}, {args.steps} steps, {args.warmup} warmup")
    r = Runner(args.workload)
    s = r.summary(args.steps, args.warmup)
    err = r.max_err()
    wl = r.wl
    bound = "mfma" if s["bound"] == "mfma" else "hbm"
    if bound == "mfma":
        roof = dict(bound="mfma", achieved=s["tflops"], peak=PEAK_TFLOPS[wl["dtype"]],
                    unit="TFLOP/s", frac=s["mfma_frac"])
    else:
        roof = dict(bound="hbm", achieved=s["gbs"], peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=s["hbm_frac"])
    roof["traffic"] = traffic_for(args.workload)
    roof["kernel"] = r.kernel
    roof["kernel_ms_mean"] = s["kernel_ms_mean"]
    roof["kernel_ms_median"] = s["kernel_ms_median"]
    roof["kernel_ms_min"] = s["kernel_ms_min"]
    roof["kernel_time_source"] = ("per timed step, events recorded by the convolution "
                                  "kernel dispatches (fusedconv_run_timed)")
    roof["weight_prep_ms_mean"] = s["weight_prep_ms_mean"]
    r.free()
    del r
    torch.cuda.empty_cache()

    flop = work(wl, wl["y"])[0]
    out = {
        "metric": METRIC,
        "value": flop / (s["wall_ms_per_step"] * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": s["wall_ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl["dtype"],
        "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": {"workload": args.workload, "x": wl["x"], "w": wl["w"], "b": wl["b"],
                   "z": wl["z"], "y": wl["y"], "attrs": wl["attrs"],
                   "route": s["route"], "split_k": s["split_k"]},
        "roofline": roof,
        "max_rel_err": err,
        "tolerance": TAU[wl["dtype"]],
    }
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(args.workload)
    if not args.no_per_config:
        per = []
        for name in WORKLOADS:
            log(f"bench: per-config {name}")
            rr = Runner(name)
            ss = rr.summary(args.per_config_steps, 3)
            ss["max_rel_err"] = rr.max_err(1500)
            rr.free()
            del rr
            torch.cuda.empty_cache()
            per.append(ss)
        out["per_config"] = per
    if not args.no_route_comparison:
        # the other routes of a workload (explicit im2col against the implicit
        # ones; the direct kernel for the fp32 convs), same timing method (the
        # planner's own choice is the per_config line)
        comp = []
        for name, wl_c in WORKLOADS.items():
            for route in wl_c.get("compare_routes", []):
                log(f"bench: route comparison {name} {route}")
                rr = Runner(name, route=route)
                ss = rr.summary(args.per_config_steps, 3)
                ss["max_rel_err"] = rr.max_err(1500)
                ss["workspace_bytes"] = rr.op.workspace_bytes
                rr.free()
                del rr
                torch.cuda.empty_cache()
                comp.append({k: ss[k] for k in ("workload", "route", "kernel", "kernel_ms_mean",
                                                 "kernel_ms_median", "weight_prep_ms_mean",
                                                 "tflops", "gbs", "max_rel_err",
                                                 "workspace_bytes")})
        out["route_comparison"] = comp
    if not args.no_backward:
        log("bench: backward of the headline convolution")
        out["backward"] = backward_timing(HEADLINE, args.per_config_steps, 3)
        torch.cuda.empty_cache()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
