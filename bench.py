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


def csrc_hash():
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "convolution_implicit_gemm_amd", "csrc", "*"))):
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traffic_for(name, kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs, if still current."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("csrc_hash") != csrc_hash() or rec.get("kernel") != kernel:
        return None
    return rec.get("bytes_per_launch")


class Runner:
    def __init__(self, name, seed_sets=None):
        import torch
        import convolution_implicit_gemm_amd as fc
        self.torch = torch
        self.name = name
        wl = WORKLOADS[name]
        self.wl = wl
        attrs = dict(wl["attrs"])
        if attrs.get("activation_params") is not None:
            attrs["activation_params"] = [float(np.float32(v)) for v in attrs["activation_params"]]
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

    def step(self, i):
        s = self.sets[i % len(self.sets)]
        return self.op(s["x"], s["w"], s["b"], s["z"], out=s["y"], workspace=self.ws)

    def time(self, steps, warmup):
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            ev[i][0].record(stream)
            self.step(i)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        kern = [a.elapsed_time(b) * 1e-3 for a, b in ev]
        return wall / steps, float(np.mean(kern)), float(np.min(kern)), float(np.median(kern))

    def max_err(self, n_points=4000):
        from oracle import oracle
        torch = self.torch
        y = self.step(0)
        torch.cuda.synchronize()
        yh = y.cpu().numpy().ravel()
        rng = np.random.default_rng(123)
        idx = rng.integers(0, yh.size, n_points)
        ref = oracle.fusedconv_at(self.inp["x"], self.inp["w"], self.inp["b"], self.inp["z"],
                                  idx=idx, **self.attrs_oracle())
        return float(np.max(np.abs(yh[idx].astype(np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-30))

    def attrs_oracle(self):
        return {k: v for k, v in self.attrs.items() if k not in ("route", "split_k")}

    def summary(self, steps, warmup):
        per_step, k_mean, k_min, k_med = self.time(steps, warmup)
        bound, t_c, t_m = bound_of(self.wl, self.flop, self.nbytes)
        tflops = self.flop / k_mean / 1e12
        gbs = self.nbytes / k_mean / 1e9
        return dict(workload=self.name, kernel=self.kernel, route=self.op.handle.route,
                    split_k=self.op.handle.split_k, dtype=self.wl["dtype"],
                    wall_ms_per_step=per_step * 1e3, kernel_ms_mean=k_mean * 1e3,
                    kernel_ms_min=k_min * 1e3, kernel_ms_median=k_med * 1e3,
                    tflops=tflops, gbs=gbs,
                    mfma_frac=tflops / PEAK_TFLOPS[self.wl["dtype"]], hbm_frac=gbs / PEAK_HBM_GBS,
                    bound=bound, bound_frac=max(t_c, t_m) / k_mean, rotating_sets=len(self.sets))

    def free(self):
        self.sets = []
        self.ws = None


def cpu_baseline(name, target_s=12.0):
    """The oracle, as it stands, on a bounded sample of the workload's images."""
    from oracle import oracle
    wl = WORKLOADS[name]
    inp = make_inputs(name)
    attrs = dict(wl["attrs"])
    n = wl["x"][0]
    flop_all, _ = work(wl, wl["y"])
    per_img = flop_all / n
    t0 = time.perf_counter()
    oracle.fusedconv(inp["x"], inp["w"], inp["b"], inp["z"], batches=(0, 1), **attrs)
    t1 = time.perf_counter() - t0
    k = int(max(1, min(n - 1, target_s / max(t1, 1e-3))))
    t0 = time.perf_counter()
    oracle.fusedconv(inp["x"], inp["w"], inp["b"], inp["z"], batches=(1, 1 + k), **attrs)
    dt = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", 0)) or os.cpu_count()
    return dict(value=per_img * k / dt / 1e12, unit="TFLOP/s", cores=cores, kind="oracle",
                sample=f"{k} of {n} images (all {wl['w'][0]} output channels), {dt:.1f} s",
                seconds=dt)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE, choices=list(WORKLOADS))
    ap.add_argument("--no-per-config", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--per-config-steps", type=int, default=20)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this FusedConv build runs on one GPU only; "
                          "bench.py measures --gpus 1"}))
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a HIP device"
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
    roof["traffic"] = traffic_for(args.workload, r.kernel)
    roof["kernel"] = r.kernel
    roof["kernel_ms_mean"] = s["kernel_ms_mean"]
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
    print(json.dumps(out))


if __name__ == "__main__":
    main()
