#!/usr/bin/env python3
"""Throughput of the fused KroQuant transform + MXFP4 quantizer on one MI355X.

One step = the fused kernel (kq_transform_quantize_mxfp4) over both FLUX.1-
schnell linear-layer inputs of one denoising step's shape: batch 4 x 4608
tokens = 18432 rows at d = 3072 and at d = 12288 (bf16, synthetic, seeded).
The same inputs are also timed through the SmoothQuant baseline kernel and the
quantize-only kernel, and through the CPU oracle on the host cores.

Algorithmic bytes per element: 2 (bf16 in) + 0.5 (E2M1 codes) + 1/32 (E8M0
scale) = 2.53125. Inputs are rotated over enough buffer sets (>= 512 MB) that
no launch is served from the 256 MB Infinity Cache.

Prints ONE JSON line on stdout (rank 0, N = 1).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

BYTES_PER_ELEM = 2.0 + 0.5 + 1.0 / 32.0
HBM_PEAK_GBPS = 8000.0
ROTATE_BYTES = 512 << 20
WORKLOAD = ("flux_18432x3072", "flux_18432x12288")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fused_flux_18432x12288.json")


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum host time spent on the CPU-oracle baseline (0 disables it)")
    ap.add_argument("--only", choices=["fused", "smoothquant", "quantize"], default=None,
                    help="time only one kernel (for profiler runs)")
    return ap.parse_args()


class Sets:
    """Rotating device buffer sets for one tensor of the workload."""

    def __init__(self, torch, w):
        self.m, self.d = w.m, w.d
        per = w.m * w.d * BYTES_PER_ELEM
        self.n = max(1, int(math.ceil(ROTATE_BYTES / per)))
        A0 = torch.from_numpy(w.A.view(np.int16)).to("cuda").view(torch.bfloat16)
        self.A = [A0] + [A0.clone() for _ in range(self.n - 1)]
        self.codes = [torch.empty((w.m, w.d // 2), dtype=torch.uint8, device="cuda") for _ in range(self.n)]
        self.scales = [torch.empty((w.m, w.d // 32), dtype=torch.uint8, device="cuda") for _ in range(self.n)]
        self.factors = torch.from_numpy(w.factors).cuda()
        self.inv = torch.from_numpy(w.inv_scale).cuda()
        self.i = 0
        self.bytes = w.m * w.d * BYTES_PER_ELEM
        self.elems = w.m * w.d

    def next(self):
        k = self.i % self.n
        self.i += 1
        return self.A[k], self.codes[k], self.scales[k]


def run_kernel(kq, kind, s: Sets, stream):
    A, c, sc = s.next()
    if kind == "fused":
        kq.transform_quantize_mxfp4(A, s.factors, codes=c, scales=sc, stream=stream)
    elif kind == "smoothquant":
        kq.smoothquant_quantize_mxfp4(A, s.inv, codes=c, scales=sc, stream=stream)
    else:
        kq.quantize_mxfp4(A, codes=c, scales=sc, stream=stream)


def time_kernel(torch, kq, kind, sets, steps, warmup):
    """Times `steps` steps (each: the kernel over every tensor of the workload).

    Returns wall ms per step (synchronize on both sides) and per-tensor HIP-event
    launch durations recorded on the launch stream.
    """
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        for s in sets:
            run_kernel(kq, kind, s, stream)
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)] for _ in sets]
    t0 = time.perf_counter()
    for it in range(steps):
        for si, s in enumerate(sets):
            e0, e1 = ev[si][it]
            e0.record(stream)
            run_kernel(kq, kind, s, stream)
            e1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    per = []
    for si in range(len(sets)):
        d = np.array([a.elapsed_time(b) for a, b in ev[si]]) * 1e3  # microseconds
        per.append(d)
    return wall_ms, per


def summarize(d_us, s: Sets):
    med = float(np.median(d_us))
    return {"m": s.m, "d": s.d, "median_us": round(med, 3), "mean_us": round(float(d_us.mean()), 3),
            "p10_us": round(float(np.percentile(d_us, 10)), 3),
            "p90_us": round(float(np.percentile(d_us, 90)), 3),
            "GBps": round(s.bytes / (med * 1e-6) / 1e9, 1),
            "Gelem_per_s": round(s.elems / (med * 1e-6) / 1e9, 2),
            "pct_hbm_peak": round(100.0 * s.bytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBPS, 1)}


def source_digest():
    import glob
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mxfp4_activation_quantizer_amd", "csrc")
    for p in sorted(glob.glob(os.path.join(csrc, "*"))):
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def traffic_for(kernel_bytes):
    """Counter-derived HBM bytes per launch of the dominant kernel, if still current."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("source_digest") != source_digest():
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(ws, seconds):
    """The oracle, as it is, on the same FLUX inputs (fused path), timed on the host."""
    import oracle
    orc = oracle.get()
    threads = oracle.default_threads()
    done_elems, t_used, reps = 0, 0.0, 0
    while t_used < seconds or reps == 0:
        for w in ws:
            t0 = time.perf_counter()
            orc.transform_quantize(w.A, w.factors, want_y=False)
            t_used += time.perf_counter() - t0
            done_elems += w.m * w.d
        reps += 1
    gbps = done_elems * BYTES_PER_ELEM / t_used / 1e9
    return {"value": round(gbps, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "oracle transform+quantize (dense fp64 K, Eq. 12) over the whole FLUX step "
                      "(18432x3072 and 18432x12288), %d pass(es), %.1f s" % (reps, t_used),
            "Gelem_per_s": round(done_elems / t_used / 1e9, 4)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this build measures one GPU only (the quantizer needs no collectives); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    import mxfp4_activation_quantizer_amd as kq
    import synth

    kq.lib()
    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    log("generating inputs " + " ".join(WORKLOAD))
    ws = [synth.workload(n) for n in WORKLOAD]
    sets = [Sets(torch, w) for w in ws]
    log("buffer sets per tensor: %s" % [s.n for s in sets])
    kinds = [args.only] if args.only else ["fused", "smoothquant", "quantize"]
    res = {}
    for kind in kinds:
        log("timing %s: %d warmup + %d steps" % (kind, args.warmup, args.steps))
        wall_ms, per = time_kernel(torch, kq, kind, sets, args.steps, args.warmup)
        res[kind] = {"wall_ms_per_step": wall_ms, "per_tensor": [summarize(d, s) for d, s in zip(per, sets)],
                     "per_tensor_mean_us": [float(d.mean()) for d in per]}
        log("%s: %.4f ms/step; %s" % (kind, wall_ms, res[kind]["per_tensor"]))
    head = res[kinds[0]]
    step_bytes = sum(s.bytes for s in sets)
    step_elems = sum(s.elems for s in sets)
    ms = head["wall_ms_per_step"]
    value = step_bytes / (ms * 1e-3) / 1e9
    # dominant kernel: the d = 12288 launch; achieved = algorithmic bytes / mean event duration
    big = max(range(len(sets)), key=lambda i: sets[i].bytes)
    mean_us = head["per_tensor_mean_us"][big]
    achieved = sets[big].bytes / (mean_us * 1e-6) / 1e9
    traffic = traffic_for(sets[big].bytes)
    out = {
        "metric": "fused KroQuant+MXFP4 quantizer GB/s & Gelem/s, % of HBM peak, vs SmoothQuant",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "flux1-schnell b4x4608 tokens: 18432x3072 + 18432x12288 bf16",
                   "kernel": kinds[0], "m": sets[0].m, "d": [s.d for s in sets],
                   "bytes_per_element": BYTES_PER_ELEM},
        "gelem_per_s": round(step_elems / (ms * 1e-3) / 1e9, 2),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "kernel": "kq::bf16_quant_kernel (%s) on %dx%d" % (kinds[0], sets[big].m, sets[big].d)},
        "kernels": {k: v["per_tensor"] for k, v in res.items()},
    }
    if "fused" in res and "smoothquant" in res:
        out["fused_vs_smoothquant_speedup"] = round(
            res["smoothquant"]["wall_ms_per_step"] / res["fused"]["wall_ms_per_step"], 3)
    if args.cpu_seconds > 0 and not args.only:
        log("CPU oracle baseline (>= %.0f s)" % args.cpu_seconds)
        out["cpu_baseline"] = cpu_baseline(ws, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
