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
# device kernels behind each timed entry point (as rocprofv3 names them)
KERNEL_NAMES = {"fused": "kq::rowwave_kernel<2, 0, 4, 4, false> (fused transform + MXFP4)",
                "smoothquant": "kq::rowwave_kernel<1, 0, 8, 4, false> (SmoothQuant + MXFP4)",
                "quantize": "kq::flat_quantize_kernel (quantize-only)"}
FUSED_KERNEL = "rowwave_kernel<2, 0, 4, 4, false>"


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum host time spent on the CPU-oracle baseline (0 disables it)")
    ap.add_argument("--only", choices=["fused", "smoothquant", "quantize", "hadamard32"], default=None,
                    help="time only one kernel (for profiler runs)")
    ap.add_argument("--eager", action="store_true",
                    help="time steps as eager launches instead of replaying one HIP graph per step")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the other configs, the MFMA form, the fold and the W4A4 GEMM timings")
    ap.add_argument("--tensor", type=int, choices=[3072, 12288], default=None,
                    help="time only the tensor with this d (for profiler runs)")
    ap.add_argument("--gemm-launches", type=int, default=0, metavar="N",
                    help="launch only the packed-scale W4A4 GEMM N times on seeded random MXFP4 operands "
                         "of --gemm-shape (for counter runs), print its event median, and exit")
    ap.add_argument("--gemm-shape", default="18432x3072x3072", help="m x n x k for --gemm-launches")
    ap.add_argument("--gemm-out", choices=("fp32", "bf16"), default="fp32", help="output type for --gemm-launches")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy, 10 times (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=5, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                         "COPY_WRITE_DIR", "OUT_JSON"),
                    help="turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of the fused d=12288 "
                         "launch and of the copy calibration into HBM bytes per launch")
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
        return self.get(k)

    def get(self, k):
        k %= self.n
        return self.A[k], self.codes[k], self.scales[k]


def run_kernel(kq, kind, s: Sets, stream, k=None):
    A, c, sc = s.next() if k is None else s.get(k)
    if kind == "fused":
        kq.transform_quantize_mxfp4(A, s.factors, codes=c, scales=sc, stream=stream)
    elif kind.startswith("fused_"):
        kq.transform_quantize_mxfp4(A, s.factors, codes=c, scales=sc, stream=stream, form=kind[len("fused_"):])
    elif kind == "smoothquant":
        kq.smoothquant_quantize_mxfp4(A, s.inv, codes=c, scales=sc, stream=stream)
    elif kind == "hadamard32":
        kq.hadamard_quantize_mxfp4(A, 32, codes=c, scales=sc, stream=stream)
    elif kind == "fwht":
        kq.hadamard_quantize_mxfp4(A, s.d, codes=c, scales=sc, stream=stream)
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


class StepGraphs:
    """One captured HIP graph per rotation index r: the step's launches (one per
    tensor of the workload) on buffer set r, replayed in turn so the rotation
    past the Infinity Cache is kept."""

    def __init__(self, torch, kq, kind, sets):
        self.torch = torch
        nrot = 1
        for s in sets:
            nrot = nrot * s.n // math.gcd(nrot, s.n)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # one eager pass on the capture stream first
            for r in range(nrot):
                for s in sets:
                    run_kernel(kq, kind, s, side, k=r)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.graphs = []
        for r in range(nrot):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for s in sets:
                    run_kernel(kq, kind, s, torch.cuda.current_stream(), k=r)
            self.graphs.append(g)
        self.i = 0

    def replay(self, n):
        for _ in range(n):
            self.graphs[self.i % len(self.graphs)].replay()
            self.i += 1

    def time(self, steps, warmup):
        """W untimed replays, then exactly `steps` timed ones bracketed by
        synchronize; returns ms per step."""
        self.replay(warmup)
        self.torch.cuda.synchronize()
        t0 = time.perf_counter()
        self.replay(steps)
        self.torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps


def time_step_graphs(torch, kq, kind, sets, steps, warmup):
    """Wall time per step with each step replayed as one captured HIP graph."""
    return StepGraphs(torch, kq, kind, sets).time(steps, warmup)


def _events_us(torch, fn, reps, warmup):
    """Per-call durations (microseconds) of fn() by HIP events on the current stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ev]) * 1e3


def extras(torch, kq, synth, flux_sets, reps=100, warmup=20):
    """Context measurements kept beside the headline step (same rotation rules):
    the PixArt-shaped inputs, the paper's power-of-two kernel-table shapes with
    the Hadamard baselines, the MFMA form of the transform on the FLUX inputs,
    the weight fold and fp32 quantizer on 3072 x 3072 weights, and the W4A4 GEMM."""
    out = {"other_configs": {}}
    out["kernel_table_pow2"] = kernel_table(torch, kq, synth, reps, warmup)
    out["production_shapes_table4"] = production_table(torch, kq, synth, reps, warmup)
    out["m_sweep_d4096_fig4"] = m_sweep(torch, kq, synth, reps, warmup)
    for name in ("pixart_attn_4096x1152", "pixart_ffn_8192x4608"):
        w = synth.workload(name)
        s = Sets(torch, w)
        per = {}
        for kind in ("fused", "smoothquant", "quantize"):
            _, d = time_kernel(torch, kq, kind, [s], reps, warmup)
            per[kind] = summarize(d[0], s)
        out["other_configs"][name] = per
        log("%s: %s" % (name, per))
        del s
    for form in ("mfma", "mfma_lds"):
        _, d = time_kernel(torch, kq, "fused_" + form, flux_sets, reps, warmup)
        out["fused_%s_form" % form] = [summarize(x, s) for x, s in zip(d, flux_sets)]
        log("%s form: %s" % (form, out["fused_%s_form" % form]))
    # weight side: fold and fp32 quantize of a 3072 x 3072 fp32 weight
    W = torch.from_numpy(synth.weights(3072, 3072, 1004)).cuda()
    fac = flux_sets[0].factors
    Wf = torch.empty_like(W)
    d_fold = _events_us(torch, lambda: kq.inverse_fold_weights(W, fac, out=Wf), reps, warmup)
    cw, sw = kq.quantize_mxfp4_f32(Wf)
    d_q32 = _events_us(torch, lambda: kq.quantize_mxfp4_f32(Wf, codes=cw, scales=sw), reps, warmup)
    nW = W.numel()
    fold_b, q32_b = nW * 8.0, nW * (4 + 0.5 + 1 / 32)
    out["weight_fold_3072x3072"] = {
        "median_us": round(float(np.median(d_fold)), 3),
        "GBps": round(fold_b / (np.median(d_fold) * 1e-6) / 1e9, 1),
        "quantize_f32_median_us": round(float(np.median(d_q32)), 3),
        "quantize_f32_GBps": round(q32_b / (np.median(d_q32) * 1e-6) / 1e9, 1),
        "note": "small (37.7 MB) and L2/Infinity-Cache resident across repeats; offline step"}
    # W4A4 GEMM on the FLUX 18432 x 3072 activations and the folded weights
    A, ca, sa = flux_sets[0].get(0)
    kq.transform_quantize_mxfp4(A, fac, codes=ca, scales=sa)
    O = torch.empty((A.shape[0], 3072), dtype=torch.float32, device="cuda")
    d_g = _events_us(torch, lambda: kq.mxfp4_gemm(ca, sa, cw, sw, out=O), 20, 3)
    flops = 2.0 * A.shape[0] * 3072 * 3072
    med = float(np.median(d_g))
    out["w4a4_gemm_18432x3072x3072"] = {"median_us": round(med, 1),
                                         "TFLOPs": round(flops / (med * 1e-6) / 1e12, 1),
                                         "pct_fp4_peak": round(100 * flops / (med * 1e-6) / 10.1e15, 2)}
    # the packed-scale kernel (256 x 256 tiles, 32 x 32 x 64 instruction): W's scales are
    # packed once (offline, like the fold), A's on every call
    psa = kq.pack_mxfp4_scales(sa)
    psw = kq.pack_mxfp4_scales(sw)
    d_pk = _events_us(torch, lambda: kq.pack_mxfp4_scales(sa, out=psa), 20, 3)
    d_gp = _events_us(torch, lambda: kq.mxfp4_gemm_packed(ca, psa, cw, psw, out=O), 20, 3)
    Ob = torch.empty((A.shape[0], 3072), dtype=torch.bfloat16, device="cuda")
    d_gb = _events_us(torch, lambda: kq.mxfp4_gemm_packed(ca, psa, cw, psw, out=Ob, bf16=True), 20, 3)
    med_pk, med_gp, med_gb = float(np.median(d_pk)), float(np.median(d_gp)), float(np.median(d_gb))
    out["w4a4_gemm_18432x3072x3072"].update({
        "packed_median_us": round(med_gp, 1), "packed_TFLOPs": round(flops / (med_gp * 1e-6) / 1e12, 1),
        "packed_pct_fp4_peak": round(100 * flops / (med_gp * 1e-6) / 10.1e15, 2),
        "pack_a_scales_us": round(med_pk, 2),
        "packed_bf16_out_median_us": round(med_gb, 1),
        "packed_bf16_out_pct_fp4_peak": round(100 * flops / (med_gb * 1e-6) / 10.1e15, 2)})
    log("weight side / gemm: %s %s" % (out["weight_fold_3072x3072"], out["w4a4_gemm_18432x3072x3072"]))
    # the same product on the 128 x 512-tile kernel, and the layer with the transform and
    # quantizer in the product's prologue against the two launches it replaces
    d_w = _events_us(torch, lambda: kq.mxfp4_gemm_wide(ca, sa, cw, sw, out=O), 20, 3)
    d_f = _events_us(torch, lambda: kq.transform_quantize_mxfp4_gemm(A, fac, cw, sw, out=O), 20, 3)
    d_q = _events_us(torch, lambda: kq.transform_quantize_mxfp4(A, fac, codes=ca, scales=sa), 20, 3)
    med_w, med_f, med_q = (float(np.median(x)) for x in (d_w, d_f, d_q))
    out["w4a4_layer_fused_18432x3072x3072"] = {
        "wide_gemm_us": round(med_w, 1), "wide_gemm_TFLOPs": round(flops / (med_w * 1e-6) / 1e12, 1),
        "wide_gemm_pct_fp4_peak": round(100 * flops / (med_w * 1e-6) / 10.1e15, 2),
        "fused_layer_us": round(med_f, 1), "fused_layer_TFLOPs": round(flops / (med_f * 1e-6) / 1e12, 1),
        "quantizer_us": round(med_q, 1),
        "pipeline_us": round(med_q + min(med, med_w), 1),
        "pipeline_packed_us": round(med_q + med_pk + med_gp, 1)}
    # the same three launches enqueued back to back and timed as one region (the sum
    # above counts each launch's event overhead)
    def pipeline_packed():
        kq.transform_quantize_mxfp4(A, fac, codes=ca, scales=sa)
        kq.pack_mxfp4_scales(sa, out=psa)
        kq.mxfp4_gemm_packed(ca, psa, cw, psw, out=O)
    out["w4a4_layer_fused_18432x3072x3072"]["pipeline_packed_region_us"] = round(
        float(np.median(_events_us(torch, pipeline_packed, 20, 3))), 1)
    # the quantizer writing the packed scale layout itself: two launches
    pq = psa
    def pipeline_packed_quantizer():
        kq.transform_quantize_mxfp4_packed(A, fac, codes=ca, packed_scales=pq)
        kq.mxfp4_gemm_packed(ca, pq, cw, psw, out=O)
    out["w4a4_layer_fused_18432x3072x3072"]["quantizer_packed_scales_us"] = round(float(np.median(
        _events_us(torch, lambda: kq.transform_quantize_mxfp4_packed(A, fac, codes=ca, packed_scales=pq), 20, 3))), 1)
    out["w4a4_layer_fused_18432x3072x3072"]["pipeline_packed_quantizer_region_us"] = round(
        float(np.median(_events_us(torch, pipeline_packed_quantizer, 20, 3))), 1)
    log("fused layer: %s" % out["w4a4_layer_fused_18432x3072x3072"])
    out["w4a4_layer_lowrank_18432x3072x3072_r128"] = lowrank_layer_timing(torch, kq, A, fac, cw, sw, W)
    log("low-rank layer: %s" % out["w4a4_layer_lowrank_18432x3072x3072_r128"])
    out["calibration_4096x3072x3072"] = calibration_timing(torch, kq, synth, A, W)
    log("calibration: %s" % out["calibration_4096x3072x3072"])
    return out


def lowrank_layer_timing(torch, kq, A, fac, cw, sw, W, r=128, reps=20):
    """Eq. 11 at inference on the FLUX 18432x3072 input with 3072x3072 weights and a
    rank-128 branch (random L, R; timing only): fused quantizer with the bf16 output,
    projection Z = X16 Q(R)^T, GEMM with the low-rank epilogue; against the plain
    quantizer + W4A4 GEMM."""
    g = torch.Generator(device="cuda").manual_seed(7)
    L = torch.randn((W.shape[0], r), device="cuda", generator=g) / r ** 0.5
    R = torch.randn((r, W.shape[1]), device="cuda", generator=g) / W.shape[1] ** 0.5
    cr, sr = kq.quantize_mxfp4_f32(R)
    cl, sl = kq.quantize_mxfp4_f32(L)
    ca, sa, y16 = kq.transform_quantize_mxfp4_y16(A, fac)
    Z = kq.lowrank_project(y16, cr, sr)
    O = kq.mxfp4_gemm_lowrank(ca, sa, cw, sw, Z, cl, sl)
    med = lambda f: round(float(np.median(_events_us(torch, f, reps, 3))), 1)
    res = {"quantize_y16_us": med(lambda: kq.transform_quantize_mxfp4_y16(A, fac, codes=ca, scales=sa, y16=y16)),
           "project_us": med(lambda: kq.lowrank_project(y16, cr, sr, out=Z)),
           "gemm_lowrank_us": med(lambda: kq.mxfp4_gemm_lowrank(ca, sa, cw, sw, Z, cl, sl, out=O)),
           "quantize_us": med(lambda: kq.transform_quantize_mxfp4(A, fac, codes=ca, scales=sa)),
           "gemm_us": med(lambda: kq.mxfp4_gemm(ca, sa, cw, sw, out=O))}
    # the low-rank epilogue on the packed-scale GEMM (W's scales packed offline, A's per call)
    psa, psw = kq.pack_mxfp4_scales(sa), kq.pack_mxfp4_scales(sw)
    res["gemm_lowrank_packed_us"] = med(lambda: kq.mxfp4_gemm_packed_lowrank(ca, psa, cw, psw, Z, cl, sl, out=O))
    res["pack_a_scales_us"] = med(lambda: kq.pack_mxfp4_scales(sa, out=psa))
    # R decoded to bf16 once per call, then the projection without in-kernel decoding
    r16 = kq.dequantize_mxfp4_bf16(cr, sr)
    res["decode_r_us"] = med(lambda: kq.dequantize_mxfp4_bf16(cr, sr, out=r16))
    res["project_bf16_us"] = med(lambda: kq.lowrank_project_bf16(y16, r16, out=Z))
    res["layer_with_branch_us"] = round(res["quantize_y16_us"] + res["project_us"] + res["gemm_lowrank_us"], 1)
    res["layer_with_branch_r16_us"] = round(res["quantize_y16_us"] + res["decode_r_us"] + res["project_bf16_us"] +
                                            res["gemm_lowrank_us"], 1)
    res["layer_with_branch_packed_us"] = round(res["quantize_y16_us"] + res["decode_r_us"] + res["project_bf16_us"] +
                                               res["pack_a_scales_us"] + res["gemm_lowrank_packed_us"], 1)
    res["layer_plain_us"] = round(res["quantize_us"] + res["gemm_us"], 1)

    # the fast route's five launches back to back, timed as one region
    def layer_packed():
        kq.transform_quantize_mxfp4_y16(A, fac, codes=ca, scales=sa, y16=y16)
        kq.dequantize_mxfp4_bf16(cr, sr, out=r16)
        kq.lowrank_project_bf16(y16, r16, out=Z)
        kq.pack_mxfp4_scales(sa, out=psa)
        kq.mxfp4_gemm_packed_lowrank(ca, psa, cw, psw, Z, cl, sl, out=O)
    res["layer_with_branch_packed_region_us"] = med(layer_packed)

    # the same with the quantizer writing the packed scales itself (four launches)
    def layer_packed_quantizer():
        kq.transform_quantize_mxfp4_packed(A, fac, codes=ca, packed_scales=psa, y16=y16)
        kq.dequantize_mxfp4_bf16(cr, sr, out=r16)
        kq.lowrank_project_bf16(y16, r16, out=Z)
        kq.mxfp4_gemm_packed_lowrank(ca, psa, cw, psw, Z, cl, sl, out=O)
    res["layer_with_branch_packed_quantizer_region_us"] = med(layer_packed_quantizer)

    # the branch's operands prepared outside the product: the projection writes Z's bf16
    # split, L is decoded to bf16 (both decodes per call, as R's above), and the packed
    # GEMM moves them straight into LDS (bit-identical to the fp32-Z form)
    Zh, Zl = kq.lowrank_project_bf16_split(y16, r16)
    l16 = kq.dequantize_mxfp4_bf16(cl, sl)
    res["project_bf16_split_us"] = med(lambda: kq.lowrank_project_bf16_split(y16, r16, Zh=Zh, Zl=Zl))
    res["decode_l_us"] = med(lambda: kq.dequantize_mxfp4_bf16(cl, sl, out=l16))
    res["gemm_lowrank_split_us"] = med(lambda: kq.mxfp4_gemm_packed_lowrank_split(ca, psa, cw, psw, Zh, Zl, l16,
                                                                                  out=O))

    def layer_split():
        kq.transform_quantize_mxfp4_packed(A, fac, codes=ca, packed_scales=psa, y16=y16)
        kq.dequantize_mxfp4_bf16(cr, sr, out=r16)
        kq.lowrank_project_bf16_split(y16, r16, Zh=Zh, Zl=Zl)
        kq.dequantize_mxfp4_bf16(cl, sl, out=l16)
        kq.mxfp4_gemm_packed_lowrank_split(ca, psa, cw, psw, Zh, Zl, l16, out=O)
    res["layer_with_branch_split_region_us"] = med(layer_split)

    # the same with R and L decoded once per weight (as W's scales are packed once):
    # three launches per call
    def layer_split_prepared():
        kq.transform_quantize_mxfp4_packed(A, fac, codes=ca, packed_scales=psa, y16=y16)
        kq.lowrank_project_bf16_split(y16, r16, Zh=Zh, Zl=Zl)
        kq.mxfp4_gemm_packed_lowrank_split(ca, psa, cw, psw, Zh, Zl, l16, out=O)
    res["layer_with_branch_split_prepared_region_us"] = med(layer_split_prepared)

    # R kept in MXFP4 (the projection's producers decode it) and L decoded once per weight
    res["project_split_mx_r_us"] = med(lambda: kq.lowrank_project_split(y16, cr, sr, Zh=Zh, Zl=Zl))

    def layer_mx_r():
        kq.transform_quantize_mxfp4_packed(A, fac, codes=ca, packed_scales=psa, y16=y16)
        kq.lowrank_project_split(y16, cr, sr, Zh=Zh, Zl=Zl)
        kq.mxfp4_gemm_packed_lowrank_split(ca, psa, cw, psw, Zh, Zl, l16, out=O)
    res["layer_with_branch_mx_r_region_us"] = med(layer_mx_r)
    return res


def calibration_timing(torch, kq, synth, A, W, steps=20):
    """Layer-wise calibration (Sec. 3.3) on 4096 FLUX rows with the 3072 x 3072 weights:
    GPU time per Adam step (three M x d x o GEMMs and the per-block chain), the fp32
    GEMM alone, and one step of the float64 oracle on the host for scale."""
    M = 4096
    A4 = A[:M].contiguous()
    cal = kq.Calibration(A4, W)
    cal.step(lr=1e-2)  # sets lambda
    d_step = _events_us(torch, lambda: cal.step(lr=1e-2), steps, 2)
    Af = A4.float()
    Cg = torch.empty((M, W.shape[0]), dtype=torch.float32, device="cuda")
    d_gemm = _events_us(torch, lambda: kq.gemm_f32(Af, W, transb=True, out=Cg), 10, 2)
    flops = 2.0 * M * W.shape[0] * W.shape[1]
    res = {"gpu_ms_per_step": round(float(np.median(d_step)) / 1e3, 3),
           "gemm_f32_4096x3072x3072_us": round(float(np.median(d_gemm)), 1),
           "gemm_f32_TFLOPs": round(flops / (np.median(d_gemm) * 1e-6) / 1e12, 1),
           "gemm_f32_frac_of_fp32_peak": round(flops / (np.median(d_gemm) * 1e-6) / 157.3e12, 3),
           "losses_after": [round(float(x), 5) for x in cal.losses.cpu().numpy()]}
    try:
        from oracle import calib as ocalib
        P = ocalib.Problem(synth.bf16_bits_to_f32(A4.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64),
                           W.cpu().numpy().astype(np.float64))
        th = ocalib.hadamard_theta(W.shape[1] // 32)
        t0 = time.perf_counter()
        P.gradient(th, 1.0, 1.0)
        res["oracle_s_per_step"] = round(time.perf_counter() - t0, 2)
    except Exception as e:  # the oracle is a reported baseline only
        res["oracle_s_per_step"] = "unavailable: %s" % e
    return res


def kernel_table(torch, kq, synth, reps, warmup):
    """The kernel-latency comparison of the paper (Sec. 4.4, Table 3) on this GPU:
    quantize-only (Q4), SmoothQuant (Scale), the fused Kronecker kernel (K2),
    block Hadamard-32 and the full-width Walsh-Hadamard transform (FWHT), each
    fused with the MXFP4 quantizer, at the table's power-of-two shapes."""
    names = ("pow2_4096x1024", "pow2_4096x4096", "pow2_4096x16384", "pow2_512x4096", "pow2_512x16384")
    return shape_table(torch, kq, synth, names, ("quantize", "smoothquant", "fused", "hadamard32", "fwht"), reps,
                       warmup)


def shape_table(torch, kq, synth, names, kinds, reps, warmup, m_override=None):
    """Per-shape medians of each kind (same rotation rules), plus SmoothQuant over
    fused and FWHT over fused where both were timed."""
    table = {}
    for name in names:
        w = synth.workload(name, m=m_override)
        s = Sets(torch, w)
        per = {}
        for kind in kinds:
            if kind == "fwht" and (w.d & (w.d - 1)) != 0:
                continue
            _, d = time_kernel(torch, kq, kind, [s], reps, warmup)
            per[kind] = summarize(d[0], s)
        if "smoothquant" in per and "fused" in per:
            per["scale_over_fused"] = round(per["smoothquant"]["median_us"] / per["fused"]["median_us"], 3)
        if "fwht" in per and "fused" in per:
            per["fwht_over_fused"] = round(per["fwht"]["median_us"] / per["fused"]["median_us"], 3)
        key = name if m_override is None else "m%d_d%d" % (w.m, w.d)
        table[key] = per
        log("%s: %s" % (key, {k: (v["median_us"] if isinstance(v, dict) else v) for k, v in per.items()}))
        del s
    return table


def production_table(torch, kq, synth, reps, warmup):
    """The paper's production-shape latency table (Appendix A, Table 4) on this GPU:
    quantize-only (Q4), SmoothQuant (Scale) and the fused Kronecker kernel at the
    FLUX.1 / PixArt-Sigma linear-layer shapes it lists."""
    names = ("prod_512x3072", "prod_512x12288", "pixart_attn_4096x1152", "prod_4096x3072", "prod_4096x3456",
             "pow2_4096x4096", "prod_4096x4608", "prod_4096x12288")
    return shape_table(torch, kq, synth, names, ("quantize", "smoothquant", "fused"), reps, warmup)


def m_sweep(torch, kq, synth, reps, warmup):
    """Latency against the token count m at d = 4096 (the paper's Sec. 4.4, Fig. 4):
    m = 2^7 .. 2^14, quantize-only, SmoothQuant, fused and the full-width FWHT."""
    out = {}
    for lg in range(7, 15):
        out.update(shape_table(torch, kq, synth, ("pow2_4096x4096",), ("quantize", "smoothquant", "fused", "fwht"),
                               reps, warmup, m_override=1 << lg))
    return out


def summarize(d_us, s: Sets):
    med = float(np.median(d_us))
    return {"m": s.m, "d": s.d, "median_us": round(med, 3), "mean_us": round(float(d_us.mean()), 3),
            "p10_us": round(float(np.percentile(d_us, 10)), 3),
            "p90_us": round(float(np.percentile(d_us, 90)), 3),
            "GBps": round(s.bytes / (med * 1e-6) / 1e9, 1),
            "Gelem_per_s": round(s.elems / (med * 1e-6) / 1e9, 2),
            "pct_hbm_peak": round(100.0 * s.bytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBPS, 1)}


def source_digest():
    """Hash of the sources the dominant (fused) kernel is built from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mxfp4_activation_quantizer_amd", "csrc")
    for f in ("kq_kernels.hip", "kq_device.hpp"):
        h.update(open(os.path.join(csrc, f), "rb").read())
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
    # the other two oracle paths on the same step, once each (context beside the fused rate)
    others = {}
    for name, fn in (("quantize_only", lambda w: orc.quantize_bf16(w.A)),
                     ("smoothquant", lambda w: orc.smoothquant_quantize(w.A, w.inv_scale))):
        t0 = time.perf_counter()
        n = 0
        for w in ws:
            fn(w)
            n += w.m * w.d
        others[name + "_Gelem_per_s"] = round(n / (time.perf_counter() - t0) / 1e9, 4)
    return {"value": round(gbps, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "oracle transform+quantize (dense fp64 K, Eq. 12) over the whole FLUX step "
                      "(18432x3072 and 18432x12288), %d pass(es), %.1f s" % (reps, t_used),
            "Gelem_per_s": round(done_elems / t_used / 1e9, 4), **others}


COPY_BYTES = 1 << 30
COPY_KERNEL = "neg"


def copy_calibration():
    """A plain streaming kernel of known traffic: y = -x over 1 GiB of fp32, i.e.
    1 GiB read + 1 GiB written per call (torch's elementwise negation kernel)."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(10):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES, "calls": 10}))


def _pmc_rows(d, counter):
    """(kernel name, grid size, value) per dispatch from a rocprofv3 --pmc csv directory."""
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") != counter:
                    continue
                rows.append((r.get("Kernel_Name", ""), int(float(r.get("Grid_Size", 0) or 0)),
                             float(r["Counter_Value"])))
    return rows


def summarize_pmc(fetch_dir, write_dir, cfetch_dir, cwrite_dir, out_json):
    """Counter-derived HBM traffic of the fused 18432x12288 launch.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what the same
    counters read for the 1 GiB copy calibration (known bytes / counted bytes).
    """
    def largest_kernel(rows, name_part):
        sel = [r for r in rows if name_part in r[0]]
        grid = max(r[1] for r in sel)
        vals = [r[2] for r in sel if r[1] == grid]
        return sum(vals) / len(vals), len(vals), sel[0][0], grid
    f_fused, n_f, kname, grid = largest_kernel(_pmc_rows(fetch_dir, "FETCH_SIZE"), FUSED_KERNEL)
    w_fused, n_w, _, _ = largest_kernel(_pmc_rows(write_dir, "WRITE_SIZE"), FUSED_KERNEL)
    f_copy, n_cf, cname, _ = largest_kernel(_pmc_rows(cfetch_dir, "FETCH_SIZE"), COPY_KERNEL)
    w_copy, n_cw, _, _ = largest_kernel(_pmc_rows(cwrite_dir, "WRITE_SIZE"), COPY_KERNEL)
    kf = COPY_BYTES / (f_copy * 1024.0)
    kw = COPY_BYTES / (w_copy * 1024.0)
    fetch_b = f_fused * 1024.0 * kf
    write_b = w_fused * 1024.0 * kw
    alg = 18432 * 12288 * BYTES_PER_ELEM
    out = {"kernel": kname, "grid_size": grid, "dispatches": [n_f, n_w],
           "fetch_kib_per_launch": round(f_fused, 1), "write_kib_per_launch": round(w_fused, 1),
           "copy_kernel": cname, "copy_fetch_kib": round(f_copy, 1), "copy_write_kib": round(w_copy, 1),
           "scale_fetch": round(kf, 4), "scale_write": round(kw, 4),
           "fetch_bytes": round(fetch_b), "write_bytes": round(write_b),
           "bytes_per_launch": round(fetch_b + write_b),
           "algorithmic_bytes_per_launch": round(alg),
           "traffic_over_algorithmic": round((fetch_b + write_b) / alg, 4),
           "source_digest": source_digest()}
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def gemm_launches(n, shape, out="fp32"):
    """The packed-scale W4A4 GEMM alone, n launches (fp32 or bf16 output), for counter and
    kernel-trace runs (k = 0 times the output stores alone)."""
    import torch

    import mxfp4_activation_quantizer_amd as kq
    m, nn, k = (int(x) for x in shape.split("x"))
    g = torch.Generator(device="cuda").manual_seed(5)
    ca = torch.randint(0, 256, (m, k // 2), dtype=torch.uint8, device="cuda", generator=g)
    cw = torch.randint(0, 256, (nn, k // 2), dtype=torch.uint8, device="cuda", generator=g)
    sa = torch.randint(118, 130, (m, k // 32), dtype=torch.uint8, device="cuda", generator=g)
    sw = torch.randint(118, 130, (nn, k // 32), dtype=torch.uint8, device="cuda", generator=g)
    psa, psw = kq.pack_mxfp4_scales(sa), kq.pack_mxfp4_scales(sw)
    bf = out == "bf16"
    O = torch.empty((m, nn), dtype=torch.bfloat16 if bf else torch.float32, device="cuda")
    d = _events_us(torch, lambda: kq.mxfp4_gemm_packed(ca, psa, cw, psw, out=O, bf16=bf), n, 2)
    log("packed gemm %s %s: %d launches, median %.1f us" % (shape, out, n, float(np.median(d))))


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gemm_launches > 0:
        gemm_launches(args.gemm_launches, args.gemm_shape, args.gemm_out)
        return
    if args.gpus != 1:
        print("bench.py: measures one GPU only (the quantizer needs no collectives); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    import mxfp4_activation_quantizer_amd as kq
    import synth

    kq.lib()
    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    names = [n for n in WORKLOAD if args.tensor is None or n.endswith("x%d" % args.tensor)]
    log("generating inputs " + " ".join(names))
    ws = [synth.workload(n) for n in names]
    sets = [Sets(torch, w) for w in ws]
    log("buffer sets per tensor: %s" % [s.n for s in sets])
    kinds = [args.only] if args.only else ["fused", "smoothquant", "quantize"]
    # Process warm-up, outside every timed region: the first graph replays and
    # launches of a process pay one-time costs (and a cold clock) that a timed
    # region must not include; every kind's step runs here a few times.
    graphs = {}
    for kind in kinds:
        if not args.eager:
            graphs[kind] = StepGraphs(torch, kq, kind, sets)
            graphs[kind].replay(20)
        for _ in range(10):
            for s in sets:
                run_kernel(kq, kind, s, torch.cuda.current_stream())
    torch.cuda.synchronize()
    res = {}
    for kind in kinds:
        log("timing %s: %d warmup + %d steps, eager launches with HIP events" % (kind, args.warmup, args.steps))
        eager_ms, per = time_kernel(torch, kq, kind, sets, args.steps, args.warmup)
        wall_ms = eager_ms
        if not args.eager:
            log("timing %s: %d warmup + %d steps, one HIP graph per step" % (kind, args.warmup, args.steps))
            wall_ms = graphs[kind].time(args.steps, args.warmup)
        res[kind] = {"wall_ms_per_step": wall_ms, "eager_ms_per_step": eager_ms,
                     "per_tensor": [summarize(d, s) for d, s in zip(per, sets)],
                     "per_tensor_mean_us": [float(d.mean()) for d in per]}
        log("%s: %.4f ms/step (eager %.4f); %s" % (kind, wall_ms, eager_ms, res[kind]["per_tensor"]))
    # fused against SmoothQuant on the same inputs: alternating blocks of the same
    # K graph-replayed steps (neither kernel always runs first or warmer)
    cmp = None
    if not args.eager and "fused" in kinds and "smoothquant" in kinds:
        blocks = {"fused": [], "smoothquant": []}
        for _ in range(3):
            for kind in ("fused", "smoothquant"):
                blocks[kind].append(graphs[kind].time(args.steps, args.warmup))
        cmp = {k: [round(x, 5) for x in v] for k, v in blocks.items()}
        cmp["speedup"] = round(float(np.median(blocks["smoothquant"]) / np.median(blocks["fused"])), 4)
        log("fused vs smoothquant, alternating blocks of %d steps: %s" % (args.steps, cmp))
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
        "step_launch": "eager" if args.eager else "hip_graph",
        "eager_ms_per_step": round(head["eager_ms_per_step"], 5),
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
                     "kernel": "%s on %dx%d" % (KERNEL_NAMES[kinds[0]], sets[big].m, sets[big].d)},
        "kernels": {k: v["per_tensor"] for k, v in res.items()},
    }
    if cmp is not None:
        out["fused_vs_smoothquant_speedup"] = cmp["speedup"]
        out["fused_vs_smoothquant_blocks_ms"] = {k: cmp[k] for k in ("fused", "smoothquant")}
    elif "fused" in res and "smoothquant" in res:
        out["fused_vs_smoothquant_speedup"] = round(
            res["smoothquant"]["wall_ms_per_step"] / res["fused"]["wall_ms_per_step"], 3)
    if not args.only and not args.no_extras:
        out["extras"] = extras(torch, kq, synth, sets)
    if args.cpu_seconds > 0 and not args.only:
        log("CPU oracle baseline (>= %.0f s)" % args.cpu_seconds)
        out["cpu_baseline"] = cpu_baseline(ws, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
