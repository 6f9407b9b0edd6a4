#!/usr/bin/env python
"""Decode-step throughput of the dequant-GEMV path on one MI355X.

A step is one batch-1 decode step of a 28-layer Qwen3-0.6B-shaped text
decoder: its 197 affine-INT8 g64 projection GEMVs in decoder order (per layer
q, k, v -> o -> gate, up -> down; then the tied 151936 x 1024 LM head), every
weight resident in HBM (633,233,408 bytes), a fresh BF16 N(0,1) input per
GEMV (turbospark-runtime 0.3.0, qwen3_asr_metal.rs -- Qwen3AsrMetalEngine::
step runs exactly this GEMV sequence once per generated token).

Prints one JSON line.  `value` is decoder tokens/s (batch 1, so 1000 /
ms_per_step); the same line carries weight GB/s and the fraction of the
8 TB/s HBM peak, the roofline of the dominant kernel measured with HIP events
on its stream, and the CPU oracle timed on the host (which also re-checks
sampled outputs of the timed buffers).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "dequant-GEMV weight GB/s & % HBM peak; decoder-step tokens/s at batch 1"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--variant", default="step", choices=["step", "graph"],
                   help="step: the whole step as one persistent launch (default); "
                        "graph: 197 GEMV launches captured in a HIP graph")
    return p.parse_args()


class DecodeStep:
    """All weights, inputs and outputs of one decode step, resident on the GPU."""

    def __init__(self, spec, dev):
        import torch

        import quantized_transformer_decode_amd as qd
        import synth
        self.qd = qd
        self.spec = spec
        self.mats = synth.decode_step_matrices(spec)
        self.blobs, self.xs, self.ys, self.x_host = [], [], [], []
        self.weight_bytes = 0
        for i, (layer, name, rows, cols, stage) in enumerate(self.mats):
            tr = synth.affine_triplet(rows, cols, key=(3, layer, i))
            blob = torch.empty(qd.affine_i8_g64_bytes(rows, cols), dtype=torch.uint8, device=dev)
            qd.affine_i8_g64_pack(
                torch.from_numpy(tr.codes.view(np.uint8).reshape(-1)).to(dev),
                torch.from_numpy(tr.scales.view(np.uint8).reshape(-1)).to(dev),
                torch.from_numpy(tr.biases.view(np.uint8).reshape(-1)).to(dev),
                rows, cols, blob)
            xb = synth.x_bf16(1, cols, key=(3, layer, 1000 + i))
            self.x_host.append(xb)
            self.xs.append(torch.from_numpy(xb.view(np.int16).copy()).to(dev).view(torch.bfloat16))
            self.ys.append(torch.empty((1, rows), dtype=torch.bfloat16, device=dev))
            self.blobs.append(blob)
            self.weight_bytes += qd.affine_i8_g64_bytes(rows, cols)
        torch.cuda.synchronize()

    def launches(self):
        return len(self.mats)

    def plan_step(self, dev):
        import torch
        qd = self.qd
        self.ops = qd.make_ops((b, x, y, rows, cols, stage) for (_, _, rows, cols, stage), b, x, y
                               in zip(self.mats, self.blobs, self.xs, self.ys))
        nbytes = qd.qgemv_affine_i8_g64_step_workspace_bytes(self.ops, 1)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.plan = qd.qgemv_affine_i8_g64_step_plan(self.ops, 1, self.ws, nbytes)

    def run_step(self, stream=None):
        self.qd.qgemv_affine_i8_g64_step_run(self.plan, stream)

    def run_eager(self, stream=None):
        for (layer, name, rows, cols, stage), blob, x, y in zip(self.mats, self.blobs, self.xs, self.ys):
            self.qd.qgemv_affine_i8_g64(blob, rows, cols, x, y, 1, stream)


def cpu_baseline(step: DecodeStep):
    """The oracle on one full decode step (all 197 GEMVs, every row), on all
    host cores; its outputs are compared with the GPU's timed buffers."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    blobs = [b.cpu().numpy() for b in step.blobs]
    ys = [y.float().cpu().numpy().astype(np.float64) for y in step.ys]
    t0 = time.perf_counter()
    refs = []
    for (layer, name, rows, cols, stage), blob, xh in zip(step.mats, blobs, step.x_host):
        refs.append(oracle.affine_gemv(blob, rows, cols, xh))
    dt = time.perf_counter() - t0
    worst = 0.0
    for got, ref in zip(ys, refs):
        half = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(got), 2.0 ** -126))) - 8)
        excess = float(np.maximum(np.abs(got - ref) - half, 0).max() / np.abs(ref).max())
        worst = max(worst, excess)
    ok = worst <= 1e-5
    return {
        "value": 1.0 / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
        "sample": "one full decode step: all 197 GEMVs, every output row, f64 (%.1f s wall)" % dt,
        "weight_GBps": step.weight_bytes / dt / 1e9,
        "parity_vs_timed_gpu_buffers": "ok" if ok else "FAIL (excess %.3g)" % worst,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU only; --gpus must be 1 "
                          "(the path runs on a single MI355X; sharding is described in the "
                          "design notes, not launched)"}))
        return 2
    import torch
    import synth
    dev = "cuda:0"
    torch.cuda.set_device(0)
    step = DecodeStep(synth.QWEN3_0_6B, dev)

    # warm (also fills the library's per-device architecture cache)
    step.run_eager()
    torch.cuda.synchronize()

    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step.run_eager()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            step.run_eager()
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()

    def timed(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(cur)
        for _ in range(steps):
            fn()
        e1.record(cur)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps, time.perf_counter() - t0

    # the launch-per-GEMV graph, kept as a reference point
    ms_graph, _ = timed(g.replay, max(10, args.steps // 4), max(2, args.warmup // 4))

    if args.variant == "step":
        step.plan_step(dev)
        ms, wall = timed(lambda: step.run_step(cur), args.steps, args.warmup)
        err = step.qd.qgemv_affine_i8_g64_step_check(step.plan)
        assert err == 0
        variant = ("one persistent launch per step (one workgroup per CU); stage s+1 "
                   "reads its inputs only after every workgroup finished stage s")
        kernel = "affine_step_kernel"
        launches = 1
    else:
        ms, wall = ms_graph, None
        variant = "hipgraph: 197 GEMV launches in decoder order"
        kernel = "affine_gemv_kernel<1,4>"
        launches = step.launches()
    tok_s = 1000.0 / ms
    gbps = step.weight_bytes / (ms * 1e-3) / 1e9

    avg_launch_s = ms * 1e-3 / launches
    bytes_per_launch = step.weight_bytes / launches
    achieved = bytes_per_launch / avg_launch_s / 1e9
    out = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "qwen3-0.6b-shaped decode step, batch 1: 197 affine-INT8 g64 "
                        "GEMVs (28 x q,k,v,o,gate,up,down + 151936x1024 LM head)",
            "batch": 1, "weight_bytes": step.weight_bytes,
            "activations": "bf16 in/out, fp32 accumulate",
            "variant": variant,
        },
        "graph_of_197_launches_ms_per_step": ms_graph,
        "weight_GBps": gbps,
        "hbm_peak_frac": gbps / HBM_PEAK_GBPS,
        "wall_s_timed": wall,
        "roofline": {
            "kernel": kernel,
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": None,
            "bytes_per_launch": bytes_per_launch,
            "avg_launch_us": avg_launch_s * 1e6,
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(step)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
