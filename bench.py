#!/usr/bin/env python
"""Throughput of the dequantize-inside-the-matmul decode path on one MI355X.

Headline step: one batch-1 decode step of a 28-layer Qwen3-0.6B-shaped text
decoder -- its 197 affine-INT8 g64 projection GEMVs in decoder order (per
layer q, k, v -> o -> gate, up -> down, then the tied 151936 x 1024 LM head),
every weight resident in HBM (633,233,408 bytes), a fresh BF16 N(0,1) input
per GEMV (turbospark-runtime 0.3.0, qwen3_asr_metal.rs --
Qwen3AsrMetalEngine::step runs this GEMV sequence once per generated token).

Prints one JSON line.  `value` is decoder tokens/s at batch 1 (1000 /
ms_per_step).  The line also carries weight GB/s and the fraction of the
8 TB/s HBM peak, the roofline of the dominant kernel (HIP events on its
stream; also against a measured practical read ceiling, the library's
streaming read probe over 2 GiB), p10/p50/p90 of single-step times, the ROCm
version and clocks, the CPU oracle timed on the host (it also re-checks the
outputs of the timed buffers), and under "rows" a measurement of every other
part of the path on its own workload:
  affine_gemv_1024       single 1024x1024 affine GEMV, batch 1
  affine_lm_head         the tied LM heads (151936 x 1024 / x 2048) at M = 1, 4, 16:
                         single large GEMVs, weights streamed past the 256 MB MALL
  affine_f16             the same 151936 x 1024 GEMV with f16 activations (the
                         page's Metal dtype) and the device tied-embedding lookup
  q4_0_ffn_pair          Whisper-base FFN pair (fc1 2048x512, fc2 512x2048), M = 1, 4
  qwen3_1_7b_step        Qwen3-1.7B-shaped decode step at M = 1, 4, 10, 16
                         (persistent at M <= 4; graphs of one launch per stage)
  whisper_large_prefill  one Whisper-large layer's six projections at 1500 frames
  whisper_large_decoder  32 layers x 6 Q4_0 GEMVs at batch 1 (one persistent launch;
                         also 128 launches with q, k, v grouped)
  q4_0_bake              f32 -> Q4_0 of one Whisper-large layer
All inputs are seeded synthetic data of the pages' shapes (see synth/).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense BF16 matrix cores
METRIC = "dequant-GEMV weight GB/s & % HBM peak; decoder-step tokens/s at batch 1"
DEV = "cuda:0"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--rows", default="all",
                   help="comma-separated extra rows to measure, 'all' or 'none'")
    p.add_argument("--no-sweep", action="store_true",
                   help="skip the order-free sweep (profiling runs that average the "
                        "headline kernel's launches)")
    p.add_argument("--copy-calibration-mb", type=int, default=0,
                   help="first run one device-to-device copy of this many MiB (the "
                        "reference dispatch for rocprofv3 FETCH_SIZE/WRITE_SIZE scaling)")
    p.add_argument("--no-env", action="store_true",
                   help="skip the rocm-smi clock query (profiled runs: under rocprofv3 --pmc "
                        "a child process would start with the GPU already initialised)")
    p.add_argument("--variant", default="step", choices=["step", "graph"],
                   help="step: the whole step as one persistent launch (default); "
                        "graph: 197 GEMV launches captured in a HIP graph")
    return p.parse_args()


# ---- helpers -------------------------------------------------------------------

def u8dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).reshape(-1).copy()).to(DEV)


def bf16dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).to(DEV).view(
        torch.bfloat16)


def event_time(fn, iters, warmup, stream=None):
    """Average ms per call of fn(), HIP events on the current stream."""
    import torch
    cur = stream or torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(cur)
    for _ in range(iters):
        fn()
    e1.record(cur)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def capture(fn):
    """Capture fn() (which launches on the current stream) into a HIP graph."""
    import torch
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        fn()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.synchronize()
    return g


def affine_blob(qd, rows, cols, key, digests=None):
    """The packed blob of one synthetic matrix; with `digests` (a list), the
    sha256 of its codes, scales and biases are appended in that order."""
    import torch
    import synth
    tr = synth.affine_triplet(rows, cols, key=key)
    if digests is not None:
        digests += [synth.sha256(tr.codes), synth.sha256(tr.scales), synth.sha256(tr.biases)]
    blob = torch.empty(qd.affine_i8_g64_bytes(rows, cols), dtype=torch.uint8, device=DEV)
    qd.affine_i8_g64_pack(u8dev(tr.codes), u8dev(tr.scales), u8dev(tr.biases), rows, cols, blob)
    return blob


# ---- the headline step ---------------------------------------------------------

class DecodeStep:
    """All weights, inputs and outputs of one affine decode step on the GPU."""

    def __init__(self, spec, m=1, cfg=3):
        import torch

        import quantized_transformer_decode_amd as qd
        import synth
        self.qd = qd
        self.m = m
        self.mats = synth.decode_step_matrices(spec)
        self.blobs, self.xs, self.ys, self.x_host = [], [], [], []
        self.digests = []  # sha256 of every generated tensor, in generation order
        self.weight_bytes = 0
        for i, (layer, name, rows, cols, stage) in enumerate(self.mats):
            self.blobs.append(affine_blob(qd, rows, cols, (cfg, layer, i), self.digests))
            xb = synth.x_bf16(m, cols, key=(cfg, layer, 1000 + i))
            self.x_host.append(xb)
            self.digests.append(synth.sha256(xb))
            self.xs.append(bf16dev(xb))
            self.ys.append(torch.empty((m, rows), dtype=torch.bfloat16, device=DEV))
            self.weight_bytes += qd.affine_i8_g64_bytes(rows, cols)
        torch.cuda.synchronize()

    def plan_step(self):
        import torch
        qd = self.qd
        self.ops = qd.make_ops((b, x, y, rows, cols, stage) for (_, _, rows, cols, stage), b, x, y
                               in zip(self.mats, self.blobs, self.xs, self.ys))
        nbytes = qd.qgemv_affine_i8_g64_step_workspace_bytes(self.ops, self.m)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
        self.plan = qd.qgemv_affine_i8_g64_step_plan(self.ops, self.m, self.ws, nbytes)

    def plan_sweep(self):
        """Upper bound, not a decode step: the same GEMVs with the order
        ignored -- ops grouped by input width into as few stages as the plan
        allows (at most 16384 staged input words per stage)."""
        import torch
        qd = self.qd
        order = sorted(range(len(self.mats)), key=lambda i: self.mats[i][3])
        specs, stage, words, cols = [], -1, 0, None
        for i in order:
            _, _, rows, c, _ = self.mats[i]
            w = self.m * ((c + 1023) // 1024) * 1024
            if c != cols or words + w > 16384:
                stage, words, cols = stage + 1, 0, c
            words += w
            specs.append((self.blobs[i], self.xs[i], self.ys[i], rows, c, stage))
        ops = qd.make_ops(specs)
        nbytes = qd.qgemv_affine_i8_g64_step_workspace_bytes(ops, self.m)
        self.sweep_ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
        self.sweep_plan = qd.qgemv_affine_i8_g64_step_plan(ops, self.m, self.sweep_ws, nbytes)
        return stage + 1

    def run_step(self, stream=None):
        self.qd.qgemv_affine_i8_g64_step_run(self.plan, stream)

    def run_eager(self, stream=None):
        for (_, _, rows, cols, _), blob, x, y in zip(self.mats, self.blobs, self.xs, self.ys):
            self.qd.qgemv_affine_i8_g64(blob, rows, cols, x, y, self.m, stream)

    def run_grouped(self, stream=None):
        """One launch per stage (113 for 28 layers): the GEMVs of a stage read
        one input, as q/k/v and gate/up do in the decoder -- here the stage's
        first input buffer."""
        i, n = 0, len(self.mats)
        while i < n:
            j = i
            while j < n and self.mats[j][4] == self.mats[i][4]:
                j += 1
            cols = self.mats[i][3]
            self.qd.qgemv_affine_i8_g64_group(
                [(self.blobs[k], self.ys[k], self.mats[k][2]) for k in range(i, j)],
                cols, self.xs[i], self.m, stream)
            i = j

    def free(self):
        self.blobs = self.xs = self.ys = None


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(step: DecodeStep):
    """The oracle on one full decode step (all 197 GEMVs, every row) on all
    host cores; its outputs are compared with the GPU's timed buffers."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    blobs = [b.cpu().numpy() for b in step.blobs]
    ys = [y.float().cpu().numpy().astype(np.float64) for y in step.ys]
    t0 = time.perf_counter()
    refs = [oracle.affine_gemv(blob, rows, cols, xh)
            for (_, _, rows, cols, _), blob, xh in zip(step.mats, blobs, step.x_host)]
    dt = time.perf_counter() - t0
    worst = 0.0
    for got, ref in zip(ys, refs):
        # each output must be the BF16 rounding of the exact value up to fp32
        # accumulation noise
        half = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(got), 2.0 ** -126))) - 8)
        worst = max(worst, float(np.maximum(np.abs(got - ref) - half, 0).max() / np.abs(ref).max()))
    return {
        "value": 1.0 / dt, "unit": "tokens/s", "cores": cores, "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": "one full decode step: all 197 GEMVs, every output row, f64 (%.2f s wall)" % dt,
        "weight_GBps": step.weight_bytes / dt / 1e9,
        "parity_vs_timed_gpu_buffers": "ok" if worst <= 1e-5 else "FAIL (excess %.3g)" % worst,
    }


def cpu_baseline_rows():
    """The oracle (f64, all host cores) on a bounded sample of every other
    config's workload, with the extrapolation to the whole workload stated
    in each entry.  Inputs are the same shapes and distributions as the GPU
    rows (seeded host tensors)."""
    import oracle
    import synth
    cores = len(os.sched_getaffinity(0))
    out = {}

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    def affine(rows, cols, key):
        tr = synth.affine_triplet(rows, cols, key=key)
        return oracle.affine_pack(tr.codes, tr.scales, tr.biases, rows, cols)

    # config 1: one 1024 x 1024 affine GEMV, batch 1
    blob = affine(1024, 1024, (1, 0, 0))
    x = synth.x_bf16(1, 1024, key=(1, 0, 1))
    dt = min(timed(lambda: oracle.affine_gemv(blob, 1024, 1024, x)) for _ in range(3))
    nb = oracle.affine_bytes(1024, 1024)
    out["affine_gemv_1024"] = {"us_per_gemv": dt * 1e6, "weight_GBps": nb / dt / 1e9,
                               "sample": "the whole GEMV (best of 3)"}
    # config 2: Whisper-base FFN pair, Q4_0 bake and GEMV at M = 1, 4
    pair = []
    t_bake = 0.0
    for name, rows, cols in synth.WHISPER_BASE_FFN:
        w = synth.w_f32(rows, cols, key=(2, 0, rows))
        t0 = time.perf_counter()
        pair.append((rows, cols, oracle.q4_0_quantize(w, rows, cols)))
        t_bake += time.perf_counter() - t0
    pb = sum(oracle.q4_0_bytes(r, c) for r, c, _ in pair)
    ffn = {"bake_us_per_pair": t_bake * 1e6}
    for m in (1, 4):
        xs = [synth.x_f32(m, c, key=(2, m, c)) for _, c, _ in pair]
        dt = min(timed(lambda: [oracle.q4_0_gemm(wq, r, c, xx) for (r, c, wq), xx in
                                zip(pair, xs)]) for _ in range(3))
        ffn[f"M{m}"] = {"us_per_pair": dt * 1e6, "weight_GBps": pb / dt / 1e9}
    ffn["sample"] = "the whole pair (best of 3)"
    out["q4_0_ffn_pair"] = ffn
    # config 4: Qwen3-1.7B step at batch 1 -- one layer's seven GEMVs timed,
    # the step is that per-weight time over all 1.83 GB of weights
    spec = synth.QWEN3_1_7B
    mats = [m_ for m_ in synth.decode_step_matrices(spec) if m_[0] == 0]
    blobs = [affine(r, c, (4, 0, i)) for i, (_, _, r, c, _) in enumerate(mats)]
    xs = [synth.x_bf16(1, c, key=(4, 0, 100 + i)) for i, (_, _, r, c, _) in enumerate(mats)]
    dt = timed(lambda: [oracle.affine_gemv(b, r, c, xx) for b, (_, _, r, c, _), xx in
                        zip(blobs, mats, xs)])
    lb = sum(oracle.affine_bytes(r, c) for _, _, r, c, _ in mats)
    step_s = dt * 1827979264 / lb
    out["qwen3_1_7b_step"] = {"tokens_per_s": 1.0 / step_s, "weight_GBps": lb / dt / 1e9,
                              "sample": "layer 0's 7 GEMVs (%d bytes) in %.3f s, scaled by "
                                        "weight bytes to the 1,827,979,264-byte step, M = 1"
                                        % (lb, dt)}
    # configs 5a / 5b: one Whisper-large layer, baked by the oracle
    lay = [(name, r, c, oracle.q4_0_quantize(synth.w_f32(r, c, key=(5, 0, k)), r, c))
           for k, (name, r, c) in enumerate(synth.WHISPER_LARGE_LAYER)]
    frames = 64
    xb = {c: synth.x_bf16(frames, c, key=(5, 99, c)) for c in (1280, 5120)}
    dt = timed(lambda: [oracle.q4_0_gemm(wq, r, c, xb[c]) for _, r, c, wq in lay])
    flops = sum(2 * frames * r * c for _, r, c, _ in lay)
    layer_s = dt * synth.WHISPER_LARGE_FRAMES / frames
    out["whisper_large_prefill"] = {
        "TFLOPs": flops / dt / 1e12, "ms_per_layer": layer_s * 1e3,
        "ms_32_layers": 32 * layer_s * 1e3,
        "sample": "one encoder layer's six GEMMs on %d of the 1500 frames (%.3f s), scaled "
                  "by frames" % (frames, dt)}
    x1 = {c: synth.x_f32(1, c, key=(5, 98, c)) for c in (1280, 5120)}
    dt = timed(lambda: [oracle.q4_0_gemm(wq, r, c, x1[c]) for _, r, c, wq in lay])
    db = sum(oracle.q4_0_bytes(r, c) for _, r, c, _ in lay)
    out["whisper_large_decoder"] = {
        "tokens_per_s": 1.0 / (32 * dt), "weight_GBps": db / dt / 1e9,
        "sample": "one decoder layer's six GEMVs at M = 1 (%.3f s), times 32 layers" % dt}
    return {"cores": cores, "cpu_model": cpu_model(), "kind": "oracle", "configs": out}


# ---- rows ------------------------------------------------------------------------

def row_affine_gemv_1024(qd):
    """Single 1024x1024 GEMV at batch 1: warm (same weights every launch) and
    cold (rotating over 482 distinct copies, 537 MB, past the 256 MB MALL)."""
    import torch
    import synth
    rows = cols = 1024
    nbytes = qd.affine_i8_g64_bytes(rows, cols)
    ncopy = 482
    base = affine_blob(qd, rows, cols, (1, 0, 0))
    copies = base.repeat(ncopy).view(ncopy, -1)
    x = bf16dev(synth.x_bf16(1, cols, key=(1, 0, 1)))
    y = torch.empty((1, rows), dtype=torch.bfloat16, device=DEV)
    gw = capture(lambda: [qd.qgemv_affine_i8_g64(base, rows, cols, x, y, 1) for _ in range(ncopy)])
    gc = capture(lambda: [qd.qgemv_affine_i8_g64(copies[i], rows, cols, x, y, 1)
                          for i in range(ncopy)])
    warm = event_time(gw.replay, 5, 2) / ncopy
    cold = event_time(gc.replay, 5, 2) / ncopy
    single = single_launch_cold(lambda i: qd.qgemv_affine_i8_g64(copies[i], rows, cols, x, y, 1),
                                ncopy)
    return {"shape": "1024x1024, M=1", "weight_bytes": nbytes,
            "us_single_launch_cold": single,
            "us_per_gemv_warm": warm * 1e3, "us_per_gemv_cold": cold * 1e3,
            "GBps_cold": nbytes / (cold * 1e-3) / 1e9,
            "hbm_peak_frac_cold": nbytes / (cold * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "note": "throughput: back-to-back launches in one HIP graph; cold rotates 482 "
                    "copies (537 MB); single launch: one launch alone on an idle GPU, its "
                    "weights last touched 537 MB earlier"}


def single_launch_cold(launch, ncopy, trials=25):
    """Time of one launch alone on an idle stream, from HIP events recorded
    just before and after it (so it includes the dispatch latency, not only
    the kernel); median and min over `trials`, in microseconds.  The caller
    has just streamed the `ncopy` copies in order, so trial t takes copy t:
    every copy a trial reads was last touched at least ncopy - trials
    copies earlier (past the MALL for the rows here)."""
    import torch
    assert trials <= ncopy // 4
    times = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for t in range(trials):
        i = t
        torch.cuda.synchronize()
        e0.record()
        launch(i)
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    times.sort()
    return {"median": times[len(times) // 2], "min": times[0], "trials": trials}


def row_affine_lm_head(qd):
    """The tied LM heads of the two decoders as single GEMVs at M = 1, 4, 16:
    151936 x 1024 (165 MB) and 151936 x 2048 (330 MB); two copies of each are
    alternated so every launch streams its weights from HBM (the pair exceeds
    the 256 MB MALL)."""
    import torch
    import synth
    out = {}
    for cols in (1024, 2048):
        rows = 151936
        nbytes = qd.affine_i8_g64_bytes(rows, cols)
        blobs = [affine_blob(qd, rows, cols, (3, 28, 7 + k)) for k in range(2)]
        res = {"weight_bytes": nbytes}
        for m in (1, 4, 16):
            x = bf16dev(synth.x_bf16(m, cols, key=(3, 29, m)))
            y = torch.empty((m, rows), dtype=torch.bfloat16, device=DEV)
            g = capture(lambda: [qd.qgemv_affine_i8_g64(blobs[i % 2], rows, cols, x, y, m)
                                 for i in range(8)])
            # the clocks settle over the first ~100 launches of a row
            ms = event_time(g.replay, 10, 12) / 8
            gbps = nbytes / (ms * 1e-3) / 1e9
            res[f"M{m}"] = {"us": ms * 1e3, "GBps": gbps, "hbm_peak_frac": gbps / HBM_PEAK_GBPS}
        out[f"{rows}x{cols}"] = res
        del blobs
        torch.cuda.empty_cache()
    return out


def row_affine_f16(qd):
    """The f16-activation GEMV (the page's Metal dtype) on the 151936 x 1024
    LM head at M = 1, 4, 16 (two alternating copies, as for BF16), and the
    device lookup of 16 tied-embedding rows of that table as f16."""
    import numpy as np
    import torch
    import synth
    rows, cols = 151936, 1024
    nbytes = qd.affine_i8_g64_bytes(rows, cols)
    blobs = [affine_blob(qd, rows, cols, (3, 28, 7 + k)) for k in range(2)]
    res = {"weight_bytes": nbytes}
    for m in (1, 4, 16):
        bits = synth.x_f16(m, cols, key=(3, 30, m))
        x = torch.from_numpy(bits.view(np.int16).copy()).to(DEV).view(torch.float16)
        y = torch.empty((m, rows), dtype=torch.float16, device=DEV)
        g = capture(lambda: [qd.qgemv_affine_i8_g64_f16(blobs[i % 2], rows, cols, x, y, m)
                             for i in range(8)])
        ms = event_time(g.replay, 10, 12) / 8
        gbps = nbytes / (ms * 1e-3) / 1e9
        res[f"M{m}"] = {"us": ms * 1e3, "GBps": gbps, "hbm_peak_frac": gbps / HBM_PEAK_GBPS}
    ids = [int(t) for t in np.linspace(0, rows - 1, 16)]
    emb = torch.empty((16, cols), dtype=torch.float16, device=DEV)
    g = capture(lambda: [qd.affine_i8_g64_embed_rows(blobs[0], rows, cols, ids, emb)
                         for _ in range(8)])
    res["embed_rows_16_tokens_us"] = event_time(g.replay, 20, 2) / 8 * 1e3
    del blobs
    torch.cuda.empty_cache()
    return res


def q4_0_from_f32(qd, w_host, rows, cols):
    import torch
    wq = torch.empty(qd.q4_0_bytes(rows, cols), dtype=torch.uint8, device=DEV)
    qd.q4_0_quantize(torch.from_numpy(w_host).to(DEV), rows, cols, wq)
    return wq


def row_q4_0_ffn_pair(qd):
    """Whisper-base FFN pair baked to Q4_0 on the GPU, GEMV at M = 1 and 4,
    cold over 455 distinct pairs (537 MB)."""
    import torch
    import synth
    npair = 455
    mats = []
    for name, rows, cols in synth.WHISPER_BASE_FFN:
        wq = q4_0_from_f32(qd, synth.w_f32(rows, cols, key=(2, 0, rows)), rows, cols)
        mats.append((rows, cols, wq, wq.repeat(npair).view(npair, -1)))
    pair_bytes = sum(qd.q4_0_bytes(r, c) for r, c, _, _ in mats)
    out = {"shapes": "fc1 2048x512 + fc2 512x2048", "pair_weight_bytes": pair_bytes}
    for m in (1, 4):
        xs = [torch.from_numpy(synth.x_f32(m, c, key=(2, m, c))).to(DEV) for r, c, _, _ in mats]
        ys = [torch.empty((m, r), device=DEV) for r, c, _, _ in mats]

        def launch(cold):
            for i in range(npair):
                for k, (r, c, wq, cp) in enumerate(mats):
                    qd.qgemv_q4_0(cp[i] if cold else wq, r, c, xs[k], ys[k], m)
        gw, gc = capture(lambda: launch(False)), capture(lambda: launch(True))
        warm = event_time(gw.replay, 3, 1) / npair
        cold = event_time(gc.replay, 3, 1) / npair
        single = single_launch_cold(
            lambda i: [qd.qgemv_q4_0(cp[i], r, c, xs[k], ys[k], m)
                       for k, (r, c, wq, cp) in enumerate(mats)], npair)
        out[f"M{m}"] = {"us_single_launch_pair_cold": single,
                        "us_per_pair_warm": warm * 1e3, "us_per_pair_cold": cold * 1e3,
                        "GBps_cold": pair_bytes / (cold * 1e-3) / 1e9}
    out["note"] = ("throughput: pairs back to back in one HIP graph; single launch: the two "
                   "GEMVs alone on an idle GPU (HIP events around both), weights cold")
    return out


def row_qwen3_1_7b_step(qd):
    """Qwen3-1.7B-shaped decode step (1,827,979,264 weight bytes) at M rows:
    M <= 4 as one persistent launch and as a graph of one launch per stage
    (the faster is reported), M = 10, 16 as a graph of one launch per stage
    (113), with the graph of 197 single-GEMV launches alongside."""
    import synth
    out = {}
    step = DecodeStep(synth.QWEN3_1_7B, m=1, cfg=4)
    wb = step.weight_bytes
    step.plan_step()
    ms1 = event_time(step.run_step, 20, 5)
    g1 = capture(step.run_grouped)
    ms1g = event_time(g1.replay, 10, 3)
    best = min(ms1, ms1g)
    out["M1"] = {"ms_per_step": best, "tokens_per_s": 1000.0 / best,
                 "weight_GBps": wb / (best * 1e-3) / 1e9,
                 "hbm_peak_frac": wb / (best * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                 "variant": "persistent step" if ms1 <= ms1g else
                            "113 launches (one per stage) in a HIP graph",
                 "ms_persistent_step": ms1, "ms_113_stage_launches": ms1g}
    ys_keep = step.ys
    for m in (4, 10, 16):
        import torch
        step.m = m
        step.xs = [bf16dev(synth.x_bf16(m, cols, key=(4, layer, 2000 + i)))
                   for i, (layer, _, rows, cols, _) in enumerate(step.mats)]
        step.ys = [torch.empty((m, rows), dtype=torch.bfloat16, device=DEV)
                   for (_, _, rows, _, _) in step.mats]
        g = capture(step.run_grouped)
        msg = event_time(g.replay, 5, 2)
        g197 = capture(step.run_eager)
        ms197 = event_time(g197.replay, 5, 2)
        row = {"ms_113_stage_launches": msg, "ms_per_step_197_launches": ms197}
        ms, variant = msg, "113 launches (one per stage, grouped same-input GEMVs) in a HIP graph"
        if m <= 4:  # the persistent step takes up to four token rows
            step.plan_step()
            msp = event_time(step.run_step, 10, 3)
            row["ms_persistent_step"] = msp
            if msp < ms:
                ms, variant = msp, "persistent step"
        row.update({"ms_per_step": ms, "tokens_per_s": m * 1000.0 / ms,
                    "weight_GBps": wb / (ms * 1e-3) / 1e9,
                    "hbm_peak_frac": wb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                    "variant": variant})
        out[f"M{m}"] = row
    del ys_keep
    step.free()
    out["weight_bytes"] = wb
    return out


def whisper_large_layers(qd, nlayers):
    """Q4_0 weights of `nlayers` Whisper-large layers, baked on the GPU."""
    import synth
    layers = []
    for layer in range(nlayers):
        layers.append([(name, rows, cols,
                        q4_0_from_f32(qd, synth.w_f32(rows, cols, key=(5, layer, k)), rows, cols))
                       for k, (name, rows, cols) in enumerate(synth.WHISPER_LARGE_LAYER)])
    return layers


def row_whisper_large_prefill(qd, layers):
    """One encoder layer's six Q4_0 projections at M = 1500 frames (MFMA)."""
    import torch
    import synth
    m = synth.WHISPER_LARGE_FRAMES
    lay = layers[0]
    xs = {c: bf16dev(synth.x_bf16(m, c, key=(5, 99, c))) for c in (1280, 5120)}
    ys = [torch.empty((m, r), device=DEV) for _, r, _, _ in lay]
    flops = sum(2 * m * r * c for _, r, c, _ in lay)
    g = capture(lambda: [qd.qgemm_q4_0_prefill(wq, r, c, xs[c], ys[k], m)
                         for k, (_, r, c, wq) in enumerate(lay)])
    ms = event_time(g.replay, 10, 3)
    # per matrix: ten back-to-back launches per graph (a graph of one ~20 us
    # launch leaves the GPU idle between replays, and the timing turns bimodal)
    per = {}
    for k, (name, r, c, wq) in enumerate(lay):
        gk = capture(lambda k=k, r=r, c=c, wq=wq: [
            qd.qgemm_q4_0_prefill(wq, r, c, xs[c], ys[k], m) for _ in range(10)])
        mk = event_time(gk.replay, 5, 2) / 10
        per[name] = {"us": mk * 1e3, "TFLOPs": 2 * m * r * c / (mk * 1e-3) / 1e12,
                     "mfma_frac": 2 * m * r * c / (mk * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS}
    tf = flops / (ms * 1e-3) / 1e12
    # the layer as the page runs it (q_linear): q, k, v in one launch (k has
    # no bias), o, fc1 with gelu_tanh, fc2 -- biases and GELU in the epilogue
    byname = {name: (r, c, wq) for name, r, c, wq in lay}
    bias = {name: torch.full((r,), 0.01, device=DEV) for name, r, _, _ in lay}
    yl = {name: torch.empty((m, r), device=DEV) for name, r, _, _ in lay}

    def linear_layer():
        qd.qlinear_q4_0_gemm([(byname[n][2], None if n == "k" else bias[n], yl[n], byname[n][0])
                              for n in ("q", "k", "v")], 1280, xs[1280], m)
        qd.qlinear_q4_0_gemm([(byname["o"][2], bias["o"], yl["o"], byname["o"][0])], 1280,
                             xs[1280], m)
        qd.qlinear_q4_0_gemm([(byname["fc1"][2], bias["fc1"], yl["fc1"], byname["fc1"][0])],
                             1280, xs[1280], m, gelu=True)
        qd.qlinear_q4_0_gemm([(byname["fc2"][2], bias["fc2"], yl["fc2"], byname["fc2"][0])],
                             5120, xs[5120], m)
    gl = capture(linear_layer)
    ms_lin = event_time(gl.replay, 10, 3)
    gq = capture(lambda: [qd.qlinear_q4_0_gemm(
        [(byname[n][2], None if n == "k" else bias[n], yl[n], byname[n][0]) for n in ("q", "k", "v")],
        1280, xs[1280], m) for _ in range(10)])
    ms_qkv = event_time(gq.replay, 5, 2) / 10
    f_qkv = 3 * 2 * m * 1280 * 1280
    return {"frames": m, "flops_per_layer": flops, "ms_per_layer": ms,
            "ms_32_layers": 32 * ms, "TFLOPs": tf, "mfma_frac": tf / BF16_MFMA_PEAK_TFLOPS,
            "per_matrix": per,
            "q_linear_layer": {
                "note": "q, k, v as one grouped launch (3 x 1280 columns), biases and "
                        "gelu_tanh (fc1) in the epilogue",
                "ms": ms_lin, "TFLOPs": flops / (ms_lin * 1e-3) / 1e12,
                "mfma_frac": flops / (ms_lin * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                "qkv_grouped_us": ms_qkv * 1e3,
                "qkv_grouped_TFLOPs": f_qkv / (ms_qkv * 1e-3) / 1e12}}


def row_whisper_large_decoder(qd, layers):
    """32 layers x (q, k, v, o, fc1, fc2) Q4_0 GEMVs at batch 1, f32: one
    launch for the self-attention q, k, v (they read one input), then o,
    fc1, fc2 -- 128 launches in a HIP graph (192 single launches reported
    alongside)."""
    import torch
    import synth
    ops = []
    wb = 0
    for layer, lay in enumerate(layers):
        for k, (name, r, c, wq) in enumerate(lay):
            x = torch.from_numpy(synth.x_f32(1, c, key=(5, layer, 100 + k))).to(DEV)
            ops.append((name, wq, r, c, x, torch.empty((1, r), device=DEV)))
            wb += qd.q4_0_bytes(r, c)

    def grouped():
        i = 0
        while i < len(ops):
            if ops[i][0] == "q":  # q, k, v share the layer's input
                qd.qgemv_q4_0_group([(w, y, r) for _, w, r, _, _, y in ops[i:i + 3]],
                                    ops[i][3], ops[i][4], 1)
                i += 3
            else:
                _, w, r, c, x, y = ops[i]
                qd.qgemv_q4_0(w, r, c, x, y, 1)
                i += 1
    g = capture(grouped)
    ms_graph = event_time(g.replay, 20, 3)
    # the same 192 GEMVs as one persistent launch (128 stages: q, k, v share
    # a stage)
    stage_of = {"q": 0, "k": 0, "v": 0, "o": 1, "fc1": 2, "fc2": 3}
    sops = qd.make_q4_0_ops((w, x, y, r, c, 4 * (i // 6) + stage_of[name])
                            for i, (name, w, r, c, x, y) in enumerate(ops))
    nbytes = qd.qgemv_q4_0_step_workspace_bytes(sops, 1)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    plan = qd.qgemv_q4_0_step_plan(sops, 1, ws, nbytes)
    gp_ = capture(lambda: qd.qgemv_q4_0_step_run(plan))
    ms_pers = event_time(gp_.replay, 20, 3)
    assert qd.qgemv_q4_0_step_check(plan) == 0
    ms = min(ms_graph, ms_pers)
    g192 = capture(lambda: [qd.qgemv_q4_0(w, r, c, x, y, 1) for _, w, r, c, x, y in ops])
    ms192 = event_time(g192.replay, 20, 3)
    # the same step as the page's q_linear calls: biases (none for k) and
    # gelu_tanh after fc1 in the epilogue
    biases = {id(y): torch.full((r,), 0.01, device=DEV) for name, _, r, _, _, y in ops
              if name != "k"}

    def linear():
        i = 0
        while i < len(ops):
            if ops[i][0] == "q":
                qd.qlinear_q4_0_gemv([(w, biases.get(id(y)), y, r)
                                      for _, w, r, _, _, y in ops[i:i + 3]],
                                     ops[i][3], ops[i][4], 1)
                i += 3
            else:
                name, w, r, c, x, y = ops[i]
                qd.qlinear_q4_0_gemv([(w, biases[id(y)], y, r)], c, x, 1, gelu=name == "fc1")
                i += 1
    gl = capture(linear)
    ms_lin = event_time(gl.replay, 20, 3)
    # variant with the cross-attention q and o of every layer (1280 x 1280
    # each; the cross-attention k and v run over the encoder frames with the
    # prefill GEMM): 8 matrices per layer, 192 launches
    cross = []
    for layer in range(len(layers)):
        for k, name in enumerate(("cross_q", "cross_o")):
            wq = q4_0_from_f32(qd, synth.w_f32(1280, 1280, key=(5, layer, 200 + k)), 1280, 1280)
            x = torch.from_numpy(synth.x_f32(1, 1280, key=(5, layer, 300 + k))).to(DEV)
            cross.append((layer, wq, x, torch.empty((1, 1280), device=DEV)))
    wb_cross = wb + sum(qd.q4_0_bytes(1280, 1280) for _ in cross)

    def with_cross():
        i = 0
        layer = 0
        while i < len(ops):
            qd.qgemv_q4_0_group([(w, y, r) for _, w, r, _, _, y in ops[i:i + 3]],
                                ops[i][3], ops[i][4], 1)
            _, w, r, c, x, y = ops[i + 3]  # self-attention o
            qd.qgemv_q4_0(w, r, c, x, y, 1)
            for _, wq, x, y in cross[2 * layer:2 * layer + 2]:
                qd.qgemv_q4_0(wq, 1280, 1280, x, y, 1)
            for _, w, r, c, x, y in ops[i + 4:i + 6]:  # fc1, fc2
                qd.qgemv_q4_0(w, r, c, x, y, 1)
            i += 6
            layer += 1
    gx = capture(with_cross)
    ms_x = event_time(gx.replay, 20, 3)
    del cross
    return {"gemvs": len(ops), "weight_bytes": wb, "ms_per_step": ms,
            "tokens_per_s": 1000.0 / ms, "weight_GBps": wb / (ms * 1e-3) / 1e9,
            "hbm_peak_frac": wb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "variant": ("one persistent launch (128 stages)" if ms_pers <= ms_graph
                        else "128 launches (q, k, v grouped) in a HIP graph"),
            "ms_persistent_step": ms_pers, "ms_128_launches": ms_graph,
            "ms_per_step_192_launches": ms192,
            "ms_per_step_q_linear": ms_lin,
            "with_cross_q_o": {"weight_bytes": wb_cross, "ms_per_step": ms_x,
                               "weight_GBps": wb_cross / (ms_x * 1e-3) / 1e9,
                               "hbm_peak_frac": wb_cross / (ms_x * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                               "variant": "8 matrices per layer (plus cross-attention q, o), "
                                          "192 launches in a HIP graph"}}


def row_q4_0_bake(qd):
    """f32 -> Q4_0 of one Whisper-large layer (19.7 M weights)."""
    import torch
    import synth
    mats = [(r, c, torch.from_numpy(synth.w_f32(r, c, key=(5, 77, k))).to(DEV),
             torch.empty(qd.q4_0_bytes(r, c), dtype=torch.uint8, device=DEV))
            for k, (_, r, c) in enumerate(synth.WHISPER_LARGE_LAYER)]
    n = sum(r * c for r, c, _, _ in mats)
    g = capture(lambda: [qd.q4_0_quantize(w, r, c, o) for r, c, w, o in mats])
    ms = event_time(g.replay, 20, 3)
    moved = n * 4 + sum(qd.q4_0_bytes(r, c) for r, c, _, _ in mats)
    return {"weights": n, "ms": ms, "Gweights_per_s": n / (ms * 1e-3) / 1e9,
            "GBps": moved / (ms * 1e-3) / 1e9,
            "hbm_peak_frac": moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}


def row_attention_decode(qd):
    """Grouped-query decode attention, f16 (the page's Metal dtype), as a
    decode step runs it: one call per layer over 28 layers' own caches
    (Qwen3-0.6B/1.7B heads: 16 query / 8 K/V heads of 128) at windows of
    128 .. 32768 rows, and the 32-head (Qwen3-4B) shape at 4096.  Bytes are
    the K and V rows of the window (+ q and out), read once per call."""
    import math
    import numpy as np
    import torch
    import synth
    layers = 28
    out = {"layers": layers, "dtype": "f16"}
    for heads, kv, d, n in ((16, 8, 128, 128), (16, 8, 128, 1024), (16, 8, 128, 4096),
                            (16, 8, 128, 32768), (32, 8, 128, 4096)):
        qb, kb, vb = synth.attention_inputs(heads, kv, d, n, key=(12, heads, n))
        def dev(bits):
            return torch.from_numpy(bits.view(np.int16).copy()).to(DEV).view(torch.float16)
        q, k0, v0 = dev(qb), dev(kb), dev(vb)
        ks = [k0.clone() for _ in range(layers)]
        vs = [v0.clone() for _ in range(layers)]
        del k0, v0
        o = torch.empty((heads, d), dtype=torch.float16, device=DEV)
        wsb = qd.attention_decode_workspace_bytes(heads, kv, d)
        ws = torch.empty(wsb // 4, dtype=torch.float32, device=DEV)
        scale = 1.0 / math.sqrt(d)
        g = capture(lambda: [qd.attention_decode(q, ks[i], vs[i], heads, kv, d, n, 0, scale, o,
                                                 ws, wsb) for i in range(layers)])
        ms = event_time(g.replay, 10, 2) / layers
        nbytes = 2 * n * kv * d * 2 + 2 * heads * d * 2
        gbps = nbytes / (ms * 1e-3) / 1e9
        out[f"h{heads}_kv{kv}_d{d}_n{n}"] = {
            "us_per_layer": ms * 1e3, "bytes_per_call": nbytes, "GBps": gbps,
            "hbm_peak_frac": gbps / HBM_PEAK_GBPS, "us_per_token_all_layers": ms * 1e3 * layers}
        del ks, vs
        torch.cuda.empty_cache()
    return out


def row_qwen3_decoder_step(qd):
    """The whole Qwen3-0.6B decoder step (28 layers: norms, q/k/v, per-head
    norms + RoPE with the cache append, attention over the cache, o,
    residuals, gate/up, SiLU-mul, down; final norm and the tied LM head),
    f16 buffers, captured once in a HIP graph and replayed token after token
    (the position advances on the device), at cache contexts of 128, 1024
    and 4096 rows (random f16 K/V rows before the first position).  Bytes
    per token: every weight blob once + the K/V rows attended."""
    import numpy as np
    import torch
    import synth
    spec = synth.QWEN3_0_6B_STEP
    m = synth.qwen3_model(spec)

    def u16dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).to(DEV)

    def blob(tr):
        b = torch.empty(qd.affine_i8_g64_bytes(tr.rows, tr.cols), dtype=torch.uint8, device=DEV)
        qd.affine_i8_g64_pack(u8dev(tr.codes), u8dev(tr.scales), u8dev(tr.biases), tr.rows,
                              tr.cols, b)
        return b

    steps, ctxs = 64, (128, 1024, 4096)
    cap = max(ctxs) + steps
    layers, wbytes = [], 0
    for L in m["layers"]:
        d = {n: blob(L[n]) for n in ("q", "k", "v", "o", "gate", "up", "down")}
        wbytes += sum(t.numel() for t in d.values())
        d.update({n: u16dev(L[n]) for n in ("in_norm", "q_norm", "k_norm", "post_norm")})
        shape = (cap, spec.kv_heads, spec.head_dim)
        d["k_cache"] = (torch.randn(shape, device=DEV) * 0.5).half()
        d["v_cache"] = torch.randn(shape, device=DEV).half()
        layers.append(d)
    embed = blob(m["embed"])
    final_norm = u16dev(m["final_norm"])
    wbytes += embed.numel()
    del m
    model = qd.qwen3_model(spec.hidden, spec.heads, spec.kv_heads, spec.head_dim, spec.inter,
                           spec.vocab, cap, float(np.float32(spec.eps)),
                           float(np.float32(spec.theta)), layers, final_norm, embed)
    wsb = qd.qwen3_step_workspace_bytes(model)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    pos = torch.zeros(1, dtype=torch.int32, device=DEV)
    x = torch.randn(spec.hidden, device=DEV).half()
    logits = torch.empty(spec.vocab, dtype=torch.float16, device=DEV)
    g = capture(lambda: qd.qwen3_step_run(model, ws, wsb, x, pos, logits, advance=True))
    out = {"model": spec.name, "layers": spec.layers, "weight_bytes": wbytes,
           "launches_per_token": spec.layers * (5 if spec.kv_heads <= 8 else 6) + 1}
    for ctx in ctxs:
        pos.fill_(ctx)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        pos.fill_(ctx)
        ms = event_time(g.replay, steps, 0)
        assert int(pos.item()) == ctx + steps
        kv_bytes = spec.layers * 2 * (ctx + steps // 2) * spec.kv_heads * spec.head_dim * 2
        gbps = (wbytes + kv_bytes) / (ms * 1e-3) / 1e9
        out[f"ctx{ctx}"] = {"ms_per_token": ms, "tokens_per_s": 1e3 / ms,
                            "GBps_weights_plus_kv": gbps, "hbm_peak_frac": gbps / HBM_PEAK_GBPS}
    assert qd.qwen3_step_check(ws) == 0
    del layers, embed, g
    torch.cuda.empty_cache()
    return out


ROWS = ("affine_gemv_1024", "affine_lm_head", "affine_f16", "q4_0_ffn_pair", "qwen3_1_7b_step", "whisper_large_prefill",
        "whisper_large_decoder", "q4_0_bake", "attention_decode", "qwen3_decoder_step")


# HBM traffic of the headline kernel per launch, from two rocprofv3 --pmc runs
# (FETCH_SIZE, WRITE_SIZE) of this script scaled by the same counters of a
# device-to-device copy of known size; the summary records the sha256 of the
# kernel's sources at measurement time and is ignored once they change.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "affine_step_kernel_qwen3_0_6b_traffic.md")
STEP_SOURCES = ("decode_step.hip", "qd_step.h", "qd_device.h", "affine_gemv.hip", "qd_api.hip")


def step_source_sha():
    import hashlib
    h = hashlib.sha256()
    for f in STEP_SOURCES:
        with open(os.path.join(ROOT, "quantized_transformer_decode_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per step (the step kernel and the streamed LM head), or None
    if absent or stale."""
    try:
        with open(TRAFFIC_FILE) as fh:
            text = fh.read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].split(": ", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("source_sha256") != step_source_sha():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def run_rows(qd, names):
    import torch
    out = {}
    layers = None
    for name in names:
        t0 = time.perf_counter()
        try:
            if name in ("whisper_large_prefill", "whisper_large_decoder") and layers is None:
                import synth
                layers = whisper_large_layers(qd, synth.WHISPER_LARGE_LAYERS)
            fn = globals()["row_" + name]
            out[name] = fn(qd, layers) if "whisper_large" in name else fn(qd)
        except Exception as e:  # a failing row is reported, not hidden
            out[name] = {"error": repr(e)}
        out[name]["bench_wall_s"] = time.perf_counter() - t0
        torch.cuda.empty_cache()
    return out


def step_distribution(fn, n, stream):
    """Per-step HIP-event times (ms) of n back-to-back calls: p10 / p50 / p90."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in evs)
    return {"n": n, "p10": t[n // 10], "p50": t[n // 2], "p90": t[(9 * n) // 10],
            "min": t[0], "max": t[-1]}


def hbm_read_ceiling(qd, nbytes=2 << 30, iters=10):
    """GB/s of the library's streaming read probe over nbytes of HBM: the
    practical ceiling the GEMV rooflines are also set against."""
    import torch
    buf = torch.ones(nbytes, dtype=torch.uint8, device=DEV)
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    ms = event_time(lambda: qd.stream_read(buf, nbytes, sink), iters, 2)
    del buf, sink
    torch.cuda.empty_cache()
    return nbytes / (ms * 1e-3) / 1e9


def environment():
    """ROCm version, device and clocks (rocm-smi; None where unavailable)."""
    import subprocess
    import torch
    env = {"device": torch.cuda.get_device_name(0),
           "compute_units": torch.cuda.get_device_properties(0).multi_processor_count,
           "torch": torch.__version__}
    try:
        with open("/opt/rocm/.info/version") as f:
            env["rocm"] = f.read().strip()
    except OSError:
        env["rocm"] = None
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True,
                           text=True, timeout=20)
        card = next(iter(json.loads(r.stdout).values()))
        env["clocks"] = {k: v for k, v in card.items() if "clock" in k.lower()}
    except Exception:  # the clocks are context only
        env["clocks"] = None
    return env


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the decode path runs on one GPU; --gpus must be 1 "
                          "(the path runs on a single MI355X; sharding is described in the "
                          "design notes, not launched)"}))
        return 2
    import torch

    import synth
    torch.cuda.set_device(0)
    if args.copy_calibration_mb:
        n = args.copy_calibration_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device=DEV)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    step = DecodeStep(synth.QWEN3_0_6B)
    qd = step.qd
    step.run_eager()  # warm (also fills the library's per-device caches)
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()

    g = capture(step.run_eager)  # the launch-per-GEMV graph, kept as a reference point
    ms_graph = event_time(g.replay, max(10, args.steps // 4), max(2, args.warmup // 4))
    gg = capture(step.run_grouped)  # one launch per stage
    ms_grouped = event_time(gg.replay, max(10, args.steps // 4), max(2, args.warmup // 4))

    if args.variant == "step":
        step.plan_step()
        t0 = time.perf_counter()
        ms = event_time(lambda: step.run_step(cur), args.steps, args.warmup, cur)
        wall = time.perf_counter() - t0
        dist = step_distribution(lambda: step.run_step(cur), min(args.steps, 200), cur)
        assert qd.qgemv_affine_i8_g64_step_check(step.plan) == 0
        ms_sweep, n_sweep = None, None
        if not args.no_sweep:
            n_sweep = step.plan_sweep()
            ms_sweep = event_time(lambda: qd.qgemv_affine_i8_g64_step_run(step.sweep_plan, cur),
                                  max(10, args.steps // 4), max(2, args.warmup // 4), cur)
            assert qd.qgemv_affine_i8_g64_step_check(step.sweep_plan) == 0
        variant = ("one persistent launch per step (one workgroup per CU); stage s+1 "
                   "reads its inputs only after every workgroup finished stage s")
        kernel, launches = f"affine_step_kernel<{step.plan.group}>", 1
        if step.plan.tail:
            variant += ("; the last stage (the LM head, one GEMV) streams as a second "
                        "launch after it")
            kernel += "+affine_gemv_m1_kernel"
    else:
        ms, wall = ms_graph, None
        dist = step_distribution(g.replay, min(args.steps, 200), cur)
        ms_sweep, n_sweep = None, None
        variant = "hipgraph: 197 GEMV launches in decoder order"
        kernel, launches = "affine_gemv_mfma_kernel", len(step.mats)
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
            "activations": "bf16 in/out, u8 codes, fp32 accumulate",
            "variant": variant,
            "inputs_sha256": {
                "tensors": len(step.digests),
                "order": "per GEMV in decoder order: codes, scales, biases, x",
                "sha256_of_digests": hashlib.sha256(
                    "".join(step.digests).encode()).hexdigest(),
            },
        },
        "weight_GBps": gbps,
        "hbm_peak_frac": gbps / HBM_PEAK_GBPS,
        "step_ms_distribution": dist,
        "graph_of_197_launches_ms_per_step": ms_graph,
        "graph_of_113_stage_launches_ms_per_step": ms_grouped,
        "independent_sweep": None if ms_sweep is None else {
            "note": "upper bound, not a decode step: the same 197 GEMVs in one persistent "
                    "launch with their order ignored (grouped by input width)",
            "stages": n_sweep, "ms": ms_sweep,
            "weight_GBps": step.weight_bytes / (ms_sweep * 1e-3) / 1e9,
            "hbm_peak_frac": step.weight_bytes / (ms_sweep * 1e-3) / 1e9 / HBM_PEAK_GBPS},
        "wall_s_timed": wall,
        "roofline": {
            "kernel": kernel, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
            "traffic": recorded_traffic() if kernel.startswith("affine_step_kernel") else None,
            "bytes_per_launch": bytes_per_launch, "avg_launch_us": avg_launch_s * 1e6,
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(step)
        out["cpu_baseline_rows"] = cpu_baseline_rows()
    step.free()
    torch.cuda.empty_cache()
    ceiling = hbm_read_ceiling(qd)
    out["hbm_read_ceiling_GBps"] = ceiling
    out["roofline"]["practical_peak"] = ceiling
    out["roofline"]["frac_of_practical"] = achieved / ceiling
    out["env"] = None if args.no_env else environment()
    names = ROWS if args.rows == "all" else [] if args.rows == "none" else args.rows.split(",")
    if names:
        out["rows"] = run_rows(qd, names)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
