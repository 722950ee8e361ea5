#!/usr/bin/env python3
"""Benchmark of libgq on one MI355X.

The timed step is one Llama-3-8B-shaped Q4_K decode step: the q, k, v, o,
gate, up and down projections of 32 distinct layers (224 gq_matvec calls,
3.93 GB of packed weights, so every call streams cold weights from HBM),
enqueued back-to-back on one stream. The step is captured once in a HIP
graph and replayed (host launch cost would otherwise exceed the GPU time of
the small projections); the eager rate is reported beside it.

value = algorithmic bytes per step (packed W + x + y of every call) / time,
in GB/s. The JSON line also carries:
  roofline      the dominant kernel (the Q4_K GEMV instance of the K = 4096
                projections) timed alone with HIP events on its stream;
  per_projection, int8_activation_step_variant, fused_step_variant
                the step's parts and variants (us per call as the median of
                5 timed loops, with mean and minimum);
  prefill_q4_k_llama3_8b
                the Llama-3-8B prefill products (M = 2..512): us, TFLOP/s,
                % of the fp16 matrix peak and % of the HBM peak;
  cpu_baseline  the C oracle on the host cores over a bounded sample, on N
                threads and on one, with the CPU model, the oracle's time per
                call of every config, and the GPU's largest relative error
                against the oracle on every config;
  workloads     the other shapes: Q8_0 lm_head (cold), the Qwen2.5-0.5B and
                SmolLM-135M decode shapes (cold over > 512 MB of rotating
                copies, and warm), the mixed formats, MoE, the prefill GEMMs
                and gq_dequant.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix peak
SMALL_M = (2, 4, 8)            # few activation rows (batched matvec or matrix cores)


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Timer:
    """HIP events on torch's current stream, which is where libgq launches.

    Before a timed loop the same work runs for at least `warm_ms` of wall
    time: the GPU's clock falls while it idles and ramps back up under load
    (an M = 512 prefill product measured 219-222 us right after an idle gap
    against 186-195 us after a few milliseconds of work), so a few calls
    timed from cold measure the ramp, not the kernel."""

    def __init__(self, torch, warm_ms: float = 20.0):
        self.torch = torch
        self.warm_ms = warm_ms

    def warm(self, fn, batch: int) -> None:
        torch = self.torch
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < self.warm_ms:
            for _ in range(max(1, batch)):
                fn()
            torch.cuda.synchronize()

    def time(self, fn, iters: int, warmup: int = 1, warm: bool = True) -> float:
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        if warm and warmup > 0:
            self.warm(fn, iters)
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(iters):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / iters  # ms per fn()

    def stats(self, fn, iters: int, reps: int = 5, warmup: int = 1):
        """(mean, median, min) ms per fn() over `reps` event-timed loops of
        `iters` calls each."""
        per = [self.time(fn, iters, warmup=warmup if r == 0 else 0) for r in range(reps)]
        return float(np.mean(per)), float(np.median(per)), float(np.min(per))


def rate_row(nbytes: int, calls: int, st) -> dict:
    """us per call (mean / median / min over the timed loops), GB/s and % of
    the HBM peak at the median."""
    mean, med, mn = (v * 1e3 / calls for v in st)
    gbps = nbytes / (med * 1e-6) / 1e9
    return dict(us_per_call=round(med, 3), us_mean=round(mean, 3), us_min=round(mn, 3),
                GBps=round(gbps, 1), pct_hbm=round(100 * gbps / HBM_PEAK_GBS, 2))


def capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm: first launches outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def gemv_bytes(fmt_row_bytes: int, rows: int, cols: int) -> int:
    return rows * fmt_row_bytes + 4 * cols + 4 * rows


DOMINANT_KERNEL = "gemv_kernel<Q4KUnit, 64, 2, 0, false>"  # unit, group width, rows per group, store epilogue, not expert-batched
# HBM bytes per launch of the dominant kernel from rocprofv3 --pmc FETCH_SIZE
# and WRITE_SIZE (bench.py --traffic-probe), each scaled by the same counter
# on a 256 MiB plain copy (FETCH x 2.000, WRITE x 1.000); set to None whenever
# the kernel changes until it is measured again.
TRAFFIC_BYTES_PER_LAUNCH = 21619395


def dominant_launches(mats):
    return [m for m in mats if m["cols"] == 4096 and m["rows"] >= 4096]


def traffic_probe(torch, gq, lib, synth, mats, stream_ptr):
    """One plain device copy of 256 MiB (the counter calibration), one pass
    over the dominant kernel's launches, then the Qwen2.5-0.5B Q8_0 lm_head
    once packed and once in the split layout (cold: fresh copies, repacked
    before the copy that flushes the caches); for rocprofv3 --pmc runs."""
    fmt, rows, cols = synth.QWEN05_LM_HEAD
    W, x = synth.matrix_and_x(fmt, rows, cols, 2, 0)
    Wd, xd = torch.from_numpy(W).cuda(), torch.from_numpy(x).cuda()
    Sd = gq.gq_q8_0_split_repack(Wd, rows, cols)
    yd = torch.empty(rows, dtype=torch.float32, device="cuda")
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    sp = stream_ptr()
    for m in dominant_launches(mats):
        lib.gq_matvec(*m["args"], sp)
    torch.cuda.synchronize()
    for f, w in ((fmt, Wd), (gq.FMT_Q8_0_SPLIT, Sd)):
        dst.copy_(src)  # evicts the lm_head from the caches
        torch.cuda.synchronize()
        assert lib.gq_matvec(f, w.data_ptr(), rows, cols, xd.data_ptr(), yd.data_ptr(), sp) == 0
        torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": src.numel(),
                      "dominant_bytes_per_launch": sum(m["bytes"] for m in dominant_launches(mats))
                      / len(dominant_launches(mats)),
                      "lm_head_bytes": {"packed": gemv_bytes(gq.gq_row_bytes(fmt, cols), rows, cols),
                                        "split": gemv_bytes(gq.gq_row_bytes(gq.FMT_Q8_0_SPLIT, cols),
                                                            rows, cols)}}), flush=True)


def decode_probe(torch, gq, lib, synth, mats, stream_ptr):
    """Eager launches for counter runs: the 224 matvecs of the decode step
    twice (q/o/gate/up run the row-group kernel instance of the roofline, k/v
    its 1024-row sibling, down the wide-row Q4_K kernel), then for layers
    0-3 the fused launches (q|k|v matvec, gate|up SwiGLU matvec, o and down
    accumulating)."""
    sp = stream_ptr()
    for _ in range(2):
        for m in mats:
            assert lib.gq_matvec(*m["args"], sp) == 0
    torch.cuda.synchronize()
    f = gq.FMT_Q4_K
    for layer in range(4):
        q, k, v, o, gate, up, down = mats[7 * layer:7 * layer + 7]
        wqkv = torch.cat([q["W"], k["W"], v["W"]])
        wgu = torch.cat([gate["W"], up["W"]])
        yqkv = torch.empty(q["rows"] + k["rows"] + v["rows"], dtype=torch.float32, device="cuda")
        h = torch.empty(gate["rows"], dtype=torch.float32, device="cuda")
        resid = torch.zeros(o["rows"], dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        assert lib.gq_matvec(f, wqkv.data_ptr(), yqkv.numel(), q["cols"], q["x"].data_ptr(),
                             yqkv.data_ptr(), sp) == 0
        assert lib.gq_matvec_acc(f, o["W"].data_ptr(), o["rows"], o["cols"], o["x"].data_ptr(),
                                 resid.data_ptr(), sp) == 0
        assert lib.gq_matvec_swiglu(f, wgu.data_ptr(), gate["rows"], gate["cols"], gate["x"].data_ptr(),
                                    h.data_ptr(), sp) == 0
        assert lib.gq_matvec_acc(f, down["W"].data_ptr(), down["rows"], down["cols"], down["x"].data_ptr(),
                                 resid.data_ptr(), sp) == 0
        torch.cuda.synchronize()
        del wqkv, wgu
    print(json.dumps({"decode_probe": "done", "step_launches": len(mats), "fused_layers": 4}), flush=True)


def prefill_probe(torch, gq, lib, synth, stream_ptr, ms=(512,)):
    """One call of each prefill product per M (after one warm-up call):
    Q4_K gate and down on the fp16 matrix cores and, at M = 512, Q6_K down,
    Q5_K gate and the Q8_0 gate packed and split (fp16 as well; the split
    layout made by one gq_q8_0_split_repack launch before its two calls);
    for rocprofv3 --pmc runs (MFMA busy cycles, executed matrix ops, waits
    and cache requests per dispatch)."""
    cases = []
    for M in ms:
        for which in ("gate", "down"):
            W, X, rows, cols = synth.prefill_inputs(which, M)
            cases.append((f"q4_k_{which}_M{M}", 12, W, X, rows, cols))
        if M == 512:
            for i in (1, 3):
                name, f, r, c, W, _ = synth.mixed_format_weight_and_x(i)
                cases.append((name, f, W, synth.activations((M, c), synth.rng_for(911, M)), r, c))
            W8 = synth.weights(gq.FMT_Q8_0, 14336, 4096, synth.rng_for(6, 0))
            X8 = synth.activations((M, 4096), synth.rng_for(911, M))
            cases.append(("q8_0_gate", gq.FMT_Q8_0, W8, X8, 14336, 4096))
            cases.append(("q8_0_split_gate", gq.FMT_Q8_0_SPLIT, W8, X8, 14336, 4096))
    out = {}
    for name, f, W, X, rows, cols in cases:
        M = X.shape[0]
        Wd, Xd = torch.from_numpy(W).cuda(), torch.from_numpy(X).cuda()
        if f == gq.FMT_Q8_0_SPLIT:
            Wd = gq.gq_q8_0_split_repack(Wd, rows, cols)
        Yd = torch.empty((M, rows), dtype=torch.float32, device="cuda")
        for _ in range(2):
            st = lib.gq_matmul(f, Wd.data_ptr(), rows, cols, Xd.data_ptr(), M, Yd.data_ptr(),
                               stream_ptr())
            assert st == 0
        torch.cuda.synchronize()
        out[name] = dict(fmt=f, rows=rows, cols=cols, M=M, flops=2.0 * M * rows * cols)
        del Wd, Xd, Yd
    print(json.dumps(out), flush=True)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=8.0)
    ap.add_argument("--prefill-probe", action="store_true",
                    help="run each prefill product twice (M from --prefill-probe-m; for counter runs) and exit")
    ap.add_argument("--prefill-probe-m", default="512",
                    help="activation rows for --prefill-probe, comma separated")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run a 256 MiB copy and one pass of the dominant kernel, then exit")
    ap.add_argument("--decode-probe", action="store_true",
                    help="run the 224-launch decode step twice and the fused launches of 4 layers "
                         "once, eagerly (for rocprofv3 counter runs), then exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: the block-quantised GEMV path runs on a single "
              f"MI355X (no collectives); --gpus {args.gpus} is not supported.", file=sys.stderr)
        return 2

    import torch

    import gguf_block_quant_gq_amd as gq
    import synth

    torch.cuda.set_device(0)
    lib = gq.load_library()
    timer = Timer(torch)
    stream_ptr = lambda: int(torch.cuda.current_stream().cuda_stream)  # noqa: E731

    if args.prefill_probe:
        prefill_probe(torch, gq, lib, synth, stream_ptr,
                      tuple(int(m) for m in args.prefill_probe_m.split(",")))
        return 0

    # ------------------------------------------------ decode step workload
    t0 = time.time()
    mats = []
    total_bytes = 0
    for layer in range(synth.LLAMA3_8B_LAYERS):
        for proj in range(7):
            name, rows, cols, _, _ = synth.llama3_8b_matrix(layer, proj)
            W, x = synth.llama3_8b_weight_and_x(layer, proj)
            Wd = torch.from_numpy(W).cuda()
            xd = torch.from_numpy(x).cuda()
            yd = torch.empty(rows, dtype=torch.float32, device="cuda")
            rb = gq.gq_row_bytes(gq.FMT_Q4_K, cols)
            nbytes = gemv_bytes(rb, rows, cols)
            total_bytes += nbytes
            mats.append(dict(name=name, rows=rows, cols=cols, W=Wd, x=xd, y=yd, bytes=nbytes,
                             args=(gq.FMT_Q4_K, Wd.data_ptr(), rows, cols, xd.data_ptr(),
                                   yd.data_ptr())))
    torch.cuda.synchronize()
    log(f"generated and uploaded 224 Q4_K matrices ({total_bytes / 1e9:.3f} GB) in "
        f"{time.time() - t0:.1f}s")

    if args.traffic_probe:
        traffic_probe(torch, gq, lib, synth, mats, stream_ptr)
        return 0
    if args.decode_probe:
        decode_probe(torch, gq, lib, synth, mats, stream_ptr)
        return 0

    def step(subset=None):
        sp = stream_ptr()
        for m in (mats if subset is None else subset):
            st = lib.gq_matvec(*m["args"], sp)
            if st != 0:
                raise gq.GQError(st, "gq_matvec")

    graph = capture(torch, step)
    # exactly W untimed steps, then K timed ones (the K-step loop is long
    # enough that the clock ramp is a small part of it)
    ms_graph = timer.time(graph.replay, args.steps, warmup=args.warmup, warm=False)
    # spread of single steps (each replay timed alone), beside the K-step mean
    one = [timer.time(graph.replay, 1, warmup=0) for _ in range(max(5, args.steps // 2))]
    ms_eager = timer.time(step, max(5, args.steps // 5), warmup=2)
    value = total_bytes / (ms_graph * 1e-3) / 1e9
    log(f"decode step: {ms_graph * 1e3:.1f} us (graph), {ms_eager * 1e3:.1f} us (eager); "
        f"{value:.0f} GB/s = {100 * value / HBM_PEAK_GBS:.1f}% of 8 TB/s")

    # per-projection rates (graph of the 32 launches of one projection)
    per_proj = {}
    for proj in range(7):
        sub = [m for m in mats if m["name"] == synth.LLAMA3_8B_LAYER[proj][0]]
        g = capture(torch, lambda sub=sub: step(sub))
        st = timer.stats(g.replay, max(2, args.steps // 10), reps=5, warmup=2)
        per_proj[sub[0]["name"]] = rate_row(sum(m["bytes"] for m in sub) // len(sub), len(sub), st)
    log(f"per projection: {per_proj}")

    # --------------------------------- roofline: the dominant GEMV kernel
    # The launches of one kernel instance, gemv_kernel<Q4KUnit, 64, 2, 1>:
    # the K = 4096 projections with >= 4096 rows (q, o, gate, up; 128 of the
    # 224 launches, 69% of the step's bytes), timed alone (graph replay, HIP
    # events on the launch stream).
    dom = dominant_launches(mats)
    gdom = capture(torch, lambda: step(dom))
    ms_dom = timer.time(gdom.replay, max(5, args.steps // 5), warmup=2)
    dom_bytes = sum(m["bytes"] for m in dom) / len(dom)
    dom_us = ms_dom * 1e3 / len(dom)
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=TRAFFIC_BYTES_PER_LAUNCH,
                    kernel=DOMINANT_KERNEL, launches_per_step=len(dom),
                    bytes_per_launch=round(dom_bytes), avg_launch_us=round(dom_us, 3))
    log(f"roofline: {roofline}")

    fused = fused_step_variant(torch, gq, lib, synth, mats, timer, stream_ptr, args)
    int8 = int8_step_variant(torch, gq, lib, synth, mats, timer, stream_ptr, args)

    extras = {}
    if not args.no_extras:
        extras = run_extras(torch, gq, lib, synth, timer, stream_ptr, args)
        del graph, gdom

    # ------------------------------------------------------ CPU baseline
    cpu = None
    if not args.no_cpu_baseline:
        gpu = gpu_config_outputs(torch, gq, synth)
        cpu = cpu_baseline(synth, args.cpu_seconds, gpu)
        log(f"cpu baseline: {cpu}")

    # config 4 (the Llama-3-8B prefill products) at the top level
    config4 = {k[len("matmul_"):]: v for k, v in extras.items()
               if k.startswith("matmul_gate_M") or k.startswith("matmul_down_M")}

    line = {
        "metric": "Q4_K/Q8_0 GEMV weight GB/s & % of 8 TB/s HBM peak; prefill GEMM TFLOP/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_graph, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "llama3_8b_decode_step_q4_k",
            "calls_per_step": len(mats),
            "layers": synth.LLAMA3_8B_LAYERS,
            "projections": [p[0] for p in synth.LLAMA3_8B_LAYER],
            "weight_bytes_per_step": int(sum(m["rows"] * gq.gq_row_bytes(12, m["cols"])
                                              for m in mats)),
            "bytes_per_step": int(total_bytes),
            "launch": "hipGraph replay of 224 gq_matvec launches on one stream",
            "eager_ms_per_step": round(ms_eager, 4),
            "eager_GBps": round(total_bytes / (ms_eager * 1e-3) / 1e9, 1),
            "step_us_median": round(float(np.median(one)) * 1e3, 1),
            "step_us_min": round(float(np.min(one)) * 1e3, 1),
            "seed": 3,
        },
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "per_projection": per_proj,
        "fused_step_variant": fused,
        "int8_activation_step_variant": int8,
        "roofline": roofline,
        "prefill_q4_k_llama3_8b": config4,
        "cpu_baseline": cpu,
        "workloads": extras,
    }
    print(json.dumps(line), flush=True)
    return 0


def fused_step_variant(torch, gq, lib, synth, mats, timer, stream_ptr, args):
    """A labelled variant of the same decode step with the fused launches of
    the pages' design: per layer one gq_matvec over the q|k|v tensor (the
    three weight matrices concatenated row-wise, as a fused attn_qkv tensor
    stores them), gq_matvec_acc for o and for down (the residual add folded
    into the store), and gq_matvec_swiglu over the gate|up tensor: 128
    launches, the same 3.93 GB of weights."""
    f = gq.FMT_Q4_K
    layers = []
    nbytes = 0
    for layer in range(synth.LLAMA3_8B_LAYERS):
        m = mats[7 * layer:7 * layer + 7]
        q, k, v, o, gate, up, down = m
        wqkv = torch.cat([q["W"], k["W"], v["W"]])
        wgu = torch.cat([gate["W"], up["W"]])
        yqkv = torch.empty(q["rows"] + k["rows"] + v["rows"], dtype=torch.float32, device="cuda")
        h = torch.empty(gate["rows"], dtype=torch.float32, device="cuda")
        resid = torch.zeros(o["rows"], dtype=torch.float32, device="cuda")
        calls = [
            (lib.gq_matvec, (f, wqkv.data_ptr(), yqkv.numel(), q["cols"], q["x"].data_ptr(),
                             yqkv.data_ptr())),
            (lib.gq_matvec_acc, (f, o["W"].data_ptr(), o["rows"], o["cols"], o["x"].data_ptr(),
                                 resid.data_ptr())),
            (lib.gq_matvec_swiglu, (f, wgu.data_ptr(), gate["rows"], gate["cols"],
                                    gate["x"].data_ptr(), h.data_ptr())),
            (lib.gq_matvec_acc, (f, down["W"].data_ptr(), down["rows"], down["cols"],
                                 down["x"].data_ptr(), resid.data_ptr())),
        ]
        w = sum(t["W"].numel() for t in m)
        vec = 4 * (q["cols"] + yqkv.numel() + o["cols"] + 2 * o["rows"] + gate["cols"]
                   + gate["rows"] + down["cols"] + 2 * down["rows"])
        nbytes += w + vec
        layers.append(dict(keep=(wqkv, wgu, yqkv, h, resid), calls=calls))

    def fstep():
        sp = stream_ptr()
        for L in layers:
            for fn, a in L["calls"]:
                st = fn(*a, sp)
                if st != 0:
                    raise gq.GQError(st, "fused step")

    g = capture(torch, fstep)
    ms = timer.time(g.replay, args.steps, warmup=args.warmup)
    gbs = nbytes / (ms * 1e-3) / 1e9
    out = dict(launch="hipGraph replay of 128 launches: q|k|v matvec, o matvec_acc, gate|up "
                      "matvec_swiglu, down matvec_acc per layer",
               launches_per_step=4 * len(layers), ms_per_step=round(ms, 4),
               bytes_per_step=nbytes, GBps=round(gbs, 1),
               pct_hbm=round(100 * gbs / HBM_PEAK_GBS, 2))
    log(f"fused decode step variant: {out}")
    del g, layers
    torch.cuda.synchronize()
    return out


def int8_step_variant(torch, gq, lib, synth, mats, timer, stream_ptr, args):
    """The same 224 matrices with int8 activations (gq_matvec_q8_1 on each
    matrix's Q8_1-quantised x, quantised beforehand): the step, each
    projection, and the quantiser's cost per call (one activation row)."""
    xq = []
    for m in mats:
        q = gq.gq_quantize_q8_1(m["x"], 1, m["cols"])
        xq.append(q)
    torch.cuda.synchronize()

    def step(idx):
        sp = stream_ptr()
        for i in idx:
            m = mats[i]
            st = lib.gq_matvec_q8_1(gq.FMT_Q4_K, m["W"].data_ptr(), m["rows"], m["cols"],
                                    xq[i].data_ptr(), m["y"].data_ptr(), sp)
            if st != 0:
                raise gq.GQError(st, "gq_matvec_q8_1")

    every = list(range(len(mats)))
    g = capture(torch, lambda: step(every))
    st = timer.stats(g.replay, max(2, args.steps // 10), reps=5, warmup=2)
    wbytes = sum(m["rows"] * gq.gq_row_bytes(12, m["cols"]) + 36 * (m["cols"] // 32) + 4 * m["rows"]
                 for m in mats)
    out = dict(launch="hipGraph replay of 224 gq_matvec_q8_1 launches (activations quantised beforehand)",
               bytes_per_step=int(wbytes), step=rate_row(wbytes, 1, st))
    per = {}
    for proj in range(7):
        idx = [i for i, m in enumerate(mats) if m["name"] == synth.LLAMA3_8B_LAYER[proj][0]]
        gp = capture(torch, lambda idx=idx: step(idx))
        stp = timer.stats(gp.replay, max(2, args.steps // 10), reps=5, warmup=2)
        m = mats[idx[0]]
        per[m["name"]] = rate_row(m["rows"] * gq.gq_row_bytes(12, m["cols"]) + 36 * (m["cols"] // 32)
                                  + 4 * m["rows"], len(idx), stp)
        del gp
    out["per_projection"] = per
    x0 = mats[0]["x"]
    q0 = torch.empty(36 * (x0.numel() // 32), dtype=torch.uint8, device="cuda")

    def quant():
        sp = stream_ptr()
        for _ in range(32):
            lib.gq_quantize_q8_1(x0.data_ptr(), 1, x0.numel(), q0.data_ptr(), sp)

    gq_ = capture(torch, quant)
    mean, med, mn = timer.stats(gq_.replay, 5, reps=5, warmup=2)
    out["quantize_4096_us_per_call"] = round(med * 1e3 / 32, 3)
    log(f"int8 activation step: {out}")
    del g, gq_
    return out


def run_extras(torch, gq, lib, synth, timer, stream_ptr, args):
    out = {}
    iters = max(10, args.steps)

    # Q8_0 lm_head, cold: rotate 4 copies (580 MB > 2 x 256 MB Infinity Cache)
    fmt, rows, cols = synth.QWEN05_LM_HEAD
    W, x = synth.matrix_and_x(fmt, rows, cols, 2, 0)
    copies = [torch.from_numpy(W).cuda() for _ in range(4)]
    xd = torch.from_numpy(x).cuda()
    yd = torch.empty(rows, dtype=torch.float32, device="cuda")
    rb = gq.gq_row_bytes(fmt, cols)
    nbytes = gemv_bytes(rb, rows, cols)

    def lm(cs):
        sp = stream_ptr()
        for c in cs:
            lib.gq_matvec(fmt, c.data_ptr(), rows, cols, xd.data_ptr(), yd.data_ptr(), sp)

    st = timer.stats(lambda: lm(copies), max(2, iters // 5), reps=5, warmup=2)
    ms_warm = timer.time(lambda: lm(copies[:1] * 4), iters, warmup=2) / 4
    out["qwen05b_lm_head_q8_0"] = dict(shape=[rows, cols], seed=2, cold_rotating_copies=len(copies),
                                       **rate_row(nbytes, len(copies), st),
                                       warm_us_per_call=round(ms_warm * 1e3, 2))
    log(f"lm_head: {out['qwen05b_lm_head_q8_0']}")

    # the same lm_head with int8 activations (cold, same copies)
    xq = gq.gq_quantize_q8_1(xd, 1, cols)

    def lm8(cs):
        sp = stream_ptr()
        for c in cs:
            lib.gq_matvec_q8_1(fmt, c.data_ptr(), rows, cols, xq.data_ptr(), yd.data_ptr(), sp)

    st = timer.stats(lambda: lm8(copies), max(2, iters // 5), reps=5, warmup=2)
    out["qwen05b_lm_head_q8_0_int8_act"] = dict(shape=[rows, cols],
                                                **rate_row(rows * rb + 36 * (cols // 32) + 4 * rows,
                                                           len(copies), st))
    log(f"lm_head int8 activations: {out['qwen05b_lm_head_q8_0_int8_act']}")

    # the same lm_head repacked into the split per-row layout (scales apart
    # from the codes), cold over 4 copies like the packed one
    srb = gq.gq_row_bytes(gq.FMT_Q8_0_SPLIT, cols)
    split = [gq.gq_q8_0_split_repack(c, rows, cols) for c in copies]
    torch.cuda.synchronize()
    sbytes = gemv_bytes(srb, rows, cols)

    def lm_split(cs):
        sp = stream_ptr()
        for c in cs:
            lib.gq_matvec(gq.FMT_Q8_0_SPLIT, c.data_ptr(), rows, cols, xd.data_ptr(), yd.data_ptr(), sp)

    ms_cold = timer.time(lambda: lm_split(split), iters, warmup=2) / len(split)
    ms_warm = timer.time(lambda: lm_split(split[:1] * 4), iters, warmup=2) / 4
    out["qwen05b_lm_head_q8_0_split"] = dict(
        shape=[rows, cols], us_per_call=round(ms_cold * 1e3, 2),
        GBps=round(sbytes / (ms_cold * 1e-3) / 1e9, 1),
        pct_hbm=round(100 * sbytes / (ms_cold * 1e-3) / 1e9 / HBM_PEAK_GBS, 1),
        warm_us_per_call=round(ms_warm * 1e3, 2))
    log(f"lm_head split layout: {out['qwen05b_lm_head_q8_0_split']}")

    def repack():
        st = lib.gq_q8_0_split_repack(copies[0].data_ptr(), rows, cols, split[0].data_ptr(), stream_ptr())
        assert st == 0

    ms = timer.time(repack, 5, warmup=1)
    out["q8_0_split_repack_lm_head"] = dict(us_per_call=round(ms * 1e3, 1),
                                            GBps=round(rows * (rb + srb) / (ms * 1e-3) / 1e9, 1))
    del split

    # gq_dequant of the lm_head (bit-exact expansion, 545 MB written)
    dq = torch.empty((rows, cols), dtype=torch.float32, device="cuda")

    def dequant():
        st = lib.gq_dequant(fmt, copies[0].data_ptr(), rows, cols, dq.data_ptr())
        assert st == 0

    ms = timer.time(dequant, 5, warmup=1)
    dbytes = rows * rb + 4 * rows * cols
    out["dequant_lm_head_q8_0"] = dict(us_per_call=round(ms * 1e3, 1),
                                       GBps=round(dbytes / (ms * 1e-3) / 1e9, 1),
                                       pct_hbm=round(100 * dbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 1))
    del dq, copies

    # configs 0 and 1 (SmolLM-135M ffn_up Q8_0, the Qwen2.5-0.5B decode
    # shapes Q4_K): cold -- one launch per copy over more than 512 MB of
    # rotating copies in one graph, so W comes from HBM -- and warm (one copy
    # replayed 20 times, labelled warm_*)
    small = [("smollm135m_ffn_up_q8_0", synth.SMOLLM_FFN_UP, 0, 0)]
    small += [(f"qwen05b_{r}x{c}_q4_k", (f, r, c), 1, i)
              for i, (f, r, c) in enumerate(synth.QWEN05_DECODE)]
    for name, (f, r, c), seed, mid in small:
        W, x = synth.matrix_and_x(f, r, c, seed, mid)
        Wd, xd2 = torch.from_numpy(W).cuda(), torch.from_numpy(x).cuda()
        y2 = torch.empty(r, dtype=torch.float32, device="cuda")
        b = gemv_bytes(gq.gq_row_bytes(f, c), r, c)
        ncopy = min(8192, -(-(520 << 20) // W.size))
        big = torch.empty((ncopy, W.size), dtype=torch.uint8, device="cuda")
        big.copy_(Wd.unsqueeze(0).expand(ncopy, -1))
        base = big.data_ptr()

        def cold(f=f, r=r, c=c, base=base, n=ncopy, size=W.size, xd2=xd2, y2=y2):
            sp = stream_ptr()
            for i in range(n):
                lib.gq_matvec(f, base + i * size, r, c, xd2.data_ptr(), y2.data_ptr(), sp)

        def call(f=f, r=r, c=c, Wd=Wd, xd2=xd2, y2=y2):
            sp = stream_ptr()
            for _ in range(20):
                lib.gq_matvec(f, Wd.data_ptr(), r, c, xd2.data_ptr(), y2.data_ptr(), sp)

        gc = capture(torch, cold)
        st = timer.stats(gc.replay, 2, reps=5, warmup=1)
        g = capture(torch, call)
        stw = timer.stats(g.replay, 10, reps=5, warmup=2)
        warm = rate_row(b, 20, stw)
        out[name] = dict(shape=[r, c], seed=seed, cold_rotating_copies=ncopy,
                         cold_bytes=int(ncopy * W.size), **rate_row(b, ncopy, st),
                         **{f"warm_{k}": v for k, v in warm.items()})
        del gc, g, big
    log(f"configs 0 and 1: { {k: v for k, v in out.items() if 'q4_k' in k or 'smollm' in k} }")

    # the formats that Q4_K_M / Q5_K_M files mix in (Q6_K lm_head and
    # ffn_down, Q5_K projections, Q5_0 896-wide tensors), cold: enough
    # rotating copies to exceed 600 MB per pass
    for i, (name, f, r, c) in enumerate(synth.MIXED_FORMATS):
        _, _, _, _, W, x = synth.mixed_format_weight_and_x(i)
        ncopy = max(1, min(16, -(-600_000_000 // W.size)))
        cs = [torch.from_numpy(W).cuda() for _ in range(ncopy)]
        xd2 = torch.from_numpy(x).cuda()
        y2 = torch.empty(r, dtype=torch.float32, device="cuda")
        b = gemv_bytes(gq.gq_row_bytes(f, c), r, c)

        def mv(f=f, r=r, c=c, cs=cs, xd2=xd2, y2=y2):
            sp = stream_ptr()
            for w in cs:
                lib.gq_matvec(f, w.data_ptr(), r, c, xd2.data_ptr(), y2.data_ptr(), sp)

        g = capture(torch, mv)
        ms = timer.time(g.replay, max(5, iters // 2), warmup=2) / ncopy
        out[name] = dict(shape=[r, c], us_per_call=round(ms * 1e3, 2),
                         GBps=round(b / (ms * 1e-3) / 1e9, 1),
                         pct_hbm=round(100 * b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 1))
        del cs, g
    log(f"mixed formats: { {k: out[k] for k, *_ in synth.MIXED_FORMATS} }")

    # mixture-of-experts decode: one expert-batched launch per layer
    # projection (Qwen3-30B-A3B-style: 128 experts of 768 x 2048, top 8;
    # Mixtral-style: 8 experts of 14336 x 4096, top 2), random distinct
    # expert ids per call. The 128-expert tensor (113 MB) fits in the 256 MB
    # Infinity Cache, so its figure is partly warm; the 8-expert one (264 MB)
    # is not.
    for name, (f, n_expert, r, c, topk) in {
            "moe_top8_of_128_768x2048_q4_k": (12, 128, 768, 2048, 8),
            "moe_top2_of_8_14336x4096_q4_k": (12, 8, 14336, 4096, 2)}.items():
        rng = synth.rng_for(6, n_expert)
        W = synth.weights(f, n_expert * r, c, rng)
        Wd = torch.from_numpy(W).cuda()
        del W
        xd2 = torch.from_numpy(synth.activations(c, rng)).cuda()
        ncall = 16
        ids = [torch.from_numpy(rng.permutation(n_expert)[:topk].astype(np.int32)).cuda()
               for _ in range(ncall)]
        Y2 = torch.empty((topk, r), dtype=torch.float32, device="cuda")
        b = topk * gemv_bytes(gq.gq_row_bytes(f, c), r, c)

        def moe(f=f, n_expert=n_expert, r=r, c=c, topk=topk, Wd=Wd, xd2=xd2, ids=ids, Y2=Y2):
            sp = stream_ptr()
            for e in ids:
                st = lib.gq_matvec_experts(f, Wd.data_ptr(), n_expert, r, c, xd2.data_ptr(), topk,
                                           e.data_ptr(), topk, Y2.data_ptr(), sp)
                assert st == 0

        g = capture(torch, moe)
        ms = timer.time(g.replay, max(5, iters // 2), warmup=2) / ncall
        out[name] = dict(us_per_call=round(ms * 1e3, 2), expert_bytes_per_call=int(b),
                         GBps=round(b / (ms * 1e-3) / 1e9, 1),
                         pct_hbm=round(100 * b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 1))
        del g
        if n_expert == 8:
            # the prefill of the same layer: 512 tokens, top 2, bucketed by
            # expert (a skewed split of the 1024 rows), one grouped call
            counts = [230, 190, 150, 130, 110, 90, 74, 50]
            Xg = torch.from_numpy(synth.activations((sum(counts), c), rng)).cuda()
            Yg = torch.empty((sum(counts), r), dtype=torch.float32, device="cuda")
            import ctypes
            carr = (ctypes.c_int64 * n_expert)(*counts)

            def grouped(f=f, r=r, c=c, Wd=Wd, Xg=Xg, Yg=Yg, carr=carr):
                st = lib.gq_matmul_experts(f, Wd.data_ptr(), n_expert, r, c, Xg.data_ptr(), carr,
                                           Yg.data_ptr(), stream_ptr())
                assert st == 0

            ms = timer.time(grouped, 5, warmup=1)
            tf = 2.0 * sum(counts) * r * c / (ms * 1e-3) / 1e12
            out["moe_prefill_512x2_of_8_14336x4096_q4_k"] = dict(
                rows_per_expert=counts, us_per_call=round(ms * 1e3, 1), TFLOPs=round(tf, 2),
                pct_mfma_f16_peak=round(100 * tf / MFMA_F16_PEAK_TFLOPS, 2))
            # the device-side steps around it: bucketing of the 1024
            # assignments (ids giving the same split, in shuffled order), the
            # gather of the 512 activation rows into bucket order, the
            # weighted scatter of the 1024 expert rows back onto 512 outputs,
            # and the whole chain with the counts copied to the host
            n_tok, k = 512, 2
            idv = rng.permutation(np.repeat(np.arange(n_expert, dtype=np.int32), counts)).astype(np.int32)
            idd = torch.from_numpy(idv).cuda()
            cnt = torch.empty(n_expert, dtype=torch.int64, device="cuda")
            ordr = torch.empty(n_tok * k, dtype=torch.int32, device="cuda")
            posd = torch.empty(n_tok * k, dtype=torch.int32, device="cuda")
            Xt = torch.from_numpy(synth.activations((n_tok, c), rng)).cuda()
            wts = torch.rand(n_tok * k, dtype=torch.float32, device="cuda")
            outd = torch.zeros((n_tok, r), dtype=torch.float32, device="cuda")

            def bucket():
                assert lib.gq_moe_bucket(idd.data_ptr(), n_tok * k, n_expert, cnt.data_ptr(), ordr.data_ptr(),
                                         posd.data_ptr(), stream_ptr()) == 0

            def gather():
                assert lib.gq_moe_gather(Xt.data_ptr(), c, k, posd.data_ptr(), n_tok * k, Xg.data_ptr(),
                                         stream_ptr()) == 0

            def scatter():
                assert lib.gq_moe_scatter(Yg.data_ptr(), r, posd.data_ptr(), wts.data_ptr(), n_tok * k, k,
                                          outd.data_ptr(), stream_ptr()) == 0

            def chain():
                bucket()
                gather()
                m = cnt.cpu().tolist()
                ca = (ctypes.c_int64 * n_expert)(*m)
                assert lib.gq_matmul_experts(f, Wd.data_ptr(), n_expert, r, c, Xg.data_ptr(), ca,
                                             Yg.data_ptr(), stream_ptr()) == 0
                scatter()

            def chain_dev():
                bucket()
                gather()
                assert lib.gq_matmul_experts_dev(f, Wd.data_ptr(), n_expert, r, c, Xg.data_ptr(), cnt.data_ptr(),
                                                 n_tok * k, Yg.data_ptr(), stream_ptr()) == 0
                scatter()

            bucket()
            torch.cuda.synchronize()
            assert cnt.cpu().tolist() == counts
            gchain = capture(torch, chain_dev)
            ms_gc = timer.time(gchain.replay, 5, warmup=1)
            del gchain
            ms_b = timer.time(bucket, 20, warmup=2)
            ms_g = timer.time(gather, 20, warmup=2)
            ms_s = timer.time(scatter, 20, warmup=2)
            ms_c = timer.time(chain, 5, warmup=1)
            gb_g = (n_tok * c * 4 + n_tok * k * c * 4) / 1e9
            gb_s = (n_tok * k * r * 4 + 2 * n_tok * r * 4) / 1e9
            out["moe_prefill_device_steps_512x2_of_8"] = dict(
                bucket_us=round(ms_b * 1e3, 2), gather_us=round(ms_g * 1e3, 2),
                gather_GBps=round(gb_g / (ms_g * 1e-3), 1), scatter_us=round(ms_s * 1e3, 2),
                scatter_GBps=round(gb_s / (ms_s * 1e-3), 1),
                chain_us=round(ms_c * 1e3, 1),
                chain="bucket + gather + counts to the host + gq_matmul_experts + scatter",
                chain_device_counts_graph_us=round(ms_gc * 1e3, 1))
            del Xg, Yg, Xt, outd
        del Wd
    log(f"moe: { {k: v for k, v in out.items() if k.startswith('moe')} }")

    # prefill products of the other formats (the Llama-3-8B Q6_K down and
    # Q5_K gate shapes and the Qwen2.5-0.5B Q5_0 4864x896, all on the fp16
    # matrix cores)
    for i in (1, 3, 7):
        name, f, r, c, W, _ = synth.mixed_format_weight_and_x(i)
        Wd = torch.from_numpy(W).cuda()
        del W
        for M in synth.PREFILL_M:
            Xd = torch.from_numpy(synth.activations((M, c), synth.rng_for(911, M))).cuda()
            Yd = torch.empty((M, r), dtype=torch.float32, device="cuda")

            def mmf(f=f, r=r, c=c, M=M, Wd=Wd, Xd=Xd, Yd=Yd):
                st = lib.gq_matmul(f, Wd.data_ptr(), r, c, Xd.data_ptr(), M, Yd.data_ptr(),
                                   stream_ptr())
                assert st == 0

            ms = float(np.median([timer.time(mmf, 10 if M < 512 else 5, warmup=1) for _ in range(3)]))
            tf = 2.0 * M * r * c / (ms * 1e-3) / 1e12
            out[f"matmul_{name}_M{M}"] = dict(us_per_call=round(ms * 1e3, 1), TFLOPs=round(tf, 2),
                                              pct_mfma_f16_peak=round(100 * tf / MFMA_F16_PEAK_TFLOPS, 2))
        del Wd
    log(f"mixed-format prefill: { {k: v for k, v in out.items() if k.startswith(('matmul_llama3', 'matmul_qwen'))} }")

    # Q8_0 prefill products at the Llama-3-8B gate and down shapes (fp16
    # matrix cores), packed and in the split per-row layout; weights seed 6,
    # matrix_id 0 (gate) / 1 (down)
    for k, (which, r, c) in enumerate((("gate", 14336, 4096), ("down", 4096, 14336))):
        Wd = torch.from_numpy(synth.weights(gq.FMT_Q8_0, r, c, synth.rng_for(6, k))).cuda()
        Sd = gq.gq_q8_0_split_repack(Wd, r, c)
        for f, Wf, tag in ((gq.FMT_Q8_0, Wd, "q8_0"), (gq.FMT_Q8_0_SPLIT, Sd, "q8_0_split")):
            for M in synth.PREFILL_M:
                Xd = torch.from_numpy(synth.activations((M, c), synth.rng_for(911, M))).cuda()
                Yd = torch.empty((M, r), dtype=torch.float32, device="cuda")

                def mq(f=f, Wf=Wf, r=r, c=c, M=M, Xd=Xd, Yd=Yd):
                    st = lib.gq_matmul(f, Wf.data_ptr(), r, c, Xd.data_ptr(), M, Yd.data_ptr(),
                                       stream_ptr())
                    assert st == 0

                _, ms, ms_min = timer.stats(mq, 10 if M < 512 else 5, reps=3, warmup=1)
                tf = 2.0 * M * r * c / (ms * 1e-3) / 1e12
                out[f"matmul_{tag}_{which}_M{M}"] = dict(
                    us_per_call=round(ms * 1e3, 1), us_min=round(ms_min * 1e3, 1), TFLOPs=round(tf, 2),
                    pct_mfma_f16_peak=round(100 * tf / MFMA_F16_PEAK_TFLOPS, 2))
        del Wd, Sd
    log(f"q8_0 prefill: { {k: v for k, v in out.items() if k.startswith('matmul_q8_0')} }")

    # Q4_K products with a few (M = 2, 4, 8) and many activation rows at the
    # Llama-3-8B prefill shapes (matrix cores)
    for which in ("gate", "down"):
        for M in SMALL_M + synth.PREFILL_M:
            W, X, rows, cols = synth.prefill_inputs(which, M)
            Wd, Xd = torch.from_numpy(W).cuda(), torch.from_numpy(X).cuda()
            Yd = torch.empty((M, rows), dtype=torch.float32, device="cuda")

            def mm(Wd=Wd, Xd=Xd, Yd=Yd, rows=rows, cols=cols, M=M):
                st = lib.gq_matmul(12, Wd.data_ptr(), rows, cols, Xd.data_ptr(), M,
                                   Yd.data_ptr(), stream_ptr())
                assert st == 0

            # median of three timed loops (a single loop of these short
            # calls is at the mercy of one slow launch)
            _, ms, ms_min = timer.stats(mm, 10 if M < 512 else 5, reps=5, warmup=1)
            flops = 2.0 * M * rows * cols
            wb = rows * gq.gq_row_bytes(12, cols) + 4 * M * (rows + cols)
            tf = flops / (ms * 1e-3) / 1e12
            key = f"matmul_{which}_M{M}"
            out[key] = dict(
                us_per_call=round(ms * 1e3, 1), us_min=round(ms_min * 1e3, 1), TFLOPs=round(tf, 2),
                pct_mfma_f16_peak=round(100 * tf / MFMA_F16_PEAK_TFLOPS, 2),
                GBps=round(wb / (ms * 1e-3) / 1e9, 1),
                pct_hbm=round(100 * wb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2))
            log(f"matmul {which} M={M}: {out[key]}")
    return out


def gpu_config_outputs(torch, gq, synth):
    """One gq_matvec / gq_matmul of every config on fresh buffers, copied to
    the host: the GPU side of the per-config error the CPU leg reports."""
    out = {}

    def mv(fmt, W, rows, cols, x):
        return gq.gq_matvec(fmt, torch.from_numpy(W).cuda(), rows, cols, torch.from_numpy(x).cuda())

    f, r, c = synth.SMOLLM_FFN_UP
    W, x = synth.matrix_and_x(f, r, c, 0, 0)
    out["config0"] = [(f, W, r, c, x[None, :], mv(f, W, r, c, x))]
    out["config1"] = []
    for i, (f, r, c) in enumerate(synth.QWEN05_DECODE):
        W, x = synth.matrix_and_x(f, r, c, 1, i)
        out["config1"].append((f, W, r, c, x[None, :], mv(f, W, r, c, x)))
    f, r, c = synth.QWEN05_LM_HEAD
    W, x = synth.matrix_and_x(f, r, c, 2, 0)
    out["config2"] = [(f, W, r, c, x[None, :], mv(f, W, r, c, x))]
    out["config3"] = []
    for proj in range(7):
        name, r, c, _, _ = synth.llama3_8b_matrix(0, proj)
        W, x = synth.llama3_8b_weight_and_x(0, proj)
        out["config3"].append((12, W, r, c, x[None, :], mv(12, W, r, c, x)))
    out["config4"] = []
    for M in (16, 64):
        for which in ("gate", "down"):
            W, X, r, c = synth.prefill_inputs(which, M)
            Y = gq.gq_matmul(12, torch.from_numpy(W).cuda(), r, c, torch.from_numpy(X).cuda())
            out["config4"].append((12, W, r, c, X, Y))
    torch.cuda.synchronize()
    for k, v in out.items():
        out[k] = [(f, W, r, c, X, Y.cpu().numpy().reshape(X.shape[0], r)) for f, W, r, c, X, Y in v]
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(synth, seconds: float, gpu=None):
    """The C oracle (dequant + f64 dot) on the host cores. value: weight GB/s
    over the q, k, v, o, gate, up, down matrices of layer 0 of the decode step
    on N threads, repeated for about `seconds`; beside it one pass on one
    thread, and the oracle's time per call of every config (N threads and one
    thread; config 3 as 32 x layer 0, config 4 at M = 512 as 8 x M = 64,
    both marked as scaled), and, with `gpu` (gpu_config_outputs), the largest
    |y - y_ref| / sum |w x| of the GPU output of each config."""
    import oracle

    try:
        threads = len(os.sched_getaffinity(0))
    except AttributeError:
        threads = os.cpu_count() or 1
    threads = max(1, min(16, threads))  # one GPU's share of the host
    mats = []
    for proj in range(7):
        name, rows, cols, _, _ = synth.llama3_8b_matrix(0, proj)
        W, x = synth.llama3_8b_weight_and_x(0, proj)
        mats.append((rows, cols, W, x))
    per_pass = sum(r * oracle.row_bytes(12, c) + 4 * (r + c) for r, c, _, _ in mats)

    def one_pass(n):
        for rows, cols, W, x in mats:
            oracle.matvec(12, W, rows, cols, x, nthreads=n)

    done = 0
    passes = 0
    t0 = time.perf_counter()
    while True:
        one_pass(threads)
        passes += 1
        done += per_pass
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    t1 = time.perf_counter()
    one_pass(1)
    dt1 = time.perf_counter() - t1

    def timed(fn, n):
        t = time.perf_counter()
        r = fn(n)
        return (time.perf_counter() - t) * 1e6, r

    per_config = {}
    errors = {}
    for key, cases in (gpu or {}).items():
        rows_out = []
        worst = 0.0
        for f, W, r, c, X, Y in cases:
            M = X.shape[0]
            t_n, (ref, S) = timed(lambda n: oracle.matmul(f, W, r, c, X, nthreads=n), threads)
            row = dict(shape=[r, c], M=M, oracle_us_nthreads=round(t_n, 1))
            if key != "config4":  # the prefill products take seconds on one thread
                row["oracle_us_1thread"] = round(timed(lambda n: oracle.matmul(f, W, r, c, X, nthreads=n), 1)[0], 1)
            rows_out.append(row)
            err = np.abs(Y.astype(np.float64) - ref)
            with np.errstate(divide="ignore", invalid="ignore"):
                rel = np.where(S > 0, err / S, np.where(err > 0, np.inf, 0.0))
            worst = max(worst, float(rel.max()))
        errors[key] = worst
        if key == "config3":
            n_us = sum(x["oracle_us_nthreads"] for x in rows_out)
            one_us = sum(x["oracle_us_1thread"] for x in rows_out)
            per_config[key] = dict(layer0=rows_out, step_oracle_us_nthreads_scaled=round(32 * n_us, 1),
                                   step_oracle_us_1thread_scaled=round(32 * one_us, 1),
                                   note="step = 32 x layer 0 (scaled, not timed)")
        elif key == "config4":
            m64 = [x for x in rows_out if x["M"] == 64]
            per_config[key] = dict(measured=rows_out,
                                   M512_oracle_us_nthreads_scaled=[dict(shape=x["shape"],
                                                                        us=round(8 * x["oracle_us_nthreads"], 1))
                                                                   for x in m64],
                                   note="M = 512 as 8 x M = 64 (scaled, not timed)")
        else:
            per_config[key] = rows_out
    return {"value": round(done / dt / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "value_1thread": round(per_pass / dt1 / 1e9, 3),
            "sample": f"{passes} pass(es) over layer 0's 7 Q4_K projections "
                      f"({per_pass / 1e6:.1f} MB per pass) of the decode step on {threads} threads, "
                      f"f64 accumulation, {dt:.1f}s; one pass on 1 thread, {dt1:.1f}s",
            "per_config": per_config,
            "max_rel_err": errors}


if __name__ == "__main__":
    sys.exit(main())
