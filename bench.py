#!/usr/bin/env python3
"""Benchmark of the quantized-matmul hot path on one MI355X.

Headline workload (decode, M = 1): the four Llama-3-8B-shaped matrices
W [4096,4096], [1024,4096], [14336,4096], [4096,14336] at 4 bits, G = 64,
fp16 activations x [1, K] ~ N(0, 1), weights ~ N(0, 0.02) with 0.1% outliers
x20, quantized on the device by aq_quantize.  One step = one y = x @ W^T per
matrix through the shape dispatch (aq_quantized_matmul), each on a cold copy
of its packed weights: the step rotates over enough distinct copies (>= 1 GiB
of packed weights in total, four times the 256 MB last-level cache) that
every launch streams its weights from HBM.  Steps are replayed from HIP
graphs (one replay runs a step on every cold copy) so host launch overhead
stays off the device timeline.

value = packed weight bytes (codes + scales + biases) of the timed steps /
the timed wall interval on the device (effective weight GB/s, the metric's
first part).  The JSON line also carries:
  roofline      the dominant decode kernel's achieved algorithmic bytes/s
                (weights + x + y per launch / average launch duration, timed
                live with HIP events on the launch stream over graphs of
                back-to-back launches) vs 8 TB/s, and its HBM traffic per
                launch from the committed counter summary when it matches the
                current kernel source;
  cpu_baseline  the CPU oracle computing the same decode step on the host
                cores (value), with "legs" timing it beside every other
                section on bounded samples of the same inputs: spec-decode
                (M = 4), MoE gather, quantize, prefill (a few rows of X
                against the whole W) and the tiny 512 x 512 case on one
                thread; nproc, OpenMP threads and the CPU model are stated;
  qmm           the metric's second part: prefill Y = X @ W^T with X bf16
                [2048, 8192] and W [28672, 8192] at 4-bit G=64 (plus 3-bit
                G=64 and 2-bit G=32), TFLOP/s vs the 2.5 PFLOP/s dense bf16 peak
                and vs an MFMA-only loop measured on the device (with the
                shader clock it runs at).
Per decode shape the line also carries the time of a plain streaming read of
the same bytes (same cold rotation and timing), a measured second denominator.
  specdec, moe  the M = 2..8 matrix-vector kernels (bf16 x, [14336, 4096] and
                [4096, 14336] at 4/64 and 8/128; also M = 16 and 64, sliced
                few-row kernel) and the MoE gather kernel
                (32 tokens, top-6 of 64 experts), % of HBM per launch on cold
                weights; plus the matrix-core gather on the same experts at
                prefill size (2048 tokens, top-6), TFLOP/s;
  quantize_dequantize  aq_quantize of the prefill-size matrix (fp32 in),
                aq_dequantize of it to bf16 (% of HBM), the integer-zero-point
                aq_quantize_zp and the range-search aq_quantize_mse over 21
                narrowed ranges;
  fp_modes      the block-scaled float modes mxfp4, nvfp4 and mxfp8: the
                decode product on the four decode matrices, with the plain
                read of the same bytes, and quantize / dequantize of the
                prefill-size matrix, per mode;
  embedding     quantized embedding lookups (rows of a [128256, 4096] 8-bit
                table dequantized to bf16) for 1 and 2048 tokens.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "QMV M=1 effective weight GB/s (% of HBM peak); QMM TFLOP/s (% MFMA peak)"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
DECODE_SHAPES = [(4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336)]
G, BITS = 64, 4
PREFILL = dict(M=2048, N=28672, K=8192, settings=[(4, 64), (3, 64), (2, 32)])
COLD_BYTES = 1 << 30


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-baseline leg")
    p.add_argument("--no-qmm", action="store_true", help="skip the prefill (QMM) section")
    p.add_argument("--no-embedding", action="store_true", help="skip the embedding section")
    p.add_argument("--no-extra", action="store_true",
                   help="skip the spec-decode (M = 2..8) and MoE gather sections")
    p.add_argument("--no-fp-modes", action="store_true",
                   help="skip the block-scaled float modes section (mxfp4, nvfp4, mxfp8)")
    p.add_argument("--qmm-iters", type=int, default=20)
    p.add_argument("--copy-probe", action="store_true",
                   help="also run a plain 512 MiB device copy (counter calibration)")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    return p.parse_args()


def _spin(torch):
    """Keep the device busy briefly so the host can queue launches ahead."""
    try:
        torch.cuda._sleep(20_000_000)
    except (AttributeError, RuntimeError):
        pass


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the kernels shard by rows or experts, see the design notes)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import group_wise_affine_aq_amd as aq
    from group_wise_affine_aq_amd import inputs

    aq.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    props = torch.cuda.get_device_properties(dev)
    print(f"# device: {props.name} ({getattr(props, 'gcnArchName', '?')}), "
          f"{props.multi_processor_count} CUs", file=sys.stderr, flush=True)

    # ---- decode workload ---------------------------------------------------------------
    mats = []
    for i, (N, K) in enumerate(DECODE_SHAPES):
        w = inputs.weights_device(N, K, device=dev, seed=0, key=(1, i), outliers=True)
        c, s, b = aq.aq_quantize(w, G, BITS)
        del w
        x = inputs.activations_device(1, K, "f16", device=dev, seed=0, key=(1, i))
        y = torch.empty((1, N), dtype=torch.float16, device=dev)
        wbytes = aq.aq_qweight_bytes(N, K, G, BITS)
        mats.append(dict(N=N, K=K, packed=(c, s, b), x=x, y=y, wbytes=wbytes,
                         algo_bytes=wbytes + 2 * K + 2 * N))
    step_wbytes = sum(m["wbytes"] for m in mats)
    copies = max(2, math.ceil(COLD_BYTES / step_wbytes))
    sets = [[m["packed"] for m in mats]]
    for _ in range(copies - 1):
        sets.append([tuple(t.clone() for t in m["packed"]) for m in mats])
    torch.cuda.synchronize()
    print(f"# decode: {len(mats)} matrices, {step_wbytes} packed bytes/step, {copies} cold copies",
          file=sys.stderr, flush=True)

    def step(ci):
        for m, (c, s, b) in zip(mats, sets[ci]):
            aq.aq_quantized_matmul(m["x"], c, s, b, G, BITS, y=m["y"])

    # Steps are replayed from HIP graphs: `round_graph` holds one step on each
    # cold copy in turn (a replay is `copies` steps), `step_graphs[ci]` one
    # step on copy ci (for the remainder), so exactly K steps run.
    for ci in range(copies):  # eager pass first (also loads the kernels)
        step(ci)
    torch.cuda.synchronize()
    gstream = torch.cuda.Stream()
    step_graphs = []
    with torch.cuda.stream(gstream):
        round_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(round_graph, stream=gstream):
            for ci in range(copies):
                step(ci)
        for ci in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=gstream):
                step(ci)
            step_graphs.append(g)
    torch.cuda.synchronize()

    def run_steps(n):
        for _ in range(n // copies):
            round_graph.replay()
        for ci in range(n % copies):
            step_graphs[ci].replay()

    run_steps(args.warmup)
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps --------------------------------------------------
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    run_steps(args.steps)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t0.elapsed_time(t1)
    ms_per_step = ms_total / args.steps
    value = step_wbytes * args.steps / (ms_total * 1e-3) / 1e9
    print(f"# timed {args.steps} steps: {ms_per_step * 1e3:.2f} us/step (device), "
          f"host wall {wall * 1e6 / args.steps:.2f} us/step", file=sys.stderr, flush=True)

    # ---- per-launch durations (HIP events on the launch stream) ---------------------------
    # For each shape: one graph of `reps` back-to-back launches over the cold
    # copies, replayed between two events on the launch stream; per-launch time
    # = elapsed / reps.  It includes the dispatch gap between consecutive graph
    # kernels, which kernel-trace durations leave out.
    reps = 2 * copies
    per_shape = []
    for j, m in enumerate(mats):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(gstream):
            with torch.cuda.graph(g, stream=gstream):
                for r in range(reps):
                    c, s, b = sets[r % copies][j]
                    aq.aq_quantized_matmul(m["x"], c, s, b, G, BITS, y=m["y"])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        durs = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            durs.append(e0.elapsed_time(e1) * 1e3 / reps)  # us per launch
        del g
        avg = sum(durs) / len(durs)
        per_shape.append(dict(shape=[m["N"], m["K"]], weight_bytes=m["wbytes"],
                              algo_bytes=m["algo_bytes"], launches=reps * 5,
                              kernel=aq.aq_qmv_describe(1, m["N"], m["K"], G, BITS, "f16"),
                              avg_us=round(avg, 3), min_us=round(min(durs), 3),
                              weight_gbs=round(m["wbytes"] / (avg * 1e-6) / 1e9, 1),
                              pct_hbm=round(100 * m["wbytes"] / (avg * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)))
        print(f"# QMV {m['N']}x{m['K']} ({per_shape[-1]['kernel']}): {avg:.2f} us/launch in-graph, "
              f"{per_shape[-1]['weight_gbs']} GB/s weights", file=sys.stderr, flush=True)
    # ---- second denominator: a plain streaming read of the same bytes -------------------
    # Same cold rotation and the same graph timing, best of a few launch shapes.
    for ps, m in zip(per_shape, mats):
        ps["read_ceiling_us"] = round(_read_ceiling_us(aq, torch, m["wbytes"], stream), 3)
        ps["read_ceiling_gbs"] = round(m["wbytes"] / (ps["read_ceiling_us"] * 1e-6) / 1e9, 1)
        ps["frac_of_read_ceiling"] = round(ps["read_ceiling_us"] / ps["avg_us"], 3)
        print(f"# plain read of {m['wbytes']} B: {ps['read_ceiling_us']:.2f} us "
              f"({ps['read_ceiling_gbs']} GB/s); kernel at {ps['frac_of_read_ceiling']:.2f} of it",
              file=sys.stderr, flush=True)
    # the sustained read rate: the same plain reads over 1 GiB per launch, where
    # the fixed cost of a launch no longer weighs
    big_us = _read_ceiling_us(aq, torch, 1 << 30, stream)
    sustained = {"bytes": 1 << 30, "avg_us": round(big_us, 2),
                 "gbs": round((1 << 30) / (big_us * 1e-6) / 1e9, 1)}
    print(f"# plain read of 1 GiB: {big_us:.1f} us ({sustained['gbs']} GB/s)", file=sys.stderr,
          flush=True)
    # context: the same product with dense bf16 weights (torch's F.linear ->
    # hipBLASLt), cold copies, on the two 33 MB shapes (112 MB of bf16 each)
    import torch.nn.functional as F
    for ps, m in zip(per_shape, mats):
        if m["N"] * m["K"] < 4096 * 14336:
            continue
        nb = m["N"] * m["K"] * 2
        dcopies = max(2, math.ceil(COLD_BYTES / nb))
        ws = [torch.empty((m["N"], m["K"]), dtype=torch.bfloat16, device=dev).normal_(0, 0.02)
              for _ in range(dcopies)]
        xb = m["x"].to(torch.bfloat16)
        F.linear(xb, ws[0])  # library set-up outside the capture
        torch.cuda.synchronize()
        us = _graph_us(torch, stream, [lambda wc=wc: F.linear(xb, wc) for wc in ws] * 2)
        ps["dense_bf16_linear_us"] = round(us, 3)
        ps["speedup_vs_dense_bf16"] = round(us / ps["avg_us"], 2)
        print(f"# dense bf16 F.linear {m['N']}x{m['K']} ({nb} B): {us:.2f} us; the 4-bit kernel is "
              f"{us / ps['avg_us']:.2f}x faster", file=sys.stderr, flush=True)
        del ws
        torch.cuda.synchronize()
    # the dominant kernel: the instantiation with the most device time per step
    by_kernel = {}
    for ps in per_shape:
        by_kernel.setdefault(ps["kernel"], []).append(ps)
    kname, group = max(by_kernel.items(), key=lambda kv: sum(p["avg_us"] for p in kv[1]))
    g_algo = sum(p["algo_bytes"] for p in group)
    g_us = sum(p["avg_us"] for p in group)
    achieved = g_algo / (g_us * 1e-6) / 1e9
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=_traffic(kname, group),
                    kernel=kname, shapes=[p["shape"] for p in group],
                    launches_per_step=len(group), avg_launch_us=round(g_us / len(group), 3),
                    algo_bytes_per_launch=round(g_algo / len(group)),
                    read_ceiling_gbs=round(g_algo / (sum(p["read_ceiling_us"] for p in group)
                                                     * 1e-6) / 1e9, 1),
                    frac_of_read_ceiling=round(sum(p["read_ceiling_us"] for p in group) / g_us, 3))

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "decode QMV M=1, W [4096,4096] [1024,4096] [14336,4096] "
                               "[4096,14336], 4-bit G=64, fp16 x, cold weights",
                   "step_weight_bytes": step_wbytes, "cold_copies": copies,
                   "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 1)},
        "roofline": roofline,
        "per_shape": per_shape,
        "sustained_read_1gib": sustained,
    }

    if args.copy_probe:
        a = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        bb = torch.empty_like(a)
        for _ in range(3):
            bb.copy_(a)
        torch.cuda.synchronize()

    # ---- CPU baseline: the CPU oracle on the same step -----------------------------------
    legs = None
    if not args.no_cpu:
        result["cpu_baseline"] = _cpu_baseline(mats, args.cpu_seconds)
        legs = result["cpu_baseline"]["legs"]

    # ---- spec-decode (M = 2..8) and MoE gather: % of HBM per launch ------------------------
    if not args.no_extra:
        result["specdec"] = _specdec(aq, inputs, dev, stream, legs)
        result["moe"] = _moe(aq, inputs, dev, stream, legs)

    # ---- quantize and dequantize (offline conversion, standalone decode) -------------------
    if not args.no_extra:
        result["quantize_dequantize"] = _quant_dequant(aq, inputs, dev, stream, legs)

    # ---- block-scaled float modes ---------------------------------------------------------
    if not args.no_fp_modes:
        result["fp_modes"] = _fp_modes(aq, inputs, dev, stream, legs)

    # ---- quantized embedding ---------------------------------------------------------------
    if not args.no_embedding:
        del round_graph, step_graphs, sets
        torch.cuda.synchronize()
        result["embedding"] = _embedding(aq, inputs, dev, stream)

    # ---- prefill (QMM) ---------------------------------------------------------------------
    if not args.no_qmm:
        if args.no_embedding:
            del round_graph, step_graphs, sets
        torch.cuda.synchronize()
        result["qmm"] = _qmm(aq, inputs, dev, args.qmm_iters, legs)

    print(json.dumps(result), flush=True)


def _read_ceiling_us(aq, torch, nbytes, stream):
    """Per-launch time of a plain streaming read of nbytes cold bytes (graph of
    back-to-back launches over >= 1 GiB of rotating buffers, HIP events): the
    best of grid-stride reads at four launch shapes and one-shot reads (all of
    a thread's loads in flight at once, a contiguous block per workgroup) at
    three, the fastest forms a sweep of 3 block sizes x 3 depths x 4 grid
    sizes found on the MI355X."""
    copies = max(2, math.ceil(COLD_BYTES / nbytes))
    bufs = [torch.empty(nbytes // 4, dtype=torch.int32, device=stream.device) for _ in range(copies)]
    for b in bufs:
        b.fill_(1)
    sink = torch.zeros(4, dtype=torch.int32, device=stream.device)
    best = float("inf")
    gs = torch.cuda.Stream()
    shapes = [("stride", 512, 4), ("stride", 1024, 4), ("stride", 2048, 1), ("stride", 512, 8),
              ("oneshot", 256, 8), ("oneshot", 512, 4), ("oneshot", 256, 4)]
    for kind, a, unroll in shapes:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(gs):
            with torch.cuda.graph(g, stream=gs):
                for i in range(copies):
                    if kind == "stride":
                        aq.aq_bench_stream_read(bufs[i], a, unroll, sink=sink)
                    else:
                        aq.aq_bench_read_oneshot(bufs[i], a, unroll, sink=sink)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e3 / copies)
        del g
    del bufs
    torch.cuda.synchronize()
    return best


def _mfma_clock(aq, torch, cus):
    """Shader clock and rate of an MFMA-only loop (one wave per SIMD on every CU)."""
    iters = 20000
    aq.aq_bench_mfma_clock(cus, 100)
    torch.cuda.synchronize()
    out = aq.aq_bench_mfma_clock(cus, iters)
    torch.cuda.synchronize()
    t = out.double().cpu()
    secs = t[:, 1].mean().item() / 1e8
    ghz = t[:, 0].mean().item() / secs / 1e9
    tflops = 4 * cus * 14 * iters * 32768 / secs / 1e12
    return round(ghz, 3), round(tflops, 1)


def _traffic(kname, group):
    """HBM bytes per launch of the roofline kernel from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known size;
    one line per decode instantiation), or None when the summary was taken
    on another kernel source or does not cover this kernel."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "qmv_decode_m1_traffic.txt")
    src = os.path.join(ROOT, "group_wise_affine_aq_amd", "csrc", "aq_qmv.hip")
    if not os.path.exists(path):
        return None
    sha, per_kernel = None, {}
    for line in open(path):
        if line.startswith("#") or ":" not in line:
            continue
        k, v = line.rsplit(":", 1)
        k, v = k.strip(), v.strip()
        if k == "source_sha256_16":
            sha = v
        elif k.startswith("hbm_bytes_per_launch "):
            per_kernel[k[len("hbm_bytes_per_launch "):]] = v
    if sha != hashlib.sha256(open(src, "rb").read()).hexdigest()[:16] or kname not in per_kernel:
        return None
    try:
        return float(per_kernel[kname])
    except ValueError:
        return None


def _host_packed(c, s, b):
    """Device packed weights -> the oracle's numpy arrays."""
    import numpy as np
    import torch
    return (c.cpu().numpy().view(np.uint32), s.view(torch.int16).cpu().numpy().view(np.uint16),
            b.view(torch.int16).cpu().numpy().view(np.uint16))


def _host_x(x, dtype):
    """Device fp16/bf16 activations -> exact float64 values."""
    import numpy as np
    import torch
    from group_wise_affine_aq_amd import inputs as _inp
    return _inp.from_bits(x.view(torch.int16).cpu().numpy().view(np.uint16), dtype)


def _cpu_timed(fn, seconds):
    """Run fn until at least `seconds` of wall time have passed (at least once);
    returns (runs, elapsed seconds)."""
    runs, t0 = 0, time.perf_counter()
    while True:
        fn()
        runs += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return runs, el


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "?"


def _cpu_baseline(mats, seconds):
    """The oracle on the decode step (all host threads OpenMP gives it), and
    the single-thread tiny case; the other sections add their legs."""
    import oracle
    from group_wise_affine_aq_amd import inputs as _inp

    host = [(_host_x(m["x"], "f16"), *_host_packed(*m["packed"]), m["K"]) for m in mats]

    def step():
        for x, c, s, b, K in host:
            oracle.matmul(x, c, s, b, K, G, BITS)

    reps, el = _cpu_timed(step, seconds)
    step_bytes = sum(m["wbytes"] for m in mats)
    cpu_gbs = step_bytes * reps / el / 1e9
    model, threads = _cpu_model(), oracle.num_threads()
    # the tiny workload (W [512, 512] 4-bit G=64, x fp16 [1, 512]) on one thread
    w = _inp.weights(512, 512, seed=0)
    c, s, b = oracle.quantize(w, G, BITS)
    x = _inp.from_bits(_inp.activations(1, 512, "f16", seed=0), "f16")
    oracle.set_num_threads(1)
    try:
        runs, t1 = _cpu_timed(lambda: oracle.matmul(x, c, s, b, 512, G, BITS), 1.0)
    finally:
        oracle.set_num_threads(threads)
    tiny_bytes = oracle.qweight_bytes(512, 512, G, BITS)
    legs = {"tiny_single_thread": {
        "workload": "W [512,512] 4-bit G=64, x fp16 [1,512]", "threads": 1,
        "us_per_call": round(t1 / runs * 1e6, 1), "gbs": round(tiny_bytes * runs / t1 / 1e9, 3),
        "sample": f"{runs} calls in {t1:.1f} s"}}
    print(f"# CPU oracle: decode {cpu_gbs:.3f} GB/s on {threads} threads; tiny case "
          f"{legs['tiny_single_thread']['us_per_call']} us on one thread", file=sys.stderr,
          flush=True)
    return {"value": round(cpu_gbs, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} full decode step(s) (4 matrices, {step_bytes} packed weight bytes, "
                      f"fp64 accumulation), {el:.1f} s on {model}",
            "nproc": os.cpu_count(), "omp_threads": threads, "cpu_model": model, "legs": legs}


def _graph_us(torch, stream, launches, reps=5):
    """Per-launch device time of `launches` (a list of callables) captured
    back-to-back in one graph and replayed between HIP events."""
    gs = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(gs):
        with torch.cuda.graph(g, stream=gs):
            for f in launches:
                f()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    durs = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        durs.append(e0.elapsed_time(e1) * 1e3 / len(launches))
    del g
    return sum(durs) / len(durs)


def _specdec(aq, inputs, dev, stream, legs=None):
    """Matrix-vector kernels for M = 2..8 rows (bf16), and the same matrices
    at 16 and 64 rows, each launch on a cold copy of the weights (>= 1 GiB
    rotated), per-launch time in a graph."""
    import torch
    cfg = inputs.WORKLOADS["specdec"]
    wid = inputs.WORKLOAD_ID["specdec"]
    out = {"workload": "spec-decode QMV, x bf16 [M, K], M in {2,3,4,6,8}; batched decode "
                       "M in {16, 64}; cold weights"}
    for (N, K) in cfg["shapes"]:
        w = inputs.weights_device(N, K, device=dev, seed=0, key=(wid,))
        for bits, g in zip(cfg["bits"], cfg["group_size"]):
            packed = aq.aq_quantize(w, g, bits)
            wbytes = aq.aq_qweight_bytes(N, K, g, bits)
            copies = max(2, math.ceil(COLD_BYTES / wbytes))
            sets = [packed] + [tuple(t.clone() for t in packed) for _ in range(copies - 1)]
            ceil_us = _read_ceiling_us(aq, torch, wbytes, stream)
            rows = {}
            for M in cfg["M"] + cfg["M_batch"]:
                x = inputs.activations_device(M, K, "bf16", device=dev, seed=0, key=(wid, N, M))
                y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
                fs = [lambda c=c, s_=s_, b=b: aq.aq_quantized_matmul(x, c, s_, b, g, bits, y=y)
                      for (c, s_, b) in sets]
                us = _graph_us(torch, stream, fs)
                gbs = wbytes / (us * 1e-6) / 1e9
                rows[f"M{M}"] = {"avg_us": round(us, 3), "weight_gbs": round(gbs, 1),
                                 "pct_hbm": round(100 * gbs / HBM_PEAK_GBS, 1),
                                 "frac_of_read_ceiling": round(ceil_us / us, 3)}
                print(f"# QMV {N}x{K} {bits}-bit G={g} M={M}: {us:.2f} us, {gbs:.0f} GB/s weights",
                      file=sys.stderr, flush=True)
            out[f"{N}x{K}_b{bits}_g{g}"] = dict(weight_bytes=wbytes,
                                                read_ceiling_us=round(ceil_us, 3), **rows)
            if legs is not None and "specdec" not in legs:
                # the oracle on the first matrix, M = 4 rows of the same x
                import oracle
                M = 4
                x = inputs.activations_device(M, K, "bf16", device=dev, seed=0, key=(wid, N, M))
                hx, hp = _host_x(x, "bf16"), _host_packed(*packed)
                runs, el = _cpu_timed(lambda: oracle.matmul(hx, *hp, K, g, bits), 1.5)
                legs["specdec"] = {"workload": f"W [{N},{K}] {bits}-bit G={g}, x bf16 [{M},{K}]",
                                   "threads": oracle.num_threads(),
                                   "gbs": round(wbytes * runs / el / 1e9, 3),
                                   "gpu_gbs": rows[f"M{M}"]["weight_gbs"],
                                   "sample": f"{runs} call(s) in {el:.1f} s"}
            del sets, packed
            torch.cuda.synchronize()
        del w
    return out


def _moe(aq, inputs, dev, stream, legs=None):
    """Gather matrix-vector kernel: 32 tokens x top-6 of 64 experts [1408, 2048]
    4-bit G=64; cold copies of the expert stack rotated (>= 1 GiB)."""
    import numpy as np
    import torch
    cfg = inputs.WORKLOADS["moe"]
    wid = inputs.WORKLOAD_ID["moe"]
    (N, K), E, T, topk = cfg["shapes"][0], cfg["experts"], cfg["tokens"], cfg["topk"]
    g, bits = cfg["group_size"][0], cfg["bits"][0]
    parts = [aq.aq_quantize(inputs.weights_device(N, K, device=dev, seed=0, key=(wid, e)), g, bits)
             for e in range(E)]
    packed = tuple(torch.stack([p[i] for p in parts]) for i in range(3))
    del parts
    ids_np = inputs.expert_ids(T, E, topk, seed=0, key=(wid,))
    ids = torch.from_numpy(ids_np).to(dev)
    x = inputs.activations_device(T, K, "f16", device=dev, seed=0, key=(wid,))
    y = torch.empty((T, topk, N), dtype=torch.float16, device=dev)
    ebytes = aq.aq_qweight_bytes(N, K, g, bits)
    copies = max(2, math.ceil(COLD_BYTES / (E * ebytes)))
    sets = [packed] + [tuple(t.clone() for t in packed) for _ in range(copies - 1)]
    fs = [lambda c=c, s_=s_, b=b: aq.aq_gather_qmv(x, c, s_, b, ids, g, bits, y=y)
          for (c, s_, b) in sets]
    us = _graph_us(torch, stream, fs)
    used = len(np.unique(ids_np))
    algo = used * ebytes + T * K * 2 + T * topk * N * 2 + T * topk * 4
    gbs = algo / (us * 1e-6) / 1e9
    print(f"# MoE gather ({used} of {E} experts used): {us:.2f} us, {gbs:.0f} GB/s algorithmic",
          file=sys.stderr, flush=True)
    res = {"workload": f"MoE gather: {E} experts [{N},{K}] {bits}-bit G={g}, x fp16 [{T},{K}], "
                       f"ids [{T},{topk}], cold weights",
           "experts_used": used, "algo_bytes": algo, "avg_us": round(us, 3),
           "gbs": round(gbs, 1), "pct_hbm": round(100 * gbs / HBM_PEAK_GBS, 1)}
    if legs is not None:
        import oracle
        hx, hp = _host_x(x, "f16"), _host_packed(*packed)
        runs, el = _cpu_timed(lambda: oracle.gather_matmul(hx, *hp, ids_np, K, g, bits), 1.5)
        legs["moe"] = {"workload": res["workload"].replace(", cold weights", ""),
                       "threads": oracle.num_threads(),
                       "gbs": round(algo * runs / el / 1e9, 3), "gpu_gbs": round(gbs, 1),
                       "sample": f"{runs} call(s) in {el:.1f} s"}
    # the same expert stack at prefill size on the matrix cores
    Tp = cfg["prefill_tokens"]
    ids_p = torch.from_numpy(inputs.expert_ids(Tp, E, topk, seed=0, key=(wid, 1))).to(dev)
    xp = inputs.activations_device(Tp, K, "f16", device=dev, seed=0, key=(wid, 1))
    yp = torch.empty((Tp, topk, N), dtype=torch.float16, device=dev)
    fs = [lambda c=c, s_=s_, b=b: aq.aq_gather_qmm(xp, c, s_, b, ids_p, g, bits, y=yp)
          for (c, s_, b) in sets[:4]]
    us = _graph_us(torch, stream, fs)
    flop = 2 * Tp * topk * N * K
    tf = flop / (us * 1e-6) / 1e12
    print(f"# MoE prefill gather ({Tp} tokens, top-{topk}): {us:.1f} us, {tf:.0f} TFLOP/s",
          file=sys.stderr, flush=True)
    res["prefill"] = {"workload": f"x fp16 [{Tp},{K}], ids [{Tp},{topk}], same experts",
                      "avg_us": round(us, 2), "flop": flop, "tflops": round(tf, 1),
                      "pct_mfma_peak": round(100 * tf / MFMA_BF16_PEAK_TFLOPS, 1)}
    del sets, packed
    torch.cuda.synchronize()
    return res


def _quant_dequant(aq, inputs, dev, stream, legs=None):
    """aq_quantize on W [28672, 8192] fp32 (4-bit G=64) and aq_dequantize of the
    result to bf16: each one pass over HBM, timed in graphs of back-to-back
    launches."""
    import torch
    N, K, g, bits = PREFILL["N"], PREFILL["K"], 64, 4
    w = inputs.weights_device(N, K, device=dev, seed=0, key=(inputs.WORKLOAD_ID["prefill"],))
    c, s_, b = aq.aq_quantize(w, g, bits)
    out = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    packed = aq.aq_qweight_bytes(N, K, g, bits)
    res = {"workload": f"W [{N},{K}] fp32 -> 4-bit G=64 and back to bf16"}
    us = _graph_us(torch, stream, [lambda: aq.aq_quantize(w, g, bits, codes=c, scales=s_, biases=b)] * 4)
    nb = 4 * N * K + packed
    res["quantize"] = {"avg_us": round(us, 2), "bytes": nb, "gbs": round(nb / (us * 1e-6) / 1e9, 1),
                       "pct_hbm": round(100 * nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)}
    us = _graph_us(torch, stream, [lambda: aq.aq_dequantize(c, s_, b, g, bits, out=out)] * 4)
    nb = packed + 2 * N * K
    res["dequantize_bf16"] = {"avg_us": round(us, 2), "bytes": nb,
                              "gbs": round(nb / (us * 1e-6) / 1e9, 1),
                              "pct_hbm": round(100 * nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)}
    # integer zero points, same matrix (zeros written too)
    zeros = torch.empty((N, K // g), dtype=torch.uint8, device=dev)
    us = _graph_us(torch, stream, [lambda: aq.aq_quantize_zp(w, g, bits, codes=c, scales=s_,
                                                             biases=b, zeros=zeros)] * 4)
    nb = 4 * N * K + packed + N * (K // g)
    res["quantize_zp"] = {"avg_us": round(us, 2), "bytes": nb,
                          "gbs": round(nb / (us * 1e-6) / 1e9, 1),
                          "pct_hbm": round(100 * nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)}
    # range search over 21 narrowed ranges (both ends moved inwards, keeping
    # 100 % .. 80 % of the width), same matrix
    steps = 21
    us = _graph_us(torch, stream,
                   [lambda: aq.aq_quantize_mse(w, g, bits, steps, codes=c, scales=s_, biases=b)] * 2)
    nb = 4 * N * K + packed
    res["quantize_mse"] = {"steps": steps, "avg_us": round(us, 2), "bytes": nb,
                           "gbs": round(nb / (us * 1e-6) / 1e9, 1),
                           "weights_per_s": round(N * K / (us * 1e-6), 1)}
    # a second denominator for these read-and-write passes: torch's device
    # copy (the runtime's copy kernel) of 512 MiB into another 512 MiB
    src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    us = _graph_us(torch, stream, [lambda: dst.copy_(src)] * 4)
    copy_gbs = 2 * src.numel() / (us * 1e-6) / 1e9
    res["device_copy"] = {"bytes": 2 * src.numel(), "avg_us": round(us, 2),
                          "gbs": round(copy_gbs, 1)}
    for key in ("quantize", "dequantize_bf16", "quantize_zp"):
        res[key]["frac_of_device_copy"] = round(res[key]["gbs"] / copy_gbs, 3)
    del src, dst
    if legs is not None:
        # the oracle quantizer on the first 1024 rows of the same W
        import oracle
        rows = 1024
        hw = w[:rows].cpu().numpy()
        runs, el = _cpu_timed(lambda: oracle.quantize(hw, g, bits), 1.5)
        nbs = 4 * rows * K + aq.aq_qweight_bytes(rows, K, g, bits)
        legs["quantize"] = {"workload": f"W [{rows} of {N} rows, {K}] fp32 -> 4-bit G=64",
                            "threads": oracle.num_threads(),
                            "gbs": round(nbs * runs / el / 1e9, 3),
                            "gpu_gbs": res["quantize"]["gbs"],
                            "sample": f"{runs} call(s) in {el:.1f} s"}
    print(f"# zero-point quantize {res['quantize_zp']['avg_us']:.1f} us "
          f"({res['quantize_zp']['gbs']} GB/s)", file=sys.stderr, flush=True)
    print(f"# quantize {res['quantize']['avg_us']:.1f} us ({res['quantize']['gbs']} GB/s), "
          f"dequantize {res['dequantize_bf16']['avg_us']:.1f} us ({res['dequantize_bf16']['gbs']} GB/s), "
          f"range-search quantize ({steps} ranges) {res['quantize_mse']['avg_us']:.1f} us; "
          f"device copy of 512 MiB {res['device_copy']['gbs']} GB/s", file=sys.stderr, flush=True)
    del w, c, s_, b, out
    torch.cuda.synchronize()
    return res


def _fp_tensor_exp(w, mode):
    """nvfp4's tensor exponent T = ceil(log2(max|W| / 2688)) (the largest group
    scale near the top of E4M3's range); 0 for the mx modes."""
    if mode != "nvfp4":
        return 0
    amax = float(w.abs().max())
    return 0 if amax == 0 else max(-100, min(100, math.ceil(math.log2(amax / 2688))))


def _fp_modes(aq, inputs, dev, stream, legs=None):
    """Block-scaled float modes (mxfp4: E2M1 codes + exponent byte per 32,
    4.25 bits/weight; nvfp4: E2M1 codes + E4M3 scale per 16, 4.5 bits;
    mxfp8: E4M3 codes + exponent byte per 32, 8.25 bits): the decode product
    on the four decode matrices (the headline weights quantized by
    aq_quantize_fp, x fp16), each launch on a cold copy (>= 1 GiB rotated),
    per-launch time in a graph, with the plain read of the same bytes beside
    it; and aq_quantize_fp / aq_dequantize_fp (bf16) on the prefill-size
    matrix."""
    import torch
    out = {"workload": "decode M=1, W [4096,4096] [1024,4096] [14336,4096] [4096,14336], "
                       "fp16 x, cold weights; M=4, 8 bf16 x on the two 33 MB matrices; the MoE "
                       "gather workload with block-scaled experts; "
                       "quantize / dequantize W [28672,8192] fp32 <-> bf16"}
    ceilings = {}
    for mode, (_, grp, bits) in aq.FP_MODES.items():
        rows = {}
        total_us = total_bytes = 0
        for i, (N, K) in enumerate(DECODE_SHAPES):
            w = inputs.weights_device(N, K, device=dev, seed=0, key=(1, i), outliers=True)
            T = _fp_tensor_exp(w, mode)
            packed = aq.aq_quantize_fp(w, mode, T)
            del w
            wbytes = N * K * bits // 8 + N * K // grp
            copies = max(2, math.ceil(COLD_BYTES / wbytes))
            sets = [packed] + [tuple(t.clone() for t in packed) for _ in range(copies - 1)]
            x = inputs.activations_device(1, K, "f16", device=dev, seed=0, key=(1, i))
            y = torch.empty((1, N), dtype=torch.float16, device=dev)
            fs = [lambda c=c, s_=s_: aq.aq_qmv_fp(x, c, s_, mode, T, y=y) for (c, s_) in sets] * 2
            us = _graph_us(torch, stream, fs)
            if wbytes not in ceilings:
                ceilings[wbytes] = _read_ceiling_us(aq, torch, wbytes, stream)
            ceil_us = ceilings[wbytes]
            gbs = wbytes / (us * 1e-6) / 1e9
            rows[f"{N}x{K}"] = {"kernel": aq.aq_qmv_fp_describe(N, K, mode), "weight_bytes": wbytes,
                                "tensor_exp": T, "avg_us": round(us, 3),
                                "weight_gbs": round(gbs, 1),
                                "pct_hbm": round(100 * gbs / HBM_PEAK_GBS, 1),
                                "read_ceiling_us": round(ceil_us, 3),
                                "frac_of_read_ceiling": round(ceil_us / us, 3)}
            total_us += us
            total_bytes += wbytes
            print(f"# {mode} QMV {N}x{K}: {us:.2f} us, {gbs:.0f} GB/s weights, "
                  f"{ceil_us / us:.2f} of the plain read", file=sys.stderr, flush=True)
            if N * K >= 4096 * 14336:
                # speculative-decoding widths on the matrix cores, bf16 x
                for M in (4, 8):
                    xm = inputs.activations_device(M, K, "bf16", device=dev, seed=0, key=(2, i))
                    ym = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
                    fm = [lambda c=c, s_=s_: aq.aq_matmul_fp(xm, c, s_, mode, T, y=ym)
                          for (c, s_) in sets] * 2
                    usm = _graph_us(torch, stream, fm)
                    gm = wbytes / (usm * 1e-6) / 1e9
                    rows[f"{N}x{K}"][f"rows_M{M}"] = {
                        "avg_us": round(usm, 3), "weight_gbs": round(gm, 1),
                        "pct_hbm": round(100 * gm / HBM_PEAK_GBS, 1),
                        "frac_of_read_ceiling": round(ceil_us / usm, 3)}
                    print(f"# {mode} M={M} bf16 {N}x{K}: {usm:.2f} us, {gm:.0f} GB/s weights, "
                          f"{ceil_us / usm:.2f} of the plain read", file=sys.stderr, flush=True)
            if legs is not None and f"{mode}_decode" not in legs:
                # the oracle on the first matrix: exact dequantize, then the product
                import oracle
                hx = _host_x(x, "f16")
                hc = packed[0].cpu().numpy().view("uint32")
                hs = packed[1].cpu().numpy()
                deq = {"mxfp4": lambda: oracle.dequantize_mxfp4_exact(hc, hs, K),
                       "mxfp8": lambda: oracle.dequantize_mxfp8_exact(hc, hs, K),
                       "nvfp4": lambda: oracle.dequantize_nvfp4_exact(hc, hs, K, T)}[mode]
                runs, el = _cpu_timed(lambda: oracle.matmul_dense(hx, deq()), 1.0)
                legs[f"{mode}_decode"] = {"workload": f"{mode} W [{N},{K}], x fp16 [1,{K}]",
                                          "threads": oracle.num_threads(),
                                          "gbs": round(wbytes * runs / el / 1e9, 3),
                                          "gpu_gbs": round(gbs, 1),
                                          "sample": f"{runs} call(s) in {el:.1f} s"}
            del sets, packed
            torch.cuda.synchronize()
        res = {"per_shape": rows, "step_us": round(total_us, 3), "step_weight_bytes": total_bytes,
               "step_weight_gbs": round(total_bytes / (total_us * 1e-6) / 1e9, 1)}
        # quantize (fp32 in) and dequantize (bf16 out) of the prefill-size matrix
        N, K = PREFILL["N"], PREFILL["K"]
        w = inputs.weights_device(N, K, device=dev, seed=0, key=(inputs.WORKLOAD_ID["prefill"],))
        T = _fp_tensor_exp(w, mode)
        c, s_ = aq.aq_quantize_fp(w, mode, T)
        deq = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
        packed = N * K * bits // 8 + N * K // grp
        us = _graph_us(torch, stream, [lambda: aq.aq_quantize_fp(w, mode, T, codes=c, scales=s_)] * 4)
        nb = 4 * N * K + packed
        res["quantize"] = {"avg_us": round(us, 2), "bytes": nb,
                           "gbs": round(nb / (us * 1e-6) / 1e9, 1),
                           "pct_hbm": round(100 * nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)}
        us = _graph_us(torch, stream, [lambda: aq.aq_dequantize_fp(c, s_, K, mode, T, out=deq)] * 4)
        nb = packed + 2 * N * K
        res["dequantize_bf16"] = {"avg_us": round(us, 2), "bytes": nb,
                                  "gbs": round(nb / (us * 1e-6) / 1e9, 1),
                                  "pct_hbm": round(100 * nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)}
        res["moe"] = _fp_moe(aq, inputs, dev, stream, mode, grp, bits)
        print(f"# {mode} step {total_us:.2f} us ({res['step_weight_gbs']} GB/s); quantize "
              f"{res['quantize']['avg_us']:.1f} us ({res['quantize']['gbs']} GB/s), dequantize "
              f"{res['dequantize_bf16']['avg_us']:.1f} us ({res['dequantize_bf16']['gbs']} GB/s)",
              file=sys.stderr, flush=True)
        out[mode] = res
        del w, c, s_, deq
        torch.cuda.synchronize()
    return out


def _fp_moe(aq, inputs, dev, stream, mode, grp, bits):
    """The MoE decode workload (32 tokens x top-6 of 64 experts [1408, 2048],
    the same seeded weights and ids as the affine gather) with the experts in a
    block-scaled mode: aq_gather_matmul_fp, cold copies of the expert stack."""
    import numpy as np
    import torch
    cfg = inputs.WORKLOADS["moe"]
    wid = inputs.WORKLOAD_ID["moe"]
    (N, K), E, T, topk = cfg["shapes"][0], cfg["experts"], cfg["tokens"], cfg["topk"]
    amax = max(float(inputs.weights_device(N, K, device=dev, seed=0, key=(wid, e)).abs().max())
               for e in range(E))
    Te = 0 if mode != "nvfp4" or amax == 0 else max(-100, min(100, math.ceil(math.log2(amax / 2688))))
    parts = [aq.aq_quantize_fp(inputs.weights_device(N, K, device=dev, seed=0, key=(wid, e)),
                               mode, Te) for e in range(E)]
    packed = tuple(torch.stack([p[i] for p in parts]) for i in range(2))
    del parts
    ids_np = inputs.expert_ids(T, E, topk, seed=0, key=(wid,))
    ids = torch.from_numpy(ids_np).to(dev)
    x = inputs.activations_device(T, K, "f16", device=dev, seed=0, key=(wid,))
    y = torch.empty((T, topk, N), dtype=torch.float16, device=dev)
    ebytes = N * K * bits // 8 + N * K // grp
    copies = max(2, math.ceil(COLD_BYTES / (E * ebytes)))
    sets = [packed] + [tuple(t.clone() for t in packed) for _ in range(copies - 1)]
    fs = [lambda c=c, s_=s_: aq.aq_gather_matmul_fp(x, c, s_, ids, mode, Te, y=y)
          for (c, s_) in sets]
    us = _graph_us(torch, stream, fs)
    used = len(np.unique(ids_np))
    algo = used * ebytes + T * K * 2 + T * topk * N * 2 + T * topk * 4
    gbs = algo / (us * 1e-6) / 1e9
    print(f"# {mode} MoE gather ({used} of {E} experts used): {us:.2f} us, {gbs:.0f} GB/s "
          "algorithmic", file=sys.stderr, flush=True)
    del sets, packed
    torch.cuda.synchronize()
    return {"workload": f"{E} experts [{N},{K}] {mode}, x fp16 [{T},{K}], ids [{T},{topk}], "
                        "cold weights",
            "experts_used": used, "algo_bytes": algo, "avg_us": round(us, 3),
            "gbs": round(gbs, 1), "pct_hbm": round(100 * gbs / HBM_PEAK_GBS, 1)}


def _embedding(aq, inputs, dev, stream):
    """Quantized embedding lookup on a [128256, 4096] 8-bit G=128 table (541 MB,
    more than the last-level cache), bf16 rows, T = 1 and T = 2048 tokens; each
    launch of a graph of back-to-back launches uses its own seeded ids."""
    import torch
    cfg = inputs.WORKLOADS["embedding"]
    (V, K), G, bits = cfg["shapes"][0], cfg["group_size"][0], cfg["bits"][0]
    w = inputs.weights_device(V, K, device=dev, seed=0, key=(inputs.WORKLOAD_ID["embedding"],))
    c, s, b = aq.aq_quantize(w, G, bits)
    del w
    out = {"workload": f"embedding table [{V},{K}] {bits}-bit G={G}, bf16 rows"}
    reps = 32
    gs = torch.cuda.Stream()
    for T in cfg["tokens"]:
        ids = [torch.from_numpy(inputs.token_ids(T, V, seed=r + 1,
                                                 key=(inputs.WORKLOAD_ID["embedding"],))).to(dev)
               for r in range(reps)]
        o = torch.empty((T, K), dtype=torch.bfloat16, device=dev)
        aq.aq_embedding(ids[0], c, s, b, G, bits, out=o)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(gs):
            with torch.cuda.graph(g, stream=gs):
                for r in range(reps):
                    aq.aq_embedding(ids[r], c, s, b, G, bits, out=o)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        durs = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            durs.append(e0.elapsed_time(e1) * 1e3 / reps)
        us = sum(durs) / len(durs)
        nbytes = T * (K * bits // 8 + (K // G) * 4) + T * K * 2 + T * 4
        out[f"T{T}"] = {"avg_us": round(us, 3), "algo_bytes": nbytes,
                        "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
                        "pct_hbm": round(100 * nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)}
        print(f"# embedding T={T}: {us:.2f} us/launch in-graph, {out[f'T{T}']['gbs']} GB/s "
              f"(rows read + written)", file=sys.stderr, flush=True)
        del g
    return out


def _qmm(aq, inputs, dev, iters, legs=None):
    import torch
    M, N, K = PREFILL["M"], PREFILL["N"], PREFILL["K"]
    x = inputs.activations_device(M, K, "bf16", device=dev, seed=0, key=(3,))
    w = inputs.weights_device(N, K, device=dev, seed=0, key=(3,))
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    out = {"workload": f"prefill X bf16 [{M},{K}] x W [{N},{K}]", "flop": 2 * M * N * K}
    flop = 2 * M * N * K
    for bits, g in PREFILL["settings"]:
        c, s, b = aq.aq_quantize(w, g, bits)
        for _ in range(10):  # the clock settles over the first launches
            aq.aq_qmm(x, c, s, b, g, bits, y=y)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(iters)]
        _spin(torch)
        for e0, e1 in evs:
            e0.record()
            aq.aq_qmm(x, c, s, b, g, bits, y=y)
            e1.record()
        torch.cuda.synchronize()
        durs = sorted(a.elapsed_time(b) for a, b in evs)
        avg = sum(durs) / len(durs)
        med = durs[len(durs) // 2]
        tf = flop / (avg * 1e-3) / 1e12
        out[f"b{bits}_g{g}"] = {"avg_ms": round(avg, 4), "median_ms": round(med, 4),
                                "tflops": round(tf, 1),
                                "pct_mfma_peak": round(100 * tf / MFMA_BF16_PEAK_TFLOPS, 1)}
        print(f"# QMM {bits}-bit G={g}: {avg:.3f} ms (median {med:.3f}), {tf:.1f} TFLOP/s",
              file=sys.stderr, flush=True)
        if legs is not None and "qmm" not in legs:
            # the oracle on the first 4 rows of X against all of W
            import oracle
            Ms = 4
            hx, hp = _host_x(x[:Ms], "bf16"), _host_packed(c, s, b)
            runs, el = _cpu_timed(lambda: oracle.matmul(hx, *hp, K, g, bits), 1.0)
            legs["qmm"] = {"workload": f"X bf16 [{Ms} of {M} rows, {K}] x W [{N},{K}] "
                                       f"{bits}-bit G={g}",
                           "threads": oracle.num_threads(),
                           "gflops": round(2 * Ms * N * K * runs / el / 1e9, 3),
                           "gpu_gflops": round(tf * 1e3, 1),
                           "sample": f"{runs} call(s) in {el:.1f} s"}
        del c, s, b
    # dense bf16 GEMM on the library GEMM (hipBLASLt) at the same shape, for context
    wd = w.to(torch.bfloat16)
    for _ in range(10):
        torch.matmul(x, wd.T)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        torch.matmul(x, wd.T)
    e1.record()
    torch.cuda.synchronize()
    avg = e0.elapsed_time(e1) / iters
    out["dense_bf16_torch_matmul"] = {"avg_ms": round(avg, 4),
                                      "tflops": round(flop / (avg * 1e-3) / 1e12, 1)}
    out["peak_tflops"] = MFMA_BF16_PEAK_TFLOPS
    # second denominator: an MFMA-only loop (no data movement) and the clock it runs at
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    ghz, tfl = _mfma_clock(aq, torch, cus)
    out["mfma_only_loop"] = {"tflops": tfl, "sclk_ghz": ghz}
    key = f"b{PREFILL['settings'][0][0]}_g{PREFILL['settings'][0][1]}"
    out[key]["frac_of_mfma_only_loop"] = round(out[key]["tflops"] / tfl, 3)
    print(f"# MFMA-only loop: {tfl:.1f} TFLOP/s at {ghz:.2f} GHz", file=sys.stderr, flush=True)
    return out


if __name__ == "__main__":
    main()
