#!/usr/bin/env python3
"""Benchmark of the fused dequantize-and-multiply on one MI355X.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--no-extras] [--no-cpu-baseline]
    python bench.py --calibrate                       # launch and streaming-read calibration
    python bench.py --summarize-trace DIR             # rocprofv3 kernel-trace summary (markdown)
    python bench.py --summarize-counters F W CF CW    # rocprofv3 FETCH/WRITE summary (markdown)

Headline (one JSON line on stdout): quantized-weight GB/s of the matrix-vector
path at one token on the seven projections of a Qwen3-Embedding-4B decoder
layer (Q4_K: 4096x2560, 1024x2560, 2560x4096, 9728x2560 twice; Q6_K:
1024x2560, 2560x9728; random N(0, 0.02^2) weights, N(0, 1) fp32 activations).
A step is one pass over the layer: the seven projections in four calls as a
decode step makes them (q+k+v and gate+up read one input each, so they share a
qmm_gemv_group call; attn_output and ffn_down alone), four launches of the
one-token GEMV kernel.  Weights rotate
through copies totalling more than 1 GiB, so each step streams them from HBM
rather than the 256 MB Infinity Cache.  Steps are timed as replays of HIP
graphs captured from the library's launches (the graph only removes host
launch overhead; the kernels are the ones an eager call runs).

Also reported:
  roofline      the step's kernel: all four launches are the one-token GEMV
                kernel (k_gemv1 and its Q4_K+Q6_K form k_gemv1_pair), run back to
                back, so its average launch duration is the HIP-event-timed step
                over four launches, and its algorithmic bytes per launch the
                layer's weights + x + y over four; against 8 TB/s.  "traffic" from the
                rocprofv3 counter summary in profiles/ when it was taken on the
                current kernel source, else null.
  cpu_baseline  the CPU oracle (NumPy dequantization + fp64 matmul) on a bounded
                sample of the same workload, in the same unit; per-config
                oracle timings (median of 3) in extras.oracle_per_config.
  extras        the other workloads, each timed over more than 1 GiB of
                distinct weight copies per sample: the single Q4_0 256x512
                matvec, 4-bit affine-group decode at 1..16 tokens (with its fp32
                VALU ceiling fraction), the prefill GEMM at 7..2048 tokens with
                both token tiles, the batch of 2 x 65 tokens on 128 x 768 in all
                five formats, the expert-indexed matvec at 2..24 tokens with ids
                re-drawn per call and its matrix-core form at 64..1024 tokens,
                and the GPU quantizer.
"""

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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix cores
# fp32 vector ALU: 256 CUs x 4 SIMDs x 16 lanes x 2 flops (fma) x 2.4 GHz = 78.6 TFLOP/s for
# one fma per lane per cycle; packed fp32 (two per lane) doubles it to 157.3, but this library
# is built without packed fp32 instructions, so 78.6 is the ceiling its fmas can reach
VALU_F32_FMA_TFLOPS = 78.6
VALU_F32_PACKED_TFLOPS = 157.3
ROTATE_BYTES = 1 << 30         # > 256 MB Infinity Cache
METRIC = "quantized-weight GB/s at n<=16 and TFLOP/s at n>=64, as % of roofline"
# the decode step's calls (indices into the layer's projections): attn_q, attn_k and
# attn_v read one input, ffn_gate and ffn_up another; attn_output and ffn_down each
# wait for the previous result
DECODE_GROUPS = [[0, 1, 2], [3], [4, 5], [6]]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-extras", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--ungrouped", action="store_true",
                   help="headline step as seven separate qmm_gemv calls (default: the independent "
                        "projections share qmm_gemv_group calls)")
    p.add_argument("--event-launches", type=int, default=64,
                   help="launches per projection in the isolated per-projection pass (0: skip it)")
    p.add_argument("--calls", type=int, default=20, help="calls per timed sample in the extras")
    p.add_argument("--rounds", type=int, default=6, help="timed samples per extra case (median)")
    p.add_argument("--copy-probe", action="store_true", help="only run a 256 MiB device copy (counter calibration)")
    p.add_argument("--calibrate", action="store_true",
                   help="only time an empty kernel and plain streaming reads of the decode-layer projection sizes")
    p.add_argument("--table-only", action="store_true",
                   help="with --summarize-trace: the per-kernel table only (a run of another workload)")
    p.add_argument("--summarize-trace", default=None, metavar="DIR",
                   help="print a markdown summary of a rocprofv3 kernel trace of this benchmark (no GPU needed)")
    p.add_argument("--summarize-sq", nargs="+", default=None, metavar="DIR",
                   help="print per-kernel SQ counter fractions from rocprofv3 --pmc runs (no GPU needed)")
    p.add_argument("--summarize-counters", nargs=4, default=None, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                   help="print a markdown summary of rocprofv3 FETCH_SIZE / WRITE_SIZE runs of this benchmark and "
                        "of --copy-probe (no GPU needed)")
    p.add_argument("--prefill-only", default=None, metavar="N[,N...]",
                   help="only time the decode layer's prefill GEMM at these token counts (for profiling)")
    p.add_argument("--formats-only", action="store_true", help="only run the per-format sweep")
    p.add_argument("--small-decode-only", default=None, metavar="N[,N...]",
                   help="only time the 4-bit-group layer at these token counts (for profiling)")
    p.add_argument("--decode-few-only", default=None, metavar="N[,N...]",
                   help="only time the decode layer at these fp16 token counts through qmm_gemv")
    p.add_argument("--moe-only", default=None, metavar="N[,N...]",
                   help="only time the expert-indexed paths at these token counts: the matvec up to 32 "
                        "tokens, the matrix-core path above (for profiling)")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest():
    """Digest of what the one-token GEMV kernel is built from (its source, the headers it
    includes and the build flags): the committed counter summaries hold for that kernel only."""
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "block_quantized_weight_matmul_amd")
    for f in ["csrc/gemv.hip", "csrc/decode.hpp", "csrc/internal.hpp", "build.py"]:
        with open(os.path.join(pkg, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------------------------------------
# device helpers

class Rotation:
    """C copies of a set of block blobs in one device buffer; copy c of blob j is a
    contiguous, 256-byte aligned slice."""

    def __init__(self, torch, blobs, min_total=ROTATE_BYTES, min_copies=2):
        self.sizes = [int(b.size) for b in blobs]
        self.offs, off = [], 0
        for s in self.sizes:
            self.offs.append(off)
            off += (s + 255) // 256 * 256
        self.copy_bytes = off
        self.copies = max(min_copies, math.ceil(min_total / self.copy_bytes))
        host = np.zeros(self.copy_bytes, np.uint8)
        for b, o in zip(blobs, self.offs):
            host[o:o + b.size] = b
        self.buf = torch.empty(self.copies * self.copy_bytes, dtype=torch.uint8, device="cuda")
        first = torch.from_numpy(host).to("cuda")
        for c in range(self.copies):
            self.buf[c * self.copy_bytes:(c + 1) * self.copy_bytes].copy_(first)
        torch.cuda.synchronize()

    def slice(self, c, j):
        o = c * self.copy_bytes + self.offs[j]
        return self.buf[o:o + self.sizes[j]]


def capture(torch, fn):
    """HIP graph of fn()'s launches (warmed up on a side stream first)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, rounds):
    """Median ms of one replay of g over `rounds` event-timed replays."""
    ts = []
    for _ in range(rounds):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b))
    return float(np.median(ts))


# ------------------------------------------------------------------------------------------------
# headline: decode layer, one token

def launch_sets(mats, call, N):
    """The launches qmm_gemv_group makes for the matrices `call` (indices into mats) at N
    tokens: in order, up to four not yet launched matrices of the first one's K (one
    format, or Q4_K with Q6_K at one token), else those of its format and K, else it
    alone."""
    left, out = list(call), []
    while left:
        i = left[0]
        for same_fmt in (False, True):
            st = [j for j in left if mats[j]["K"] == mats[i]["K"]
                  and (not same_fmt or mats[j]["fmt"] == mats[i]["fmt"])][:4]
            fmts = {mats[j]["fmt"] for j in st}
            if len(st) > 1 and (len(fmts) == 1 and (N == 1 or mats[i]["fmt"] != "q8_0")
                                or (fmts <= {"q4_k", "q6_k"} and N == 1)):
                break
        else:
            st = [i]
        out.append(st)
        left = [j for j in left if j not in st]
    return out


def headline_launches(W):
    """Launches of one headline step and the mean algorithmic bytes (quantized weights
    + fp32 x + fp32 y) per launch."""
    mats = [{"fmt": f, "K": K, "M": M} for _, M, K, f in W.DECODE_SHAPES]
    n = sum(len(launch_sets(mats, c, 1)) for c in DECODE_GROUPS)
    alg = sum(M * {"q4_k": 144, "q6_k": 210}[fmt] * K // 256 + 4 * K + 4 * M for _, M, K, fmt in W.DECODE_SHAPES)
    return n, alg / n


def decode_layer(torch, q, W, args):
    t0 = time.time()
    mats = [W.decode_weights(i) for i in range(len(W.DECODE_SHAPES))]
    log(f"[bench] decode layer generated in {time.time() - t0:.1f}s")
    rot = Rotation(torch, [m["blob"] for m in mats])
    P = len(mats)
    handles = [[q.QMatrix(rot.slice(c, j), m["fmt"], m["M"], m["K"]) for j, m in enumerate(mats)]
               for c in range(rot.copies)]
    xs = [torch.from_numpy(W.decode_x(j, 1)).to("cuda") for j in range(P)]
    ys = [torch.empty((1, m["M"]), dtype=torch.float32, device="cuda") for m in mats]
    layer_weight_bytes = sum(int(m["blob"].size) for m in mats)
    layer_alg_bytes = sum(int(m["blob"].size) + 4 * m["K"] + 4 * m["M"] for m in mats)

    # the step's calls: the layer's independent projections share a call (query, key
    # and value read the same normed input in a layer, as do gate and up); the
    # library gives matrices of one format and K one launch
    calls = [[j] for j in range(P)] if args.ungrouped else DECODE_GROUPS
    sets = [s for c in calls for s in launch_sets(mats, c, 1)]
    launches = len(sets)

    def step(c):
        for grp in calls:
            if len(grp) == 1:
                q.qmm_gemv(handles[c][grp[0]].handle, xs[grp[0]], 1, ys[grp[0]])
            else:
                q.qmm_gemv_group([handles[c][j].handle for j in grp], [xs[j] for j in grp], 1, [ys[j] for j in grp])

    full = capture(torch, lambda: [step(c) for c in range(rot.copies)])
    singles = [capture(torch, lambda c=c: step(c)) for c in range(rot.copies)]

    def run(nsteps):
        for _ in range(nsteps // rot.copies):
            full.replay()
        for c in range(nsteps % rot.copies):
            singles[c].replay()

    run(args.warmup)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    ev0.record()
    run(args.steps)
    ev1.record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_start
    ev_ms = ev0.elapsed_time(ev1)
    ms_per_step = wall_s * 1e3 / args.steps
    value = layer_weight_bytes * args.steps / wall_s / 1e9

    # isolated per-projection pass: for each projection, a graph of R back-to-back launches
    # of that projection alone (rotating copies), timed with HIP events; a launch that
    # follows a launch of the same kernel overlaps it more than in the layer step, so
    # these are context, not the roofline's launch time
    R = args.event_launches
    mean_us = np.zeros(P)
    for j in range(P if R > 0 else 0):
        g = capture(torch, lambda j=j: [q.qmm_gemv(handles[r % rot.copies][j].handle, xs[j], 1, ys[j])
                                       for r in range(R)])
        mean_us[j] = time_graph(torch, g, 5) * 1e3 / R
        del g
    projections = [{"name": m["name"], "fmt": m["fmt"], "M": m["M"], "K": m["K"], "weight_bytes": int(m["blob"].size),
                    "isolated_us": round(float(mean_us[j]), 3),
                    "isolated_weight_gbs": round(m["blob"].size / (mean_us[j] * 1e-6) / 1e9, 1)}
                   for j, m in enumerate(mats)]
    # the roofline's kernel: every launch of the step is the one-token GEMV (k_gemv1, or
    # k_gemv1_pair for the Q4_K + Q6_K call) and they run back to back, so the event-timed step over its launches is their
    # average duration (the rocprofv3 trace in profiles/ checks this against
    # per-dispatch durations)
    step_us = ev_ms / args.steps * 1e3
    avg_us = step_us / launches
    alg_per_launch = layer_alg_bytes / launches
    out = {
        "value": value, "ms_per_step": ms_per_step, "event_ms_per_step": ev_ms / args.steps,
        "layer_weight_bytes": layer_weight_bytes, "layer_alg_bytes": layer_alg_bytes,
        "copies": rot.copies, "rotation_bytes": rot.copies * rot.copy_bytes,
        "projections": projections,
        "calls": [[mats[j]["name"] for j in c] for c in calls],
        "launch_sets": [[mats[j]["name"] for j in st] for st in sets],
        "kernel": {"launches_per_step": launches, "avg_us": avg_us, "alg_bytes_per_launch": alg_per_launch,
                   "achieved_gbs": alg_per_launch / (avg_us * 1e-6) / 1e9},
        "sum_isolated_us": float(mean_us.sum()),
    }
    del handles, full, singles
    return out, mats


COUNTER_SUMMARY = os.path.join(ROOT, "profiles", "gemv_decode_layer_counters.md")
TRACE_SUMMARY = os.path.join(ROOT, "profiles", "gemv_decode_layer_kernel_trace.md")


def _summary_values(path):
    vals = {}
    if os.path.exists(path):
        for line in open(path):
            if ":" in line and line.strip().startswith("- "):
                k, _, v = line.strip()[2:].partition(":")
                vals[k.strip()] = v.strip()
    return vals


def traffic_from_profile(digest):
    """HBM bytes per launch of the step's kernel from the committed counter summary, if it
    was taken on this kernel source."""
    vals = _summary_values(COUNTER_SUMMARY)
    if not vals:
        return None, "no counter summary"
    if vals.get("source_digest") != digest:
        return None, "counters taken on another kernel source"
    try:
        return float(vals["traffic_bytes_per_launch"]), "rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated"
    except (KeyError, ValueError):
        return None, "summary incomplete"


# ------------------------------------------------------------------------------------------------
# CPU oracle baseline

def cpu_baseline(mats, min_seconds=10.0):
    """The oracle on the headline workload itself: whole passes over the decode layer's
    seven projections at one token, repeated until about min_seconds of CPU work."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        blas_threads = None
    from qmm_synth import workloads as W
    xs = [W.decode_x(j, 1) for j in range(len(mats))]
    t0 = time.perf_counter()
    nbytes, passes = 0, 0
    while passes == 0 or time.perf_counter() - t0 < min_seconds:
        for m, x in zip(mats, xs):
            oracle.matmul_ref(x, oracle.dequantize(m["fmt"], m["blob"], m["M"], m["K"]))
            nbytes += int(m["blob"].size)
        passes += 1
    dt = time.perf_counter() - t0
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": (f"{passes} pass(es) over all seven projections of the decode layer at one token "
                       f"({nbytes} quantized bytes): NumPy dequantization (single-threaded) + fp64 matmul "
                       f"(BLAS threads available: {blas_threads}), {dt:.1f} s; cores counts the "
                       f"dequantization thread, which takes >99% of the time")}


def _median3(fn):
    ts = []
    for _ in range(3):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts))


def oracle_per_config(W, mats):
    """The oracle (dequantization + fp64 products, as the parity tests run it) on one bounded
    sample of each workload, median of 3 runs: its throughput in the workload's own unit."""
    import oracle
    out = []
    d = W.single_matvec()
    t = _median3(lambda: oracle.matmul_ref(d["x"], oracle.dequantize(d["fmt"], d["blob"], d["M"], d["K"])))
    out.append({"config": "Q4_0 256x512 matvec, 1 token", "sample": "whole", "s": t,
                "weight_gbs": d["blob"].size / t / 1e9})
    for j in (1, 6):  # attn_k (Q4_K) and ffn_down (Q6_K)
        m = mats[j]
        x = W.decode_x(j, 1)
        t = _median3(lambda: oracle.matmul_ref(x, oracle.dequantize(m["fmt"], m["blob"], m["M"], m["K"])))
        out.append({"config": "decode layer, 1 fp32 token", "sample": m["name"], "s": t,
                    "weight_gbs": m["blob"].size / t / 1e9})
    sm = W.small_decode_weights(0)
    x = W.small_decode_x(0, 16)
    t = _median3(lambda: oracle.matmul_ref(x, oracle.dequantize("a4g64", sm["blob"], sm["M"], sm["K"])))
    out.append({"config": "A4G64 layer, 16 fp16 tokens", "sample": sm["name"], "s": t,
                "weight_gbs": sm["blob"].size / t / 1e9, "gflops": 2 * 16 * sm["M"] * sm["K"] / t / 1e9})
    m = mats[1]
    x = W.prefill_x(1, 512)
    t = _median3(lambda: oracle.matmul_ref(x, oracle.dequantize(m["fmt"], m["blob"], m["M"], m["K"])))
    out.append({"config": "prefill GEMM, 512 fp16 tokens", "sample": m["name"], "s": t,
                "gflops": 2 * 512 * m["M"] * m["K"] / t / 1e9})
    pb = W.prefill_batch(2)
    t = _median3(lambda: oracle.matmul_ref(pb["x"], oracle.dequantize(pb["fmt"], pb["blob"], pb["M"], pb["K"])))
    out.append({"config": "batch 2 x 65 tokens, 128 x 768", "sample": pb["fmt"], "s": t,
                "gflops": 2 * 130 * pb["M"] * pb["K"] / t / 1e9})
    ids = W.moe_ids(2, 0)
    used = sorted(set(ids.reshape(-1).tolist()))
    x = W.moe_x(2)
    blobs = {e: W.moe_expert(e) for e in used}

    def moe():
        ws = [None] * W.MOE_EXPERTS
        for e in used:
            ws[e] = oracle.dequantize("q4_0", blobs[e], W.MOE_M, W.MOE_K)
        zero = np.zeros((W.MOE_M, W.MOE_K), np.float32)
        oracle.matmul_id_ref(x, ids, [w if w is not None else zero for w in ws])
    t = _median3(moe)
    out.append({"config": "expert-indexed matvec, 2 tokens x 8 slots", "sample": f"{len(used)} distinct experts",
                "s": t, "weight_gbs": len(used) * blobs[used[0]].size / t / 1e9})
    return {"kind": "oracle", "cores": 1, "note": "NumPy dequantization (single-threaded) dominates; fp64 "
            "products through BLAS", "results": out}


# ------------------------------------------------------------------------------------------------
# extras

def extra_single_matvec(torch, q, W, args):
    d = W.single_matvec()
    rot = Rotation(torch, [d["blob"]])
    hs = [q.QMatrix(rot.slice(c, 0), d["fmt"], d["M"], d["K"]) for c in range(rot.copies)]
    x = torch.from_numpy(d["x"]).to("cuda")
    y = torch.empty((1, d["M"]), device="cuda")
    # one sample = one call on every copy (> 1 GiB of distinct weights)
    g = capture(torch, lambda: [q.qmm_gemv(h.handle, x, 1, y) for h in hs])
    us = time_graph(torch, g, args.rounds) * 1e3 / len(hs)
    del g
    return {"workload": "Q4_0 256x512, 1 fp32 token", "us_per_call": us, "copies": rot.copies,
            "weight_gbs": d["blob"].size / (us * 1e-6) / 1e9,
            "frac_hbm": d["blob"].size / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "note": "a 73,728-byte matrix: the call is bound by the launch, not by its bytes"}


def extra_small_decode(torch, q, W, args):
    mats = [W.small_decode_weights(i) for i in range(len(W.SMALL_DECODE_SHAPES))]
    rot = Rotation(torch, [m["blob"] for m in mats])
    hs = [[q.QMatrix(rot.slice(c, j), m["fmt"], m["M"], m["K"]) for j, m in enumerate(mats)]
          for c in range(rot.copies)]
    wbytes = sum(int(m["blob"].size) for m in mats)
    res = []
    tokens = [int(t) for t in args.small_decode_only.split(",")] if args.small_decode_only else W.SMALL_DECODE_TOKENS
    for n in tokens:
        xs = [torch.from_numpy(W.small_decode_x(j, n)).to("cuda") for j in range(len(mats))]
        ys = [torch.empty((n, m["M"]), device="cuda") for m in mats]
        layers = rot.copies  # one sample = one layer pass on every copy (> 1 GiB)

        def fn():
            for c in range(layers):
                for grp in DECODE_GROUPS:  # the layer's calls, as in the headline
                    if len(grp) == 1:
                        q.qmm_gemv(hs[c][grp[0]].handle, xs[grp[0]], n, ys[grp[0]])
                    else:
                        q.qmm_gemv_group([hs[c][j].handle for j in grp], [xs[j] for j in grp], n,
                                         [ys[j] for j in grp])
        g = capture(torch, fn)
        us = time_graph(torch, g, args.rounds) * 1e3 / layers
        del g
        flops = 2 * n * sum(m["M"] * m["K"] for m in mats)
        tflops = flops / (us * 1e-6) / 1e12
        # 1..4 tokens: the vector kernels, one fp32 fma per weight and token (fp32 vector
        # ceiling); 5..32: the matrix-core kernel (codes and activations as exact fp16
        # operands), whose products take a small share of the fp16 peak: the weight
        # stream is the roofline there
        mc = n >= 5
        row = {"n": n, "us_per_layer": us, "weight_gbs": wbytes / (us * 1e-6) / 1e9,
               "frac_hbm": wbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
               "tflops": tflops,
               "path": "matrix cores" if mc else "vector",
               "frac_valu_fma": None if mc else tflops / VALU_F32_FMA_TFLOPS,
               "frac_valu_packed": None if mc else tflops / VALU_F32_PACKED_TFLOPS,
               "frac_mfma_f16": tflops / MFMA_F16_PEAK_TFLOPS if mc else None,
               "binding": "hbm"}
        if n >= 4:
            # the same layer through the matrix-matrix path (qmm_gemm_ws, auto tile; fp16
            # staging of the weights, so a looser bound than the matrix-vector path's)
            wss = []
            for j in range(len(mats)):
                nb = q.qmm_gemm_workspace_bytes(hs[0][j].handle, n)
                wss.append(torch.empty((nb + 15) // 16 * 4, device="cuda") if nb else None)

            def fm():
                for c in range(layers):
                    for j in range(len(mats)):
                        q.qmm_gemm_ws(hs[c][j].handle, xs[j], n, ys[j], 0, wss[j])
            g = capture(torch, fm)
            us_mm = time_graph(torch, g, args.rounds) * 1e3 / layers
            del g, wss
            row["gemm_us_per_layer"] = us_mm
        res.append(row)
    return {"workload": "Qwen3-0.6B layer, A4G64 (group 64), fp16 tokens; q+k+v and gate+up share qmm_gemv_group "
                        "calls (one launch each at one token)", "layer_weight_bytes": wbytes,
            "copies": rot.copies, "rotation_bytes": rot.copies * rot.copy_bytes,
            "valu_peaks_tflops": {"fma": VALU_F32_FMA_TFLOPS, "packed": VALU_F32_PACKED_TFLOPS},
            "results": res}


def extra_decode_few(torch, q, W, mats, args):
    """The decode layer (the headline's seven projections) at a few fp16 tokens through
    qmm_gemv: the same launches as the headline at one token; past one token the q+k
    pair and gate+up share grouped calls (grouped calls mix Q4_K with Q6_K only at one
    token), v, attn_output and ffn_down take their own.  Both formats take the matrix
    cores from 5 tokens, the vector kernels below.  Beside it, the same
    layer through the matrix-matrix path (qmm_gemm_ws, weights staged in fp16)."""
    rot = Rotation(torch, [m["blob"] for m in mats])
    hs = [[q.QMatrix(rot.slice(c, j), m["fmt"], m["M"], m["K"]) for j, m in enumerate(mats)]
          for c in range(rot.copies)]
    wbytes = sum(int(m["blob"].size) for m in mats)
    groups_n = [[0, 1], [2], [3], [4, 5], [6]]
    res = []
    tokens = [int(t) for t in args.decode_few_only.split(",")] if args.decode_few_only else [1, 2, 4, 8, 16]
    for n in tokens:
        xs = [torch.from_numpy(W.prefill_x(j, n)).to("cuda") for j in range(len(mats))]
        ys = [torch.empty((n, m["M"]), device="cuda") for m in mats]
        layers = rot.copies
        groups = DECODE_GROUPS if n == 1 else groups_n

        def fn():
            for c in range(layers):
                for grp in groups:
                    if len(grp) == 1:
                        q.qmm_gemv(hs[c][grp[0]].handle, xs[grp[0]], n, ys[grp[0]])
                    else:
                        q.qmm_gemv_group([hs[c][j].handle for j in grp], [xs[j] for j in grp], n,
                                         [ys[j] for j in grp])
        g = capture(torch, fn)
        us = time_graph(torch, g, args.rounds) * 1e3 / layers
        del g
        gbs = wbytes / (us * 1e-6) / 1e9
        row = {"n": n, "us_per_layer": us, "weight_gbs": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
               "launches": len(groups),
               "path": "matrix cores" if n >= 5 else "vector"}
        if n >= 2:
            wss = []
            for j in range(len(mats)):
                nb = q.qmm_gemm_workspace_bytes(hs[0][j].handle, n)
                wss.append(torch.empty((nb + 15) // 16 * 4, device="cuda") if nb else None)

            def fm():
                for c in range(layers):
                    for j in range(len(mats)):
                        q.qmm_gemm_ws(hs[c][j].handle, xs[j], n, ys[j], 0, wss[j])
            g = capture(torch, fm)
            row["gemm_us_per_layer"] = time_graph(torch, g, args.rounds) * 1e3 / layers
            del g, wss
        res.append(row)
    return {"workload": "decode layer (Q4_K / Q6_K, the headline's seven projections), fp16 tokens "
                        "(seeds of the prefill rows), weights rotated over >1 GiB per sample",
            "layer_weight_bytes": wbytes, "copies": rot.copies, "rotation_bytes": rot.copies * rot.copy_bytes,
            "results": res}


def extra_prefill(torch, q, W, mats, args):
    # weight copies rotate over >1 GiB, as for the decode layer, and every sample
    # passes over all of them: at few tokens the path streams its weights, which
    # must not come from a warm cache
    rot = Rotation(torch, [m["blob"] for m in mats])
    hss = [[q.QMatrix(rot.slice(c, j), m["fmt"], m["M"], m["K"]) for j, m in enumerate(mats)]
           for c in range(rot.copies)]
    flops_tok = 2 * sum(m["M"] * m["K"] for m in mats)
    wbytes = sum(int(m["blob"].size) for m in mats)
    res = []
    tokens = [int(t) for t in args.prefill_only.split(",")] if args.prefill_only else W.PREFILL_TOKENS
    for n in tokens:
        xs = [torch.from_numpy(W.prefill_x(j, n)).to("cuda") for j in range(len(mats))]
        ys = [torch.empty((n, m["M"]), device="cuda") for m in mats]
        # the workspace of the K-split calls (QMatrix.gemm's path)
        wss = []
        for j in range(len(mats)):
            nb = q.qmm_gemm_workspace_bytes(hss[0][j].handle, n)
            wss.append(torch.empty((nb + 15) // 16 * 4, device="cuda") if nb else None)
        calls = rot.copies
        per_tile = {}
        for tile in (32, 64):
            g = capture(torch, lambda tile=tile: [q.qmm_gemm_ws(hss[c][j].handle, xs[j], n, ys[j], tile, wss[j])
                                                  for c in range(calls) for j in range(len(mats))])
            per_tile[tile] = g
        ts = {32: [], 64: []}
        for r in range(args.rounds):
            order = (32, 64) if r % 2 == 0 else (64, 32)
            for tile in order:
                ts[tile].append(time_graph(torch, per_tile[tile], 1) * 1e3 / calls)
        chosen = q.qmm_tile_for_tokens(n)
        us = {t: float(np.median(v)) for t, v in ts.items()}
        res.append({"n": n, "chosen_tile": chosen, "k_split": any(w is not None for w in wss),
                    "us_per_layer": us[chosen],
                    "us_tile32": us[32], "us_tile64": us[64], "ratio_64_over_32": us[64] / us[32],
                    "tflops": flops_tok * n / (us[chosen] * 1e-6) / 1e12,
                    "frac_mfma": flops_tok * n / (us[chosen] * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS,
                    "weight_gbs": wbytes / (us[chosen] * 1e-6) / 1e9,
                    "frac_hbm": wbytes / (us[chosen] * 1e-6) / 1e9 / HBM_PEAK_GBS})
        del per_tile, xs, ys, wss
    return {"workload": "decode-layer shapes as prefill GEMM, fp16 tokens, auto tile, "
                        "weights rotated over >1 GiB per sample",
            "copies": rot.copies, "rotation_bytes": rot.copies * rot.copy_bytes, "results": res}


def extra_prefill_batch(torch, q, W, args):
    """A batch of two 65-token sequences (flattened to 130 tokens) on a 128 x 768 matrix in
    every format, both tiles; weights rotated over > 1 GiB per sample."""
    res = []
    for fi, fmt in enumerate(W.FORMAT_ORDER):
        d = W.prefill_batch(fi)
        n = d["x"].shape[0]
        rot = Rotation(torch, [d["blob"]])
        hs = [q.QMatrix(rot.slice(c, 0), fmt, d["M"], d["K"]) for c in range(rot.copies)]
        x = torch.from_numpy(d["x"]).to("cuda")
        y = torch.empty((n, d["M"]), device="cuda")
        nb = q.qmm_gemm_workspace_bytes(hs[0].handle, n)
        ws = torch.empty((nb + 15) // 16 * 4, device="cuda") if nb else None
        graphs = {t: capture(torch, lambda t=t: [q.qmm_gemm_ws(h.handle, x, n, y, t, ws) for h in hs])
                  for t in (32, 64)}
        ts = {32: [], 64: []}
        for r in range(args.rounds):
            for t in ((32, 64) if r % 2 == 0 else (64, 32)):
                ts[t].append(time_graph(torch, graphs[t], 1) * 1e3 / len(hs))
        us = {t: float(np.median(v)) for t, v in ts.items()}
        chosen = q.qmm_tile_for_tokens(n)
        flops = 2 * d["M"] * d["K"] * n
        res.append({"fmt": fmt, "chosen_tile": chosen, "us_per_call": us[chosen], "us_tile32": us[32],
                    "us_tile64": us[64], "k_split": nb > 0, "weight_bytes": int(d["blob"].size),
                    "tflops": flops / (us[chosen] * 1e-6) / 1e12,
                    "frac_mfma": flops / (us[chosen] * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS,
                    "weight_gbs": d["blob"].size / (us[chosen] * 1e-6) / 1e9,
                    "frac_hbm": d["blob"].size / (us[chosen] * 1e-6) / 1e9 / HBM_PEAK_GBS,
                    "copies": rot.copies})
        del graphs, hs, rot, x, y, ws
        torch.cuda.empty_cache()
    return {"workload": "batch of 2 x 65 fp16 tokens (flattened to 130) on 128 x 768, qmm_gemm_ws, "
                        "weights rotated over >1 GiB per sample; 1.4 MFLOP-scale calls bound by their launch",
            "results": res}


def extra_formats(torch, q, W, args):
    """Every block format on one 4096 x 4096 matrix: the one-token and the 16-token (fp16)
    matrix-vector calls (quantized-weight GB/s) and the 512-token matrix-core call
    (TFLOP/s), weights rotated over > 1 GiB of copies per sample."""
    res = []
    for fmt in W.ALL_FORMATS:
        d = W.format_sweep_weights(fmt)
        rot = Rotation(torch, [d["blob"]])
        hs = [q.QMatrix(rot.slice(c, 0), fmt, d["M"], d["K"]) for c in range(rot.copies)]
        row = {"fmt": fmt, "weight_bytes": int(d["blob"].size), "bits_per_weight": d["blob"].size * 8 / (d["M"] * d["K"]),
               "copies": rot.copies}
        x1 = torch.from_numpy(W.format_sweep_x(1)).to("cuda")
        y1 = torch.empty((1, d["M"]), device="cuda")
        g = capture(torch, lambda: [q.qmm_gemv(h.handle, x1, 1, y1) for h in hs])
        us = time_graph(torch, g, args.rounds) * 1e3 / len(hs)
        del g
        row["gemv_n1_us"] = us
        row["gemv_n1_weight_gbs"] = d["blob"].size / (us * 1e-6) / 1e9
        row["gemv_n1_frac_hbm"] = row["gemv_n1_weight_gbs"] / HBM_PEAK_GBS
        # 16 fp16 tokens (qmm_gemv): the matrix cores take every format from at most 16
        x16 = torch.from_numpy(W.format_sweep_x(16)).to("cuda").half()
        y16 = torch.empty((16, d["M"]), device="cuda")
        g = capture(torch, lambda: [q.qmm_gemv(h.handle, x16, 16, y16) for h in hs])
        us = time_graph(torch, g, args.rounds) * 1e3 / len(hs)
        del g
        row["gemv_n16_f16_us"] = us
        row["gemv_n16_f16_weight_gbs"] = d["blob"].size / (us * 1e-6) / 1e9
        row["gemv_n16_f16_tflops"] = 2.0 * d["M"] * d["K"] * 16 / (us * 1e-6) / 1e12
        n = 512
        xn = torch.from_numpy(W.format_sweep_x(n)).to("cuda")
        yn = torch.empty((n, d["M"]), device="cuda")
        nb = q.qmm_gemm_workspace_bytes(hs[0].handle, n)
        ws = torch.empty((nb + 15) // 16 * 4, device="cuda") if nb else None
        g = capture(torch, lambda: [q.qmm_gemm_ws(h.handle, xn, n, yn, 0, ws) for h in hs])
        us = time_graph(torch, g, max(2, args.rounds // 2)) * 1e3 / len(hs)
        del g
        row["gemm_n512_us"] = us
        row["gemm_n512_tflops"] = 2.0 * d["M"] * d["K"] * n / (us * 1e-6) / 1e12
        row["gemm_n512_frac_mfma"] = row["gemm_n512_tflops"] / MFMA_F16_PEAK_TFLOPS
        res.append(row)
        del hs, rot, x1, y1, xn, yn, ws
        torch.cuda.empty_cache()
    return {"workload": "every block format, 4096 x 4096, N(0,0.02^2) weights; 1 fp32 token and 16 fp16 "
                        "tokens (qmm_gemv), 512 fp16 tokens (qmm_gemm_ws, auto tile); weights rotated over "
                        ">1 GiB per sample",
            "results": res}


def extra_moe(torch, q, W, args):
    t0 = time.time()
    stack = W.moe_stack()
    log(f"[bench] expert stack generated in {time.time() - t0:.1f}s")
    rot = Rotation(torch, [stack])
    E, M, K, S = W.MOE_EXPERTS, W.MOE_M, W.MOE_K, W.MOE_SLOTS
    hs = [q.QMatrix(rot.slice(c, 0), "q4_0", M, K, E) for c in range(rot.copies)]
    ebytes = stack.size // E
    res = []
    C = 64
    only = [int(t) for t in args.moe_only.split(",")] if args.moe_only else None
    for n in ([t for t in only if t <= 32] if only else W.MOE_TOKENS):
        ids_h = [W.moe_ids(n, c) for c in range(C)]
        ids = [torch.from_numpy(i).to("cuda") for i in ids_h]
        x = torch.from_numpy(W.moe_x(n)).to("cuda")
        y = torch.empty((n, S, M), device="cuda")
        calls = C
        g = capture(torch, lambda: [q.qmm_gemm_id(hs[c % rot.copies].handle, x, n, S, 1, ids[c], y)
                                    for c in range(calls)])
        us = time_graph(torch, g, args.rounds) * 1e3 / calls
        distinct = float(np.mean([len(np.unique(i)) for i in ids_h]))
        gbs = distinct * ebytes / (us * 1e-6) / 1e9
        res.append({"n": n, "us_per_call": us, "distinct_experts": distinct,
                    "distinct_weight_gbs": gbs, "frac_hbm": gbs / HBM_PEAK_GBS})
    # prefill-sized calls on the matrix cores (qmm_gemm_id_tiled), fp16 activations
    pre = []
    C = 8
    for n in ([t for t in only if t > 32] if only else W.MOE_PREFILL_TOKENS):
        ids_h = [W.moe_ids(n, c) for c in range(C)]
        ids = [torch.from_numpy(i).to("cuda") for i in ids_h]
        x = torch.from_numpy(W.moe_prefill_x(n)).to("cuda")
        y = torch.empty((n, S, M), device="cuda")
        g = capture(torch, lambda: [q.qmm_gemm_id_tiled(hs[c % rot.copies].handle, x, n, S, 1, ids[c], y)
                                    for c in range(C)])
        us = time_graph(torch, g, args.rounds) * 1e3 / C
        distinct = float(np.mean([len(np.unique(i)) for i in ids_h]))
        tflops = 2.0 * M * K * n * S / (us * 1e-6) / 1e12
        pre.append({"n": n, "us_per_call": us, "distinct_experts": distinct, "tflops": tflops,
                    "frac_mfma": tflops / MFMA_F16_PEAK_TFLOPS,
                    "distinct_weight_gbs": distinct * ebytes / (us * 1e-6) / 1e9})
    return {"workload": "128 experts x Q4_0 4096x512, 8 ids per token, ids re-drawn per call",
            "copies": rot.copies, "results": res,
            "prefill_tiled": {"workload": "same experts, fp16 tokens, qmm_gemm_id_tiled, auto tile", "results": pre}}


def extra_quantize(torch, q, W, mats, args):
    """The GPU quantizer on the decode layer's fp32 weights (regenerated from the
    same seeds), fp32 bytes read per second."""
    res = []
    for j, m in enumerate(mats):
        if m["name"] not in ("ffn_gate", "ffn_down"):
            continue
        w = torch.from_numpy(W.decode_weights_fp32(j)).to("cuda")
        out = torch.empty(m["blob"].size, dtype=torch.uint8, device="cuda")
        g = capture(torch, lambda: [q.qmm_quantize(m["fmt"], w, m["M"], m["K"], out) for _ in range(5)])
        us = time_graph(torch, g, args.rounds) * 1e3 / 5
        res.append({"proj": m["name"], "fmt": m["fmt"], "M": m["M"], "K": m["K"], "us": us,
                    "fp32_gbs": w.numel() * 4 / (us * 1e-6) / 1e9,
                    "same_bytes_as_data": bool(np.array_equal(out.cpu().numpy(), m["blob"]))})
        del w, out
    return {"workload": "qmm_quantize of decode-layer weights (fp32 in, blocks out)", "results": res}


# ------------------------------------------------------------------------------------------------

def calibrate(torch, W):
    """Reference points for the one-token GEMV, both as replays of HIP graphs over rotating
    copies (> 1 GiB): the launch of a one-element in-place add (an empty kernel), and a
    plain streaming read of each decode-layer projection's byte count (torch's int32 sum
    over the bytes) and of the whole layer in one launch."""
    out = {}
    t = torch.zeros(1, device="cuda")
    g = capture(torch, lambda: [t.add_(1) for _ in range(1000)])
    out["empty_kernel_us"] = time_graph(torch, g, 5) * 1e3 / 1000
    del g
    sizes = [(name, M * {"q4_k": 144, "q6_k": 210}[fmt] * K // 256) for name, M, K, fmt in W.DECODE_SHAPES]
    per = dict(sizes)
    # the headline step's launch sets (grouped calls) and the whole layer in one launch
    mats = [{"fmt": f, "K": K, "M": M, "name": n} for n, M, K, f in W.DECODE_SHAPES]
    for c in DECODE_GROUPS:
        for st in launch_sets(mats, c, 1):
            if len(st) > 1:
                names = [mats[j]["name"] for j in st]
                sizes.append(("+".join(names), sum(per[n] for n in names)))
    sizes.append(("whole layer", sum(per.values())))
    reads = []
    for name, nbytes in sizes:
        per = (nbytes + 4095) // 4096 * 4096
        copies = max(2, -(-ROTATE_BYTES // per))
        buf = torch.ones(copies * per, dtype=torch.uint8, device="cuda")
        row = {"name": name, "bytes": nbytes}
        # (a) a row-wise max over the bytes as int32 rows of 1024: one kernel reading every
        # byte once and writing 1/1024 of it
        rows = [buf[c * per:(c + 1) * per].view(torch.int32).view(-1, 1024) for c in range(copies)]
        g = capture(torch, lambda: [r.amax(dim=1) for r in rows])
        row["rowmax_us"] = time_graph(torch, g, 5) * 1e3 / copies
        del g
        # (b) a device copy of half the bytes (reads nbytes / 2, writes nbytes / 2)
        half = per // 2
        g = capture(torch, lambda: [buf[c * per + half:c * per + 2 * half].copy_(buf[c * per:c * per + half])
                                    for c in range(copies)])
        row["copy_half_us"] = time_graph(torch, g, 5) * 1e3 / copies
        del g, rows
        row["stream_us"] = min(row["rowmax_us"], row["copy_half_us"])
        row["stream_gbs"] = nbytes / (row["stream_us"] * 1e-6) / 1e9
        reads.append(row)
        del buf
        torch.cuda.empty_cache()
    out["streaming_read"] = reads
    # torch's dense fp16 GEMM (hipBLASLt) on the decode-layer shapes: the same products
    # with the weights already fp16, y = x W^T with W^T stored [K, M] (no transposed view),
    # two weight copies alternating
    dense = []
    for n in (512, 2048):
        tot_us, tot_fl = 0.0, 0.0
        for name, M, K, fmt in W.DECODE_SHAPES:
            wts = [torch.randn(K, M, device="cuda").mul_(0.02).half() for _ in range(2)]
            x = torch.randn(n, K, device="cuda").half()
            ys = [torch.empty(n, M, device="cuda", dtype=torch.float16) for _ in range(2)]
            g = capture(torch, lambda: [torch.mm(x, wts[c % 2], out=ys[c % 2]) for c in range(8)])
            us = time_graph(torch, g, 5) * 1e3 / 8
            del g, wts, ys
            fl = 2.0 * n * M * K
            tot_us += us
            tot_fl += fl
            dense.append({"n": n, "name": name, "us": round(us, 2), "tflops": round(fl / (us * 1e-6) / 1e12, 1)})
        dense.append({"n": n, "name": "layer", "us": round(tot_us, 2), "tflops": round(tot_fl / (tot_us * 1e-6) / 1e12, 1)})
        torch.cuda.empty_cache()
    out["dense_fp16_gemm"] = dense
    return out


def _csv_rows(root, suffix):
    import csv
    rows = []
    for path in sorted(glob.glob(os.path.join(root, "**", f"*{suffix}"), recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def _col(row, *names):
    for n in names:
        if n in row:
            return row[n]
    raise KeyError(names)


def summarize_trace(root, table_only=False):
    """Markdown summary of a rocprofv3 --kernel-trace run of this benchmark (with the
    headline's one-token GEMV figures unless table_only: a run of another workload)."""
    from qmm_synth import workloads as W
    rows = _csv_rows(root, "kernel_trace.csv")
    if not rows:
        raise SystemExit(f"no *kernel_trace.csv under {root}")
    stats = {}
    for r in rows:
        name = _col(r, "Kernel_Name", "Kernel-Name")
        dur = (int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp"))) / 1e3
        grid = int(_col(r, "Grid_Size_X", "Grid_Size"))
        wg = int(_col(r, "Workgroup_Size_X", "Workgroup_Size"))
        stats.setdefault((name, grid, wg), []).append(dur)
    lines = ["| kernel | grid x | workgroup | dispatches | median us | mean us |", "|---|---|---|---|---|---|"]
    gemv = []
    for (name, grid, wg), ds in sorted(stats.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{name}` | {grid} | {wg} | {len(ds)} | {np.median(ds):.2f} | {np.mean(ds):.2f} |")
        if "k_gemv1" in name:
            gemv.extend(ds)
    if not gemv or table_only:  # another workload: the table only
        print("\n".join(lines))
        return
    nl, alg = headline_launches(W)
    mean = float(np.mean(gemv)) if gemv else float("nan")
    lines += ["", f"All one-token GEMV dispatches (k_gemv1 and k_gemv1_pair): {len(gemv)}, mean {mean:.3f} us; "
              f"{nl} per step -> {nl * mean:.2f} us of kernel time per step; "
              f"algorithmic bytes per launch {alg:.0f} -> {alg / (mean * 1e-6) / 1e9:.1f} GB/s "
              f"= {alg / (mean * 1e-6) / 1e9 / HBM_PEAK_GBS:.4f} of 8 TB/s.", "",
              "Machine-readable:", "",
              f"- source_digest: {source_digest()}",
              f"- gemv1_dispatches: {len(gemv)}",
              f"- gemv1_mean_us: {mean:.4f}",
              f"- alg_bytes_per_launch: {alg:.0f}"]
    print("\n".join(lines))


def summarize_sq(dirs, top=8):
    """Per kernel (name and grid) of rocprofv3 --pmc runs over the same workload: the SQ
    counters summed over its dispatches, as fractions of wave-cycles and per wave."""
    agg, disp = {}, {}
    for d in dirs:
        for r in _csv_rows(d, "counter_collection.csv"):
            k = f"{_col(r, 'Kernel_Name')[:60]} grid {_col(r, 'Grid_Size', 'Grid_Size_X')}"
            a = agg.setdefault(k, {})
            a[_col(r, "Counter_Name")] = a.get(_col(r, "Counter_Name"), 0.0) + float(_col(r, "Counter_Value"))
            disp.setdefault((k, d), set()).add(_col(r, "Dispatch_Id"))
    out = []
    for k, v in sorted(agg.items(), key=lambda kv: -kv[1].get("SQ_WAVE_CYCLES", 0))[:top]:
        nd = max(len(disp.get((k, d), ())) for d in dirs)
        wc = v.get("SQ_WAVE_CYCLES", 0) or 1.0
        waves = v.get("SQ_WAVES", 0) or 1.0
        out.append(f"{k}: {nd} dispatches, {waves / nd:.0f} waves each")
        out.append("   of wave-cycles: VALU %.2f, LDS %.2f, VMEM %.2f, waiting %.2f, dependency stalls %.2f" % (
            v.get("SQ_ACTIVE_INST_VALU", 0) / wc, v.get("SQ_ACTIVE_INST_LDS", 0) / wc,
            v.get("SQ_ACTIVE_INST_VMEM", 0) / wc, v.get("SQ_WAIT_ANY", 0) / wc, v.get("SQ_WAIT_INST_ANY", 0) / wc))
        out.append("   per wave: VALU %.0f, MFMA %.0f, LDS %.0f, VMEM reads %.0f instructions" % (
            v.get("SQ_INSTS_VALU", 0) / waves, v.get("SQ_INSTS_MFMA", 0) / waves, v.get("SQ_INSTS_LDS", 0) / waves,
            v.get("SQ_INSTS_VMEM_RD", 0) / waves))
    print("\n".join(out))


def summarize_counters(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    """Markdown summary of rocprofv3 FETCH_SIZE / WRITE_SIZE passes over this benchmark's
    headline (kernels k_gemv1, k_gemv1_pair) and over --copy-probe (the calibration copy)."""
    from qmm_synth import workloads as W

    def per_dispatch(root, counter, match):
        vals = {}
        for r in _csv_rows(root, "counter_collection.csv"):
            if _col(r, "Counter_Name") != counter or match not in _col(r, "Kernel_Name"):
                continue
            key = _col(r, "Dispatch_Id")
            vals[key] = vals.get(key, 0.0) + float(_col(r, "Counter_Value"))
        return list(vals.values())

    f = per_dispatch(fetch_dir, "FETCH_SIZE", "k_gemv1")
    w = per_dispatch(write_dir, "WRITE_SIZE", "k_gemv1")
    cf = per_dispatch(copy_fetch_dir, "FETCH_SIZE", "copyBuffer")
    cw = per_dispatch(copy_write_dir, "WRITE_SIZE", "copyBuffer")
    moved_kib = (256 << 20) / 1024
    ff, wf = moved_kib / float(np.mean(cf)), moved_kib / float(np.mean(cw))
    traffic = (float(np.mean(f)) * ff + float(np.mean(w)) * wf) * 1024
    nl, alg = headline_launches(W)
    lines = ["| quantity | value |", "|---|---|",
             f"| k_gemv1 / k_gemv1_pair dispatches (fetch pass / write pass) | {len(f)} / {len(w)} |",
             f"| FETCH_SIZE per dispatch (KiB, raw) | {np.mean(f):.1f} |",
             f"| WRITE_SIZE per dispatch (KiB, raw) | {np.mean(w):.2f} |",
             f"| copy probe: FETCH_SIZE / WRITE_SIZE for {moved_kib:.0f} KiB moved | {np.mean(cf):.1f} / {np.mean(cw):.1f} KiB |",
             f"| calibration factor fetch / write | {ff:.4f} / {wf:.4f} |",
             f"| HBM traffic per launch (bytes, calibrated) | {traffic:.0f} |",
             f"| algorithmic bytes per launch (weights + x + y of the layer over its {nl} launches) | {alg:.0f} |",
             f"| traffic / algorithmic | {traffic / alg:.3f} |",
             "", "Machine-readable (read by bench.py; valid only for this kernel source):", "",
             f"- source_digest: {source_digest()}",
             f"- traffic_bytes_per_launch: {traffic:.0f}",
             f"- fetch_factor: {ff:.4f}",
             f"- write_factor: {wf:.4f}"]
    print("\n".join(lines))


def copy_probe(torch):
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 5}))


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.table_only)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.summarize_sq:
        summarize_sq(args.summarize_sq)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the library has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import block_quantized_weight_matmul_amd as q
    from qmm_synth import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe(torch)
        return
    if args.calibrate:
        print(json.dumps({"calibration": calibrate(torch, W)}), flush=True)
        return
    if args.moe_only:
        print(json.dumps({"expert_matvec": extra_moe(torch, q, W, args)}), flush=True)
        return
    if args.formats_only:
        print(json.dumps({"formats": extra_formats(torch, q, W, args)}), flush=True)
        return
    if args.small_decode_only:
        print(json.dumps({"small_decode_a4g64": extra_small_decode(torch, q, W, args)}), flush=True)
        return
    if args.decode_few_only:
        mats = [W.decode_weights(j) for j in range(len(W.DECODE_SHAPES))]
        print(json.dumps({"decode_layer_few_tokens": extra_decode_few(torch, q, W, mats, args)}), flush=True)
        return
    if args.prefill_only:
        mats = [W.decode_weights(j) for j in range(len(W.DECODE_SHAPES))]
        print(json.dumps({"prefill_gemm": extra_prefill(torch, q, W, mats, args)}), flush=True)
        return

    head, mats = decode_layer(torch, q, W, args)
    log(f"[bench] decode layer: {head['value']:.1f} GB/s, {head['ms_per_step'] * 1e3:.2f} us/step")
    digest = source_digest()
    kern = head["kernel"]
    traffic, traffic_note = traffic_from_profile(digest)
    result = {
        "metric": METRIC,
        "value": round(head["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "decode GEMV, 1 fp32 token, seven Qwen3-Embedding-4B layer projections "
                        "(Q4_K x5, Q6_K x2), weights N(0,0.02^2) quantized, rotated over >1 GiB",
            "tokens": 1,
            "layer_weight_bytes": head["layer_weight_bytes"],
            "frac_hbm": head["value"] / HBM_PEAK_GBS,
            "event_ms_per_step": head["event_ms_per_step"],
            "sum_of_isolated_kernel_us": head["sum_isolated_us"],
            "copies": head["copies"],
            "rotation_bytes": head["rotation_bytes"],
            "source_digest": digest,
            "projections": head["projections"],
            "calls": head["calls"],
        },
        "roofline": {
            "kernel": "qmm::k_gemv1 / k_gemv1_pair (one-token GEMV; the step's launches: "
                      + ", ".join("+".join(c) for c in head["launch_sets"]) + ")",
            "bound": "hbm",
            "achieved": round(kern["achieved_gbs"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": kern["achieved_gbs"] / HBM_PEAK_GBS,
            "traffic": traffic,
            "traffic_note": traffic_note,
            "avg_launch_us": kern["avg_us"],
            "alg_bytes_per_launch": kern["alg_bytes_per_launch"],
            "launches_per_step": kern["launches_per_step"],
            "launch_time_source": "HIP events around the timed region (graph replays on the current stream) / "
                                  "launches; per-dispatch trace durations in profiles/ add up to the step",
        },
    }
    extras = {}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(mats)
        log(f"[bench] cpu baseline: {result['cpu_baseline']['value']:.4f} GB/s")
        t0 = time.time()
        extras["oracle_per_config"] = oracle_per_config(W, mats)
        log(f"[bench] oracle per config done in {time.time() - t0:.1f}s")
    if not args.no_extras:
        for name, fn in (("single_matvec", lambda: extra_single_matvec(torch, q, W, args)),
                         ("small_decode_a4g64", lambda: extra_small_decode(torch, q, W, args)),
                         ("decode_layer_few_tokens", lambda: extra_decode_few(torch, q, W, mats, args)),
                         ("prefill_gemm", lambda: extra_prefill(torch, q, W, mats, args)),
                         ("prefill_batch_2x65", lambda: extra_prefill_batch(torch, q, W, args)),
                         ("formats", lambda: extra_formats(torch, q, W, args)),
                         ("expert_matvec", lambda: extra_moe(torch, q, W, args)),
                         ("quantize", lambda: extra_quantize(torch, q, W, mats, args))):
            t0 = time.time()
            extras[name] = fn()
            log(f"[bench] extra {name} done in {time.time() - t0:.1f}s")
            torch.cuda.empty_cache()
    if extras:
        result["extras"] = extras
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
