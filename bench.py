#!/usr/bin/env python3
"""Benchmark of the fused dequantize-and-multiply on one MI355X.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--no-extras] [--no-cpu-baseline]

Headline (one JSON line on stdout): quantized-weight GB/s of the matrix-vector
path at one token on the seven projections of a Qwen3-Embedding-4B decoder
layer (Q4_K: 4096x2560, 1024x2560, 2560x4096, 9728x2560 twice; Q6_K:
1024x2560, 2560x9728; random N(0, 0.02^2) weights, N(0, 1) fp32 activations).
A step is one pass over the layer: seven GEMV launches.  Weights rotate
through copies totalling more than 1 GiB, so each step streams them from HBM
rather than the 256 MB Infinity Cache.  Steps are timed as replays of HIP
graphs captured from the library's launches (the graph only removes host
launch overhead; the kernels are the ones an eager call runs).

Also reported:
  roofline      the dominant kernel (the GEMV instance with the most time per
                step): algorithmic bytes per launch / its mean launch time, from
                HIP events around a graph of back-to-back launches of each
                projection, against 8 TB/s; "traffic" from the rocprofv3 counter
                summary in profiles/ when it was taken on the current kernel
                source, else null.
  cpu_baseline  the CPU oracle (NumPy dequantization + fp64 matmul) on a bounded
                sample of the same workload, in the same unit.
  extras        the other workloads: the single Q4_0 256x512 matvec, 4-bit
                affine-group decode at 1..16 tokens, the prefill GEMM at
                7..2048 tokens with both token tiles, and the expert-indexed
                matvec at 2..24 tokens with ids re-drawn per call.
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
ROTATE_BYTES = 1 << 30         # > 256 MB Infinity Cache
METRIC = "quantized-weight GB/s at n<=16 and TFLOP/s at n>=64, as % of roofline"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-extras", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--event-launches", type=int, default=64, help="launches per projection in the per-kernel pass")
    p.add_argument("--calls", type=int, default=20, help="calls per timed sample in the extras")
    p.add_argument("--rounds", type=int, default=6, help="timed samples per extra case (median)")
    p.add_argument("--copy-probe", action="store_true", help="only run a 256 MiB device copy (counter calibration)")
    p.add_argument("--prefill-only", default=None, metavar="N[,N...]",
                   help="only time the decode layer's prefill GEMM at these token counts (for profiling)")
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

    def step(c):
        for j in range(P):
            q.qmm_gemv(handles[c][j].handle, xs[j], 1, ys[j])

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

    # per-kernel pass: for each projection, a graph of R back-to-back launches (rotating
    # copies) timed with HIP events on the stream it is replayed on; mean per launch
    R = args.event_launches
    mean_us = np.zeros(P)
    for j in range(P):
        g = capture(torch, lambda j=j: [q.qmm_gemv(handles[r % rot.copies][j].handle, xs[j], 1, ys[j])
                                       for r in range(R)])
        mean_us[j] = time_graph(torch, g, 5) * 1e3 / R
        del g
    # kernels are instantiated per block format (the token bucket is fixed at one token)
    per_kernel = {}
    for j, m in enumerate(mats):
        k = per_kernel.setdefault(m["fmt"], {"launches": 0, "us": 0.0, "alg_bytes": 0, "weight_bytes": 0,
                                             "projections": []})
        k["launches"] += 1
        k["us"] += float(mean_us[j])
        k["alg_bytes"] += int(m["blob"].size) + 4 * m["K"] + 4 * m["M"]
        k["weight_bytes"] += int(m["blob"].size)
        k["projections"].append(m["name"])
    dom_fmt = max(per_kernel, key=lambda f: per_kernel[f]["us"])
    dk = per_kernel[dom_fmt]
    avg_us = dk["us"] / dk["launches"]
    alg_per_launch = dk["alg_bytes"] / dk["launches"]
    achieved = alg_per_launch / (avg_us * 1e-6) / 1e9
    projections = [{"name": m["name"], "fmt": m["fmt"], "M": m["M"], "K": m["K"], "weight_bytes": int(m["blob"].size),
                    "mean_us": round(float(mean_us[j]), 3),
                    "weight_gbs": round(m["blob"].size / (mean_us[j] * 1e-6) / 1e9, 1)}
                   for j, m in enumerate(mats)]
    out = {
        "value": value, "ms_per_step": ms_per_step, "event_ms_per_step": ev_ms / args.steps,
        "layer_weight_bytes": layer_weight_bytes, "layer_alg_bytes": layer_alg_bytes,
        "copies": rot.copies, "rotation_bytes": rot.copies * rot.copy_bytes,
        "projections": projections,
        "dominant": {"fmt": dom_fmt, "launches_per_step": dk["launches"], "avg_us": avg_us,
                     "alg_bytes_per_launch": alg_per_launch, "achieved_gbs": achieved,
                     "projections": dk["projections"]},
        "sum_kernel_us": float(mean_us.sum()),
    }
    del handles, full, singles
    return out, mats


def traffic_from_profile(fmt, digest):
    """HBM bytes per launch from the committed counter summary, if it matches this source."""
    path = os.path.join(ROOT, "profiles", f"gemv_{fmt}_decode_layer_counters.md")
    if not os.path.exists(path):
        return None, "no counter summary"
    vals = {}
    for line in open(path):
        if ":" in line and line.strip().startswith("- "):
            k, _, v = line.strip()[2:].partition(":")
            vals[k.strip()] = v.strip()
    if vals.get("source_digest") != digest:
        return None, "counters taken on another kernel source"
    try:
        return float(vals["traffic_bytes_per_launch"]), "rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated"
    except (KeyError, ValueError):
        return None, "summary incomplete"


# ------------------------------------------------------------------------------------------------
# CPU oracle baseline

def cpu_baseline(mats):
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        blas_threads = None
    names = ("ffn_gate", "ffn_down")
    sample = [m for m in mats if m["name"] in names]
    from qmm_synth import workloads as W
    t0 = time.perf_counter()
    nbytes = 0
    for m in sample:
        w = oracle.dequantize(m["fmt"], m["blob"], m["M"], m["K"])
        x = W.decode_x([d[0] for d in W.DECODE_SHAPES].index(m["name"]), 1)
        oracle.matmul_ref(x, w)
        nbytes += int(m["blob"].size)
    dt = time.perf_counter() - t0
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": (f"{'+'.join(names)} of the same layer ({nbytes} quantized bytes, "
                       f"{nbytes / sum(m['blob'].size for m in mats):.0%} of it) at one token: NumPy "
                       f"dequantization (single-threaded) + fp64 matmul (BLAS threads available: "
                       f"{blas_threads}), {dt:.1f} s; cores counts the dequantization thread, which "
                       f"takes >99% of the time")}


# ------------------------------------------------------------------------------------------------
# extras

def extra_single_matvec(torch, q, W, args):
    d = W.single_matvec()
    rot = Rotation(torch, [d["blob"]], min_total=64 << 20)
    hs = [q.QMatrix(rot.slice(c, 0), d["fmt"], d["M"], d["K"]) for c in range(rot.copies)]
    x = torch.from_numpy(d["x"]).to("cuda")
    y = torch.empty((1, d["M"]), device="cuda")
    g = capture(torch, lambda: [q.qmm_gemv(hs[i % rot.copies].handle, x, 1, y) for i in range(args.calls)])
    us = time_graph(torch, g, args.rounds) * 1e3 / args.calls
    return {"workload": "Q4_0 256x512, 1 fp32 token", "us_per_call": us,
            "weight_gbs": d["blob"].size / (us * 1e-6) / 1e9,
            "frac_hbm": d["blob"].size / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}


def extra_small_decode(torch, q, W, args):
    mats = [W.small_decode_weights(i) for i in range(len(W.SMALL_DECODE_SHAPES))]
    rot = Rotation(torch, [m["blob"] for m in mats])
    hs = [[q.QMatrix(rot.slice(c, j), m["fmt"], m["M"], m["K"]) for j, m in enumerate(mats)]
          for c in range(rot.copies)]
    wbytes = sum(int(m["blob"].size) for m in mats)
    res = []
    for n in W.SMALL_DECODE_TOKENS:
        xs = [torch.from_numpy(W.small_decode_x(j, n)).to("cuda") for j in range(len(mats))]
        ys = [torch.empty((n, m["M"]), device="cuda") for m in mats]
        layers = min(args.calls, rot.copies)

        def fn():
            for c in range(layers):
                for j in range(len(mats)):
                    q.qmm_gemv(hs[c][j].handle, xs[j], n, ys[j])
        g = capture(torch, fn)
        us = time_graph(torch, g, args.rounds) * 1e3 / layers
        flops = 2 * n * sum(m["M"] * m["K"] for m in mats)
        res.append({"n": n, "us_per_layer": us, "weight_gbs": wbytes / (us * 1e-6) / 1e9,
                    "frac_hbm": wbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                    "tflops": flops / (us * 1e-6) / 1e12})
    return {"workload": "Qwen3-0.6B layer, A4G64 (group 64), fp16 tokens", "layer_weight_bytes": wbytes,
            "copies": rot.copies, "results": res}


def extra_prefill(torch, q, W, mats, args):
    # weight copies rotate over >1 GiB, as for the decode layer: at few tokens the
    # path streams its weights, which must not come from a warm cache
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
        # the workspace of the K-split few-token calls (QMatrix.gemm's path)
        wss = []
        for j in range(len(mats)):
            nb = q.qmm_gemm_workspace_bytes(hss[0][j].handle, n)
            wss.append(torch.empty((nb + 15) // 16 * 4, device="cuda") if nb else None)
        calls = max(1, min(args.calls, rot.copies, int(2e10 // (flops_tok * n)) or 1))
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
                    "weight_gbs": wbytes / (us[chosen] * 1e-6) / 1e9})
        del per_tile
    return {"workload": "decode-layer shapes as prefill GEMM, fp16 tokens, auto tile, weights rotated",
            "copies": rot.copies, "results": res}


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
    if args.moe_only:
        print(json.dumps({"expert_matvec": extra_moe(torch, q, W, args)}), flush=True)
        return
    if args.prefill_only:
        mats = [W.decode_weights(j) for j in range(len(W.DECODE_SHAPES))]
        print(json.dumps({"prefill_gemm": extra_prefill(torch, q, W, mats, args)}), flush=True)
        return

    head, mats = decode_layer(torch, q, W, args)
    log(f"[bench] decode layer: {head['value']:.1f} GB/s, {head['ms_per_step'] * 1e3:.2f} us/step")
    digest = source_digest()
    dom = head["dominant"]
    traffic, traffic_note = traffic_from_profile(dom["fmt"], digest)
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
            "sum_of_kernel_us": head["sum_kernel_us"],
            "copies": head["copies"],
            "source_digest": digest,
            "projections": head["projections"],
        },
        "roofline": {
            "kernel": f"qmm::k_gemv1<{dom['fmt']}, fp32 x> (one-token GEMV)",
            "bound": "hbm",
            "achieved": round(dom["achieved_gbs"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": dom["achieved_gbs"] / HBM_PEAK_GBS,
            "traffic": traffic,
            "traffic_note": traffic_note,
            "avg_launch_us": dom["avg_us"],
            "alg_bytes_per_launch": dom["alg_bytes_per_launch"],
            "launches_per_step": dom["launches_per_step"],
            "projections": dom["projections"],
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(mats)
        log(f"[bench] cpu baseline: {result['cpu_baseline']['value']:.4f} GB/s")
    if not args.no_extras:
        extras = {}
        for name, fn in (("single_matvec", lambda: extra_single_matvec(torch, q, W, args)),
                         ("small_decode_a4g64", lambda: extra_small_decode(torch, q, W, args)),
                         ("prefill_gemm", lambda: extra_prefill(torch, q, W, mats, args)),
                         ("expert_matvec", lambda: extra_moe(torch, q, W, args)),
                         ("quantize", lambda: extra_quantize(torch, q, W, mats, args))):
            t0 = time.time()
            extras[name] = fn()
            log(f"[bench] extra {name} done in {time.time() - t0:.1f}s")
            torch.cuda.empty_cache()
        result["extras"] = extras
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
