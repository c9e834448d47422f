"""The committed headline profiles agree with each other and with the roofline the
benchmark reports: the trace's mean GEMV dispatch and the live event-timed launch
give the same fraction of 8 TB/s within 5%, and the counter summary was taken on
the same kernel source as the trace.  (CPU only: reads profiles/.)"""

import os
import re

import bench
from qmm_synth import workloads as W
from tests.conftest import ROOT

TRACE = os.path.join(ROOT, "profiles", "gemv_decode_layer_kernel_trace.md")
COUNTERS = os.path.join(ROOT, "profiles", "gemv_decode_layer_counters.md")


def machine_readable(path):
    vals = {}
    for line in open(path):
        m = re.match(r"- (\w+): (\S+)$", line.strip())
        if m:
            vals[m.group(1)] = m.group(2)
    return vals


def test_trace_bytes_are_the_benchmark_definition():
    t = machine_readable(TRACE)
    launches, alg = bench.headline_launches(W)
    assert int(t["alg_bytes_per_launch"]) == round(alg)
    assert launches == 4


def test_trace_and_live_roofline_agree():
    t = machine_readable(TRACE)
    text = open(TRACE).read()
    m = re.search(r"launches, ([\d.]+) us \(([\d.]+) us per step event-timed, frac\s+([\d.]+)\)", text)
    assert m, "live figure not found in the trace summary"
    live_us, live_frac = float(m.group(1)), float(m.group(3))
    alg = float(t["alg_bytes_per_launch"])
    assert abs(alg / (live_us * 1e-6) / 1e9 / bench.HBM_PEAK_GBS - live_frac) < 1e-3
    trace_frac = alg / (float(t["gemv1_mean_us"]) * 1e-6) / 1e9 / bench.HBM_PEAK_GBS
    assert abs(trace_frac / live_frac - 1) < 0.05, (trace_frac, live_frac)


def test_counters_taken_on_the_traced_source():
    assert machine_readable(COUNTERS)["source_digest"] == machine_readable(TRACE)["source_digest"]
