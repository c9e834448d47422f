"""Shared helpers of the GPU parity tests: device upload, comparisons, reporting."""

import numpy as np
import torch

import oracle
from qmm_synth import quantize, workloads

DEV = "cuda"
FORMATS = ["q4_0", "q8_0", "q4_k", "q6_k", "a4g64", "q4_1", "q5_0", "q5_1", "q2_k", "q3_k", "q5_k"]
# byte offsets of each format's fp16 scale fields (kept finite in random-byte blocks)
SCALE_OFFSETS = {"q4_0": [0], "q8_0": [0], "q4_k": [0, 2], "q6_k": [0], "a4g64": [0, 2], "q4_1": [0, 2],
                 "q5_0": [0], "q5_1": [0, 2], "q2_k": [0, 2], "q3_k": [0], "q5_k": [0, 2]}
# the formats the GPU quantizer (and the oracle's reference quantizer) encode
QUANT_FORMATS = ["q4_0", "q8_0", "q4_k", "q6_k", "a4g64"]


def to_dev(a):
    return torch.from_numpy(np.array(a, order="C")).to(DEV)


def to_host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def make_matrix(fmt, M, K, seed, scale=0.02):
    g = np.random.default_rng(seed)
    w = (g.normal(0.0, scale, size=(M, K))).astype(np.float32)
    return quantize(fmt, w)


def assert_within(y, y_ref, S, tol, label=""):
    """|y - y_ref| <= tol * S elementwise (y fp32 from the device, refs fp64)."""
    y = np.asarray(y, dtype=np.float64)
    assert y.shape == y_ref.shape, (y.shape, y_ref.shape)
    assert np.all(np.isfinite(y)), f"{label}: non-finite output"
    err = np.abs(y - y_ref)
    bad = err > tol * S
    if np.any(bad):
        i = np.unravel_index(np.argmax(np.where(bad, err / np.maximum(S, 1e-300), 0)), y.shape)
        raise AssertionError(f"{label}: {bad.sum()} of {y.size} outside {tol}*S; worst at {i}: "
                             f"y={y[i]!r} ref={y_ref[i]!r} S={S[i]!r}")
    return float(np.max(err / np.maximum(S, 1e-300))) if y.size else 0.0


def count_differences(a, b):
    """Number of elements whose fp32 bit patterns differ (bit-for-bit comparison)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    assert a.shape == b.shape
    return int(np.count_nonzero(a.view(np.uint32) != b.view(np.uint32)))


__all__ = ["DEV", "FORMATS", "QUANT_FORMATS", "SCALE_OFFSETS", "to_dev", "to_host", "make_matrix", "assert_within", "count_differences",
           "oracle", "quantize", "workloads"]
