"""Matrix-matrix path (qmm_gemm) against the oracle, and the two token tiles against
each other.

Tolerance: |y - y_ref| <= 2e-3 * S.  The path stages weights as fp16 (round
to nearest even of the exact fp32 weight, relative error <= 2^-11) and fp32
activations as fp16 (<= 2^-11 more; fp16 activations are exact), multiplies
exactly and accumulates in fp32, so its error is about 1e-3 * S at most.  A
tighter check compares with the product of the staged fp16 values in fp64,
which leaves only the fp32 accumulation: 1e-5 * S16.

Tiles: the candle pull request "Metal: 64-token tile for the quantized
matrix-matrix kernel" (section "Same results, bit for bit") requires every
output to be equal bit for bit at the 32- and 64-token tiles, on 7, 32, 33 and
130 tokens and a batch of 2 x 65, with a guard that the result is not all zero."""

import ctypes
import numpy as np
import pytest
import torch

import block_quantized_weight_matmul_amd as q
from block_quantized_weight_matmul_amd import _lib as L
from tests.gpu_helpers import FORMATS, assert_within, count_differences, make_matrix, oracle, to_dev, to_host

pytestmark = pytest.mark.gpu

TOL = 2e-3
TOL16 = 1e-5

# (tokens, rows, K) of the page's byte-identity test; "1x33x200x512" reads as
# batch x tokens x rows x K, so the 7/32/33-token shapes use 200 rows and K = 512.
PAGE_SHAPES = [(7, 200, 512), (32, 200, 512), (33, 200, 512), (130, 96, 512), (130, 128, 768)]


def _data(fmt, N, M, K, xdtype, seed):
    blob = make_matrix(fmt, M, K, seed)
    w = oracle.dequantize(fmt, blob, M, K)
    g = np.random.default_rng(list(seed) + [9])
    x = g.standard_normal((N, K)).astype(np.float32).astype(xdtype)
    return blob, w, x


def _check(fmt, N, M, K, xdtype, seed, tiles=("auto", 32, 64)):
    blob, w, x = _data(fmt, N, M, K, xdtype, seed)
    qm = q.QMatrix(to_dev(blob), fmt, M, K)
    xd = to_dev(x)
    ys = {t: to_host(qm.gemm(xd, tile=t)) for t in tiles}
    y_ref = oracle.matmul_ref(x, w)
    S = oracle.tolerance_scale(x, w)
    w16 = oracle.staged_fp16(w).astype(np.float32)
    x16 = x.astype(np.float16).astype(np.float32)
    y16 = oracle.matmul_ref(x16, w16)
    S16 = oracle.tolerance_scale(x16, w16)
    for t, y in ys.items():
        label = f"gemm {fmt} N={N} M={M} K={K} tile={t} {np.dtype(xdtype).name}"
        assert_within(y, y_ref, S, TOL, label)
        assert_within(y, y16, S16, TOL16, label + " (vs fp16-staged product)")
        assert np.any(y != 0), label + ": all zero"
    return ys


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("shape", PAGE_SHAPES, ids=[f"{n}x{m}x{k}" for n, m, k in PAGE_SHAPES])
def test_tiles_bit_identical(fmt, shape):
    N, M, K = shape
    ys = _check(fmt, N, M, K, np.float16, [51, N, M, K])
    assert count_differences(ys[32], ys[64]) == 0, f"{fmt} {shape}: tiles differ"
    chosen = oracle.tile_for_tokens(N)
    assert count_differences(ys["auto"], ys[chosen]) == 0


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("N", [1, 31, 64, 65, 100, 257])
def test_gemm_ragged(fmt, N):
    bw = oracle.block_weights(fmt)
    K = 768 if 768 % bw == 0 else 3 * bw
    ys = _check(fmt, N, 131, K, np.float32, [52, N])
    assert count_differences(ys[32], ys[64]) == 0


@pytest.mark.parametrize("fmt", FORMATS)
def test_gemm_k_not_multiple_of_stage(fmt):
    """K = 3 blocks of 32 or 64 (not a multiple of the 128-deep LDS stage)."""
    if oracle.block_weights(fmt) > 64:
        pytest.skip("super-block formats have K % 256 == 0")
    K = 3 * oracle.block_weights(fmt)
    _check(fmt, 40, 70, K, np.float32, [53])


@pytest.mark.parametrize("fmt", FORMATS)
def test_gemm_one_hot_is_staged_weight(fmt):
    """x = e_k per token: y[t] must equal the fp16-staged weights w16[:, k] exactly."""
    bw = oracle.block_weights(fmt)
    K = 512 if 512 % bw == 0 else 2 * bw
    M = 80
    blob = make_matrix(fmt, M, K, [54])
    w16 = oracle.staged_fp16(oracle.dequantize(fmt, blob, M, K)).astype(np.float32)
    ks = list(range(0, K, 7))[:70]
    x = np.zeros((len(ks), K), np.float16)
    for t, k in enumerate(ks):
        x[t, k] = 1.0
    qm = q.QMatrix(to_dev(blob), fmt, M, K)
    for tile in (32, 64):
        y = to_host(qm.gemm(to_dev(x), tile=tile))
        for t, k in enumerate(ks):
            assert np.array_equal(y[t], w16[:, k]), f"{fmt} tile {tile}: token {t} (k={k})"


def test_gemm_deterministic_and_zero_tokens():
    fmt, M, K = "q4_k", 192, 512
    blob, w, x = _data(fmt, 77, M, K, np.float16, [55])
    qm = q.QMatrix(to_dev(blob), fmt, M, K)
    xd = to_dev(x)
    a, b = to_host(qm.gemm(xd, 64)), to_host(qm.gemm(xd, 64))
    assert count_differences(a, b) == 0
    y = torch.full((1, M), 3.0, device="cuda")
    # N = 0 through the C ABI itself (the binding wants x [0, K], which holds no pointer)
    assert L.lib.qmm_gemm(qm.handle, ctypes.c_void_p(xd.data_ptr()), 1, 0, ctypes.c_void_p(y.data_ptr()), 0, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
    assert np.all(to_host(y) == 3.0)


@pytest.mark.parametrize("fmt", FORMATS)
def test_gemm_split_and_unsplit(fmt):
    """qmm_gemm runs every K stage in one workgroup; qmm_gemm_ws (what QMatrix.gemm
    calls) divides K among the waves of a workgroup up to 16 tokens (no workspace) and
    among workgroups above, for few tokens, summing the partial slabs in split order.
    Both meet the bound, both are tile-identical, and the split call is deterministic."""
    bw = oracle.block_weights(fmt)
    K = 2560 if 2560 % bw == 0 else 2048
    M = 200
    for N in (7, 33, 130):
        blob, w, x = _data(fmt, N, M, K, np.float16, [56, N])
        qm = q.QMatrix(to_dev(blob), fmt, M, K)
        xd = to_dev(x)
        nb = q.qmm_gemm_workspace_bytes(qm.handle, N)
        assert (nb == 0) if N <= 16 else (nb > 0), (N, nb)
        y_ref, S = oracle.matmul_ref(x, w), oracle.tolerance_scale(x, w)
        outs = {}
        for t in (32, 64):
            y = torch.empty((N, M), device="cuda")
            q.qmm_gemm(qm.handle, xd, N, y, t)
            outs[("unsplit", t)] = to_host(y)
            outs[("split", t)] = to_host(qm.gemm(xd, tile=t))
        for (kind, t), y in outs.items():
            assert_within(y, y_ref, S, TOL, f"gemm {kind} {fmt} N={N} tile={t}")
        for kind in ("unsplit", "split"):
            assert count_differences(outs[(kind, 32)], outs[(kind, 64)]) == 0, (fmt, N, kind)
        assert count_differences(outs[("split", 64)], to_host(qm.gemm(xd, tile=64))) == 0


def test_gemm_workspace_is_zero_for_many_tokens():
    fmt, M, K = "q4_k", 4096, 2560
    qm = q.QMatrix(to_dev(make_matrix(fmt, M, K, [57])), fmt, M, K)
    assert q.qmm_gemm_workspace_bytes(qm.handle, 2048) == 0
    assert q.qmm_gemm_workspace_bytes(qm.handle, 7) == 0   # the waves of a workgroup split K
    assert q.qmm_gemm_workspace_bytes(qm.handle, 33) > 0  # workgroups split K
    assert q.qmm_gemm_workspace_bytes(qm.handle, 0) == 0


SK_SHAPES = [(1, 67, 768), (7, 300, 2560), (16, 33, 9728), (11, 130, 4096), (5, 20, 96)]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("xdtype", [np.float16, np.float32])
def test_gemm_few_tokens_workgroup_split(fmt, xdtype):
    """Up to 16 tokens the split entry points divide K among the waves of one workgroup:
    the oracle's bounds, both tiles and the rule's choice bit-identical; K of one to
    152 stages, an odd count of 32-weight units (a last
    stage half past K), rows that are not a multiple of 16."""
    bw = oracle.block_weights(fmt)
    for N, M, K in SK_SHAPES:
        if K % bw:
            K = (K + bw - 1) // bw * bw
        ys = _check(fmt, N, M, K, xdtype, [57, N, M, K])
        assert count_differences(ys[32], ys[64]) == 0, (fmt, N, K)
        assert count_differences(ys["auto"], ys[32]) == 0, (fmt, N, K)


@pytest.mark.parametrize("fmt", FORMATS)
def test_gemm_few_tokens_one_hot_is_staged_weight(fmt):
    """One-hot tokens through the workgroup split: y[t] equals the staged weights
    w16[:, k] exactly (one nonzero product, the other waves adding zeros)."""
    bw = oracle.block_weights(fmt)
    K = 2560 if 2560 % bw == 0 else 2048
    M = 70
    blob = make_matrix(fmt, M, K, [58])
    w16 = oracle.staged_fp16(oracle.dequantize(fmt, blob, M, K)).astype(np.float32)
    qm = q.QMatrix(to_dev(blob), fmt, M, K)
    ks = [0, 31, 32, 63, 64, 255, 256, 777, 1023, 1024, 1500, K - 33, K - 1]
    for xdt in (np.float16, np.float32):
        x = np.zeros((len(ks), K), xdt)
        for t, k in enumerate(ks):
            x[t, k] = 1.0
        y = to_host(qm.gemm(to_dev(x), tile=32))
        for t, k in enumerate(ks):
            assert np.array_equal(y[t], w16[:, k]), f"{fmt} {np.dtype(xdt).name}: token {t} (k={k})"
