"""Expert-indexed matrix-matrix path (qmm_gemm_id_tiled: MUL_MAT_ID of the llama.cpp
pull request "metal : fix idle threads in mul_mv_iq3_xxs for ne00 < 1024", on the
token-tiled matrix cores of the candle pull request "Metal: 64-token tile for the
quantized matrix-matrix kernel") against the oracle.

Tolerance as for qmm_gemm: 2e-3 * S against the exact product, 1e-5 * S16 against
the product of the fp16-staged operands.  Every output row must equal, bit for
bit, qmm_gemm of its expert on its activation row, for either tile."""

import numpy as np
import pytest
import torch

import block_quantized_weight_matmul_amd as q
from tests.gpu_helpers import FORMATS, assert_within, count_differences, make_matrix, oracle, to_dev, to_host

pytestmark = pytest.mark.gpu

TOL = 2e-3
TOL16 = 1e-5


def _stack(fmt, E, M, K, seed):
    blob = np.concatenate([make_matrix(fmt, M, K, [seed, e]) for e in range(E)])
    rb = oracle.row_bytes(fmt, K)
    ws = [oracle.dequantize(fmt, blob[e * M * rb:(e + 1) * M * rb], M, K) for e in range(E)]
    return blob, ws


def _ids(g, N, S, E):
    return np.stack([g.choice(E, S, replace=False) for _ in range(N)]).astype(np.int32)


def _check(fmt, y, x, ids, ws, label):
    assert_within(y, oracle.matmul_id_ref(x, ids, ws), oracle.tolerance_scale_id(x, ids, ws), TOL, label)
    w16 = [oracle.staged_fp16(w).astype(np.float32) for w in ws]
    x16 = x.astype(np.float16).astype(np.float32)
    assert_within(y, oracle.matmul_id_ref(x16, ids, w16), oracle.tolerance_scale_id(x16, ids, w16), TOL16,
                  label + " (vs fp16-staged product)")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("N,S", [(33, 8), (100, 4), (64, 8)])
def test_gemm_id_tiled_parity_and_tiles(fmt, N, S):
    """(64, 8): 51 pairs per expert on average, past the 48 that selects the
    128-token super-tile, and each expert's pairs within one super-tile."""
    E, M = 10, 96
    K = 512 if 512 % oracle.block_weights(fmt) == 0 else 2 * oracle.block_weights(fmt)
    blob, ws = _stack(fmt, E, M, K, 81)
    g = np.random.default_rng([82, N, S])
    ids = _ids(g, N, S, E)
    x = g.standard_normal((N, S, K)).astype(np.float32)
    qm = q.QMatrix(to_dev(blob), fmt, M, K, E)
    xd, idd = to_dev(x), to_dev(ids)
    ys = {t: to_host(qm.gemm_id_tiled(xd, idd, tile=t)) for t in ("auto", 32, 64)}
    _check(fmt, ys[64], x, ids, ws, f"gemm_id_tiled {fmt} N={N} S={S}")
    assert count_differences(ys[32], ys[64]) == 0, f"{fmt}: tiles differ"
    assert count_differences(ys["auto"], ys[64]) == 0


@pytest.mark.parametrize("fmt", FORMATS)
def test_gemm_id_tiled_rows_equal_dense_gemm(fmt):
    """Output row (t, s) = qmm_gemm (unsplit) of expert ids[t, s] on x[t, s], bit for
    bit; many pairs per expert (several super-tiles, the last one partial)."""
    E, M, N, S = 3, 80, 150, 4
    K = 1024 if 1024 % oracle.block_weights(fmt) == 0 else 4 * oracle.block_weights(fmt)
    blob, ws = _stack(fmt, E, M, K, 83)
    rb = oracle.row_bytes(fmt, K)
    g = np.random.default_rng(83)
    ids = g.integers(0, E, size=(N, S)).astype(np.int32)
    x = g.standard_normal((N, S, K)).astype(np.float16)
    qs = q.QMatrix(to_dev(blob), fmt, M, K, E)
    y = to_host(qs.gemm_id_tiled(to_dev(x), to_dev(ids)))
    flat_x, flat_ids, flat_y = x.reshape(N * S, K), ids.reshape(-1), y.reshape(N * S, M)
    for e in range(E):
        sel = np.nonzero(flat_ids == e)[0]
        dense = q.QMatrix(to_dev(blob[e * M * rb:(e + 1) * M * rb]), fmt, M, K)
        xe = to_dev(np.ascontiguousarray(flat_x[sel]))
        ye = torch.empty((len(sel), M), device="cuda")
        q.qmm_gemm(dense.handle, xe, len(sel), ye, 64)
        assert count_differences(flat_y[sel], to_host(ye)) == 0, f"{fmt} expert {e}"


@pytest.mark.parametrize("xdtype", [np.float32, np.float16])
def test_gemm_id_tiled_shared_x(xdtype):
    fmt, E, M, K, N, S = "q4_k", 8, 130, 512, 70, 4
    blob, ws = _stack(fmt, E, M, K, 84)
    g = np.random.default_rng(84)
    ids = _ids(g, N, S, E)
    x = g.standard_normal((N, K)).astype(np.float32).astype(xdtype)
    qm = q.QMatrix(to_dev(blob), fmt, M, K, E)
    y = to_host(qm.gemm_id_tiled(to_dev(x), to_dev(ids)))
    assert_within(y, oracle.matmul_id_ref(x, ids, ws), oracle.tolerance_scale_id(x, ids, ws), TOL,
                  "gemm_id_tiled shared x")


def test_gemm_id_tiled_invalid_ids_give_nan_rows():
    fmt, E, M, K, N, S = "q8_0", 6, 100, 256, 40, 3
    blob, ws = _stack(fmt, E, M, K, 85)
    g = np.random.default_rng(85)
    ids = _ids(g, N, S, E)
    ids[0, 1] = -1
    ids[20, 0] = E
    ids[39, 2] = 1 << 30
    x = g.standard_normal((N, S, K)).astype(np.float32)
    qm = q.QMatrix(to_dev(blob), fmt, M, K, E)
    y = to_host(qm.gemm_id_tiled(to_dev(x), to_dev(ids)))
    ref = oracle.matmul_id_ref(x, ids, ws)
    bad = (ids < 0) | (ids >= E)
    assert np.all(np.isnan(y[bad]))
    assert_within(y[~bad], ref[~bad], oracle.tolerance_scale_id(x, ids, ws)[~bad], TOL, "valid rows")


def test_gemm_id_tiled_zero_tokens_and_errors():
    import ctypes
    from block_quantized_weight_matmul_amd import _lib as L
    fmt, E, M, K = "q4_0", 2, 32, 64
    blob, _ = _stack(fmt, E, M, K, 86)
    qm = q.QMatrix(to_dev(blob), fmt, M, K, E)
    ids = torch.zeros((1, 1), dtype=torch.int32, device="cuda")
    x = torch.zeros((1, 1, K), device="cuda")
    y = torch.full((1, 1, M), 5.0, device="cuda")
    assert L.lib.qmm_gemm_id_tiled(qm.handle, ctypes.c_void_p(x.data_ptr()), 0, 0, 1, 1, ctypes.c_void_p(ids.data_ptr()), ctypes.c_void_p(y.data_ptr()), 0, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
    assert np.all(to_host(y) == 5.0)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    xp, yp, ip = (ctypes.c_void_p(t.data_ptr()) for t in (x, y, ids))
    assert L.lib.qmm_gemm_id_tiled(qm.handle, xp, 0, 1, 0, 1, ip, yp, 0, s) == -3       # S = 0
    assert L.lib.qmm_gemm_id_tiled(qm.handle, xp, 0, 1 << 17, 4, 1, ip, yp, 0, s) == -3  # too many pairs
    assert L.lib.qmm_gemm_id_tiled(qm.handle, xp, 0, 1, 1, 1, ip, yp, 48, s) == -1      # bad tile
