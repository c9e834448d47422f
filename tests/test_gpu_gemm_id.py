"""Expert-indexed matrix-vector path (qmm_gemm_id, MUL_MAT_ID in the llama.cpp pull
request "metal : fix idle threads in mul_mv_iq3_xxs for ne00 < 1024") against
the oracle: tolerance 1e-5 * S, exact equality with the dense path when every
slot picks one expert, NaN rows for ids outside [0, E)."""

import ctypes
import numpy as np
import pytest
import torch

import block_quantized_weight_matmul_amd as q
from block_quantized_weight_matmul_amd import _lib as L
from tests.gpu_helpers import FORMATS, assert_within, count_differences, make_matrix, oracle, to_dev, to_host

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _stack(fmt, E, M, K, seed):
    blob = np.concatenate([make_matrix(fmt, M, K, [seed, e]) for e in range(E)])
    rb = oracle.row_bytes(fmt, K)
    ws = [oracle.dequantize(fmt, blob[e * M * rb:(e + 1) * M * rb], M, K) for e in range(E)]
    return blob, ws


def _ids(g, N, S, E):
    return np.stack([g.choice(E, S, replace=False) for _ in range(N)]).astype(np.int32)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("N,S", [(1, 1), (2, 4), (5, 8), (12, 8), (24, 8), (32, 2)])
def test_gemm_id_per_slot(fmt, N, S):
    E, M = 10, 96
    K = 512 if 512 % oracle.block_weights(fmt) == 0 else 2 * oracle.block_weights(fmt)
    blob, ws = _stack(fmt, E, M, K, 61)
    g = np.random.default_rng([62, N, S])
    ids = _ids(g, N, S, E)
    x = g.standard_normal((N, S, K)).astype(np.float32)
    qm = q.QMatrix(to_dev(blob), fmt, M, K, E)
    y = to_host(qm.gemm_id(to_dev(x), to_dev(ids)))
    assert_within(y, oracle.matmul_id_ref(x, ids, ws), oracle.tolerance_scale_id(x, ids, ws), TOL,
                  f"gemm_id {fmt} N={N} S={S}")


@pytest.mark.parametrize("xdtype", [np.float32, np.float16])
def test_gemm_id_shared_x(xdtype):
    fmt, E, M, K, N, S = "q4_0", 16, 130, 512, 7, 4
    blob, ws = _stack(fmt, E, M, K, 63)
    g = np.random.default_rng(63)
    ids = _ids(g, N, S, E)
    x = g.standard_normal((N, K)).astype(np.float32).astype(xdtype)
    qm = q.QMatrix(to_dev(blob), fmt, M, K, E)
    y = to_host(qm.gemm_id(to_dev(x), to_dev(ids)))
    assert_within(y, oracle.matmul_id_ref(x, ids, ws), oracle.tolerance_scale_id(x, ids, ws), TOL,
                  "gemm_id shared x")


@pytest.mark.parametrize("fmt,K", [(f, 1024 if 1024 % oracle.block_weights(f) == 0 else 4 * oracle.block_weights(f))
                                   for f in FORMATS] + [("q4_0", 512)])
def test_gemm_id_equals_dense_for_one_expert(fmt, K):
    """Every slot routed to expert e: identical bits to the dense path on expert e
    (Q4_0 at K = 512 takes the narrow-row kernel)."""
    E, M, N, S = 4, 70, 3, 2
    blob, ws = _stack(fmt, E, M, K, 64)
    rb = oracle.row_bytes(fmt, K)
    g = np.random.default_rng(64)
    x = g.standard_normal((N, S, K)).astype(np.float32)
    qs = q.QMatrix(to_dev(blob), fmt, M, K, E)
    for e in range(E):
        ids = np.full((N, S), e, np.int32)
        y = to_host(qs.gemm_id(to_dev(x), to_dev(ids)))
        dense = q.QMatrix(to_dev(blob[e * M * rb:(e + 1) * M * rb]), fmt, M, K)
        yd = to_host(dense.gemv(to_dev(x.reshape(N * S, K)))).reshape(N, S, M)
        assert count_differences(y, yd) == 0, f"{fmt} expert {e}"


def test_gemm_id_invalid_ids_give_nan_rows():
    fmt, E, M, K, N, S = "q8_0", 6, 100, 256, 4, 3
    blob, ws = _stack(fmt, E, M, K, 65)
    g = np.random.default_rng(65)
    ids = _ids(g, N, S, E)
    ids[0, 1] = -1
    ids[2, 0] = E
    ids[3, 2] = 1 << 30
    x = g.standard_normal((N, S, K)).astype(np.float32)
    qm = q.QMatrix(to_dev(blob), fmt, M, K, E)
    y = to_host(qm.gemm_id(to_dev(x), to_dev(ids)))
    ref = oracle.matmul_id_ref(x, ids, ws)
    bad = (ids < 0) | (ids >= E)
    assert np.all(np.isnan(y[bad]))
    assert_within(y[~bad], ref[~bad], oracle.tolerance_scale_id(x, ids, ws)[~bad], TOL, "valid rows")


def test_gemm_id_duplicate_ids_many_pairs():
    """Duplicate ids within tokens: 32 tokens x 8 slots all on 2 experts (128 pairs
    per expert, several passes of the token bucket)."""
    fmt, E, M, K, N, S = "a4g64", 3, 64, 512, 32, 8
    blob, ws = _stack(fmt, E, M, K, 66)
    g = np.random.default_rng(66)
    ids = g.integers(1, 3, size=(N, S)).astype(np.int32)
    x = g.standard_normal((N, S, K)).astype(np.float16)
    qm = q.QMatrix(to_dev(blob), fmt, M, K, E)
    y = to_host(qm.gemm_id(to_dev(x), to_dev(ids)))
    assert_within(y, oracle.matmul_id_ref(x, ids, ws), oracle.tolerance_scale_id(x, ids, ws), TOL, "dups")


def test_gemm_id_zero_tokens_is_noop():
    fmt, E, M, K = "q4_0", 2, 32, 64
    blob, _ = _stack(fmt, E, M, K, 67)
    qm = q.QMatrix(to_dev(blob), fmt, M, K, E)
    ids = torch.zeros((1, 1), dtype=torch.int32, device="cuda")
    x = torch.zeros((1, 1, K), device="cuda")
    y = torch.full((1, 1, M), 5.0, device="cuda")
    assert L.lib.qmm_gemm_id(qm.handle, ctypes.c_void_p(x.data_ptr()), 0, 0, 1, 1, ctypes.c_void_p(ids.data_ptr()), ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
    assert np.all(to_host(y) == 5.0)


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0", "q6_k"])
def test_gemm_id_experts_not_dword_aligned(fmt):
    """Experts of an odd number of blocks of 18, 34 or 210 bytes: expert e > 0
    starts 2 bytes off a dword boundary."""
    E, M, N, S = 5, 3, 4, 3
    K = oracle.block_weights(fmt)
    assert (M * oracle.row_bytes(fmt, K)) % 4 == 2
    blob, ws = _stack(fmt, E, M, K, 68)
    g = np.random.default_rng(68)
    ids = _ids(g, N, S, E)
    x = g.standard_normal((N, S, K)).astype(np.float32)
    qm = q.QMatrix(to_dev(blob), fmt, M, K, E)
    y = to_host(qm.gemm_id(to_dev(x), to_dev(ids)))
    assert_within(y, oracle.matmul_id_ref(x, ids, ws), oracle.tolerance_scale_id(x, ids, ws), TOL, "odd experts")
    for e in range(E):
        got = to_host(qm.dequantize(e))
        assert np.array_equal(got, ws[e]), f"expert {e}"


@pytest.mark.parametrize("fmt", ["q4_0", "q4_k", "q6_k", "a4g64"])
def test_gemm_id_tall_experts(fmt):
    """Tall experts and many distinct ones: every expert's rows span many row
    slices of the launch."""
    E, M, K, N, S = 32, 2048, 512, 8, 8
    blob, ws = _stack(fmt, E, M, K, 69)
    g = np.random.default_rng(69)
    ids = _ids(g, N, S, E)
    x = g.standard_normal((N, S, K)).astype(np.float32)
    qm = q.QMatrix(to_dev(blob), fmt, M, K, E)
    y = to_host(qm.gemm_id(to_dev(x), to_dev(ids)))
    assert_within(y, oracle.matmul_id_ref(x, ids, ws), oracle.tolerance_scale_id(x, ids, ws), TOL,
                  f"slices {fmt}")


def test_gemm_id_tall_experts_many_pairs_and_bad_ids():
    """All pairs on two tall experts: several passes of pairs per row slice, many
    row slices, with ids outside [0, E) among them (NaN rows)."""
    fmt, E, M, K, N, S = "q4_0", 32, 2048, 512, 8, 8
    blob, ws = _stack(fmt, E, M, K, 70)
    g = np.random.default_rng(70)
    ids = g.integers(3, 5, size=(N, S)).astype(np.int32)
    ids[1, 2] = -3
    ids[5, 7] = E
    x = g.standard_normal((N, S, K)).astype(np.float32)
    qm = q.QMatrix(to_dev(blob), fmt, M, K, E)
    y = to_host(qm.gemm_id(to_dev(x), to_dev(ids)))
    bad = (ids < 0) | (ids >= E)
    assert np.all(np.isnan(y[bad]))
    ids_ok = np.where(bad, 3, ids)
    ref = oracle.matmul_id_ref(x, ids_ok, ws)
    sc = oracle.tolerance_scale_id(x, ids_ok, ws)
    assert_within(y[~bad], ref[~bad], sc[~bad], TOL, "slices and passes")


@pytest.mark.parametrize("N,S,xdtype", [(1, 1, np.float32), (24, 8, np.float32), (9, 8, np.float16), (32, 24, np.float32)])
def test_gemm_id_narrow_rows_many_chunks(N, S, xdtype):
    """Q4_0 at K = 512 (the route-once kernel from 65 to 512 pairs, the row-slice
    kernel at fewer or more): a row count that is no multiple of a step, experts with many pairs (several
    chunks of two), an expert's chunks split among waves; within the bound, and some
    outputs bit for bit the one-token dense call on their expert."""
    fmt, E, M, K = "q4_0", 16, 4100, 512
    blob, ws = _stack(fmt, E, M, K, 71)
    g = np.random.default_rng([71, N, S])
    ids = g.integers(0, E, size=(N, S)).astype(np.int32)
    x = g.standard_normal((N, S, K)).astype(xdtype)
    qm = q.QMatrix(to_dev(blob), fmt, M, K, E)
    y = to_host(qm.gemm_id(to_dev(x), to_dev(ids)))
    assert_within(y, oracle.matmul_id_ref(x, ids, ws), oracle.tolerance_scale_id(x, ids, ws), TOL, "narrow rows")
    rb = oracle.row_bytes(fmt, K)
    for t, s in {(0, 0), (N - 1, S - 1), (N // 2, S // 2)}:
        e = int(ids[t, s])
        dense = q.QMatrix(to_dev(blob[e * M * rb:(e + 1) * M * rb]), fmt, M, K)
        yd = to_host(dense.gemv(to_dev(x[t, s][None, :].copy())))
        assert count_differences(y[t, s][None, :], yd) == 0, (t, s, e)


def test_gemm_id_narrow_rows_all_ids_invalid():
    """Every id outside [0, E): every output row NaN, no expert streamed."""
    fmt, E, M, K, N, S = "q4_0", 4, 70, 512, 3, 2
    blob, _ = _stack(fmt, E, M, K, 72)
    qm = q.QMatrix(to_dev(blob), fmt, M, K, E)
    ids = np.array([[4, -1], [7, 4], [-5, 100]], np.int32)
    x = np.random.default_rng(72).standard_normal((N, S, K)).astype(np.float32)
    y = to_host(qm.gemm_id(to_dev(x), to_dev(ids)))
    assert np.all(np.isnan(y))


def test_gemm_id_narrow_rows_bad_ids_many_pairs():
    """Q4_0 at K = 512 past 64 pairs (the route-once kernel) with ids outside [0, E)
    among them: NaN rows for those, the others within the bound."""
    fmt, E, M, K, N, S = "q4_0", 12, 1000, 512, 16, 8
    blob, ws = _stack(fmt, E, M, K, 73)
    g = np.random.default_rng(73)
    ids = g.integers(0, E, size=(N, S)).astype(np.int32)
    ids[0, 0], ids[7, 3], ids[15, 7] = -1, E, 1 << 20
    x = g.standard_normal((N, S, K)).astype(np.float32)
    qm = q.QMatrix(to_dev(blob), fmt, M, K, E)
    y = to_host(qm.gemm_id(to_dev(x), to_dev(ids)))
    bad = (ids < 0) | (ids >= E)
    assert np.all(np.isnan(y[bad]))
    ids_ok = np.where(bad, 0, ids)
    ref = oracle.matmul_id_ref(x, ids_ok, ws)
    sc = oracle.tolerance_scale_id(x, ids_ok, ws)
    assert_within(y[~bad], ref[~bad], sc[~bad], TOL, "bad ids, many pairs")


def test_gemm_id_narrow_rows_many_experts():
    """Q4_0 at K = 512 on 8192 experts of 5 rows with 512 pairs, the route-once kernel's
    largest call: a presence bitmap of 256 words (several per scanning lane), several
    ranks per lane in the offset scan, and one expert with several pairs."""
    fmt, E, M, K, N, S = "q4_0", 8192, 5, 512, 32, 16
    blob = make_matrix(fmt, E * M, K, [74])
    w_all = oracle.dequantize(fmt, blob, E * M, K)
    ws = [w_all[e * M:(e + 1) * M] for e in range(E)]
    g = np.random.default_rng(74)
    ids = g.integers(0, E, size=(N, S)).astype(np.int32)
    ids[3, :4] = 17
    x = g.standard_normal((N, S, K)).astype(np.float32)
    qm = q.QMatrix(to_dev(blob), fmt, M, K, E)
    y = to_host(qm.gemm_id(to_dev(x), to_dev(ids)))
    assert_within(y, oracle.matmul_id_ref(x, ids, ws), oracle.tolerance_scale_id(x, ids, ws), TOL, "8192 experts")
