"""Matrix-vector path (qmm_gemv) against the oracle.

Tolerance: |y - y_ref| <= 1e-5 * S with S = sum_k |x w| (fp32 accumulation of
exact fp32 weights; each lane sums 32 products in a fresh chain, partial sums
then add up over at most K/32 chunks and a log2(64)-step butterfly, so the
worst-case bound is (32 + K/32/lanes + 6) * 2^-24 * S, below 1e-5 * S for every
K here).  One-hot activations must reproduce the dequantized weights exactly."""

import ctypes
import numpy as np
import pytest
import torch

import block_quantized_weight_matmul_amd as q
from block_quantized_weight_matmul_amd import _lib as L
from tests.gpu_helpers import FORMATS, assert_within, make_matrix, oracle, to_dev, to_host

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _run(fmt, M, K, N, xdtype, seed):
    blob = make_matrix(fmt, M, K, seed)
    w = oracle.dequantize(fmt, blob, M, K)
    g = np.random.default_rng([seed, 1] if isinstance(seed, int) else list(seed) + [1])
    x = g.standard_normal((N, K)).astype(np.float32).astype(xdtype)
    qm = q.QMatrix(to_dev(blob), fmt, M, K)
    y = to_host(qm.gemv(to_dev(x)))
    return assert_within(y, oracle.matmul_ref(x, w), oracle.tolerance_scale(x, w), TOL,
                         f"gemv {fmt} M={M} K={K} N={N} {np.dtype(xdtype).name}")


# fp16 tokens take the matrix cores from a format's token count on (the library's dispatch)
MC_FORMATS = list(FORMATS)
MC_MIN_TOKENS = {f: 5 for f in FORMATS}


def _ks(fmt):
    bw = oracle.block_weights(fmt)
    return sorted({k for k in (bw, 256, 512, 768, 1024, 2560) if k % bw == 0})


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 8, 11, 16, 24, 32])
def test_gemv_tokens(fmt, N):
    for K in _ks(fmt):
        _run(fmt, 67, K, N, np.float32, [41, N, K])


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("M", [1, 5, 64, 257])
def test_gemv_rows_fp16(fmt, M):
    for K in _ks(fmt):
        _run(fmt, M, K, 3, np.float16, [42, M, K])


@pytest.mark.parametrize("fmt", FORMATS)
def test_gemv_narrow_k_rows(fmt):
    """The matrix-vector shapes of the llama.cpp review thread: m = 4096 at k = 512,
    768, 1024 (one token)."""
    for K in (512, 768, 1024):
        if K % oracle.block_weights(fmt) == 0:
            _run(fmt, 4096, K, 1, np.float32, [43, K])


@pytest.mark.parametrize("fmt", FORMATS)
def test_gemv_one_hot_is_exact(fmt):
    """x = e_k per token: each output must equal w[:, k] exactly, which also proves
    every (row, chunk) pair is computed once: a chunk done twice would give 2w,
    a skipped one 0."""
    bw = oracle.block_weights(fmt)
    K = 1024 if 1024 % bw == 0 else 4 * bw
    M = 133
    blob = make_matrix(fmt, M, K, [44])
    w = oracle.dequantize(fmt, blob, M, K)
    qm = q.QMatrix(to_dev(blob), fmt, M, K)
    ks = list(range(0, K, K // 32))[:32]
    ks[-1] = K - 1
    x = np.zeros((len(ks), K), np.float32)
    for t, k in enumerate(ks):
        x[t, k] = 1.0
    y = to_host(qm.gemv(to_dev(x)))
    for t, k in enumerate(ks):
        assert np.array_equal(y[t], w[:, k]), f"{fmt}: token {t} (k={k})"


def test_gemv_zero_tokens_is_noop():
    fmt, M, K = "q4_0", 32, 64
    qm = q.QMatrix(to_dev(make_matrix(fmt, M, K, [45])), fmt, M, K)
    x = torch.zeros((1, K), device="cuda")
    y = torch.full((1, M), 7.0, device="cuda")
    assert L.lib.qmm_gemv(qm.handle, ctypes.c_void_p(x.data_ptr()), 0, 0, ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
    assert np.all(to_host(y) == 7.0)


def test_gemv_deterministic():
    fmt, M, K = "q6_k", 300, 2560
    qm = q.QMatrix(to_dev(make_matrix(fmt, M, K, [46])), fmt, M, K)
    x = to_dev(np.random.default_rng(46).standard_normal((5, K)).astype(np.float32))
    a, b = to_host(qm.gemv(x)), to_host(qm.gemv(x))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("xdtype", [np.float32, np.float16])
def test_gemv_tokens_long_rows(fmt, xdtype):
    """Rows long enough that a call's activations are staged a few tokens at a
    time (several passes, the last one shorter)."""
    for K, N in ((8192, 3), (9728, 16)):
        if K % oracle.block_weights(fmt) == 0:
            _run(fmt, 300, K, N, xdtype, [47, K, N])


@pytest.mark.parametrize("fmt", FORMATS)
def test_gemv_tokens_match_single_token_calls(fmt):
    """Every vector path sums the same unit partials in the same order, so a call with N
    tokens returns, bit for bit, what N one-token calls return (fp16 tokens take the
    matrix cores from a few on, by format: up to there, here; from there, below)."""
    M, K = 300, 2560 if 2560 % oracle.block_weights(fmt) == 0 else 2048
    qm = q.QMatrix(to_dev(make_matrix(fmt, M, K, [48])), fmt, M, K)
    cases = [(np.float32, 11)]
    if MC_MIN_TOKENS[fmt] > 2:
        cases.append((np.float16, MC_MIN_TOKENS[fmt] - 1))
    for xdtype, N in cases:
        x = to_dev(np.random.default_rng(48).standard_normal((N, K)).astype(xdtype))
        full = to_host(qm.gemv(x))
        for t in range(N):
            one = to_host(qm.gemv(x[t:t + 1].contiguous()))
            assert np.array_equal(full[t:t + 1].view(np.uint32), one.view(np.uint32)), (fmt, xdtype, t)


# matrices of a grouped call: two (format, K) classes with several members (one of five:
# more than one launch holds), rows that are not a multiple of any workgroup's rows,
# and matrices that take a launch of their own
GROUP = [("q4_k", 300, 2560), ("q4_k", 1000, 2560), ("q6_k", 500, 2560), ("q4_k", 64, 512), ("q4_k", 7, 2560),
         ("q4_0", 200, 512), ("q4_k", 2049, 2560), ("q4_k", 33, 2560), ("q4_0", 96, 512)]


@pytest.mark.parametrize("xdt", [np.float32, np.float16])
@pytest.mark.parametrize("N", [1, 3, 16])
def test_gemv_group_matches_single_calls(N, xdt):
    """qmm_gemv_group gives every output the bits of its own qmm_gemv call (a grouped
    one-token or few-token launch runs each matrix's rows exactly as the single launch
    does), within the oracle's bound."""
    qms, xs, ws, xh = [], [], [], []
    for i, (fmt, M, K) in enumerate(GROUP):
        blob = make_matrix(fmt, M, K, [44, i])
        ws.append(oracle.dequantize(fmt, blob, M, K))
        qms.append(q.QMatrix(to_dev(blob), fmt, M, K))
        x = np.random.default_rng([45, i, N]).standard_normal((N, K)).astype(np.float32).astype(xdt)
        xh.append(x)
        xs.append(to_dev(x))
    ys = [torch.full((N, qm.M), float("nan"), device="cuda") for qm in qms]
    q.qmm_gemv_group([qm.handle for qm in qms], xs, N, ys)
    for i, (qm, x, y) in enumerate(zip(qms, xs, ys)):
        single = to_host(qm.gemv(x))
        got = to_host(y)
        assert np.array_equal(got.view(np.uint32), single.view(np.uint32)), (GROUP[i], N)
        assert_within(got, oracle.matmul_ref(xh[i], ws[i]), oracle.tolerance_scale(xh[i], ws[i]), TOL,
                      f"gemv_group {GROUP[i]} N={N}")


def test_gemv_group_edge_cases():
    blob = make_matrix("q4_k", 64, 256, [46])
    qm = q.QMatrix(to_dev(blob), "q4_k", 64, 256)
    x = to_dev(np.ones((1, 256), np.float32))
    q.qmm_gemv_group([], [], 1, [])                       # nothing to do
    # one matrix: the single call's bits
    y1 = torch.empty((1, 64), device="cuda")
    q.qmm_gemv_group([qm.handle], [x], 1, [y1])
    assert np.array_equal(to_host(y1), to_host(qm.gemv(x)))
    # argument errors come before any launch
    lib = L.lib
    ha = (ctypes.c_void_p * 1)(qm.handle.value)
    xa = (ctypes.c_void_p * 1)(x.data_ptr())
    ya = (ctypes.c_void_p * 1)(y1.data_ptr())
    y0 = torch.full((1, 64), 7.0, device="cuda")
    assert lib.qmm_gemv_group(ha, xa, L.DTYPES["f32"], 0, (ctypes.c_void_p * 1)(y0.data_ptr()), 1, None) == 0
    assert bool((y0 == 7.0).all())                             # zero tokens: nothing written
    assert lib.qmm_gemv_group(ha, xa, L.DTYPES["f32"], 33, ya, 1, None) == -3
    xa_bad = (ctypes.c_void_p * 1)(x.data_ptr() + 4)
    assert lib.qmm_gemv_group(ha, xa_bad, L.DTYPES["f32"], 1, ya, 1, None) == -4
    assert lib.qmm_gemv_group(ha, xa, L.DTYPES["f32"], 1, ya, 65, None) == -1


@pytest.mark.parametrize("scale_log2", [-96, -112])
@pytest.mark.parametrize("fmt", ["q4_0", "q8_0", "q4_k", "q6_k", "a4g64", "q5_k", "q3_k"])
def test_gemv_small_activations(fmt, scale_log2):
    """fp32 activations of magnitude 2^-96 and 2^-112 (normal, far below any real
    activation): the matrix-vector paths multiply codes as fp16 subnormals
    (code * 2^-24) with coefficients scaled by 2^24, so their products are
    2^-24-scaled copies of the plain chain's; they stay normal fp32 numbers down to
    |x| ~ 2^-100, and below that lose only absolute precision of order 2^-149 per
    product, far inside 1e-5 * S at these scales (one-token, few-token and general
    paths)."""
    bw = oracle.block_weights(fmt)
    K = 2560 if 2560 % bw == 0 else 2048
    M = 130
    blob = make_matrix(fmt, M, K, [47, -scale_log2])
    w = oracle.dequantize(fmt, blob, M, K)
    qm = q.QMatrix(to_dev(blob), fmt, M, K)
    for N in (1, 3, 32):
        g = np.random.default_rng([48, N, -scale_log2])
        z = g.standard_normal((N, K))
        x = (np.sign(z) * np.maximum(np.abs(z), 2.0 ** -10) * 2.0 ** scale_log2).astype(np.float32)
        assert np.all(np.abs(x[x != 0]) >= np.finfo(np.float32).tiny)  # normal fp32 inputs
        y = to_host(qm.gemv(to_dev(x)))
        assert_within(y, oracle.matmul_ref(x, w), oracle.tolerance_scale(x, w), TOL,
                      f"gemv {fmt} N={N} |x|~2^{scale_log2}")


@pytest.mark.parametrize("fmt,M,K", [("q4_k", 13000, 2560), ("q6_k", 4000, 9728)])
def test_gemv_eight_rows_per_thread(fmt, M, K):
    """Tall one-token calls, past four rows per thread at one workgroup per CU: the
    eight-row kernel, on every row (its results within the bound, sampled rows against
    the oracle), fp32 and fp16 activations, and a ragged last workgroup."""
    blob = make_matrix(fmt, M, K, [49, M])
    qm = q.QMatrix(to_dev(blob), fmt, M, K)
    rb = oracle.row_bytes(fmt, K)
    rows = np.unique(np.concatenate([np.arange(0, 40), np.random.default_rng([50, M]).integers(0, M, 200),
                                     np.arange(M - 40, M)]))
    w = oracle.dequantize(fmt, blob.reshape(M, rb)[rows].reshape(-1), len(rows), K)
    for xdt in (np.float32, np.float16):
        x = np.random.default_rng([51, M]).standard_normal((1, K)).astype(np.float32).astype(xdt)
        y = to_host(qm.gemv(to_dev(x)))
        assert np.all(np.isfinite(y))
        assert_within(y[:, rows], oracle.matmul_ref(x, w), oracle.tolerance_scale(x, w), TOL,
                      f"gemv {fmt} M={M} K={K} {np.dtype(xdt).name}")


# fp16 tokens from 5 to 32 take the matrix-core kernels (2 and 4: the vector path): rows of one
# block up to long K (one to several units or groups per wave, a last wave with fewer, one
# wave), for 4-bit groups a K past the kernel's range (the vector path), rows that are not
# a multiple of 16, and one or two 16-token blocks
@pytest.mark.parametrize("fmt", MC_FORMATS)
@pytest.mark.parametrize("N", [2, 4, 5, 16, 17, 32])
def test_gemv_matrix_cores_fp16(fmt, N):
    bw = oracle.block_weights(fmt)
    shapes = ((67, 64), (67, 320), (35, 1024), (16, 2048), (130, 3072), (33, 4096), (20, 4160), (1, 1088), (9, 9728))
    for M, K in shapes:
        K = (K + bw - 1) // bw * bw
        _run(fmt, M, K, N, np.float16, [52, M, K, N])


@pytest.mark.parametrize("fmt", MC_FORMATS)
def test_gemv_matrix_cores_one_hot_is_exact(fmt):
    """fp16 one-hot tokens through the matrix-core kernels: the code sum is q exactly and
    the activation sum 1, so each output is round(a * q + b), the fp32 weight."""
    M, K = 133, 1024
    blob = make_matrix(fmt, M, K, [53])
    w = oracle.dequantize(fmt, blob, M, K)
    qm = q.QMatrix(to_dev(blob), fmt, M, K)
    for ks in (list(range(0, K, 32)), list(range(31, K, 64))[:16] + [K - 1]):
        x = np.zeros((len(ks), K), np.float16)
        for t, k in enumerate(ks):
            x[t, k] = 1.0
        y = to_host(qm.gemv(to_dev(x)))
        for t, k in enumerate(ks):
            assert np.array_equal(y[t], w[:, k]), f"token {t} (k={k})"


@pytest.mark.parametrize("fmt", MC_FORMATS)
def test_gemv_matrix_cores_subnormal_tokens(fmt):
    """fp16 activations in the subnormal range (2^-24 .. 2^-15): exact inputs of the
    matrix cores, whose products (code * 2^-24 * x, down to 2^-48) stay normal fp32."""
    M, K = 96, 2048
    blob = make_matrix(fmt, M, K, [54])
    w = oracle.dequantize(fmt, blob, M, K)
    qm = q.QMatrix(to_dev(blob), fmt, M, K)
    g = np.random.default_rng(54)
    x = (g.integers(-1023, 1024, (32, K)) * 2.0 ** -24).astype(np.float16)
    assert np.all(np.abs(x.astype(np.float32)) < 2.0 ** -14)
    y = to_host(qm.gemv(to_dev(x)))
    assert_within(y, oracle.matmul_ref(x, w), oracle.tolerance_scale(x, w), TOL, "gemv a4g64 subnormal fp16 tokens")


@pytest.mark.parametrize("fmt", MC_FORMATS)
def test_gemv_matrix_cores_match_other_token_counts(fmt):
    """On the matrix cores a token's outputs depend on its own activations, K and the
    kernel's fixed order only: a 32-token call returns, bit for bit, what calls on
    windows of its tokens return, down to the fewest the matrix cores take (one and two
    16-token blocks)."""
    M, K, N = 300, 2048, 32
    w_ = MC_MIN_TOKENS[fmt]
    qm = q.QMatrix(to_dev(make_matrix(fmt, M, K, [55])), fmt, M, K)
    x = to_dev(np.random.default_rng([55, N]).standard_normal((N, K)).astype(np.float16))
    full = to_host(qm.gemv(x))
    for s0, n in {(0, w_), (N - w_, w_), (3, max(w_, 17)), (5, max(w_, 20))}:
        part = to_host(qm.gemv(x[s0:s0 + n].contiguous()))
        assert np.array_equal(full[s0:s0 + n].view(np.uint32), part.view(np.uint32)), (s0, n)


def test_gemv_matrix_cores_two_row_tiles():
    """Tall enough (more 16-row tiles than CUs) for two row tiles per wave: ragged last
    workgroup, one and two token blocks, and one-hot tokens exact."""
    fmt, M, K = "a4g64", 4100, 1024
    blob = make_matrix(fmt, M, K, [56])
    w = oracle.dequantize(fmt, blob, M, K)
    qm = q.QMatrix(to_dev(blob), fmt, M, K)
    for N in (5, 17):
        x = np.random.default_rng([56, N]).standard_normal((N, K)).astype(np.float16)
        y = to_host(qm.gemv(to_dev(x)))
        assert_within(y, oracle.matmul_ref(x, w), oracle.tolerance_scale(x, w), TOL, f"gemv a4g64 M={M} N={N}")
    ks = [0, 63, 64, 511, 777, 1023]
    x = np.zeros((len(ks), K), np.float16)
    for t, k in enumerate(ks):
        x[t, k] = 1.0
    y = to_host(qm.gemv(to_dev(x)))
    for t, k in enumerate(ks):
        assert np.array_equal(y[t], w[:, k]), f"token {t} (k={k})"


@pytest.mark.parametrize("N", [5, 16, 24])
def test_gemv_group_matrix_cores_match_single_calls(N):
    """fp16 tokens on the matrix cores in grouped calls: a launch of the group's total rows
    (5200 4-bit-group rows here, more 16-row tiles than CUs: two row tiles per wave; Q4_K
    and Q6_K rows together, Q3_K alone) gives every output the bits of its own single call,
    within the bound."""
    shapes = [("a4g64", 2048, 1024), ("a4g64", 1024, 1024), ("a4g64", 2128, 1024), ("a4g64", 37, 2048),
              ("q4_k", 300, 2560), ("q4_k", 77, 2560), ("q6_k", 100, 2560), ("q3_k", 50, 1024)]
    qms, xs, ws, xh = [], [], [], []
    for i, (fmt, M, K) in enumerate(shapes):
        blob = make_matrix(fmt, M, K, [59, i])
        ws.append(oracle.dequantize(fmt, blob, M, K))
        qms.append(q.QMatrix(to_dev(blob), fmt, M, K))
        x = np.random.default_rng([60, i, N]).standard_normal((N, K)).astype(np.float16)
        xh.append(x)
        xs.append(to_dev(x))
    ys = [torch.full((N, qm.M), float("nan"), device="cuda") for qm in qms]
    q.qmm_gemv_group([qm.handle for qm in qms], xs, N, ys)
    for i, (qm, x, y) in enumerate(zip(qms, xs, ys)):
        single = to_host(qm.gemv(x))
        got = to_host(y)
        assert np.array_equal(got.view(np.uint32), single.view(np.uint32)), (shapes[i], N)
        assert_within(got, oracle.matmul_ref(xh[i], ws[i]), oracle.tolerance_scale(xh[i], ws[i]), TOL,
                      f"gemv_group {shapes[i]} N={N}")
