"""qmm_gemm_noalloc, the matrix-matrix entry point that allocates nothing, through the
C ABI: bit for bit the results of qmm_gemm_ws (the same kernels and K split, with the
split's partial products in the library's own device scratch instead of a caller's
workspace), on two calls in a row, the second with a smaller input, and within the
oracle's bound; calls whose split would need more than the scratch holds are refused
before any launch."""

import ctypes

import numpy as np
import pytest
import torch

import block_quantized_weight_matmul_amd as q
from block_quantized_weight_matmul_amd import _lib as L
from tests.gpu_helpers import FORMATS, assert_within, count_differences, make_matrix, oracle, to_dev, to_host

pytestmark = pytest.mark.gpu


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _noalloc(h, x, N, y, tile):
    xt = 1 if x.dtype == torch.float16 else 0
    return L.lib.qmm_gemm_noalloc(h, ctypes.c_void_p(x.data_ptr()), xt, N, ctypes.c_void_p(y.data_ptr()), tile,
                                  _stream())


def _with_workspace(qm, x, N, tile):
    y = torch.empty((N, qm.M), device="cuda")
    nb = q.qmm_gemm_workspace_bytes(qm.handle, N)
    ws = torch.empty((nb + 15) // 16 * 4, device="cuda") if nb else None
    q.qmm_gemm_ws(qm.handle, x, N, y, tile, ws)
    return y, nb


@pytest.mark.parametrize("fmt", FORMATS)
def test_noalloc_equals_workspace_entry(fmt):
    M, K = 1024, 2560
    blob = make_matrix(fmt, M, K, [91, FORMATS.index(fmt)])
    w = oracle.dequantize(fmt, blob, M, K)
    qm = q.QMatrix(to_dev(blob), fmt, M, K)
    g = np.random.default_rng([92, FORMATS.index(fmt)])
    # two calls in a row, the second smaller: 33 fp16 tokens (K split among workgroups), then
    # 7 fp32 tokens (among the waves of a workgroup), then 130 and 96 tokens (the plan of the
    # wide calls)
    for N, dt in ((33, np.float16), (7, np.float32), (130, np.float16), (96, np.float32)):
        x = g.standard_normal((N, K)).astype(dt)
        xd = to_dev(x)
        for tile in (0, 32, 64):
            ref, nb = _with_workspace(qm, xd, N, tile)
            if 16 < N <= 64:
                assert nb > 0, "the few-token call should split K among workgroups"
            if N <= 16:
                assert nb == 0, "up to 16 tokens the waves of a workgroup split K"
            y = torch.full((N, M), float("nan"), device="cuda")
            assert _noalloc(qm.handle, xd, N, y, tile) == 0, L.lib.qmm_last_error().decode()
            got = to_host(y)
            assert count_differences(got, to_host(ref)) == 0, (fmt, N, tile)
        assert_within(got, oracle.matmul_ref(x, w), oracle.tolerance_scale(x, w), 2e-3, f"{fmt} N={N}")


def test_noalloc_back_to_back_on_one_stream():
    # two calls queued without a synchronisation between them: the stream orders them,
    # and the second (smaller) one rewrites the scratch it reads
    fmt, M, K = "q4_k", 512, 4096
    blob = make_matrix(fmt, M, K, [93])
    qm = q.QMatrix(to_dev(blob), fmt, M, K)
    g = np.random.default_rng(94)
    xa = to_dev(g.standard_normal((40, K)).astype(np.float16))
    xb = to_dev(g.standard_normal((9, K)).astype(np.float16))
    ya = torch.empty((40, M), device="cuda")
    yb = torch.empty((9, M), device="cuda")
    assert _noalloc(qm.handle, xa, 40, ya, 0) == 0
    assert _noalloc(qm.handle, xb, 9, yb, 0) == 0
    ra, _ = _with_workspace(qm, xa, 40, 0)
    rb, _ = _with_workspace(qm, xb, 9, 0)
    assert count_differences(to_host(ya), to_host(ra)) == 0
    assert count_differences(to_host(yb), to_host(rb)) == 0


def test_noalloc_scratch_serves_the_prefill_workloads():
    """Every decode-layer projection at every prefill token count (and far beyond) fits the
    scratch, so the entry point serves the benchmark's matrix-matrix workloads; any call
    found above it is refused before a launch, with y untouched."""
    from qmm_synth import workloads as W
    assert L.NOALLOC_SCRATCH_BYTES == 64 << 20
    for name, M, K, fmt in W.DECODE_SHAPES:
        blocks = torch.zeros(M * oracle.row_bytes(fmt, K), dtype=torch.uint8, device="cuda")
        qm = q.QMatrix(blocks, fmt, M, K)
        for N in W.PREFILL_TOKENS + [130, 4096, 16384]:
            need = q.qmm_gemm_workspace_bytes(qm.handle, N)
            if need <= L.NOALLOC_SCRATCH_BYTES:
                continue
            x = torch.zeros((N, K), dtype=torch.float16, device="cuda")
            y = torch.full((N, M), 7.0, device="cuda")
            assert _noalloc(qm.handle, x, N, y, 0) == -3, (name, N)
            assert b"scratch" in L.lib.qmm_last_error()
            assert bool(torch.all(y == 7.0))
        # a few-token call of each shape through the entry point
        x = torch.zeros((7, K), dtype=torch.float16, device="cuda")
        y = torch.full((7, M), 7.0, device="cuda")
        assert _noalloc(qm.handle, x, 7, y, 0) == 0
        assert bool(torch.all(y == 0.0))
