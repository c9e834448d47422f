"""C-ABI behaviour on the device: error codes, shape and alignment checks, stream
order, and that the HIP library (not a fallback) is what the process loaded."""

import ctypes

import numpy as np
import pytest
import torch

import block_quantized_weight_matmul_amd as q
from block_quantized_weight_matmul_amd import _lib as L
from tests.gpu_helpers import assert_within, make_matrix, oracle, to_dev, to_host

pytestmark = pytest.mark.gpu


def _status(fn, *args):
    return fn(*args)


def test_native_library_is_loaded():
    maps = open("/proc/self/maps").read()
    assert L.LIB_PATH in maps
    assert torch.cuda.get_device_properties(0).gcnArchName.startswith("gfx950")


def test_create_errors_on_device_pointers():
    fmt, M, K = "q4_0", 8, 64
    blob = to_dev(np.zeros(M * oracle.row_bytes(fmt, K) + 64, np.uint8))
    h = ctypes.c_void_p()
    p = blob.data_ptr()
    assert L.lib.qmm_create(ctypes.byref(h), 0, ctypes.c_void_p(p + 2), 1, M, K) == -4
    assert L.lib.qmm_create(ctypes.byref(h), 11, ctypes.c_void_p(p), 1, M, K) == -2
    assert L.lib.qmm_create(ctypes.byref(h), 0, ctypes.c_void_p(p), 1, M, 40) == -3
    assert L.lib.qmm_create(ctypes.byref(h), 0, ctypes.c_void_p(p), 1, M, K) == 0
    assert L.lib.qmm_destroy(h) == 0


def test_call_errors():
    fmt, M, K = "q4_0", 16, 64
    qm = q.QMatrix(to_dev(make_matrix(fmt, M, K, [71])), fmt, M, K)
    h = qm.handle
    x = torch.zeros((40, K), device="cuda")
    y = torch.zeros((40, M), device="cuda")
    xp, yp = ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr())
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.lib.qmm_gemv(h, xp, 0, 33, yp, s) == -3            # N > 32
    assert L.lib.qmm_gemv(h, xp, 0, -1, yp, s) == -3
    assert L.lib.qmm_gemv(h, xp, 7, 1, yp, s) == -2             # bad dtype
    assert L.lib.qmm_gemv(h, ctypes.c_void_p(x.data_ptr() + 4), 0, 1, yp, s) == -4
    assert L.lib.qmm_gemv(h, xp, 0, 1, ctypes.c_void_p(y.data_ptr() + 2), s) == -4
    assert L.lib.qmm_gemv(h, None, 0, 1, yp, s) == -1
    assert L.lib.qmm_gemm(h, xp, 0, 1, yp, 48, s) == -1         # bad tile
    assert L.lib.qmm_gemm(h, xp, 0, -5, yp, 0, s) == -3
    # a split call needs its workspace: missing, too small or misaligned is refused
    # (K = 2048 gives a 40-token call K stages to split among workgroups)
    long_rows = q.QMatrix(to_dev(make_matrix(fmt, M, 2048, [74])), fmt, M, 2048)
    h = long_rows.handle
    xl = torch.zeros((40, 2048), device="cuda")
    xp = ctypes.c_void_p(xl.data_ptr())
    need = L.lib.qmm_gemm_workspace_bytes(h, 40)
    assert need > 0
    assert L.lib.qmm_gemm_workspace_bytes(h, 7) == 0   # the waves of a workgroup split K
    ws = torch.zeros(need // 4 + 8, device="cuda")
    wp = ctypes.c_void_p(ws.data_ptr())
    assert L.lib.qmm_gemm_ws(h, xp, 0, 40, yp, 0, None, 0, s) == -1
    assert L.lib.qmm_gemm_ws(h, xp, 0, 40, yp, 0, wp, need - 4, s) == -1
    assert "needs" in L.lib.qmm_last_error().decode()
    assert L.lib.qmm_gemm_ws(h, xp, 0, 40, yp, 0, ctypes.c_void_p(ws.data_ptr() + 4), need, s) == -4
    assert L.lib.qmm_gemm_ws(h, xp, 0, 40, yp, 48, wp, need, s) == -1   # bad tile
    h, xp = qm.handle, ctypes.c_void_p(x.data_ptr())
    assert L.lib.qmm_dequantize(h, 1, yp, 0, s) == -3           # expert out of range
    ids = torch.zeros((2, 2), dtype=torch.int32, device="cuda")
    ip = ctypes.c_void_p(ids.data_ptr())
    assert L.lib.qmm_gemm_id(h, xp, 0, 2, 0, 1, ip, yp, s) == -3     # S = 0
    assert L.lib.qmm_gemm_id(h, xp, 0, 2, 65, 1, ip, yp, s) == -3    # S > 64
    assert L.lib.qmm_gemm_id(h, xp, 0, 2, 2, 2, ip, yp, s) == -1     # x_per_slot
    assert L.lib.qmm_gemm_id(h, xp, 0, 2, 2, 1, ctypes.c_void_p(ids.data_ptr() + 2), yp, s) == -4
    assert "ids" in L.lib.qmm_last_error().decode()
    stack = q.QMatrix(to_dev(np.concatenate([make_matrix(fmt, M, K, [72, e]) for e in range(2)])), fmt, M, K, 2)
    assert L.lib.qmm_gemv(stack.handle, xp, 0, 1, yp, s) == -1   # dense call on a stack
    with pytest.raises(q.QmmError):
        qm.gemv(torch.zeros((33, K), device="cuda"))
    # the matrix-matrix path takes K below 2^22; the check comes before any launch,
    # so the (too small) block buffer is never read
    wide = ctypes.c_void_p()
    blk = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    assert L.lib.qmm_create(ctypes.byref(wide), 0, ctypes.c_void_p(blk.data_ptr()), 1, 1, 1 << 22) == 0
    assert L.lib.qmm_gemm(wide, xp, 0, 1, yp, 0, s) == -3
    assert "K below" in L.lib.qmm_last_error().decode()
    assert L.lib.qmm_destroy(wide) == 0


def test_stream_order_on_side_stream():
    fmt, M, K, N = "q4_k", 512, 2560, 4
    blob = make_matrix(fmt, M, K, [73])
    w = oracle.dequantize(fmt, blob, M, K)
    x = np.random.default_rng(73).standard_normal((N, K)).astype(np.float32)
    qm = q.QMatrix(to_dev(blob), fmt, M, K)
    side = torch.cuda.Stream()
    xd = to_dev(x)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        y = torch.empty((N, M), device="cuda")
        xs = xd * 2.0                       # produced on the side stream
        q.qmm_gemv(qm.handle, xs, N, y)     # must see xs (same stream)
        y2 = y * 0.5                        # must see y
    side.synchronize()
    assert_within(to_host(y2), oracle.matmul_ref(x, w), oracle.tolerance_scale(x, w), 1e-5, "side stream")
