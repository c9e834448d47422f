"""The Python binding's argument checks (CPU only, no device work).

The kernels trust the N, S, M and K they are given, so a tensor whose shape,
dtype or placement does not match the handle must be refused in the binding,
before any pointer reaches the library.  Every case here raises ValueError
before a C call is made (the tensors are host tensors: a call that got past the
checks would be refused for that instead, which the last cases pin)."""

import ctypes

import pytest
import torch

import block_quantized_weight_matmul_amd as q

M, K, E = 48, 256, 3


@pytest.fixture
def handle():
    """A handle known to the binding's registry (no library object behind it: every call
    below must fail before reaching the library)."""
    h = ctypes.c_void_p(0x5EED0)
    q._HANDLES[h.value] = q._Meta(q.TYPES["q4_k"], M, K, 1, 0)
    yield h
    q._HANDLES.pop(h.value, None)


@pytest.fixture
def stack_handle():
    h = ctypes.c_void_p(0x5EED8)
    q._HANDLES[h.value] = q._Meta(q.TYPES["q4_0"], M, K, E, 0)
    yield h
    q._HANDLES.pop(h.value, None)


def qmatrix_stub(n_experts=1):
    qm = object.__new__(q.QMatrix)
    qm.qtype, qm.M, qm.K, qm.n_experts, qm.row_bytes = "q4_k", M, K, n_experts, 144
    qm._h = None
    return qm


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def expect(fn, text):
    with pytest.raises(ValueError, match=text):
        fn()


def test_unknown_handle_is_refused():
    expect(lambda: q.qmm_gemv(ctypes.c_void_p(0x1234), f32(1, K), 1, f32(1, M)), "unknown handle")


def test_gemv_shapes(handle):
    expect(lambda: q.qmm_gemv(handle, f32(K), 1, f32(1, M)), "x has shape")          # 1-D x
    expect(lambda: q.qmm_gemv(handle, f32(2, K), 1, f32(1, M)), "x has shape")       # rows != N
    expect(lambda: q.qmm_gemv(handle, f32(1, K + 32), 1, f32(1, M)), "x has shape")  # wrong K
    expect(lambda: q.qmm_gemv(handle, f32(1, K), 1, f32(1, M + 1)), "y has shape")
    expect(lambda: q.qmm_gemv(handle, f32(1, K), 1, f32(M)), "y has shape")
    expect(lambda: q.qmm_gemv(handle, f32(1, K), 1, f32(1, M).half()), "y has dtype")
    expect(lambda: q.qmm_gemv(handle, f32(1, K).double(), 1, f32(1, M)), "x has dtype")
    expect(lambda: q.qmm_gemv(handle, f32(1, K), -1, f32(1, M)), "N=-1")


def test_gemm_shapes(handle):
    expect(lambda: q.qmm_gemm(handle, f32(7, K), 8, f32(8, M)), "x has shape")
    expect(lambda: q.qmm_gemm(handle, f32(8, K), 8, f32(8, M - 1)), "y has shape")
    expect(lambda: q.qmm_gemm_ws(handle, f32(8, K), 8, f32(7, M)), "y has shape")
    expect(lambda: q.qmm_gemm_ws(handle, f32(8, 2 * K), 8, f32(8, M)), "x has shape")


def test_id_shapes(stack_handle):
    h = stack_handle
    ids = torch.zeros((4, 2), dtype=torch.int32)
    expect(lambda: q.qmm_gemm_id(h, f32(4, 2, K), 4, 2, 1, ids.long(), f32(4, 2, M)), "ids has dtype")
    expect(lambda: q.qmm_gemm_id(h, f32(4, 2, K), 4, 3, 1, ids, f32(4, 3, M)), "x has shape")
    expect(lambda: q.qmm_gemm_id(h, f32(4, 2, K), 4, 2, 0, ids, f32(4, 2, M)), "x has shape")  # shared x is [N, K]
    expect(lambda: q.qmm_gemm_id(h, f32(4, K), 4, 2, 1, ids, f32(4, 2, M)), "x has shape")
    expect(lambda: q.qmm_gemm_id(h, f32(4, 2, K), 4, 2, 1, ids, f32(4, M)), "y has shape")
    expect(lambda: q.qmm_gemm_id(h, f32(4, 2, K), 4, 2, 2, ids, f32(4, 2, M)), "x_per_slot")
    expect(lambda: q.qmm_gemm_id_tiled(h, f32(5, 2, K), 4, 2, 1, ids, f32(4, 2, M)), "x has shape")
    expect(lambda: q.qmm_gemm_id_tiled(h, f32(4, 2, K), 4, 2, 1, ids[:3], f32(4, 2, M)), "ids has shape")


def test_dequantize_and_quantize_shapes(handle, stack_handle):
    expect(lambda: q.qmm_dequantize(handle, 0, f32(M, K + 1)), "out has shape")
    expect(lambda: q.qmm_dequantize(handle, 1, f32(M, K)), "expert=1")
    expect(lambda: q.qmm_dequantize(stack_handle, 3, f32(M, K)), "expert=3")
    expect(lambda: q.qmm_quantize("q4_k", f32(M, K), M, K, torch.zeros(M * 144 - 1, dtype=torch.uint8)),
           "blocks has shape")
    expect(lambda: q.qmm_quantize("q4_k", f32(M, K - 1), M, K, torch.zeros(M * 144, dtype=torch.uint8)),
           "w has shape")
    expect(lambda: q.qmm_quantize("q4_k", f32(M, 100), M, 100, torch.zeros(1, dtype=torch.uint8)), "not a positive")


def test_qmatrix_methods_check_ranks_and_ids():
    qm = qmatrix_stub()
    expect(lambda: qm.gemv(f32(K)), "dimensions")          # 1-D x would read K x K activations
    expect(lambda: qm.gemm(f32(2, 3, K)), "dimensions")
    expect(lambda: qm.gemm(f32(4, K + 1)), "matrix has K")
    st = qmatrix_stub(E)
    ids = torch.zeros((4, 2), dtype=torch.int32)
    expect(lambda: st.gemm_id(f32(4, 3, K), ids), "leading shape")
    expect(lambda: st.gemm_id(f32(5, K), ids), "leading shape")
    expect(lambda: st.gemm_id_tiled(f32(4, 2, K), ids.view(8)), "int32")
    expect(lambda: st.gemm_id_tiled(f32(4, 2, K), ids.float()), "int32")


def test_host_tensors_are_refused(handle, stack_handle):
    # right shapes, but host memory: refused by the binding, never passed on
    expect(lambda: q.qmm_gemv(handle, f32(2, K), 2, f32(2, M)), "device tensor")
    expect(lambda: q.qmm_gemm(handle, f32(9, K).half(), 9, f32(9, M)), "device tensor")
    ids = torch.zeros((2, 2), dtype=torch.int32)
    expect(lambda: q.qmm_gemm_id(stack_handle, f32(2, 2, K), 2, 2, 1, ids, f32(2, 2, M)), "device tensor")


def test_gemv_group_checks(handle, stack_handle):
    f16 = lambda *s: torch.zeros(s, dtype=torch.float16)
    q.qmm_gemv_group([], [], 1, [])  # nothing to do: no check can fail, nothing is called
    expect(lambda: q.qmm_gemv_group([handle], [f32(1, K)], 1, []), "same length")
    expect(lambda: q.qmm_gemv_group([handle, handle], [f32(1, K), f16(1, K)], 1, [f32(1, M), f32(1, M)]),
           "same dtype")
    expect(lambda: q.qmm_gemv_group([handle], [f32(2, K)], 1, [f32(1, M)]), r"xs\[0\] has shape")
    expect(lambda: q.qmm_gemv_group([handle, handle], [f32(1, K), f32(1, K)], 1, [f32(1, M), f32(1, M + 1)]),
           r"ys\[1\] has shape")
    expect(lambda: q.qmm_gemv_group([ctypes.c_void_p(0x1234)], [f32(1, K)], 1, [f32(1, M)]), "unknown handle")
    # a handle on another device
    other = ctypes.c_void_p(0x5EEE0)
    q._HANDLES[other.value] = q._Meta(q.TYPES["q4_k"], M, K, 1, 1)
    try:
        expect(lambda: q.qmm_gemv_group([handle, other], [f32(1, K)] * 2, 1, [f32(1, M)] * 2), "same device")
    finally:
        q._HANDLES.pop(other.value, None)
    # shapes right, host tensors: refused for placement, still before any C call
    expect(lambda: q.qmm_gemv_group([handle], [f32(1, K)], 1, [f32(1, M)]), "device tensor")
