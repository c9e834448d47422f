"""ctypes loader for libqmm.so (the C ABI of include/qmm.h).

The library is built in-tree by ``python block_quantized_weight_matmul_amd/build.py``.
There is no fallback: importing this module without the built library raises.
"""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqmm.so")

QMM_OK = 0
STATUS = {
    0: "QMM_OK", -1: "QMM_E_ARG", -2: "QMM_E_TYPE", -3: "QMM_E_SHAPE",
    -4: "QMM_E_ALIGN", -5: "QMM_E_DEVICE", -6: "QMM_E_HIP",
}
TYPES = {"q4_0": 0, "q8_0": 1, "q4_k": 2, "q6_k": 3, "a4g64": 4,
         "q4_1": 5, "q5_0": 6, "q5_1": 7, "q2_k": 8, "q3_k": 9, "q5_k": 10}
DTYPES = {"f32": 0, "f16": 1}
TILES = {"auto": 0, 32: 32, 64: 64}
NOALLOC_SCRATCH_BYTES = 64 << 20  # QMM_NOALLOC_SCRATCH_BYTES of include/qmm.h


class QmmError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python block_quantized_weight_matmul_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
    sigs = {
        "qmm_create": (c_int, [ctypes.POINTER(vp), c_int, vp, i64, i64, i64]),
        "qmm_destroy": (c_int, [vp]),
        "qmm_gemv": (c_int, [vp, vp, c_int, i64, vp, vp]),
        "qmm_gemv_group": (c_int, [ctypes.POINTER(vp), ctypes.POINTER(vp), c_int, i64, ctypes.POINTER(vp), c_int, vp]),
        "qmm_gemm": (c_int, [vp, vp, c_int, i64, vp, c_int, vp]),
        "qmm_gemm_ws": (c_int, [vp, vp, c_int, i64, vp, c_int, vp, ctypes.c_size_t, vp]),
        "qmm_gemm_workspace_bytes": (ctypes.c_size_t, [vp, i64]),
        "qmm_gemm_noalloc": (c_int, [vp, vp, c_int, i64, vp, c_int, vp]),
        "qmm_gemm_id": (c_int, [vp, vp, c_int, i64, i64, c_int, vp, vp, vp]),
        "qmm_gemm_id_tiled": (c_int, [vp, vp, c_int, i64, i64, c_int, vp, vp, c_int, vp]),
        "qmm_dequantize": (c_int, [vp, i64, vp, c_int, vp]),
        "qmm_quantize": (c_int, [c_int, vp, i64, i64, vp, vp]),
        "qmm_tile_for_tokens": (c_int, [i64]),
        "qmm_row_bytes": (ctypes.c_size_t, [c_int, i64]),
        "qmm_block_weights": (c_int, [c_int]),
        "qmm_block_bytes": (c_int, [c_int]),
        "qmm_status_string": (ctypes.c_char_p, [c_int]),
        "qmm_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    del i32
    return lib


lib = _load()


def check(status):
    if status != QMM_OK:
        raise QmmError(status, lib.qmm_last_error().decode())
    return status
