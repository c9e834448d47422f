"""Fused dequantize-and-multiply of block-quantized weights on MI355X (gfx950).

Thin Python binding over the C ABI in include/qmm.h (libqmm.so, built in-tree).
PyTorch supplies device memory and the current stream; every step of the
computation runs in the library's HIP kernels.  The functions below only
check tensor metadata, allocate outputs with torch and marshal pointers.

    qm = QMatrix(blocks_u8_cuda, "q4_k", M, K)
    y = qm.gemv(x)               # 1..32 tokens, fp32 accumulation
    y = qm.gemm(x, tile="auto")  # any N, fp16 matrix cores, 32/64-token tile
                                 # (K split over a torch-allocated workspace for few tokens)
    y = qm_stack.gemm_id(x, ids) # expert-indexed matrix-vector
    y = qm_stack.gemm_id_tiled(x, ids)  # expert-indexed, matrix cores, any N
    w = qm.dequantize()          # exact fp32 weights (or fp16 staging values)
"""

import ctypes

import torch

from ._lib import DTYPES, LIB_PATH, QMM_OK, STATUS, TILES, TYPES, QmmError, check, lib  # noqa: F401

__all__ = [
    "QMatrix", "QmmError", "LIB_PATH", "TYPES",
    "qmm_create", "qmm_destroy", "qmm_gemv", "qmm_gemm", "qmm_gemm_ws", "qmm_gemm_workspace_bytes",
    "qmm_gemm_id", "qmm_gemm_id_tiled", "qmm_dequantize", "qmm_quantize", "quantize",
    "qmm_tile_for_tokens", "qmm_row_bytes", "qmm_block_weights", "qmm_block_bytes",
]

_XT = {torch.float32: DTYPES["f32"], torch.float16: DTYPES["f16"]}


def _type_id(qtype):
    if isinstance(qtype, str):
        if qtype not in TYPES:
            raise ValueError(f"unknown block type {qtype!r}; one of {sorted(TYPES)}")
        return TYPES[qtype]
    return int(qtype)


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev_ptr(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _xt(x):
    if x.dtype not in _XT:
        raise ValueError("activations must be float32 or float16")
    return _XT[x.dtype]


# --- functions with the C names --------------------------------------------------------------

def qmm_tile_for_tokens(n: int) -> int:
    return lib.qmm_tile_for_tokens(int(n))


def qmm_row_bytes(qtype, K: int) -> int:
    return lib.qmm_row_bytes(_type_id(qtype), int(K))


def qmm_block_weights(qtype) -> int:
    return lib.qmm_block_weights(_type_id(qtype))


def qmm_block_bytes(qtype) -> int:
    return lib.qmm_block_bytes(_type_id(qtype))


def qmm_quantize(qtype, w: torch.Tensor, M: int, K: int, blocks: torch.Tensor, stream=None) -> None:
    check(lib.qmm_quantize(_type_id(qtype), _dev_ptr(w, "w"), int(M), int(K), _dev_ptr(blocks, "blocks"),
                           _stream(stream)))


def quantize(w: torch.Tensor, qtype) -> torch.Tensor:
    """fp32 [M, K] device tensor -> uint8 device tensor of M rows of blocks."""
    if w.dtype != torch.float32 or w.dim() != 2:
        raise ValueError("w must be a float32 [M, K] tensor")
    M, K = w.shape
    nbytes = qmm_row_bytes(qtype, K) * M
    if nbytes == 0 and M:
        raise ValueError(f"K={K} is not a multiple of the block of {qtype!r}")
    blocks = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=w.device)[:nbytes]
    qmm_quantize(qtype, w, M, K, blocks)
    return blocks


def qmm_create(blocks: torch.Tensor, qtype, M: int, K: int, n_experts: int = 1) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    check(lib.qmm_create(ctypes.byref(h), _type_id(qtype), _dev_ptr(blocks, "blocks"),
                         int(n_experts), int(M), int(K)))
    return h


def qmm_destroy(h) -> None:
    check(lib.qmm_destroy(h))


def qmm_gemv(h, x: torch.Tensor, N: int, y: torch.Tensor, stream=None) -> None:
    check(lib.qmm_gemv(h, _dev_ptr(x, "x"), _xt(x), int(N), _dev_ptr(y, "y"), _stream(stream)))


def qmm_gemm(h, x: torch.Tensor, N: int, y: torch.Tensor, tile=0, stream=None) -> None:
    t = TILES[tile] if tile in TILES else int(tile)
    check(lib.qmm_gemm(h, _dev_ptr(x, "x"), _xt(x), int(N), _dev_ptr(y, "y"), t, _stream(stream)))


def qmm_gemm_workspace_bytes(h, N: int) -> int:
    return lib.qmm_gemm_workspace_bytes(h, int(N))


def qmm_gemm_ws(h, x: torch.Tensor, N: int, y: torch.Tensor, tile=0, ws: torch.Tensor = None, stream=None) -> None:
    t = TILES[tile] if tile in TILES else int(tile)
    if ws is None:
        wp, wb = ctypes.c_void_p(0), 0
    else:
        wp, wb = _dev_ptr(ws, "ws"), ws.numel() * ws.element_size()
    check(lib.qmm_gemm_ws(h, _dev_ptr(x, "x"), _xt(x), int(N), _dev_ptr(y, "y"), t, wp, wb, _stream(stream)))


def qmm_gemm_id_tiled(h, x: torch.Tensor, N: int, S: int, x_per_slot: int, ids: torch.Tensor, y: torch.Tensor,
                      tile=0, stream=None) -> None:
    t = TILES[tile] if tile in TILES else int(tile)
    check(lib.qmm_gemm_id_tiled(h, _dev_ptr(x, "x"), _xt(x), int(N), int(S), int(x_per_slot),
                                _dev_ptr(ids, "ids"), _dev_ptr(y, "y"), t, _stream(stream)))


def qmm_gemm_id(h, x: torch.Tensor, N: int, S: int, x_per_slot: int, ids: torch.Tensor, y: torch.Tensor,
                stream=None) -> None:
    check(lib.qmm_gemm_id(h, _dev_ptr(x, "x"), _xt(x), int(N), int(S), int(x_per_slot),
                          _dev_ptr(ids, "ids"), _dev_ptr(y, "y"), _stream(stream)))


def qmm_dequantize(h, expert: int, out: torch.Tensor, stream=None) -> None:
    ot = _XT.get(out.dtype)
    if ot is None:
        raise ValueError("out must be float32 or float16")
    check(lib.qmm_dequantize(h, int(expert), _dev_ptr(out, "out"), ot, _stream(stream)))


# --- convenience object -------------------------------------------------------------------------

class QMatrix:
    """A block-quantized weight tensor on the device (one matrix, or E stacked experts).

    ``blocks`` is a contiguous uint8 device tensor of n_experts * M * row_bytes(K)
    bytes; it is borrowed (kept referenced here) for the life of the object.
    """

    def __init__(self, blocks: torch.Tensor, qtype, M: int, K: int, n_experts: int = 1):
        if blocks.dtype != torch.uint8:
            raise ValueError("blocks must be a uint8 tensor")
        rb = qmm_row_bytes(qtype, K)
        if rb == 0:
            raise QmmError(-3, f"K={K} is not a positive multiple of the {qtype} block")
        if blocks.numel() != n_experts * M * rb:
            raise ValueError(f"blocks holds {blocks.numel()} bytes, expected {n_experts * M * rb}")
        self.qtype, self.M, self.K, self.n_experts, self.row_bytes = qtype, int(M), int(K), int(n_experts), rb
        self._blocks = blocks
        self._h = qmm_create(blocks, qtype, M, K, n_experts)

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value is not None:
            lib.qmm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self):
        return self._h

    def _check_x(self, x, rows_shape):
        if x.shape[-1] != self.K:
            raise ValueError(f"x has K={x.shape[-1]}, matrix has K={self.K}")
        if x.device.type != "cuda":
            raise ValueError("x must be a device tensor")

    def gemv(self, x: torch.Tensor, out: torch.Tensor = None) -> torch.Tensor:
        """x [N, K] (N <= 32) -> y [N, M] fp32."""
        self._check_x(x, 2)
        N = x.shape[0]
        y = out if out is not None else torch.empty((N, self.M), dtype=torch.float32, device=x.device)
        qmm_gemv(self._h, x, N, y)
        return y

    def gemm(self, x: torch.Tensor, tile="auto", out: torch.Tensor = None) -> torch.Tensor:
        """x [N, K] -> y [N, M] fp32 through the fp16 matrix-core path; tile "auto", 32 or 64."""
        self._check_x(x, 2)
        N = x.shape[0]
        y = out if out is not None else torch.empty((N, self.M), dtype=torch.float32, device=x.device)
        nb = qmm_gemm_workspace_bytes(self._h, N)
        ws = torch.empty((nb + 15) // 16 * 4, dtype=torch.float32, device=x.device) if nb else None
        qmm_gemm_ws(self._h, x, N, y, tile, ws)
        return y

    def gemm_id(self, x: torch.Tensor, ids: torch.Tensor, out: torch.Tensor = None) -> torch.Tensor:
        """ids [N, S] int32; x [N, S, K] (one row per slot) or [N, K] -> y [N, S, M] fp32."""
        if ids.dtype != torch.int32 or ids.dim() != 2:
            raise ValueError("ids must be an int32 [N, S] tensor")
        self._check_x(x, 3)
        N, S = ids.shape
        x_per_slot = 1 if x.dim() == 3 else 0
        y = out if out is not None else torch.empty((N, S, self.M), dtype=torch.float32, device=x.device)
        qmm_gemm_id(self._h, x, N, S, x_per_slot, ids, y)
        return y

    def gemm_id_tiled(self, x: torch.Tensor, ids: torch.Tensor, tile="auto", out: torch.Tensor = None) -> torch.Tensor:
        """Prefill-sized expert-indexed product on the matrix cores (any N): ids [N, S]
        int32; x [N, S, K] or [N, K] -> y [N, S, M] fp32; tile "auto", 32 or 64."""
        if ids.dtype != torch.int32 or ids.dim() != 2:
            raise ValueError("ids must be an int32 [N, S] tensor")
        self._check_x(x, 3)
        N, S = ids.shape
        x_per_slot = 1 if x.dim() == 3 else 0
        y = out if out is not None else torch.empty((N, S, self.M), dtype=torch.float32, device=x.device)
        qmm_gemm_id_tiled(self._h, x, N, S, x_per_slot, ids, y, tile)
        return y

    def dequantize(self, expert: int = 0, dtype=torch.float32) -> torch.Tensor:
        out = torch.empty((self.M, self.K), dtype=dtype, device=self._blocks.device)
        qmm_dequantize(self._h, expert, out)
        return out
