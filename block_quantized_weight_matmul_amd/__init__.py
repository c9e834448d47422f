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

from ._lib import DTYPES, LIB_PATH, NOALLOC_SCRATCH_BYTES, QMM_OK, STATUS, TILES, TYPES, QmmError, check, lib  # noqa: F401

__all__ = [
    "QMatrix", "QmmError", "LIB_PATH", "TYPES",
    "qmm_create", "qmm_destroy", "qmm_gemv", "qmm_gemv_group", "qmm_gemm", "qmm_gemm_ws", "qmm_gemm_workspace_bytes",
    "qmm_gemm_noalloc",
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


def _xt(x):
    if x.dtype not in _XT:
        raise ValueError("activations must be float32 or float16")
    return _XT[x.dtype]


# --- argument checks ---------------------------------------------------------------------------
# Every tensor is checked against the handle's shape before a pointer reaches the library: the
# kernels trust N, S, M and K, so a mis-shaped tensor would be read or written past its end on
# the device.  Shape and dtype are checked first, then device placement and layout.

class _Meta:
    __slots__ = ("qtype", "M", "K", "n_experts", "device")

    def __init__(self, qtype, M, K, n_experts, device):
        self.qtype, self.M, self.K, self.n_experts, self.device = qtype, M, K, n_experts, device


# handle value -> _Meta of the matrix it describes (filled by qmm_create)
_HANDLES = {}


def _meta(h):
    key = h.value if isinstance(h, ctypes.c_void_p) else int(h or 0)
    m = _HANDLES.get(key)
    if m is None:
        raise ValueError("unknown handle: create it with qmm_create (or QMatrix)")
    return m


def _need(device, *specs):
    """specs: (tensor, name, shape or None, dtypes or None).  All shapes and dtypes are
    checked before any placement, then each tensor must be a contiguous tensor on
    `device` (the matrix's device; None: any device).  Returns their pointers."""
    for t, name, shape, dtypes in specs:
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a torch tensor")
        if dtypes is not None and t.dtype not in dtypes:
            raise ValueError(f"{name} has dtype {t.dtype}; expected one of {[str(d) for d in dtypes]}")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}; expected {tuple(shape)}")
    ptrs = []
    for t, name, _, _ in specs:
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if device is not None and t.device.index != device:
            raise ValueError(f"{name} is on cuda:{t.device.index}; the matrix is on cuda:{device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        ptrs.append(ctypes.c_void_p(t.data_ptr()))
    return ptrs if len(ptrs) > 1 else ptrs[0]


_ACT = (torch.float32, torch.float16)
_F32 = (torch.float32,)


def _count(v, name, lo, hi=None):
    v = int(v)
    if v < lo or (hi is not None and v > hi):
        raise ValueError(f"{name}={v} outside [{lo}, {hi if hi is not None else 'inf'})")
    return v


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
    M, K = _count(M, "M", 0), _count(K, "K", 1)
    rb = qmm_row_bytes(qtype, K)
    if rb == 0:
        raise ValueError(f"K={K} is not a positive multiple of the {qtype!r} block")
    wp, bp = _need(None, (w, "w", (M, K), _F32), (blocks, "blocks", (M * rb,), (torch.uint8,)))
    if w.device != blocks.device:
        raise ValueError("w and blocks must be on the same device")
    check(lib.qmm_quantize(_type_id(qtype), wp, M, K, bp, _stream(stream)))


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
    t = _type_id(qtype)
    M, K, E = _count(M, "M", 1), _count(K, "K", 1), _count(n_experts, "n_experts", 1)
    rb = lib.qmm_row_bytes(t, K)
    if rb == 0:
        raise ValueError(f"K={K} is not a positive multiple of the {qtype!r} block")
    bp = _need(None, (blocks, "blocks", (E * M * rb,), (torch.uint8,)))
    h = ctypes.c_void_p()
    check(lib.qmm_create(ctypes.byref(h), t, bp, E, M, K))
    _HANDLES[h.value] = _Meta(t, M, K, E, blocks.device.index)
    return h


def qmm_destroy(h) -> None:
    key = h.value if isinstance(h, ctypes.c_void_p) else h
    _HANDLES.pop(key, None)
    check(lib.qmm_destroy(h))


def qmm_gemv(h, x: torch.Tensor, N: int, y: torch.Tensor, stream=None) -> None:
    m = _meta(h)
    N = _count(N, "N", 0)
    xp, yp = _need(m.device, (x, "x", (N, m.K), _ACT), (y, "y", (N, m.M), _F32))
    check(lib.qmm_gemv(h, xp, _xt(x), N, yp, _stream(stream)))


def qmm_gemv_group(hs, xs, N: int, ys, stream=None) -> None:
    """qmm_gemv on each (hs[i], xs[i], ys[i]); one-token matrices of one format and K
    share launches.  Every x has the same dtype; every tensor is on the handles' device."""
    hs, xs, ys = list(hs), list(xs), list(ys)
    if not (len(hs) == len(xs) == len(ys)):
        raise ValueError("hs, xs and ys must have the same length")
    N = _count(N, "N", 0)
    if not hs:
        return
    if len({x.dtype for x in xs}) > 1:
        raise ValueError("every x must have the same dtype")
    n = len(hs)
    metas = [_meta(h) for h in hs]
    if len({m.device for m in metas}) > 1:
        raise ValueError("every handle must be on the same device")
    specs = []
    for i, (m, x, y) in enumerate(zip(metas, xs, ys)):
        specs += [(x, f"xs[{i}]", (N, m.K), _ACT), (y, f"ys[{i}]", (N, m.M), _F32)]
    ptrs = _need(metas[0].device, *specs)
    ha = (ctypes.c_void_p * n)(*[h if isinstance(h, int) else h.value for h in hs])
    xa = (ctypes.c_void_p * n)(*[p.value for p in ptrs[0::2]])
    ya = (ctypes.c_void_p * n)(*[p.value for p in ptrs[1::2]])
    check(lib.qmm_gemv_group(ha, xa, _xt(xs[0]), N, ya, n, _stream(stream)))


def qmm_gemm(h, x: torch.Tensor, N: int, y: torch.Tensor, tile=0, stream=None) -> None:
    m = _meta(h)
    N = _count(N, "N", 0)
    t = TILES[tile] if tile in TILES else int(tile)
    xp, yp = _need(m.device, (x, "x", (N, m.K), _ACT), (y, "y", (N, m.M), _F32))
    check(lib.qmm_gemm(h, xp, _xt(x), N, yp, t, _stream(stream)))


def qmm_gemm_workspace_bytes(h, N: int) -> int:
    return lib.qmm_gemm_workspace_bytes(h, int(N))


def qmm_gemm_ws(h, x: torch.Tensor, N: int, y: torch.Tensor, tile=0, ws: torch.Tensor = None, stream=None) -> None:
    m = _meta(h)
    N = _count(N, "N", 0)
    t = TILES[tile] if tile in TILES else int(tile)
    if ws is None:
        xp, yp = _need(m.device, (x, "x", (N, m.K), _ACT), (y, "y", (N, m.M), _F32))
        wp, wb = ctypes.c_void_p(0), 0
    else:
        xp, yp, wp = _need(m.device, (x, "x", (N, m.K), _ACT), (y, "y", (N, m.M), _F32), (ws, "ws", None, None))
        wb = ws.numel() * ws.element_size()
    check(lib.qmm_gemm_ws(h, xp, _xt(x), N, yp, t, wp, wb, _stream(stream)))


def qmm_gemm_noalloc(h, x: torch.Tensor, N: int, y: torch.Tensor, tile=0, stream=None) -> None:
    m = _meta(h)
    N = _count(N, "N", 0)
    t = TILES[tile] if tile in TILES else int(tile)
    xp, yp = _need(m.device, (x, "x", (N, m.K), _ACT), (y, "y", (N, m.M), _F32))
    check(lib.qmm_gemm_noalloc(h, xp, _xt(x), N, yp, t, _stream(stream)))


def _id_args(m, x, N, S, x_per_slot, ids, y):
    N, S = _count(N, "N", 0), _count(S, "S", 1)
    if x_per_slot not in (0, 1):
        raise ValueError("x_per_slot must be 0 or 1")
    xp, ip, yp = _need(m.device, (x, "x", (N, S, m.K) if x_per_slot else (N, m.K), _ACT),
                       (ids, "ids", (N, S), (torch.int32,)), (y, "y", (N, S, m.M), _F32))
    return N, S, xp, ip, yp


def qmm_gemm_id_tiled(h, x: torch.Tensor, N: int, S: int, x_per_slot: int, ids: torch.Tensor, y: torch.Tensor,
                      tile=0, stream=None) -> None:
    m = _meta(h)
    t = TILES[tile] if tile in TILES else int(tile)
    N, S, xp, ip, yp = _id_args(m, x, N, S, x_per_slot, ids, y)
    check(lib.qmm_gemm_id_tiled(h, xp, _xt(x), N, S, int(x_per_slot), ip, yp, t, _stream(stream)))


def qmm_gemm_id(h, x: torch.Tensor, N: int, S: int, x_per_slot: int, ids: torch.Tensor, y: torch.Tensor,
                stream=None) -> None:
    m = _meta(h)
    N, S, xp, ip, yp = _id_args(m, x, N, S, x_per_slot, ids, y)
    check(lib.qmm_gemm_id(h, xp, _xt(x), N, S, int(x_per_slot), ip, yp, _stream(stream)))


def qmm_dequantize(h, expert: int, out: torch.Tensor, stream=None) -> None:
    m = _meta(h)
    expert = _count(expert, "expert", 0, m.n_experts - 1)
    op = _need(m.device, (out, "out", (m.M, m.K), _ACT))
    check(lib.qmm_dequantize(h, expert, op, _XT[out.dtype], _stream(stream)))


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
            qmm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self):
        return self._h

    def _rows(self, x, dims):
        """Leading dimensions of x ([N, K] when dims == 2); x must end in K."""
        if not isinstance(x, torch.Tensor) or x.dim() not in dims:
            raise ValueError(f"x must be a tensor of {' or '.join(str(d) for d in dims)} dimensions")
        if x.shape[-1] != self.K:
            raise ValueError(f"x has K={x.shape[-1]}, matrix has K={self.K}")
        return tuple(x.shape[:-1])

    def _ids(self, x, ids):
        if not isinstance(ids, torch.Tensor) or ids.dtype != torch.int32 or ids.dim() != 2:
            raise ValueError("ids must be an int32 [N, S] tensor")
        N, S = ids.shape
        lead = self._rows(x, (2, 3))
        if lead != ((N, S) if x.dim() == 3 else (N,)):
            raise ValueError(f"x has leading shape {lead}; ids [N, S] = {(N, S)} needs [N, S, K] or [N, K]")
        return N, S, 1 if x.dim() == 3 else 0

    def gemv(self, x: torch.Tensor, out: torch.Tensor = None) -> torch.Tensor:
        """x [N, K] (N <= 32) -> y [N, M] fp32."""
        (N,) = self._rows(x, (2,))
        y = out if out is not None else torch.empty((N, self.M), dtype=torch.float32, device=x.device)
        qmm_gemv(self._h, x, N, y)
        return y

    def gemm(self, x: torch.Tensor, tile="auto", out: torch.Tensor = None) -> torch.Tensor:
        """x [N, K] -> y [N, M] fp32 through the fp16 matrix-core path; tile "auto", 32 or 64."""
        (N,) = self._rows(x, (2,))
        y = out if out is not None else torch.empty((N, self.M), dtype=torch.float32, device=x.device)
        nb = qmm_gemm_workspace_bytes(self._h, N)
        ws = torch.empty((nb + 15) // 16 * 4, dtype=torch.float32, device=x.device) if nb else None
        qmm_gemm_ws(self._h, x, N, y, tile, ws)
        return y

    def gemm_id(self, x: torch.Tensor, ids: torch.Tensor, out: torch.Tensor = None) -> torch.Tensor:
        """ids [N, S] int32; x [N, S, K] (one row per slot) or [N, K] -> y [N, S, M] fp32."""
        N, S, x_per_slot = self._ids(x, ids)
        y = out if out is not None else torch.empty((N, S, self.M), dtype=torch.float32, device=x.device)
        qmm_gemm_id(self._h, x, N, S, x_per_slot, ids, y)
        return y

    def gemm_id_tiled(self, x: torch.Tensor, ids: torch.Tensor, tile="auto", out: torch.Tensor = None) -> torch.Tensor:
        """Prefill-sized expert-indexed product on the matrix cores (any N): ids [N, S]
        int32; x [N, S, K] or [N, K] -> y [N, S, M] fp32; tile "auto", 32 or 64."""
        N, S, x_per_slot = self._ids(x, ids)
        y = out if out is not None else torch.empty((N, S, self.M), dtype=torch.float32, device=x.device)
        qmm_gemm_id_tiled(self._h, x, N, S, x_per_slot, ids, y, tile)
        return y

    def dequantize(self, expert: int = 0, dtype=torch.float32) -> torch.Tensor:
        out = torch.empty((self.M, self.K), dtype=dtype, device=self._blocks.device)
        qmm_dequantize(self._h, expert, out)
        return out
