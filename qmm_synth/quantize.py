"""Deterministic encoders fp32 -> blocks, used to make test and benchmark data.

The pages quantize random weights to each type before timing (candle pull
request "Metal: 64-token tile for the quantized matrix-matrix kernel",
section "Numbers": "The weights are random, quantized to those types") but
print no quantizer.  These are plain closed-form encoders (real libraries use
iterative searches; the result only has to be a valid block):

Q4_0   w* = the element of largest |w| (first on a tie); d = fp16(w* / -8);
       q = min(15, floor(w/d + 8.5)); an all-zero block gets d = 0, q = 8.
Q8_0   d = fp16(max|w| / 127); q = clamp(round_half_away(w/d), -127, 127).
Q4_K   per 32-sub-block j: lo_j = min(0, min w), hi_j = max w;
       dmin = fp16 rounded up of max_j(-lo_j)/63, m_j = ceil(-lo_j/dmin);
       d = fp16 rounded up of max_j((hi_j + dmin*m_j)/15)/63,
       sc_j = ceil((hi_j + dmin*m_j)/(15*d));
       q = clamp(round_half_away((w + dmin*m_j)/(d*sc_j)), 0, 15).
Q6_K   a_j = max|w| per 16-sub-block; d = fp16 rounded up of max_j a_j/(31*127);
       sc_j = ceil(a_j/(31*d)); q = clamp(round_half_away(w/(d*sc_j)) + 32, 0, 63).
A4G64  bias = fp16 rounded down of min w; scale = fp16 rounded up of
       (max w - bias)/15; q = clamp(round_half_away((w - bias)/scale), 0, 15).

The byte layout each encoder writes is the library's block layout (fp16
little-endian; nibble and bit placement as documented with each packer).
"""

import numpy as np


def _f16_rne(v):
    return np.asarray(v, dtype=np.float64).astype(np.float16)


def _f16_up(v):
    v = np.asarray(v, dtype=np.float64)
    h = v.astype(np.float16)
    low = h.astype(np.float64) < v
    h = np.where(low, np.nextafter(h, np.float16(np.inf)), h)
    return h.astype(np.float16)


def _f16_down(v):
    v = np.asarray(v, dtype=np.float64)
    h = v.astype(np.float16)
    high = h.astype(np.float64) > v
    h = np.where(high, np.nextafter(h, np.float16(-np.inf)), h)
    return h.astype(np.float16)


def _round_half_away(v):
    return np.sign(v) * np.floor(np.abs(v) + 0.5)


def _safe_div(a, b):
    b = np.asarray(b, dtype=np.float64)
    return np.divide(a, b, out=np.zeros(np.broadcast(a, b).shape), where=(b != 0))


def _f16_bytes(h: np.ndarray) -> np.ndarray:
    """fp16 array [n] -> little-endian bytes [n, 2]."""
    return np.ascontiguousarray(h.astype("<f2")).view(np.uint8).reshape(-1, 2)


def _quant_q4_0(w: np.ndarray) -> np.ndarray:
    wb = w.reshape(-1, 32).astype(np.float64)
    idx = np.argmax(np.abs(wb), axis=1)
    wstar = wb[np.arange(wb.shape[0]), idx]
    d16 = _f16_rne(wstar / -8.0)
    d = d16.astype(np.float64)[:, None]
    q = np.floor(_safe_div(wb, d) + 8.5)
    q = np.where(d == 0, 8, q)
    q = np.clip(q, 0, 15).astype(np.uint8)
    out = np.empty((wb.shape[0], 18), dtype=np.uint8)
    out[:, 0:2] = _f16_bytes(d16)
    out[:, 2:18] = q[:, :16] | (q[:, 16:] << 4)
    return out


def _quant_q8_0(w: np.ndarray) -> np.ndarray:
    wb = w.reshape(-1, 32).astype(np.float64)
    d16 = _f16_rne(np.abs(wb).max(axis=1) / 127.0)
    d = d16.astype(np.float64)[:, None]
    q = np.clip(_round_half_away(_safe_div(wb, d)), -127, 127).astype(np.int8)
    out = np.empty((wb.shape[0], 34), dtype=np.uint8)
    out[:, 0:2] = _f16_bytes(d16)
    out[:, 2:34] = q.view(np.uint8)
    return out


def _pack_6bit_fields(fields: np.ndarray) -> np.ndarray:
    """[nb, 16] values 0..63 -> [nb, 12] bytes of a little-endian bit string, field f at bit 6f."""
    out = np.zeros((fields.shape[0], 12), dtype=np.uint16)
    for f in range(16):
        v = fields[:, f].astype(np.uint16)
        byte, shift = divmod(6 * f, 8)
        out[:, byte] |= (v << shift) & 0xFF
        if shift + 6 > 8:
            out[:, byte + 1] |= v >> (8 - shift)
    return out.astype(np.uint8)


def _quant_q4_k(w: np.ndarray) -> np.ndarray:
    wb = w.reshape(-1, 8, 32).astype(np.float64)
    lo = np.minimum(0.0, wb.min(axis=2))
    hi = wb.max(axis=2)
    dmin16 = _f16_up((-lo).max(axis=1) / 63.0)
    dmin = dmin16.astype(np.float64)[:, None]
    m = np.clip(np.ceil(_safe_div(-lo, dmin)), 0, 63)
    dm = dmin * m
    span = hi + dm                                   # >= 0 by construction
    d16 = _f16_up((span / 15.0).max(axis=1) / 63.0)
    d = d16.astype(np.float64)[:, None]
    sc = np.clip(np.ceil(_safe_div(span, 15.0 * d)), 0, 63)
    step = (d * sc)[:, :, None]
    q = np.clip(_round_half_away(_safe_div(wb + dm[:, :, None], step)), 0, 15)
    q = np.where(step == 0, 0, q).astype(np.uint8).reshape(-1, 256)
    out = np.empty((wb.shape[0], 144), dtype=np.uint8)
    out[:, 0:2] = _f16_bytes(d16)
    out[:, 2:4] = _f16_bytes(dmin16)
    out[:, 4:16] = _pack_6bit_fields(np.concatenate([sc, m], axis=1).astype(np.int64))
    for p in range(4):
        out[:, 16 + 32 * p: 48 + 32 * p] = q[:, 64 * p: 64 * p + 32] | (q[:, 64 * p + 32: 64 * p + 64] << 4)
    return out


def _quant_q6_k(w: np.ndarray) -> np.ndarray:
    wb = w.reshape(-1, 16, 16).astype(np.float64)
    a = np.abs(wb).max(axis=2)
    d16 = _f16_up(a.max(axis=1) / (31.0 * 127.0))
    d = d16.astype(np.float64)[:, None]
    sc = np.clip(np.ceil(_safe_div(a, 31.0 * d)), 0, 127)
    step = (d * sc)[:, :, None]
    q = np.clip(_round_half_away(_safe_div(wb, step)) + 32, 0, 63)
    q = np.where(step == 0, 32, q).astype(np.uint8).reshape(-1, 256)
    out = np.empty((wb.shape[0], 210), dtype=np.uint8)
    out[:, 0:2] = _f16_bytes(d16)
    out[:, 2:18] = sc.astype(np.int8).view(np.uint8)
    out[:, 18:146] = (q[:, :128] & 0x0F) | ((q[:, 128:] & 0x0F) << 4)
    qh = np.zeros((wb.shape[0], 64), dtype=np.uint8)
    for b in range(4):
        qh |= ((q[:, 64 * b: 64 * b + 64] >> 4) & 0x3) << (2 * b)
    out[:, 146:210] = qh
    return out


def _quant_a4g64(w: np.ndarray) -> np.ndarray:
    wb = w.reshape(-1, 64).astype(np.float64)
    bias16 = _f16_down(wb.min(axis=1))
    bias = bias16.astype(np.float64)[:, None]
    scale16 = _f16_up((wb.max(axis=1) - bias[:, 0]) / 15.0)
    scale = scale16.astype(np.float64)[:, None]
    q = np.clip(_round_half_away(_safe_div(wb - bias, scale)), 0, 15)
    q = np.where(scale == 0, 0, q).astype(np.uint8)
    out = np.empty((wb.shape[0], 36), dtype=np.uint8)
    out[:, 0:2] = _f16_bytes(scale16)
    out[:, 2:4] = _f16_bytes(bias16)
    out[:, 4:36] = q[:, :32] | (q[:, 32:] << 4)
    return out


QUANTIZERS = {
    "q4_0": (32, _quant_q4_0),
    "q8_0": (32, _quant_q8_0),
    "q4_k": (256, _quant_q4_k),
    "q6_k": (256, _quant_q6_k),
    "a4g64": (64, _quant_a4g64),
}


def quantize(fmt: str, w: np.ndarray, chunk_rows: int = 1024) -> np.ndarray:
    """fp32 [M, K] -> flat uint8 blob of M rows of packed blocks (rows back to back)."""
    bw, fn = QUANTIZERS[fmt]
    w = np.asarray(w, dtype=np.float32)
    M, K = w.shape
    if K % bw:
        raise ValueError(f"K={K} is not a multiple of the {fmt} block ({bw})")
    parts = [fn(w[r: r + chunk_rows]).reshape(-1) for r in range(0, M, chunk_rows)]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.uint8)
