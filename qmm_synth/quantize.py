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
Q4_1, Q5_1   as A4G64 over 32 weights, with 15 or 31 levels (m is the bias).
Q5_0   as Q4_0 with d = fp16(w* / -16) and q = min(31, floor(w/d + 16.5)).
Q2_K, Q5_K   as Q4_K over 16-weight sub-blocks with 4-bit fields and 3 levels
       (Q2_K), or 32-weight sub-blocks with 6-bit fields and 31 levels (Q5_K).
Q3_K   per 16-sub-block: the extreme w*_j sets a signed scale that maps it to
       the code -4 (see _quant_q3_k).

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


def _affine_32(w: np.ndarray, levels: int):
    """(d16, m16, q) of the scale-and-minimum encoders: m = fp16 rounded down of min w,
    d = fp16 rounded up of (max w - m) / levels, q = clamp(rha((w - m) / d), 0, levels)."""
    wb = w.reshape(-1, 32).astype(np.float64)
    m16 = _f16_down(wb.min(axis=1))
    m = m16.astype(np.float64)[:, None]
    d16 = _f16_up((wb.max(axis=1) - m[:, 0]) / levels)
    d = d16.astype(np.float64)[:, None]
    q = np.clip(_round_half_away(_safe_div(wb - m, d)), 0, levels)
    q = np.where(d == 0, 0, q).astype(np.uint8)
    return d16, m16, q


def _quant_q4_1(w: np.ndarray) -> np.ndarray:
    d16, m16, q = _affine_32(w, 15)
    out = np.empty((q.shape[0], 20), dtype=np.uint8)
    out[:, 0:2] = _f16_bytes(d16)
    out[:, 2:4] = _f16_bytes(m16)
    out[:, 4:20] = q[:, :16] | (q[:, 16:] << 4)
    return out


def _qh_bytes(q: np.ndarray) -> np.ndarray:
    """[nb, 32] 5-bit codes -> [nb, 4] little-endian bytes of their top bits (bit i = code i)."""
    bits = ((q >> 4) & 1).astype(np.uint64)
    word = (bits << np.arange(32, dtype=np.uint64)[None, :]).sum(axis=1).astype(np.uint32)
    return word.astype("<u4").view(np.uint8).reshape(-1, 4)


def _quant_q5_0(w: np.ndarray) -> np.ndarray:
    wb = w.reshape(-1, 32).astype(np.float64)
    idx = np.argmax(np.abs(wb), axis=1)
    wstar = wb[np.arange(wb.shape[0]), idx]
    d16 = _f16_rne(wstar / -16.0)
    d = d16.astype(np.float64)[:, None]
    q = np.floor(_safe_div(wb, d) + 16.5)
    q = np.where(d == 0, 16, q)
    q = np.clip(q, 0, 31).astype(np.uint8)
    out = np.empty((wb.shape[0], 22), dtype=np.uint8)
    out[:, 0:2] = _f16_bytes(d16)
    out[:, 2:6] = _qh_bytes(q)
    out[:, 6:22] = (q[:, :16] & 15) | ((q[:, 16:] & 15) << 4)
    return out


def _quant_q5_1(w: np.ndarray) -> np.ndarray:
    d16, m16, q = _affine_32(w, 31)
    out = np.empty((q.shape[0], 24), dtype=np.uint8)
    out[:, 0:2] = _f16_bytes(d16)
    out[:, 2:4] = _f16_bytes(m16)
    out[:, 4:8] = _qh_bytes(q)
    out[:, 8:24] = (q[:, :16] & 15) | ((q[:, 16:] & 15) << 4)
    return out


def _scale_min_k(wb: np.ndarray, levels: int, field_max: int):
    """Covering encoder of the scale-and-minimum K-quants, per sub-block j (wb [nb, J, S]):
    lo_j = min(0, min w), hi_j = max w, dmin = up(max_j(-lo_j) / field_max),
    m_j = ceil(-lo_j / dmin), span_j = hi_j + dmin m_j, d = up(max_j(span_j / levels) / field_max),
    sc_j = ceil(span_j / (levels d)), q = clamp(rha((w + dmin m_j) / (d sc_j)), 0, levels)."""
    lo = np.minimum(0.0, wb.min(axis=2))
    hi = wb.max(axis=2)
    dmin16 = _f16_up((-lo).max(axis=1) / field_max)
    dmin = dmin16.astype(np.float64)[:, None]
    m = np.clip(np.ceil(_safe_div(-lo, dmin)), 0, field_max)
    dm = dmin * m
    span = hi + dm
    d16 = _f16_up((span / levels).max(axis=1) / field_max)
    d = d16.astype(np.float64)[:, None]
    sc = np.clip(np.ceil(_safe_div(span, levels * d)), 0, field_max)
    step = (d * sc)[:, :, None]
    q = np.clip(_round_half_away(_safe_div(wb + dm[:, :, None], step)), 0, levels)
    q = np.where(step == 0, 0, q).astype(np.uint8).reshape(wb.shape[0], -1)
    return d16, dmin16, sc.astype(np.int64), m.astype(np.int64), q


def _quant_q2_k(w: np.ndarray) -> np.ndarray:
    wb = w.reshape(-1, 16, 16).astype(np.float64)
    d16, dmin16, sc, m, q = _scale_min_k(wb, 3, 15)
    out = np.empty((wb.shape[0], 84), dtype=np.uint8)
    out[:, 0:2] = _f16_bytes(d16)
    out[:, 2:4] = _f16_bytes(dmin16)
    out[:, 4:20] = (sc | (m << 4)).astype(np.uint8)
    qs = np.zeros((wb.shape[0], 64), dtype=np.uint8)
    for b in range(4):
        qs |= q[:, 64 * b: 64 * b + 64] << (2 * b)
    out[:, 20:84] = qs
    return out


def _quant_q3_k(w: np.ndarray) -> np.ndarray:
    """w*_j = the signed element of largest magnitude of 16-sub-block j (first on a tie);
    d = up(max_j |w*_j| / 124); s_j = -sign(w*_j) ceil(|w*_j| / (4 d)) (at most 31 in
    magnitude), stored as s_j + 32; q = clamp(rha(w / (d s_j)) + 4, 0, 7) (4 when d s_j = 0).
    The extreme w*_j maps to the code -4 side, the wide end of -4..3."""
    wb = w.reshape(-1, 16, 16).astype(np.float64)
    idx = np.argmax(np.abs(wb), axis=2)
    wstar = np.take_along_axis(wb, idx[:, :, None], axis=2)[:, :, 0]
    d16 = _f16_up(np.abs(wstar).max(axis=1) / 124.0)
    d = d16.astype(np.float64)[:, None]
    mag = np.clip(np.ceil(_safe_div(np.abs(wstar), 4.0 * d)), 0, 31)
    s = np.where(wstar > 0, -mag, mag)
    step = (d * s)[:, :, None]
    q = np.clip(_round_half_away(_safe_div(wb, step)) + 4, 0, 7)
    q = np.where(step == 0, 4, q).astype(np.uint8).reshape(-1, 256)
    out = np.empty((wb.shape[0], 110), dtype=np.uint8)
    out[:, 0:2] = _f16_bytes(d16)
    out[:, 2:14] = _pack_6bit_fields((s + 32).astype(np.int64))
    ql = np.zeros((wb.shape[0], 64), dtype=np.uint8)
    for b in range(4):
        ql |= (q[:, 64 * b: 64 * b + 64] & 3) << (2 * b)
    out[:, 14:78] = ql
    qh = np.zeros((wb.shape[0], 32), dtype=np.uint8)
    for b in range(8):
        qh |= ((q[:, 32 * b: 32 * b + 32] >> 2) & 1) << b
    out[:, 78:110] = qh
    return out


def _quant_q5_k(w: np.ndarray) -> np.ndarray:
    wb = w.reshape(-1, 8, 32).astype(np.float64)
    d16, dmin16, sc, m, q = _scale_min_k(wb, 31, 63)
    out = np.empty((wb.shape[0], 176), dtype=np.uint8)
    out[:, 0:2] = _f16_bytes(d16)
    out[:, 2:4] = _f16_bytes(dmin16)
    out[:, 4:16] = _pack_6bit_fields(np.concatenate([sc, m], axis=1))
    qh = np.zeros((wb.shape[0], 32), dtype=np.uint8)
    for b in range(8):
        qh |= ((q[:, 32 * b: 32 * b + 32] >> 4) & 1) << b
    out[:, 16:48] = qh
    for p in range(4):
        out[:, 48 + 32 * p: 80 + 32 * p] = (q[:, 64 * p: 64 * p + 32] & 15) | ((q[:, 64 * p + 32: 64 * p + 64] & 15) << 4)
    return out


QUANTIZERS = {
    "q4_0": (32, _quant_q4_0),
    "q8_0": (32, _quant_q8_0),
    "q4_k": (256, _quant_q4_k),
    "q6_k": (256, _quant_q6_k),
    "a4g64": (64, _quant_a4g64),
    "q4_1": (32, _quant_q4_1),
    "q5_0": (32, _quant_q5_0),
    "q5_1": (32, _quant_q5_1),
    "q2_k": (256, _quant_q2_k),
    "q3_k": (256, _quant_q3_k),
    "q5_k": (256, _quant_q5_k),
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
