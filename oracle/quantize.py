"""Reference quantizers fp32 -> blocks (TEST INFRASTRUCTURE ONLY: see the package
docstring).  The library's GPU quantizer (qmm_quantize) is checked byte for
byte against these.

The pages quantize random weights to each type before timing (candle pull
request "Metal: 64-token tile for the quantized matrix-matrix kernel", section
"Numbers") but print no quantizer, so the closed forms below are this
library's readings (one per format; real libraries search iteratively).  All
arithmetic is in fp64 on the exact fp32 inputs, in the order written; fp16
roundings are to nearest even ("rne"), or the nearest fp16 at or above ("up")
or at or below ("down") the fp64 value:

  Q4_0   w* = element of largest |w| (first on a tie); d = rne(w* / -8);
         q = min(15, floor(w / d + 8.5)), q = 8 when d = 0.
  Q8_0   d = rne(max|w| / 127); q = clamp(rha(w / d), -127, 127), 0 when d = 0.
  Q4_K   per 32-weight sub-block j: lo_j = min(0, min w), hi_j = max w;
         dmin = up(max_j(-lo_j) / 63); m_j = clamp(ceil(-lo_j / dmin), 0, 63);
         span_j = hi_j + dmin * m_j; d = up(max_j(span_j / 15) / 63);
         sc_j = clamp(ceil(span_j / (15 d)), 0, 63); q = clamp(rha((w + dmin m_j)
         / (d sc_j)), 0, 15), 0 when d sc_j = 0; a zero divisor gives 0 before
         the ceil.
  Q6_K   a_j = max|w| per 16-weight sub-block; d = up(max_j a_j / 3937);
         sc_j = clamp(ceil(a_j / (31 d)), 0, 127); q = clamp(rha(w / (d sc_j)) + 32,
         0, 63), 32 when d sc_j = 0.
  A4G64  bias = down(min w); scale = up((max w - bias) / 15);
         q = clamp(rha((w - bias) / scale), 0, 15), 0 when scale = 0.

rha(v) = sign(v) * floor(|v| + 0.5) (round half away from zero).  Block byte
layouts are those of ``formats``.  Plain Python scalar loops: small inputs only.
"""

import math
import struct

import numpy as np

from .formats import block_weights


def _f16_bits(v: float) -> int:
    return struct.unpack("<H", struct.pack("<e", v))[0]


def _f16_value(bits: int) -> float:
    return struct.unpack("<e", struct.pack("<H", bits))[0]


def f16_rne(v: float) -> int:
    """fp16 bits nearest to v (ties to even)."""
    return _f16_bits(v)


def f16_up(v: float) -> int:
    """fp16 bits of the least fp16 value >= v."""
    h = _f16_bits(v)
    if _f16_value(h) < v:
        h = 0x0001 if h in (0x0000, 0x8000) else (h - 1 if h & 0x8000 else h + 1)
    return h


def f16_down(v: float) -> int:
    """fp16 bits of the greatest fp16 value <= v."""
    h = _f16_bits(v)
    if _f16_value(h) > v:
        h = 0x8001 if h in (0x0000, 0x8000) else (h + 1 if h & 0x8000 else h - 1)
    return h


def rha(v: float) -> float:
    return math.copysign(math.floor(abs(v) + 0.5), v) if v != 0 else 0.0


def _div(a: float, b: float) -> float:
    return a / b if b != 0 else 0.0


def _clamp(v, lo, hi):
    return lo if v < lo else (hi if v > hi else v)


def _le16(bits: int):
    return [bits & 0xFF, bits >> 8]


def quant_q4_0(w):
    wstar = w[0]
    for v in w:
        if abs(v) > abs(wstar):
            wstar = v
    hd = f16_rne(wstar / -8.0)
    d = _f16_value(hd)
    q = [8 if d == 0 else int(_clamp(math.floor(v / d + 8.5), 0, 15)) for v in w]
    return _le16(hd) + [q[i] | (q[i + 16] << 4) for i in range(16)]


def quant_q8_0(w):
    hd = f16_rne(max(abs(v) for v in w) / 127.0)
    d = _f16_value(hd)
    q = [int(_clamp(rha(_div(v, d)), -127, 127)) for v in w]
    return _le16(hd) + [c & 0xFF for c in q]


def quant_q4_k(w):
    subs = [w[32 * j: 32 * j + 32] for j in range(8)]
    lo = [min(0.0, min(s)) for s in subs]
    hi = [max(s) for s in subs]
    hdm = f16_up(max(-l for l in lo) / 63.0)
    dmin = _f16_value(hdm)
    m = [int(_clamp(math.ceil(_div(-l, dmin)), 0, 63)) for l in lo]
    span = [hi[j] + dmin * m[j] for j in range(8)]
    hd = f16_up(max(s / 15.0 for s in span) / 63.0)
    d = _f16_value(hd)
    sc = [int(_clamp(math.ceil(_div(span[j], 15.0 * d)), 0, 63)) for j in range(8)]
    q = []
    for j in range(8):
        step = d * sc[j]
        q += [0 if step == 0 else int(_clamp(rha((v + dmin * m[j]) / step), 0, 15)) for v in subs[j]]
    bits = 0
    for f, v in enumerate(sc + m):               # 6-bit fields, field f at bit 6f
        bits |= v << (6 * f)
    fields = [(bits >> (8 * i)) & 0xFF for i in range(12)]
    qs = []
    for p in range(4):                           # low nibble: sub-block 2p, high: 2p + 1
        qs += [q[64 * p + i] | (q[64 * p + 32 + i] << 4) for i in range(32)]
    return _le16(hd) + _le16(hdm) + fields + qs


def quant_q6_k(w):
    a = [max(abs(v) for v in w[16 * j: 16 * j + 16]) for j in range(16)]
    hd = f16_up(max(a) / 3937.0)
    d = _f16_value(hd)
    sc = [int(_clamp(math.ceil(_div(a[j], 31.0 * d)), 0, 127)) for j in range(16)]
    q = []
    for j in range(16):
        step = d * sc[j]
        q += [32 if step == 0 else int(_clamp(rha(v / step) + 32, 0, 63)) for v in w[16 * j: 16 * j + 16]]
    ql = [(q[i] & 0xF) | ((q[i + 128] & 0xF) << 4) for i in range(128)]
    qh = [sum(((q[64 * b + i] >> 4) & 3) << (2 * b) for b in range(4)) for i in range(64)]
    return _le16(hd) + [s & 0xFF for s in sc] + ql + qh


def quant_a4g64(w):
    hb = f16_down(min(w))
    bias = _f16_value(hb)
    hs = f16_up((max(w) - bias) / 15.0)
    scale = _f16_value(hs)
    q = [0 if scale == 0 else int(_clamp(rha((v - bias) / scale), 0, 15)) for v in w]
    return _le16(hs) + _le16(hb) + [q[i] | (q[i + 32] << 4) for i in range(32)]


_QUANT = {"q4_0": quant_q4_0, "q8_0": quant_q8_0, "q4_k": quant_q4_k, "q6_k": quant_q6_k, "a4g64": quant_a4g64}
# the formats with a reference quantizer (the library's GPU quantizer covers the same ones)
QUANT_FORMATS = tuple(_QUANT)


def quantize_blocks(fmt: str, w: np.ndarray) -> np.ndarray:
    """fp32 [M, K] -> uint8 blob of M rows of blocks (rows back to back)."""
    w = np.asarray(w, dtype=np.float32)
    M, K = w.shape
    bw = block_weights(fmt)
    if K % bw:
        raise ValueError(f"K={K} is not a multiple of the {fmt} block ({bw})")
    fn = _QUANT[fmt]
    out = []
    for r in range(M):
        row = [float(v) for v in w[r]]
        for b in range(0, K, bw):
            out += fn(row[b: b + bw])
    return np.array(out, dtype=np.uint8)
