"""Block layouts and dequantization to fp32 -- CPU oracle (test infrastructure only).

The pages name the block formats but print no byte layout: the candle pull
request "Metal: 64-token tile for the quantized matrix-matrix kernel"
(section "What changes") lists Q4_0, Q4_1, Q5_0, Q5_1, Q8_0 and the K-quants
Q2_K, Q3_K, Q4_K, Q5_K and Q6_K among the types its kernel serves, and the
tiny-llm pull request "perf: Optimize quantized matmul for small decode
batches" (section "Benchmark setup") runs an MLX 4-bit model, i.e. 4-bit codes
with a scale and a bias per group.  Formulas are given for four of them by the
workloads (Q4_0, Q4_K, Q6_K, the 4-bit groups); for the others the plainest
reading of their names is taken -- an "_0" type is a symmetric scale times a
code centred on zero, an "_1" type a scale and a minimum, a K-quant a 256-weight
super-block with an fp16 scale (and minimum) and small integer scales (and
minimums) per sub-block -- with the code widths the names give:

    Q4_0   32 weights, fp16 d,                     w = d * (q - 8),          q in 0..15
    Q4_1   32 weights, fp16 d, m,                  w = d * q + m,            q in 0..15
    Q5_0   32 weights, fp16 d,                     w = d * (q - 16),         q in 0..31
    Q5_1   32 weights, fp16 d, m,                  w = d * q + m,            q in 0..31
    Q8_0   32 weights, fp16 d,                     w = d * q,                q in -128..127
    Q2_K   256 = 16 x 16, fp16 d, dmin,
           4-bit sc_j and m_j per 16-sub-block,    w = d*sc_j*q - dmin*m_j,  q in 0..3
    Q3_K   256 = 16 x 16, fp16 d,
           6-bit s_j per 16-sub-block,             w = d*(s_j-32)*(q-4),     q in 0..7
    Q4_K   256 = 8 x 32, fp16 d, dmin,
           6-bit sc_j and m_j per 32-sub-block,    w = d*sc_j*q - dmin*m_j,  q in 0..15
    Q5_K   256 = 8 x 32, as Q4_K with 5-bit codes, w = d*sc_j*q - dmin*m_j,  q in 0..31
    Q6_K   256 = 16 x 16, fp16 d, int8 sc_j,       w = d * sc_j * (q - 32),  q in 0..63
    A4G64  64 weights, fp16 scale and bias,        w = scale * q + bias,     q in 0..15

Byte layouts (this library's own; the pages are silent).  fp16 fields are
little-endian IEEE binary16; "bit string" means a little-endian string of
equal-width fields, field f at bits [width*f, width*(f+1)).

    Q4_0   18 B : [0,2) d | [2,18) qs[16]; weight i (0..15) = low nibble of qs[i],
                  weight i+16 = high nibble of qs[i].
    Q4_1   20 B : [0,2) d | [2,4) m | [4,20) qs[16] as Q4_0.
    Q5_0   22 B : [0,2) d | [2,6) qh, 32-bit little-endian: bit i is the fifth
                  (top) bit of weight i | [6,22) qs[16], low four bits as Q4_0.
    Q5_1   24 B : [0,2) d | [2,4) m | [4,8) qh | [8,24) qs[16], as Q5_0.
    Q8_0   34 B : [0,2) d | [2,34) int8 q[32]; weight i = q[i].
    Q2_K   84 B : [0,2) d | [2,4) dmin | [4,20) sm[16]: sc_j = low nibble of sm[j],
                  m_j = high nibble | [20,84) qs[64]: weight i = bits 2(i//64) ..
                  2(i//64)+1 of qs[i % 64]; sub-block j = i // 16.
    Q3_K  110 B : [0,2) d | [2,14) a 96-bit string of sixteen 6-bit fields s_j |
                  [14,78) ql[64]: the low two bits of weight i are bits 2(i//64) ..
                  2(i//64)+1 of ql[i % 64] | [78,110) qh[32]: the top bit of weight i
                  is bit i//32 of qh[i % 32]; q = low2 | top << 2; sub-block j = i // 16.
    Q4_K  144 B : [0,2) d | [2,4) dmin | [4,16) a 96-bit string of sixteen 6-bit
                  fields: fields 0..7 are sc_0..sc_7, fields 8..15 are m_0..m_7 |
                  [16,144) qs[128]: for p in 0..3 and i in 0..31, weight 64p+i = low
                  nibble of qs[32p+i] (sub-block 2p) and weight 64p+32+i = high nibble
                  (sub-block 2p+1).
    Q5_K  176 B : [0,2) d | [2,4) dmin | [4,16) sc/m bit string as Q4_K | [16,48)
                  qh[32]: the top bit of weight i is bit i//32 of qh[i % 32] |
                  [48,176) qs[128], low four bits as Q4_K; q = low4 | top << 4.
    Q6_K  210 B : [0,2) d | [2,18) int8 sc[16] | [18,146) ql[128]: weight i
                  (0..127) takes the low nibble of ql[i], weight i+128 the high
                  nibble | [146,210) qh[64]: bits 2b..2b+1 of qh[i] are the top two
                  bits of weight i+64b (b = 0..3).  q = low4 | high2 << 4;
                  sub-block j = weight // 16.
    A4G64  36 B : [0,2) scale | [2,4) bias | [4,36) qs[32]; weight i (0..31) = low
                  nibble of qs[i], weight i+32 = high nibble.

A row of W is its K/block_weights blocks back to back; row r starts at byte
r * row_bytes(K); expert e of a stacked tensor starts at e * M * row_bytes(K).

Exactness: every product in these formulas is exact in fp32 (at most 23
significant bits from an 11-bit fp16 significand times a code of at most 12
bits), so the only rounding is the single add or subtract of the formats with
a minimum or bias (Q4_1, Q5_1, Q2_K, Q4_K, Q5_K, A4G64).  The dequantized value
is therefore the fp32 round-to-nearest-even of the exact real value of the
formula.  The functions below evaluate the products in fp32 (and assert that
they are exact) and then do the one add or subtract in fp32.
"""

import numpy as np

# format name -> (weights per block, bytes per block)
FORMATS = {
    "q4_0": (32, 18),
    "q8_0": (32, 34),
    "q4_k": (256, 144),
    "q6_k": (256, 210),
    "a4g64": (64, 36),
    "q4_1": (32, 20),
    "q5_0": (32, 22),
    "q5_1": (32, 24),
    "q2_k": (256, 84),
    "q3_k": (256, 110),
    "q5_k": (256, 176),
}


def block_weights(fmt: str) -> int:
    return FORMATS[fmt][0]


def block_bytes(fmt: str) -> int:
    return FORMATS[fmt][1]


def row_bytes(fmt: str, K: int) -> int:
    """Bytes of one row of K weights; 0 when K is not a positive multiple of the block."""
    bw, bb = FORMATS[fmt]
    if K <= 0 or K % bw:
        return 0
    return (K // bw) * bb


def _fp16_field(blocks: np.ndarray, off: int) -> np.ndarray:
    """The little-endian fp16 at byte offset ``off`` of every block, as exact fp32."""
    bits = blocks[:, off].astype(np.uint16) | (blocks[:, off + 1].astype(np.uint16) << 8)
    return bits.view(np.float16).astype(np.float32)


def _exact_product(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """a*b in fp32, asserting that the fp32 product equals the exact (fp64) product."""
    p32 = np.multiply(a.astype(np.float32), b.astype(np.float32), dtype=np.float32)
    p64 = a.astype(np.float64) * b.astype(np.float64)
    assert np.array_equal(p32.astype(np.float64), p64), "product not exact in fp32"
    return p32


def _dequant_q4_0(blocks: np.ndarray) -> np.ndarray:
    d = _fp16_field(blocks, 0)
    qs = blocks[:, 2:18].astype(np.int32)
    q = np.concatenate([qs & 0x0F, qs >> 4], axis=1)  # weights 0..15, then 16..31
    return _exact_product(d[:, None], q - 8)


def _dequant_q8_0(blocks: np.ndarray) -> np.ndarray:
    d = _fp16_field(blocks, 0)
    q = blocks[:, 2:34].view(np.int8).astype(np.int32)
    return _exact_product(d[:, None], q)


def _six_bit_fields(blocks: np.ndarray, off: int) -> np.ndarray:
    """The sixteen 6-bit fields of the 96-bit string at bytes [off, off+12): [nb, 16]."""
    raw = blocks[:, off:off + 12].astype(np.int64)
    fields = np.empty((blocks.shape[0], 16), dtype=np.int64)
    for f in range(16):
        bit = 6 * f
        byte, shift = divmod(bit, 8)
        two = raw[:, byte] | (raw[:, byte + 1] << 8) if byte + 1 < 12 else raw[:, byte]
        fields[:, f] = (two >> shift) & 0x3F
    return fields


def _q4_k_fields(blocks: np.ndarray):
    """The sixteen 6-bit fields of the Q4_K (and Q5_K) bit string: (sc[nb,8], m[nb,8])."""
    fields = _six_bit_fields(blocks, 4)
    return fields[:, :8], fields[:, 8:]


def _le32(blocks: np.ndarray, off: int) -> np.ndarray:
    """The little-endian 32-bit word at byte offset ``off`` of every block, [nb] int64."""
    return sum(blocks[:, off + b].astype(np.int64) << (8 * b) for b in range(4))


def _dequant_q4_k(blocks: np.ndarray) -> np.ndarray:
    d = _fp16_field(blocks, 0)
    dmin = _fp16_field(blocks, 2)
    sc, m = _q4_k_fields(blocks)
    qs = blocks[:, 16:144].astype(np.int32).reshape(-1, 4, 32)
    q = np.empty((blocks.shape[0], 256), dtype=np.int32)
    for p in range(4):
        q[:, 64 * p: 64 * p + 32] = qs[:, p, :] & 0x0F
        q[:, 64 * p + 32: 64 * p + 64] = qs[:, p, :] >> 4
    j = np.arange(256) // 32                       # sub-block of each weight
    d_sc = _exact_product(d[:, None], sc)          # [nb, 8]
    scaled = _exact_product(d_sc[:, j], q)         # d*sc_j*q
    mins = _exact_product(dmin[:, None], m)        # dmin*m_j
    return np.subtract(scaled, mins[:, j], dtype=np.float32)


def _dequant_q6_k(blocks: np.ndarray) -> np.ndarray:
    d = _fp16_field(blocks, 0)
    sc = blocks[:, 2:18].view(np.int8).astype(np.int32)
    ql = blocks[:, 18:146].astype(np.int32)
    qh = blocks[:, 146:210].astype(np.int32)
    i = np.arange(256)
    low4 = np.where(i < 128, ql[:, i % 128] & 0x0F, ql[:, i % 128] >> 4)
    high2 = (qh[:, i % 64] >> (2 * (i // 64))) & 0x3
    q = low4 | (high2 << 4)
    code = sc[:, i // 16] * (q - 32)               # exact integer, |code| <= 4096
    return _exact_product(d[:, None], code)


def _dequant_a4g64(blocks: np.ndarray) -> np.ndarray:
    scale = _fp16_field(blocks, 0)
    bias = _fp16_field(blocks, 2)
    qs = blocks[:, 4:36].astype(np.int32)
    q = np.concatenate([qs & 0x0F, qs >> 4], axis=1)
    return np.add(_exact_product(scale[:, None], q), bias[:, None], dtype=np.float32)


def _dequant_q4_1(blocks: np.ndarray) -> np.ndarray:
    d = _fp16_field(blocks, 0)
    m = _fp16_field(blocks, 2)
    qs = blocks[:, 4:20].astype(np.int32)
    q = np.concatenate([qs & 0x0F, qs >> 4], axis=1)
    return np.add(_exact_product(d[:, None], q), m[:, None], dtype=np.float32)


def _five_bit_codes(qs: np.ndarray, qh: np.ndarray) -> np.ndarray:
    """32 five-bit codes of a Q5_0/Q5_1 block: low nibbles as Q4_0, bit i of qh on top."""
    low = np.concatenate([qs & 0x0F, qs >> 4], axis=1).astype(np.int64)
    top = (qh[:, None] >> np.arange(32)[None, :]) & 1
    return (low | (top << 4)).astype(np.int32)


def _dequant_q5_0(blocks: np.ndarray) -> np.ndarray:
    d = _fp16_field(blocks, 0)
    q = _five_bit_codes(blocks[:, 6:22].astype(np.int32), _le32(blocks, 2))
    return _exact_product(d[:, None], q - 16)


def _dequant_q5_1(blocks: np.ndarray) -> np.ndarray:
    d = _fp16_field(blocks, 0)
    m = _fp16_field(blocks, 2)
    q = _five_bit_codes(blocks[:, 8:24].astype(np.int32), _le32(blocks, 4))
    return np.add(_exact_product(d[:, None], q), m[:, None], dtype=np.float32)


def _dequant_q2_k(blocks: np.ndarray) -> np.ndarray:
    d = _fp16_field(blocks, 0)
    dmin = _fp16_field(blocks, 2)
    sm = blocks[:, 4:20].astype(np.int32)
    sc, m = sm & 0x0F, sm >> 4                      # [nb, 16]
    qs = blocks[:, 20:84].astype(np.int32)
    i = np.arange(256)
    q = (qs[:, i % 64] >> (2 * (i // 64))) & 0x3
    j = i // 16
    d_sc = _exact_product(d[:, None], sc)
    scaled = _exact_product(d_sc[:, j], q)
    mins = _exact_product(dmin[:, None], m)
    return np.subtract(scaled, mins[:, j], dtype=np.float32)


def _dequant_q3_k(blocks: np.ndarray) -> np.ndarray:
    d = _fp16_field(blocks, 0)
    s = _six_bit_fields(blocks, 2) - 32             # signed scales, [nb, 16]
    ql = blocks[:, 14:78].astype(np.int32)
    qh = blocks[:, 78:110].astype(np.int32)
    i = np.arange(256)
    q = ((ql[:, i % 64] >> (2 * (i // 64))) & 0x3) | (((qh[:, i % 32] >> (i // 32)) & 1) << 2)
    code = s[:, i // 16] * (q - 4)                  # exact integer, |code| <= 128
    return _exact_product(d[:, None], code)


def _dequant_q5_k(blocks: np.ndarray) -> np.ndarray:
    d = _fp16_field(blocks, 0)
    dmin = _fp16_field(blocks, 2)
    sc, m = _q4_k_fields(blocks)
    qh = blocks[:, 16:48].astype(np.int32)
    qs = blocks[:, 48:176].astype(np.int32).reshape(-1, 4, 32)
    low = np.empty((blocks.shape[0], 256), dtype=np.int32)
    for p in range(4):
        low[:, 64 * p: 64 * p + 32] = qs[:, p, :] & 0x0F
        low[:, 64 * p + 32: 64 * p + 64] = qs[:, p, :] >> 4
    i = np.arange(256)
    q = low | (((qh[:, i % 32] >> (i // 32)) & 1) << 4)
    j = i // 32
    d_sc = _exact_product(d[:, None], sc)
    scaled = _exact_product(d_sc[:, j], q)
    mins = _exact_product(dmin[:, None], m)
    return np.subtract(scaled, mins[:, j], dtype=np.float32)


_DEQUANT = {
    "q4_0": _dequant_q4_0,
    "q8_0": _dequant_q8_0,
    "q4_k": _dequant_q4_k,
    "q6_k": _dequant_q6_k,
    "a4g64": _dequant_a4g64,
    "q4_1": _dequant_q4_1,
    "q5_0": _dequant_q5_0,
    "q5_1": _dequant_q5_1,
    "q2_k": _dequant_q2_k,
    "q3_k": _dequant_q3_k,
    "q5_k": _dequant_q5_k,
}


def dequantize_blocks(fmt: str, blocks: np.ndarray) -> np.ndarray:
    """[nblocks, block_bytes] uint8 -> [nblocks, block_weights] fp32."""
    bw, bb = FORMATS[fmt]
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(-1, bb)
    out = _DEQUANT[fmt](blocks)
    assert out.dtype == np.float32 and out.shape == (blocks.shape[0], bw)
    return out


def dequantize(fmt: str, blob: np.ndarray, M: int, K: int) -> np.ndarray:
    """Whole matrix: ``blob`` holds M rows of row_bytes(fmt, K) bytes -> [M, K] fp32."""
    rb = row_bytes(fmt, K)
    if rb == 0:
        raise ValueError(f"K={K} is not a positive multiple of the {fmt} block")
    blob = np.ascontiguousarray(blob, dtype=np.uint8).reshape(-1)
    if blob.size != M * rb:
        raise ValueError(f"expected {M * rb} bytes, got {blob.size}")
    return dequantize_blocks(fmt, blob).reshape(M, K)


def staged_fp16(w: np.ndarray) -> np.ndarray:
    """The fp16 value a weight takes when staged for the fp16 matrix-core product:
    round-to-nearest-even of the fp32 dequantized value (NumPy's cast is RNE; a
    magnitude at or above the overflow tie 65520 becomes an infinity, as IEEE
    rounding defines).  The candle pull request "Metal: 64-token tile for the
    quantized matrix-matrix kernel" (section "Why the tile sets the weight reuse")
    decodes each weight tile into threadgroup memory for the matrix product; read
    here as the fp32 weight rounded once more, to fp16."""
    with np.errstate(over="ignore"):
        return np.asarray(w, dtype=np.float32).astype(np.float16)
