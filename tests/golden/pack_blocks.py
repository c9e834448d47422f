#!/usr/bin/env python3
"""Writes tests/golden/blocks.txt: hand-chosen block fields packed into bytes.

    python tests/golden/pack_blocks.py          # rewrite blocks.txt
    python tests/golden/pack_blocks.py --check  # exit 1 if blocks.txt is stale

Each case below names its fields (fp16 scale bit patterns, integer scales and
mins, the code of every weight) and its expected dequantized weights, derived
by hand from the format's formula and written as a closed form per case.  The
packers are plain integer bit placement following the layouts of the block
formats (fp16 fields little-endian); nothing here decodes a block or imports
the oracle, so the oracle's decoders are checked against values that do not
come from them.

The formats are the ones the candle pull request "Metal: 64-token tile for the
quantized matrix-matrix kernel" (section "What changes") lists for its kernel,
plus the 4-bit affine groups of the tiny-llm pull request "perf: Optimize
quantized matmul for small decode batches" (section "Benchmark setup").
"""

import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "blocks.txt")


# ---------------------------------------------------------------------------------------------
# packers: field values -> block bytes

def h16(bits):
    """fp16 bit pattern -> 2 little-endian bytes."""
    assert 0 <= bits < 1 << 16
    return bytes([bits & 0xFF, bits >> 8])


def nibbles(lo, hi):
    """byte i = lo[i] | hi[i] << 4."""
    assert len(lo) == len(hi)
    assert all(0 <= v < 16 for v in lo + hi)
    return bytes(a | (b << 4) for a, b in zip(lo, hi))


def bitstring(fields, width):
    """Little-endian bit string of equal-width fields: field f at bits [width*f, width*(f+1))."""
    v = 0
    for f, x in enumerate(fields):
        assert 0 <= x < 1 << width
        v |= x << (width * f)
    nbytes = (width * len(fields) + 7) // 8
    return v.to_bytes(nbytes, "little")


def pack_q4_0(d, codes):
    assert len(codes) == 32
    return h16(d) + nibbles(codes[:16], codes[16:])


def pack_q8_0(d, q):
    assert len(q) == 32 and all(-128 <= v < 128 for v in q)
    return h16(d) + bytes(v & 0xFF for v in q)


def pack_q4_k(d, dmin, sc, m, codes):
    """sc, m: eight 6-bit values each; codes: 256 4-bit values.  Code bytes: for
    p = 0..3, byte 32p + i holds weight 64p + i (low nibble) and 64p + 32 + i (high)."""
    assert len(sc) == len(m) == 8 and len(codes) == 256
    qs = b"".join(nibbles(codes[64 * p: 64 * p + 32], codes[64 * p + 32: 64 * p + 64]) for p in range(4))
    return h16(d) + h16(dmin) + bitstring(list(sc) + list(m), 6) + qs


def pack_q6_k(d, sc, codes):
    """sc: sixteen int8; codes: 256 6-bit values.  ql[i] (i < 128): low nibbles of
    weights i and i + 128; qh[i] (i < 64): bit pair b holds the top two bits of
    weight i + 64b."""
    assert len(sc) == 16 and len(codes) == 256 and all(0 <= c < 64 for c in codes)
    ql = nibbles([c & 15 for c in codes[:128]], [c & 15 for c in codes[128:]])
    qh = bytes(sum(((codes[i + 64 * b] >> 4) & 3) << (2 * b) for b in range(4)) for i in range(64))
    return h16(d) + bytes(v & 0xFF for v in sc) + ql + qh


def pack_a4g64(scale, bias, codes):
    assert len(codes) == 64
    return h16(scale) + h16(bias) + nibbles(codes[:32], codes[32:])


def pack_q4_1(d, m, codes):
    assert len(codes) == 32
    return h16(d) + h16(m) + nibbles(codes[:16], codes[16:])


def top_bits(codes, bit):
    """32-bit little-endian word whose bit i is bit `bit` of codes[i]."""
    return sum(((c >> bit) & 1) << i for i, c in enumerate(codes)).to_bytes(4, "little")


def pack_q5_0(d, codes):
    assert len(codes) == 32 and all(0 <= c < 32 for c in codes)
    low = [c & 15 for c in codes]
    return h16(d) + top_bits(codes, 4) + nibbles(low[:16], low[16:])


def pack_q5_1(d, m, codes):
    assert len(codes) == 32 and all(0 <= c < 32 for c in codes)
    low = [c & 15 for c in codes]
    return h16(d) + h16(m) + top_bits(codes, 4) + nibbles(low[:16], low[16:])


def pack_q2_k(d, dmin, sc, m, codes):
    """sc, m: sixteen 4-bit values; codes: 256 2-bit values; qs[i] (i < 64) holds weight
    i + 64b in bits 2b..2b+1."""
    assert len(sc) == len(m) == 16 and len(codes) == 256 and all(0 <= c < 4 for c in codes)
    sm = nibbles(list(sc), list(m))
    qs = bytes(sum(codes[i + 64 * b] << (2 * b) for b in range(4)) for i in range(64))
    return h16(d) + h16(dmin) + sm + qs


def pack_q3_k(d, s, codes):
    """s: sixteen 6-bit stored scales (signed scale s - 32); codes: 256 3-bit values.
    ql[i] (i < 64): bits 2b..2b+1 are the low two bits of weight i + 64b; qh[i] (i < 32):
    bit b is the top bit of weight i + 32b."""
    assert len(s) == 16 and len(codes) == 256 and all(0 <= c < 8 for c in codes)
    ql = bytes(sum((codes[i + 64 * b] & 3) << (2 * b) for b in range(4)) for i in range(64))
    qh = bytes(sum(((codes[i + 32 * b] >> 2) & 1) << b for b in range(8)) for i in range(32))
    return h16(d) + bitstring(list(s), 6) + ql + qh


def pack_q5_k(d, dmin, sc, m, codes):
    """As Q4_K with 5-bit codes: qh[i] (i < 32) bit b is the top bit of weight i + 32b."""
    assert len(sc) == len(m) == 8 and len(codes) == 256 and all(0 <= c < 32 for c in codes)
    low = [c & 15 for c in codes]
    qh = bytes(sum(((codes[i + 32 * b] >> 4) & 1) << b for b in range(8)) for i in range(32))
    qs = b"".join(nibbles(low[64 * p: 64 * p + 32], low[64 * p + 32: 64 * p + 64]) for p in range(4))
    return h16(d) + h16(dmin) + bitstring(list(sc) + list(m), 6) + qh + qs


# ---------------------------------------------------------------------------------------------
# cases: (name, fmt, comment, bytes, scale text, expected integers)

def rep(v, n):
    return [v] * n


def cases():
    out = []

    def add(name, fmt, comment, data, scale, ints):
        out.append((name, fmt, comment, data, scale, ints))

    # Q4_0: w = d * (q - 8)
    codes = list(range(16)) + [15 - i for i in range(16)]
    add("q4_0_unit_scale_codes_ascending_then_descending", "q4_0",
        "d=1; weights 0..15 have codes 0..15, weights 16..31 codes 15..0",
        pack_q4_0(0x3C00, codes), "1", [c - 8 for c in codes])
    add("q4_0_negative_scale", "q4_0", "d=-0.5, every code 3: w = -0.5*(3-8) = 2.5",
        pack_q4_0(0xB800, rep(3, 32)), "0.5", rep(5, 32))
    codes = [0] + rep(15, 31)
    add("q4_0_subnormal_scale", "q4_0", "d=2^-24 (smallest fp16 subnormal); weight 0 code 0, all others code 15",
        pack_q4_0(0x0001, codes), "2**-24", [c - 8 for c in codes])
    add("q4_0_zero_scale", "q4_0", "d=0; low nibbles 2, high nibbles 1",
        pack_q4_0(0x0000, rep(2, 16) + rep(1, 16)), "1", rep(0, 32))

    # Q8_0: w = d * q
    q = [i - 16 for i in range(32)]
    add("q8_0_signed_codes", "q8_0", "d=0.25, q[i] = i-16", pack_q8_0(0x3400, q), "0.25", q)
    q = [127, -128] + rep(1, 30)
    add("q8_0_extreme_codes", "q8_0", "d=1; codes 127, -128, then 1", pack_q8_0(0x3C00, q), "1", q)
    add("q8_0_negative_subnormal_scale", "q8_0", "d=-3*2^-24, every code 2",
        pack_q8_0(0x8003, rep(2, 32)), "2**-24", rep(-6, 32))

    # Q4_K: w = d*sc_j*q - dmin*m_j, j = weight // 32
    sub = lambda j: 10 if j % 2 == 0 else 5  # noqa: E731  (low nibble 10, high nibble 5)
    codes = [sub(i // 32) for i in range(256)]
    add("q4_k_scale_and_min_per_subblock", "q4_k",
        "d=1, dmin=1, sc_j=j+1, m_j=j; every code byte 0x5a: code 10 in even sub-blocks, 5 in odd "
        "ones; w = (j+1)*code - j",
        pack_q4_k(0x3C00, 0x3C00, [j + 1 for j in range(8)], list(range(8)), codes), "1",
        [(i // 32 + 1) * codes[i] - i // 32 for i in range(256)])
    codes = []
    for p in range(4):
        codes += [(i + p) % 16 for i in range(32)] + [(31 - i) % 16 for i in range(32)]
    add("q4_k_code_positions", "q4_k",
        "d=1, dmin=0, sc_j=1, m_j=0: w = q.  code byte 32p+i = ((i+p)%16) | ((31-i)%16)<<4",
        pack_q4_k(0x3C00, 0x0000, rep(1, 8), rep(0, 8), codes), "1", codes)
    sc = [0, 0, 0, 0, 0, 63, 0, 0]
    m = [0, 0, 37, 0, 0, 0, 0, 0]
    add("q4_k_single_fields", "q4_k",
        "d=2, dmin=0.5, only sc_5=63 and m_2=37 nonzero, every code 15: sub-block 5 2*63*15 = 1890, "
        "sub-block 2 -0.5*37 = -18.5, others 0",
        pack_q4_k(0x4000, 0x3800, sc, m, rep(15, 256)), "0.5",
        rep(0, 64) + rep(-37, 32) + rep(0, 64) + rep(3780, 32) + rep(0, 64))
    add("q4_k_single_rounding_ties_to_even", "q4_k",
        "d=2048, dmin=2^-11, sc_0=sc_1=8, m_0=1, m_1=3, code 1 in sub-blocks 0 and 1, 0 elsewhere. "
        "Sub-block 0: 2^14 - 2^-11 is halfway between the fp32 neighbours 2^14-2^-10 and 2^14 -> even: "
        "2^14.  Sub-block 1: 2^14 - 3*2^-11 is halfway between 2^14-2^-10 and 2^14-2^-9 -> even: 2^14-2^-9",
        pack_q4_k(0x6800, 0x1000, [8, 8] + rep(0, 6), [1, 3] + rep(0, 6), rep(1, 64) + rep(0, 192)),
        "2**-9", rep(8388608, 32) + rep(8388607, 32) + rep(0, 192))
    add("q4_k_fp16_staging_double_rounding", "q4_k",
        "d=1025*2^-9 (fp16 0x4001), dmin=381*2^-24 (subnormal), sc_0=1, m_0=43, weight 0 code 1, "
        "other codes 0, other sub-blocks zero.  Weight 0: exact 2+2^-10+2^-24 (33570817 units of "
        "2^-24) rounds in fp32 to 2+2^-10 (33570816); weights 1..31: -381*43 = -16383 units.  The fp16 "
        "rounding of the fp32 weight 2+2^-10 is a tie -> 2.0, while one rounding of the exact value "
        "would give 2+2^-9",
        pack_q4_k(0x4001, 0x017D, [1] + rep(0, 7), [43] + rep(0, 7), [1] + rep(0, 255)),
        "2**-24", [33570816] + rep(-16383, 31) + rep(0, 224))

    # Q6_K: w = d*sc_j*(q-32), j = weight // 16
    add("q6_k_signed_scales", "q6_k",
        "d=1, sc_j = j-8, every code 0: w = (j-8)*(0-32) = 256-32j per 16-weight sub-block "
        "(sc=-3 gives +96)",
        pack_q6_k(0x3C00, [j - 8 for j in range(16)], rep(0, 256)), "1",
        [256 - 32 * (i // 16) for i in range(256)])
    codes = [(i + 17 * (i // 64)) % 64 for i in range(256)]
    add("q6_k_code_positions", "q6_k", "d=0.5, sc_j=1, code of weight i = (i + 17*(i//64)) % 64: w = 0.5*(code-32)",
        pack_q6_k(0x3800, rep(1, 16), codes), "0.5", [c - 32 for c in codes])
    add("q6_k_extreme_scales", "q6_k",
        "d=1, sc_0=127 with code 63 (weights 0..15), sc_1=-128 with code 0 (weights 16..31), other "
        "sc 0: 127*31 = 3937 ; -128*-32 = 4096",
        pack_q6_k(0x3C00, [127, -128] + rep(0, 14), rep(63, 16) + rep(0, 240)), "1",
        rep(3937, 16) + rep(4096, 16) + rep(0, 224))

    # A4G64: w = scale*q + bias
    codes = [i % 16 for i in range(32)] + [15 - (i % 16) for i in range(32)]
    add("a4g64_scale_and_bias", "a4g64",
        "scale=0.5, bias=-4; weights 0..31 codes i%16, weights 32..63 codes 15-(i%16)",
        pack_a4g64(0x3800, 0xC400, codes), "0.5", [c - 8 for c in codes])
    add("a4g64_single_rounding_ties_to_even", "a4g64",
        "scale=2048, bias=3*2^-10; code 8 (weights 0..31): 2^14 + 1.5*2^-9 is halfway between "
        "2^14+2^-9 and 2^14+2^-8 -> even: 2^14+2^-8 ; code 0 (weights 32..63): exactly 3*2^-10",
        pack_a4g64(0x6800, 0x1A00, rep(8, 32) + rep(0, 32)), "2**-10", rep(16777220, 32) + rep(3, 32))
    add("a4g64_fp16_staging_double_rounding", "a4g64",
        "scale=683/1024 (fp16 0x3956), bias=2^-24; weight 0 code 3, others 0.  Weight 0: exact "
        "2049/1024 + 2^-24 = 33570817 units of 2^-24, fp32 2+2^-10 (33570816); fp16 staging of that is "
        "a tie -> 2.0, one rounding of the exact value would give 2+2^-9.  Others: the bias, 1 unit",
        pack_a4g64(0x3956, 0x0001, [3] + rep(0, 63)), "2**-24", [33570816] + rep(1, 63))

    # Q4_1: w = d*q + m
    codes = [i % 16 for i in range(16)] + [15 - (i % 16) for i in range(16)]
    add("q4_1_scale_and_min", "q4_1", "d=0.5, m=-4; weights 0..15 codes 0..15, weights 16..31 codes 15..0",
        pack_q4_1(0x3800, 0xC400, codes), "0.5", [c - 8 for c in codes])
    add("q4_1_single_rounding_ties_to_even", "q4_1",
        "d=2048, m=3*2^-10; code 8 (weights 0..15): 2^14 + 1.5*2^-9 is halfway between 2^14+2^-9 and "
        "2^14+2^-8 -> even: 2^14+2^-8 ; code 0 (weights 16..31): exactly 3*2^-10",
        pack_q4_1(0x6800, 0x1A00, rep(8, 16) + rep(0, 16)), "2**-10", rep(16777220, 16) + rep(3, 16))
    add("q4_1_fp16_staging_double_rounding", "q4_1",
        "d=683/1024 (fp16 0x3956), m=2^-24; weight 0 code 3, others 0: exact 33570817 units of 2^-24, "
        "fp32 33570816 (2+2^-10, an fp16 tie -> 2.0 when staged); others the minimum, 1 unit",
        pack_q4_1(0x3956, 0x0001, [3] + rep(0, 31)), "2**-24", [33570816] + rep(1, 31))
    add("q4_1_negative_subnormal_scale", "q4_1", "d=-3*2^-24, m=2^-14; code 15 everywhere: -45 + 1024 units",
        pack_q4_1(0x8003, 0x0400, rep(15, 32)), "2**-24", rep(979, 32))

    # Q5_0: w = d*(q-16)
    codes = list(range(32))
    add("q5_0_codes_and_top_bits", "q5_0", "d=1; weight i has code i (top bit set from weight 16 on): w = i-16",
        pack_q5_0(0x3C00, codes), "1", [c - 16 for c in codes])
    codes = [(7 * i + 3) % 32 for i in range(32)]
    add("q5_0_scattered_top_bits", "q5_0", "d=0.25; code of weight i = (7i+3) % 32: w = 0.25*(code-16)",
        pack_q5_0(0x3400, codes), "0.25", [c - 16 for c in codes])
    add("q5_0_negative_subnormal_scale", "q5_0", "d=-3*2^-24, every code 31: w = -3*15 units",
        pack_q5_0(0x8003, rep(31, 32)), "2**-24", rep(-45, 32))

    # Q5_1: w = d*q + m
    codes = [(11 * i) % 32 for i in range(32)]
    add("q5_1_scale_and_min", "q5_1", "d=0.25, m=-1; code of weight i = 11i % 32: w = 0.25*code - 1",
        pack_q5_1(0x3400, 0xBC00, codes), "0.25", [c - 4 for c in codes])
    add("q5_1_fp16_staging_double_rounding", "q5_1",
        "d=683/1024 (fp16 0x3956), m=2^-24; weight 0 code 3, weight 1 code 19 (top bit), others 0.  "
        "Weight 0: fp32 2+2^-10, an fp16 tie; weight 1: 19*683/1024 + 2^-24 = 212615169 units -> fp32 "
        "212615168 (ulp 16 units); others 1 unit",
        pack_q5_1(0x3956, 0x0001, [3, 19] + rep(0, 30)), "2**-24", [33570816, 212615168] + rep(1, 30))

    # Q2_K: w = d*sc_j*q - dmin*m_j, j = weight // 16
    codes = [(i + i // 64) % 4 for i in range(256)]
    add("q2_k_scale_and_min_per_subblock", "q2_k",
        "d=1, dmin=1, sc_j=j, m_j=15-j, code of weight i = (i + i//64) % 4: w = j*code - (15-j)",
        pack_q2_k(0x3C00, 0x3C00, list(range(16)), [15 - j for j in range(16)], codes), "1",
        [(i // 16) * codes[i] - (15 - i // 16) for i in range(256)])
    add("q2_k_single_rounding_ties_to_even", "q2_k",
        "d=2048, dmin=2^-11, sc_0=8, m_0=1, code 1 in sub-block 0, other sub-blocks zero: "
        "2^14 - 2^-11 is halfway between 2^14-2^-10 and 2^14 -> even: 2^14",
        pack_q2_k(0x6800, 0x1000, [8] + rep(0, 15), [1] + rep(0, 15), rep(1, 16) + rep(0, 240)),
        "2**-9", rep(8388608, 16) + rep(0, 240))
    add("q2_k_fp16_staging_double_rounding", "q2_k",
        "d=1+2^-10 (0x3c01), dmin=2^-24, sc_0=1, m_0=1, weight 0 code 3, other codes 0, other "
        "sub-blocks zero.  Weight 0: exact 3+3*2^-10-2^-24 rounds in fp32 to 3+3*2^-10 "
        "(50380800 units of 2^-24), an fp16 tie -> 3+2^-8 when staged, while one rounding of the "
        "exact value would give 3+2^-9; weights 1..15: -1 unit",
        pack_q2_k(0x3C01, 0x0001, [1] + rep(0, 15), [1] + rep(0, 15), [3] + rep(0, 255)),
        "2**-24", [50380800] + rep(-1, 15) + rep(0, 240))

    # Q3_K: w = d*(s_j-32)*(q-4), j = weight // 16
    add("q3_k_signed_scales", "q3_k", "d=1, stored s_j = 24+j (signed j-8), every code 0: w = (j-8)*(-4) = 32-4j",
        pack_q3_k(0x3C00, [24 + j for j in range(16)], rep(0, 256)), "1",
        [32 - 4 * (i // 16) for i in range(256)])
    codes = [(i + 3 * (i // 64)) % 8 for i in range(256)]
    add("q3_k_code_positions", "q3_k", "d=0.5, every stored s_j = 33 (signed 1), code of weight i = "
        "(i + 3*(i//64)) % 8: w = 0.5*(code-4)",
        pack_q3_k(0x3800, rep(33, 16), codes), "0.5", [c - 4 for c in codes])
    add("q3_k_extreme_scales", "q3_k", "d=1, s_0 = 0 (signed -32) with code 0: 128 ; s_1 = 63 (signed 31) with "
        "code 7: 93 ; other stored scales 32 (signed 0)",
        pack_q3_k(0x3C00, [0, 63] + rep(32, 14), rep(0, 16) + rep(7, 16) + rep(0, 224)), "1",
        rep(128, 16) + rep(93, 16) + rep(0, 224))
    add("q3_k_negative_subnormal_scale", "q3_k", "d=-2^-24, stored s_j = 40 (signed 8), every code 7: -24 units",
        pack_q3_k(0x8001, rep(40, 16), rep(7, 256)), "2**-24", rep(-24, 256))

    # Q5_K: w = d*sc_j*q - dmin*m_j, j = weight // 32
    codes = [(i + 5 * (i // 32)) % 32 for i in range(256)]
    add("q5_k_scale_and_min_per_subblock", "q5_k",
        "d=1, dmin=1, sc_j=j+1, m_j=j; code of weight i = (i + 5*(i//32)) % 32: w = (j+1)*code - j",
        pack_q5_k(0x3C00, 0x3C00, [j + 1 for j in range(8)], list(range(8)), codes), "1",
        [(i // 32 + 1) * codes[i] - i // 32 for i in range(256)])
    add("q5_k_fp16_staging_double_rounding", "q5_k",
        "d=1025*2^-9 (0x4001), dmin=381*2^-24, sc_0=1, m_0=43, weight 0 code 1, other codes 0, other "
        "sub-blocks zero: as the Q4_K case, weight 0 fp32 2+2^-10 (an fp16 tie), weights 1..31 -16383 units",
        pack_q5_k(0x4001, 0x017D, [1] + rep(0, 7), [43] + rep(0, 7), [1] + rep(0, 255)),
        "2**-24", [33570816] + rep(-16383, 31) + rep(0, 224))
    add("q5_k_top_bits_only", "q5_k", "d=2, dmin=0, sc_j=1, m_j=0, every code 16 (only the top bit): w = 32",
        pack_q5_k(0x4000, 0x0000, rep(1, 8), rep(0, 8), rep(16, 256)), "1", rep(32, 256))
    return out


HEADER = """\
# Hand-built blocks with hand-derived dequantized values, one per case.
# WRITTEN BY tests/golden/pack_blocks.py -- edit the cases there and rerun it.
#
# The pages name the block formats without printing a layout: the candle pull
# request "Metal: 64-token tile for the quantized matrix-matrix kernel",
# section "What changes", lists Q4_0, Q8_0, Q4_K and Q6_K among the types its
# kernel serves; the tiny-llm pull request "perf: Optimize quantized matmul for
# small decode batches", section "Benchmark setup", runs an MLX 4-bit model
# (4-bit codes with a scale and a bias per group; here groups of 64, A4G64).
# The section also lists Q4_1, Q5_0, Q5_1, Q2_K, Q3_K and Q5_K, whose formulas are
# read from their names (documented with the oracle).
# Formulas and byte layouts are this library's (documented with the oracle):
#   Q4_0  w = d*(q-8)          Q8_0  w = d*q          A4G64  w = scale*q + bias
#   Q4_1  w = d*q + m          Q5_0  w = d*(q-16)     Q5_1   w = d*q + m
#   Q4_K  w = d*sc_j*q - dmin*m_j   (6-bit sc/m in a 96-bit little-endian string)
#   Q5_K  as Q4_K with a fifth code bit (qh)
#   Q2_K  w = d*sc_j*q - dmin*m_j   (4-bit sc/m per 16 weights; 2-bit codes)
#   Q3_K  w = d*(s_j-32)*(q-4)      (6-bit s per 16 weights; 2+1-bit codes)
#   Q6_K  w = d*sc_j*(q-32)         (int8 sc per 16 weights; 4+2-bit codes)
# Each case: the block's bytes (hex, packed from the field values in the
# comment by plain integer bit placement), then the expected weights as
# integers times an exact power-of-two scale ("v*n" repeats v n times), derived
# by hand from the formula.
"""


def render():
    lines = [HEADER]
    for name, fmt, comment, data, scale, ints in cases():
        lines.append(f"case {name}")
        lines.append(f"fmt {fmt}")
        lines.append(f"# {comment}")
        lines.append("hex " + data.hex())
        lines.append(f"scale {scale}")
        toks, i = [], 0
        while i < len(ints):
            j = i
            while j < len(ints) and ints[j] == ints[i]:
                j += 1
            toks.append(str(ints[i]) if j - i == 1 else f"{ints[i]}*{j - i}")
            i = j
        lines.append("ints " + " ".join(toks))
        lines.append("end")
        lines.append("")
    return "\n".join(lines)


def main():
    text = render()
    if "--check" in sys.argv:
        cur = open(OUT).read() if os.path.exists(OUT) else ""
        if cur != text:
            print(f"{OUT} is stale: rerun {os.path.basename(__file__)}", file=sys.stderr)
            sys.exit(1)
        return
    with open(OUT, "w") as f:
        f.write(text)
    print(f"wrote {OUT} ({len(cases())} cases)")


if __name__ == "__main__":
    main()
