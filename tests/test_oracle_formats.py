"""Pins of the oracle's block decoders (CPU only).

* hand-built blocks with hand-derived values (tests/golden/blocks.txt):
  every field, nibble half, bit position and sign convention of each layout,
  subnormal and zero scales, and the single fp32 rounding (ties to even) of
  the Q4_K and A4G64 add/subtract;
* round trips through the synthetic-data encoders, with the error bound each
  encoder guarantees (a misplaced nibble or scale breaks the bound by orders
  of magnitude);
* structural invariants on random bytes.
"""

import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from qmm_synth import quantize
from tests.golden_io import GOLDEN, read_blocks

CASES = read_blocks()
# byte offsets of each format's fp16 scale fields
SCALE_OFFSETS = {"q4_0": [0], "q8_0": [0], "q4_k": [0, 2], "q6_k": [0], "a4g64": [0, 2], "q4_1": [0, 2],
                 "q5_0": [0], "q5_1": [0, 2], "q2_k": [0, 2], "q3_k": [0], "q5_k": [0, 2]}


def test_golden_covers_every_format():
    assert {c["fmt"] for c in CASES} == set(oracle.FORMATS)


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_golden_block(case):
    fmt = case["fmt"]
    assert len(case["data"]) == oracle.block_bytes(fmt)
    assert len(case["expect"]) == oracle.block_weights(fmt)
    got = oracle.dequantize_blocks(fmt, np.frombuffer(case["data"], dtype=np.uint8))[0]
    assert got.dtype == np.float32
    for i, (g, e) in enumerate(zip(got.tolist(), case["expect"])):
        # every expected value is an exact dyadic rational representable in fp32;
        # compare by value so +0 == -0
        assert Fraction(g) == e, f"{case['name']}: weight {i}: got {g}, expected {float(e)}"


def test_block_geometry():
    assert oracle.FORMATS == {
        "q4_0": (32, 18), "q8_0": (32, 34), "q4_k": (256, 144), "q6_k": (256, 210), "a4g64": (64, 36),
        "q4_1": (32, 20), "q5_0": (32, 22), "q5_1": (32, 24), "q2_k": (256, 84), "q3_k": (256, 110),
        "q5_k": (256, 176)}
    # bits per weight: 4.5, 8.5, 4.5, 6.5625, 4.5, 5, 5.5, 6, 2.625, 3.4375, 5.5
    assert oracle.row_bytes("q2_k", 2560) == 840 and oracle.row_bytes("q3_k", 2560) == 1100
    assert oracle.row_bytes("q5_k", 2560) == 1760 and oracle.row_bytes("q5_0", 512) == 352
    assert oracle.row_bytes("q4_0", 512) == 288
    assert oracle.row_bytes("q4_k", 2560) == 1440
    assert oracle.row_bytes("q6_k", 9728) == 7980
    assert oracle.row_bytes("a4g64", 1024) == 576
    assert oracle.row_bytes("q8_0", 768) == 816
    for fmt in oracle.FORMATS:
        assert oracle.row_bytes(fmt, 0) == 0
        assert oracle.row_bytes(fmt, oracle.block_weights(fmt) + 16) == 0


def test_dequantize_matrix_row_order():
    # Two rows with different scales: row r must start at byte r*row_bytes.
    b0 = bytes.fromhex("003c" + "88" * 16)   # d=1, code 8 everywhere -> 0
    b1 = bytes.fromhex("0040" + "99" * 16)   # d=2, code 9 everywhere -> 2
    blob = np.frombuffer(b0 + b0 + b1 + b1, dtype=np.uint8)
    w = oracle.dequantize("q4_0", blob, 2, 64)
    assert w.shape == (2, 64)
    assert np.all(w[0] == 0) and np.all(w[1] == 2)


def _bound(fmt, blocks_u8, w_true, w_hat):
    """Per-weight error bound the encoder guarantees (see qmm_synth.quantize)."""
    bw, bb = oracle.FORMATS[fmt]
    nb = blocks_u8.size // bb
    blk = blocks_u8.reshape(nb, bb)
    f16 = lambda off: (blk[:, off].astype(np.uint16) | (blk[:, off + 1].astype(np.uint16) << 8)).view(np.float16).astype(np.float64)
    rel = 1 + 2.0 ** -20
    if fmt == "q4_0":
        d = np.abs(f16(0))[:, None]
        qs = blk[:, 2:18]
        q = np.concatenate([qs & 15, qs >> 4], axis=1)
        return np.where(q == 15, d * (1 + 2.0 ** -7), d / 2 * rel)
    if fmt == "q8_0":
        return np.repeat(np.abs(f16(0))[:, None] / 2 * rel, 32, axis=1)
    if fmt == "a4g64":
        return np.repeat(f16(0)[:, None] / 2 * rel, 64, axis=1) + 2.0 ** -24 * np.abs(w_hat.reshape(nb, 64))
    if fmt == "q4_k":
        raw = blk[:, 4:16].astype(np.int64)
        bits = sum(raw[:, i] << (8 * i) for i in range(12))
        sc = np.stack([(bits >> (6 * j)) & 63 for j in range(8)], axis=1).astype(np.float64)
        step = f16(0)[:, None] * sc
        return np.repeat(step / 2 * rel, 32, axis=1) + 2.0 ** -24 * np.abs(w_hat.reshape(nb, 256))
    if fmt == "q6_k":
        sc = np.abs(blk[:, 2:18].view(np.int8).astype(np.float64))
        return np.repeat(f16(0)[:, None] * sc / 2 * rel, 16, axis=1)
    if fmt in ("q4_1", "q5_1"):
        return np.repeat(f16(0)[:, None] / 2 * rel, 32, axis=1) + 2.0 ** -24 * np.abs(w_hat.reshape(nb, 32))
    if fmt == "q5_0":
        d = np.abs(f16(0))[:, None]
        qs = blk[:, 6:22]
        qh = sum(blk[:, 2 + b].astype(np.int64) << (8 * b) for b in range(4))
        q = np.concatenate([qs & 15, qs >> 4], axis=1) | (((qh[:, None] >> np.arange(32)) & 1) << 4)
        return np.where(q == 31, d * (1 + 2.0 ** -7), d / 2 * rel)
    if fmt == "q2_k":
        sc = (blk[:, 4:20] & 15).astype(np.float64)
        step = f16(0)[:, None] * sc
        return np.repeat(step / 2 * rel, 16, axis=1) + 2.0 ** -24 * np.abs(w_hat.reshape(nb, 256))
    if fmt == "q3_k":
        bits = [int.from_bytes(bytes(row), "little") for row in blk[:, 2:14]]   # 96-bit strings
        s = np.array([[((b >> (6 * j)) & 63) - 32 for j in range(16)] for b in bits], np.float64)
        step = np.repeat(np.abs(f16(0)[:, None] * s), 16, axis=1)
        code = np.divide(w_hat.reshape(nb, 256), np.where(step == 0, 1, np.repeat(f16(0)[:, None] * s, 16, axis=1)))
        # the far end of the codes (+3) may hold a clamped value: one full step there
        return np.where(np.abs(code - 3) < 1e-9, step * rel, step / 2 * rel)
    if fmt == "q5_k":
        raw = blk[:, 4:16].astype(np.int64)
        bits = sum(raw[:, i] << (8 * i) for i in range(12))
        sc = np.stack([(bits >> (6 * j)) & 63 for j in range(8)], axis=1).astype(np.float64)
        step = f16(0)[:, None] * sc
        return np.repeat(step / 2 * rel, 32, axis=1) + 2.0 ** -24 * np.abs(w_hat.reshape(nb, 256))
    raise AssertionError(fmt)


@pytest.mark.parametrize("fmt", list(oracle.FORMATS))
@pytest.mark.parametrize("dist", ["normal", "uniform_pos", "all_negative", "spiky", "constant", "zeros"])
def test_round_trip_bound(fmt, dist):
    g = np.random.default_rng([7, list(oracle.FORMATS).index(fmt), len(dist)])
    M, K = 6, 512
    if dist == "normal":
        w = g.normal(0, 0.02, (M, K))
    elif dist == "uniform_pos":
        w = g.uniform(0.001, 3.0, (M, K))
    elif dist == "all_negative":
        w = -g.uniform(0.5, 2.0, (M, K))
    elif dist == "spiky":
        w = g.normal(0, 1e-3, (M, K))
        w[:, ::37] = 5.0
    elif dist == "constant":
        w = np.full((M, K), 0.3125)
    else:
        w = np.zeros((M, K))
    w = w.astype(np.float32)
    blob = quantize(fmt, w)
    assert blob.size == M * oracle.row_bytes(fmt, K)
    w_hat = oracle.dequantize(fmt, blob, M, K)
    err = np.abs(w.astype(np.float64) - w_hat.astype(np.float64)).reshape(-1, oracle.block_weights(fmt))
    bound = _bound(fmt, blob, w, w_hat)
    assert np.all(err <= bound + 1e-30), f"max excess {np.max(err - bound)}"


def test_q4_0_extreme_maps_to_code_zero():
    # d = w*/-8 sends the largest-magnitude element to code 0 exactly (d*(0-8) = w*).
    w = np.zeros((1, 32), np.float32)
    w[0, 5] = -1.0
    w[0, 7] = 0.5
    blob = quantize("q4_0", w)
    w_hat = oracle.dequantize("q4_0", blob, 1, 32)
    assert w_hat[0, 5] == -1.0 and w_hat[0, 7] == 0.5


def test_quantizer_deterministic():
    w = np.random.default_rng(3).normal(0, 0.02, (8, 768)).astype(np.float32)
    for fmt in ("q4_0", "q8_0", "q4_k", "q6_k", "a4g64"):
        K = 768
        assert np.array_equal(quantize(fmt, w[:, :K]), quantize(fmt, w[:, :K].copy()))


@pytest.mark.parametrize("fmt", list(oracle.FORMATS))
def test_random_bytes_structure(fmt):
    """On arbitrary bytes the decoded weight divided by its block scale is an integer
    of the format's code range (Q4_0, Q8_0, Q6_K), and results are finite."""
    bw, bb = oracle.FORMATS[fmt]
    g = np.random.default_rng([11, bb])
    blk = g.integers(0, 256, size=(64, bb), dtype=np.uint8)
    # keep fp16 scale fields finite and normal-sized
    for off in SCALE_OFFSETS[fmt]:
        blk[:, off + 1] &= 0x3B
    w = oracle.dequantize_blocks(fmt, blk).astype(np.float64)
    assert np.all(np.isfinite(w))
    d = (blk[:, 0].astype(np.uint16) | (blk[:, 1].astype(np.uint16) << 8)).view(np.float16).astype(np.float64)[:, None]
    nz = d[:, 0] != 0
    if fmt == "q4_0":
        r = w[nz] / d[nz]
        assert np.all(r == np.round(r)) and r.min() >= -8 and r.max() <= 7
    elif fmt == "q8_0":
        r = w[nz] / d[nz]
        assert np.all(r == np.round(r)) and r.min() >= -128 and r.max() <= 127
    elif fmt == "q6_k":
        r = w[nz] / d[nz]
        assert np.all(r == np.round(r)) and np.abs(r).max() <= 4096
    elif fmt == "q5_0":
        r = w[nz] / d[nz]
        assert np.all(r == np.round(r)) and r.min() >= -16 and r.max() <= 15
        assert r.min() == -16 and r.max() == 15       # the top bit reaches both ends on random bytes
    elif fmt == "q3_k":
        r = w[nz] / d[nz]
        assert np.all(r == np.round(r)) and np.abs(r).max() <= 128
    elif fmt in ("q4_1", "q5_1"):
        # (w - m) / d is a code 0..15 or 0..31 wherever the add was exact
        m = (blk[:, 2].astype(np.uint16) | (blk[:, 3].astype(np.uint16) << 8)).view(np.float16).astype(np.float64)
        r = (w - m[:, None])[nz] / d[nz]
        near = np.abs(r - np.round(r)) < 1e-3
        assert near.mean() > 0.9 and np.round(r[near]).max() <= (15 if fmt == "q4_1" else 31)


# --- the fp16 staging value of the matrix-matrix path -----------------------------------------
# staged_fp16 is the fp16 round-to-nearest-even (ties to even) of the fp32 dequantized weight.
# Pins from the IEEE binary16 grid: ulp 2^-10 in [1, 2), 2^-9 in [2, 4), subnormal step 2^-24,
# largest finite 65504 (the next value up would be 65536, so 65520 is the overflow tie).

STAGING_PINS = [
    (1.0 + 2.0 ** -11, 1.0),                  # tie below an even significand -> down
    (1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -9),  # tie above an odd significand -> up (to even)
    (1.0 + 2.0 ** -11 + 2.0 ** -20, 1.0 + 2.0 ** -10),  # just above the tie -> up
    (2.0 + 2.0 ** -10, 2.0),                  # the staging tie of the double-rounding golden blocks
    (-(2.0 + 3 * 2.0 ** -10), -(2.0 + 2.0 ** -8)),
    (2.0 ** -25, 0.0),                        # half the smallest subnormal: tie to even zero
    (3 * 2.0 ** -25, 2.0 ** -23),             # 1.5 subnormal steps -> 2 steps
    (2.0 ** -24, 2.0 ** -24),                 # subnormals are kept, not flushed
    (1023 * 2.0 ** -24, 1023 * 2.0 ** -24),
    (65504.0, 65504.0),
    (65519.0, 65504.0),                       # below the overflow tie
    (65520.0, float("inf")),                  # the overflow tie rounds to infinity
    (-65520.0, float("-inf")),
]


@pytest.mark.parametrize("w,expect", STAGING_PINS)
def test_staged_fp16_pins(w, expect):
    w32 = np.float32(w)
    assert float(w32) == w  # every input above is an fp32 value
    got = oracle.staged_fp16(np.array([w32]))
    assert got.dtype == np.float16
    assert float(got[0]) == expect


def test_staged_fp16_keeps_signed_zero():
    got = oracle.staged_fp16(np.array([-0.0, 0.0, -2.0 ** -26], np.float32))
    assert np.signbit(got).tolist() == [True, False, True]
    assert got.tolist() == [0.0, 0.0, 0.0]


def test_staged_fp16_of_double_rounding_blocks():
    # the golden blocks built so that rounding the exact weight once to fp16 would give
    # another value than staging does: staging rounds the fp32 weight (an fp16 tie) to even
    cases = [c for c in CASES if c["name"].endswith("_fp16_staging_double_rounding")]
    assert {c["fmt"] for c in cases} == {"q4_k", "a4g64", "q4_1", "q5_1", "q2_k", "q5_k"}
    for case in cases:
        w = oracle.dequantize_blocks(case["fmt"], np.frombuffer(case["data"], np.uint8))[0]
        if case["fmt"] == "q2_k":
            # exact 3 + 3*2^-10 - 2^-24 -> fp32 3 + 3*2^-10, between 3+2^-9 and 3+2^-8
            tie, exact, even, one_rounding = 3 + 3 * 2.0 ** -10, Fraction(3) + Fraction(3, 1024) - Fraction(1, 2 ** 24), \
                3 + 2.0 ** -8, 3 + 2.0 ** -9
        else:
            # exact 2 + 2^-10 (+ or -) 2^-24 -> fp32 2 + 2^-10, between 2 and 2+2^-9
            tie, exact, even, one_rounding = 2 + 2.0 ** -10, None, 2.0, 2 + 2.0 ** -9
        assert float(w[0]) == tie
        assert float(oracle.staged_fp16(w)[0]) == even
        if exact is not None:
            assert float(np.float16(float(exact))) == one_rounding


def test_golden_file_matches_its_packer():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(GOLDEN, "pack_blocks.py"), "--check"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
