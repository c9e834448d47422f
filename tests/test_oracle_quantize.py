"""Pins of the oracle's reference quantizers (CPU only).

* hand-derived bytes: all-zero blocks of every format, exactly representable
  ramps (every code 0..15 at a known scale), the first-on-a-tie rule of Q4_0;
* the fp16 rounding helpers against fp16 neighbours;
* round trips within each format's error bound, on several distributions
  (the bound is computed from the block's own scales, so a misplaced nibble,
  bit pair or scale breaks it by orders of magnitude);
* agreement with the independently written test-data encoders."""

import importlib
import struct

import numpy as np
import pytest

import oracle
from oracle import quantize as oq
from oracle.quantize import QUANT_FORMATS
from tests.test_oracle_formats import _bound

encoders = importlib.import_module("qmm_synth.quantize")


def _h(v):
    return struct.unpack("<H", struct.pack("<e", v))[0]


def test_f16_helpers():
    third = 1.0 / 3.0
    up, down, near = oq.f16_up(third), oq.f16_down(third), oq.f16_rne(third)
    assert up == down + 1 and near in (up, down)
    assert struct.unpack("<e", struct.pack("<H", down))[0] < third < struct.unpack("<e", struct.pack("<H", up))[0]
    for exact in (0.0, 0.25, -3.5, 65504.0, 2.0 ** -24):
        assert oq.f16_up(exact) == oq.f16_down(exact) == _h(exact)
    assert oq.f16_up(1e-9) == 0x0001 and oq.f16_down(-1e-9) == 0x8001
    assert oq.f16_up(-1e-9) in (0x8000, 0x0000) and oq.f16_down(1e-9) == 0x0000
    assert oq.rha(2.5) == 3.0 and oq.rha(-2.5) == -3.0 and oq.rha(2.49) == 2.0 and oq.rha(0.0) == 0.0


@pytest.mark.parametrize("fmt", list(QUANT_FORMATS))
def test_zero_blocks(fmt):
    blob = oracle.quantize_blocks(fmt, np.zeros((1, oracle.block_weights(fmt)), np.float32))
    expect = {
        "q4_0": [0x00, 0x80] + [0x88] * 16,            # d = 0 / -8 = -0, every code 8
        "q8_0": [0] * 34,
        "q4_k": [0, 0, 0x00, 0x80] + [0] * 140,        # d = 0, dmin = -(0) / 63 = -0, scales and codes 0
        "q6_k": [0] * 146 + [0xAA] * 64,               # codes 32: high pair 2 in every slot
        "a4g64": [0] * 36,
    }[fmt]
    assert blob.tolist() == expect


def test_q4_0_ramp_and_tie():
    w = np.array([[-2.0 + 0.25 * (i % 16) for i in range(32)]], np.float32)  # w* = -2 -> d = 0.25
    blob = oracle.quantize_blocks("q4_0", w).tolist()
    assert blob[:2] == [0x00, 0x34]                     # fp16 0.25
    assert blob[2:] == [c | (c << 4) for c in range(16)]
    # +1 and -1 share the largest magnitude: the first one sets the sign of d
    t = np.zeros((1, 32), np.float32)
    t[0, 3], t[0, 9] = 1.0, -1.0
    b = oracle.quantize_blocks("q4_0", t).tolist()
    assert b[:2] == list(struct.pack("<e", -0.125))


def test_a4g64_ramp():
    w = np.array([[-1.0 + 0.5 * (i % 16) for i in range(64)]], np.float32)  # bias -1, scale 0.5
    blob = oracle.quantize_blocks("a4g64", w).tolist()
    assert blob[:4] == list(struct.pack("<e", 0.5)) + list(struct.pack("<e", -1.0))
    assert blob[4:] == [(i % 16) | ((i % 16) << 4) for i in range(32)]


def test_q8_0_ramp():
    w = np.array([[0.5 * (i - 16) for i in range(32)]], np.float32)  # max|w| = 8 -> d = rne(8/127)
    blob = oracle.quantize_blocks("q8_0", w)
    d = struct.unpack("<e", blob[:2].tobytes())[0]
    assert blob[:2].tolist() == list(struct.pack("<e", 8.0 / 127.0))
    q = blob[2:].view(np.int8).astype(np.float64)
    assert np.all(q == np.sign(w[0]) * np.floor(np.abs(w[0] / d) + 0.5))


@pytest.mark.parametrize("fmt", list(QUANT_FORMATS))
@pytest.mark.parametrize("dist", ["normal", "uniform_pos", "all_negative", "spiky", "constant"])
def test_round_trip_bound(fmt, dist):
    g = np.random.default_rng([8, list(QUANT_FORMATS).index(fmt), len(dist)])
    M, K = 3, 512
    if dist == "normal":
        w = g.normal(0, 0.02, (M, K))
    elif dist == "uniform_pos":
        w = g.uniform(0.001, 3.0, (M, K))
    elif dist == "all_negative":
        w = -g.uniform(0.5, 2.0, (M, K))
    elif dist == "spiky":
        w = g.normal(0, 1e-3, (M, K))
        w[:, ::37] = 5.0
    else:
        w = np.full((M, K), 0.3125)
    w = w.astype(np.float32)
    blob = oracle.quantize_blocks(fmt, w)
    assert blob.size == M * oracle.row_bytes(fmt, K)
    w_hat = oracle.dequantize(fmt, blob, M, K)
    err = np.abs(w.astype(np.float64) - w_hat.astype(np.float64)).reshape(-1, oracle.block_weights(fmt))
    assert np.all(err <= _bound(fmt, blob, w, w_hat) + 1e-30)


@pytest.mark.parametrize("fmt", list(QUANT_FORMATS))
def test_agrees_with_test_data_encoders(fmt):
    w = np.random.default_rng(9).normal(0, 0.5, (4, 512)).astype(np.float32)
    w[1, :64] = 0.0
    assert np.array_equal(oracle.quantize_blocks(fmt, w), encoders.quantize(fmt, w))
