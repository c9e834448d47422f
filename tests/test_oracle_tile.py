"""Pins of the oracle's token-tile rule (CPU only).

Candle pull request "Metal: 64-token tile for the quantized matrix-matrix
kernel": the rule (section "Where the 64-token tile is used"), the pins of its
padding test (section "Same results, bit for bit", the test
mm_tile_for_tokens_follows_padding), and the "chosen" column of the ratio
table (section "Numbers", stored in tests/golden/tile_choice.txt).
"""

import oracle
from tests.golden_io import read_tile_choice


def test_printed_table():
    rows = read_tile_choice()
    assert len(rows) == 27
    for n, mod, chosen in rows:
        assert n % 64 == mod
        assert oracle.tile_for_tokens(n) == chosen, n


def test_restated_rule():
    # "a multiple of 64, or leaves more than 32 over a multiple of 64"; up to 32 tokens: 32
    for n in range(1, 5000):
        expect = 64 if (n % 64 == 0 or n % 64 > 32) else 32
        assert oracle.tile_for_tokens(n) == expect, n
        if n <= 32:
            assert oracle.tile_for_tokens(n) == 32


PINS = {2: 32, 32: 32, 33: 64, 64: 64, 96: 32, 100: 64, 128: 64, 136: 32, 2048: 64}


def test_padding_test_pins():
    for n, t in PINS.items():
        assert oracle.tile_for_tokens(n) == t


def test_pins_catch_strict_inequality():
    # the page's mutation: with <= changed to <, the pin at 33 tokens fails
    def mutated(n):
        return 64 if oracle.pad_tokens(n, 64) < oracle.pad_tokens(n, 32) else 32
    failing = [n for n, t in PINS.items() if mutated(n) != t]
    assert 33 in failing


def test_pad_tokens():
    assert oracle.pad_tokens(0, 32) == 0
    assert oracle.pad_tokens(7, 32) == 25
    assert oracle.pad_tokens(130, 64) == 62
    assert oracle.pad_tokens(130, 32) == 30
    assert oracle.tile_for_tokens(130) == 32
