"""The token-tile rule of the matrix-matrix path -- CPU oracle (test infrastructure only).

Candle pull request "Metal: 64-token tile for the quantized matrix-matrix
kernel", section "Where the 64-token tile is used": the 64-token tile is used
only when it pads no more tokens than the 32-token tile.  Written out: a tile
of T tokens pads ``T * ceil(N / T) - N`` tokens, and the rule picks 64 when
that padding at T = 64 is at most the padding at T = 32, else 32.  (The page
restates it as "a multiple of 64, or more than 32 over a multiple of 64";
the tests check the two statements agree.)  At N = 0 both paddings are zero,
so the rule gives 64; nothing is launched for zero tokens.
"""


def pad_tokens(n: int, tile: int) -> int:
    """Tokens of padding when n tokens are covered by tiles of ``tile`` tokens."""
    if n < 0 or tile <= 0:
        raise ValueError("n must be >= 0 and tile > 0")
    return tile * (-(-n // tile)) - n


def tile_for_tokens(n: int) -> int:
    """32 or 64: the wider tile only when it pads no more tokens."""
    return 64 if pad_tokens(n, 64) <= pad_tokens(n, 32) else 32
