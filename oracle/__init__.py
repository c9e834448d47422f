"""Plain CPU oracle for the fused dequantize-and-multiply of block-quantized weights.

TEST INFRASTRUCTURE ONLY.  This package is the slow, obviously-correct
reference that the HIP path is checked against.  Only the test-suite, the
smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The product path (``block_quantized_weight_matmul_amd``)
never imports, calls or links anything here, and nothing here imports the
product path: the two share no code, no tables and no constants.

Contents
--------
``formats``  byte layout of each block format and its dequantization to fp32
             (one function per format, scalar per-field formulas vectorised
             over blocks with NumPy).
``matmul``   the dense product ``y = x . W^T`` and the expert-indexed product
             in fp64, plus the tolerance scale ``S = |x| . |W|^T``.
``quantize`` reference quantizers fp32 -> blocks (``quantize_blocks``), the
             check for the library's GPU quantizer.
``tile``     the 32/64-token tile rule of the candle pull request
             "Metal: 64-token tile for the quantized matrix-matrix kernel",
             section "Where the 64-token tile is used".

Every function is pinned by ``tests/test_oracle_*.py`` against hand-computed
blocks, closed forms, exact rational arithmetic and the values the pages print.
"""

from .formats import (  # noqa: F401
    FORMATS,
    block_weights,
    block_bytes,
    row_bytes,
    dequantize,
    dequantize_blocks,
    staged_fp16,
)
from .matmul import matmul_ref, matmul_id_ref, tolerance_scale, tolerance_scale_id  # noqa: F401
from .tile import tile_for_tokens, pad_tokens  # noqa: F401
from .quantize import quantize_blocks  # noqa: F401
