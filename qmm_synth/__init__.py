"""Seeded synthetic inputs for the block-quantized matmul: weights, activations, ids.

This module is the ONLY code that both the CPU oracle's tests and the HIP
path's tests/bench use.  It holds no dequantization and no product: it draws
random fp32 weights, encodes them into blocks (the quantizers below are test
data generators; any deterministic encoder would do, since parity is checked
on the fixed blocks they produce), and draws activations and expert ids.

``quantize``   fp32 [M, K] -> packed blocks (uint8) for each format.
``workloads``  the named, seeded workloads (shapes, formats, seeds).
"""

from .quantize import quantize, QUANTIZERS  # noqa: F401
from . import workloads  # noqa: F401
