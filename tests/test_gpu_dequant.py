"""Decoders on the GPU, bit for bit against the oracle (qmm_dequantize).

fp32 output: the exact dequantized weights (the oracle's values, compared by
bit pattern after +0/-0 normalisation, which the formulas leave open).  fp16
output: the values the matrix-matrix path stages, i.e. round-to-nearest-even
of those (the oracle's staged_fp16)."""

import numpy as np
import pytest
import torch

import block_quantized_weight_matmul_amd as q
from tests.golden_io import read_blocks
from tests.gpu_helpers import FORMATS, SCALE_OFFSETS, make_matrix, oracle, to_dev, to_host

pytestmark = pytest.mark.gpu


def _same(a, b):
    a = np.asarray(a, np.float32) + np.float32(0)
    b = np.asarray(b, np.float32) + np.float32(0)
    return np.array_equal(a.view(np.uint32), b.view(np.uint32))


def _check(fmt, blob, M, K, experts=1):
    qm = q.QMatrix(to_dev(blob), fmt, M, K, experts)
    rb = oracle.row_bytes(fmt, K)
    for e in range(experts):
        ref = oracle.dequantize(fmt, blob[e * M * rb:(e + 1) * M * rb], M, K)
        got32 = to_host(qm.dequantize(e, torch.float32))
        assert _same(got32, ref), f"{fmt} {M}x{K} expert {e}: fp32 differs at {np.argwhere(got32 != ref)[:5]}"
        got16 = to_host(qm.dequantize(e, torch.float16))
        assert _same(got16.astype(np.float32), oracle.staged_fp16(ref).astype(np.float32)), \
            f"{fmt} {M}x{K} expert {e}: fp16 staging differs"


@pytest.mark.parametrize("fmt", FORMATS)
def test_golden_blocks_on_device(fmt):
    cases = [c for c in read_blocks() if c["fmt"] == fmt]
    blob = np.frombuffer(b"".join(c["data"] for c in cases), np.uint8)
    bw = oracle.block_weights(fmt)
    qm = q.QMatrix(to_dev(blob), fmt, len(cases), bw)
    got = to_host(qm.dequantize())
    for r, c in enumerate(cases):
        assert [float(v) for v in got[r]] == [float(v) for v in c["expect"]], c["name"]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("M,nblk", [(1, 1), (3, 2), (67, 3), (130, 12)])
def test_random_matrices(fmt, M, nblk):
    K = nblk * oracle.block_weights(fmt)
    _check(fmt, make_matrix(fmt, M, K, [31, M, nblk]), M, K)


@pytest.mark.parametrize("fmt", FORMATS)
def test_random_bytes(fmt):
    """Arbitrary code bytes and scale fields (finite fp16 scales)."""
    bw, bb = oracle.FORMATS[fmt]
    g = np.random.default_rng([32, bb])
    M, nblk = 37, 5
    blk = g.integers(0, 256, size=(M * nblk, bb), dtype=np.uint8)
    for off in SCALE_OFFSETS[fmt]:
        blk[:, off + 1] &= 0xBF      # exponent field <= 15: finite, either sign
    _check(fmt, blk.reshape(-1), M, nblk * bw)


@pytest.mark.parametrize("fmt", FORMATS)
def test_experts_stacked(fmt):
    K = 2 * oracle.block_weights(fmt)
    M, E = 19, 3
    blob = np.concatenate([make_matrix(fmt, M, K, [33, e]) for e in range(E)])
    _check(fmt, blob, M, K, experts=E)
