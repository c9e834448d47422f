"""One-hot sweeps through every hot-path kernel, on the formats' edge cases.

With activation token t equal to the unit vector e_k, output (t, r) is the single
product w[r, k] * 1 plus exact zeros, so every path must return the weight itself:
the matrix-vector paths (fp32 arithmetic) the exact dequantized weight, the
matrix-core paths the fp16 value they stage, i.e. the fp16 rounding of that
weight (candle pull request "Metal: 64-token tile for the quantized
matrix-matrix kernel", section "Why the tile sets the weight reuse": each
weight tile is decoded once for the product).  A unit decoded twice would give
2w, a skipped one 0, a misplaced code or scale another weight (the llama.cpp
pull request "metal : fix idle threads in mul_mv_iq3_xxs for ne00 < 1024",
section "Additional information": every (row, chunk) pair is computed once).

The matrices are built from the hand-built golden blocks (tests/golden/blocks.txt:
subnormal and zero scales, signed Q6_K scales, the Q8_0 code -128, the fp32 ties
of the Q4_K/A4G64 add, and blocks whose fp16 staging is a tie that one rounding of
the exact value would break the other way) and from random bytes with finite fp16
scales, some of them subnormal -- inputs the test-data encoders never produce.
Expected values are the oracle's, compared by value (+0 == -0)."""

import numpy as np
import pytest
import torch

import block_quantized_weight_matmul_amd as q
from tests.golden_io import read_blocks
from tests.gpu_helpers import FORMATS, SCALE_OFFSETS, oracle, to_dev, to_host

pytestmark = pytest.mark.gpu

# blocks per row: K = 512 for every format (Q4_0 rows of 16 blocks take the narrow
# expert-indexed kernel), 72 rows (a ragged second 64-row tile), 3 experts
BLOCKS_PER_ROW = {"q4_0": 16, "q8_0": 16, "q4_k": 2, "q6_k": 2, "a4g64": 8, "q4_1": 16, "q5_0": 16, "q5_1": 16,
                  "q2_k": 2, "q3_k": 2, "q5_k": 2}
M, E = 72, 3


def block_pool(fmt):
    """Golden blocks, then random-byte blocks: fp16 scale fields with an exponent of at
    most 15 (finite, below 2 in magnitude, either sign), every fifth one subnormal."""
    bb = oracle.block_bytes(fmt)
    golden = [np.frombuffer(c["data"], np.uint8) for c in read_blocks() if c["fmt"] == fmt]
    g = np.random.default_rng([41, bb])
    rnd = g.integers(0, 256, size=(61, bb), dtype=np.uint8)
    for off in SCALE_OFFSETS[fmt]:
        rnd[:, off + 1] &= 0xBF
        rnd[::5, off + 1] &= 0x83     # exponent field 0: a subnormal (or zero) scale
    return np.concatenate([np.stack(golden), rnd])


def matrix(fmt, shift=0):
    pool = block_pool(fmt)
    nb = BLOCKS_PER_ROW[fmt]
    idx = (np.arange(M * nb) + shift) % len(pool)
    return np.ascontiguousarray(pool[idx]).reshape(-1)


def K_of(fmt):
    return BLOCKS_PER_ROW[fmt] * oracle.block_weights(fmt)


def one_hot(ks, K, dtype):
    x = np.zeros((len(ks), K), dtype)
    x[np.arange(len(ks)), ks] = 1
    return x


def same_values(got, want, label):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (label, got.shape, want.shape)
    bad = got != want
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{label}: {int(bad.sum())} of {bad.size} differ; first at {i}: "
                             f"got {got[i]!r}, expected {want[i]!r}")


def staged(w):
    return oracle.staged_fp16(w).astype(np.float64)


def test_pool_holds_the_edge_cases():
    # the sweeps below see: signed Q6_K scales down to -128, the Q8_0 code -128,
    # subnormal scales in every format, and the two double-rounding blocks
    assert (block_pool("q6_k")[:, 2:18].view(np.int8) == -128).any()
    assert (block_pool("q6_k")[:, 2:18].view(np.int8) < 0).mean() > 0.3
    assert (block_pool("q8_0")[:, 2:34] == 0x80).any()
    for fmt in FORMATS:
        d = block_pool(fmt)[:, 0:2].copy().view(np.float16)[:, 0]
        assert ((d != 0) & (np.abs(d.astype(np.float32)) < 2.0 ** -14)).any(), fmt
    names = [c["name"] for c in read_blocks()]
    for fmt in ("q4_k", "a4g64", "q4_1", "q5_1", "q2_k", "q5_k"):
        assert f"{fmt}_fp16_staging_double_rounding" in names


@pytest.mark.parametrize("xdt", [np.float32, np.float16])
@pytest.mark.parametrize("fmt", FORMATS)
def test_gemv_one_hot(fmt, xdt):
    K = K_of(fmt)
    blob = matrix(fmt)
    w = oracle.dequantize(fmt, blob, M, K)
    qm = q.QMatrix(to_dev(blob), fmt, M, K)
    # one token per call (the one-token kernel), every column
    ys = [qm.gemv(to_dev(one_hot([k], K, xdt))) for k in range(K)]
    same_values(to_host(torch.cat(ys)), w.T, f"{fmt} gemv N=1")
    # 32 tokens per call (the few-token kernels), and a ragged 3-token call
    for n in (32, 3):
        ys = [qm.gemv(to_dev(one_hot(list(range(k0, min(K, k0 + n))), K, xdt))) for k0 in range(0, K, n)]
        same_values(to_host(torch.cat(ys)), w.T, f"{fmt} gemv N={n}")


@pytest.mark.parametrize("xdt", [np.float32, np.float16])
@pytest.mark.parametrize("fmt", FORMATS)
def test_gemm_one_hot(fmt, xdt):
    K = K_of(fmt)
    blob = matrix(fmt)
    want = staged(oracle.dequantize(fmt, blob, M, K)).T
    qm = q.QMatrix(to_dev(blob), fmt, M, K)
    x = to_dev(one_hot(list(range(K)), K, xdt))
    for tile in (32, 64):
        y = torch.empty((K, M), device="cuda")
        q.qmm_gemm(qm.handle, x, K, y, tile)                   # unsplit
        same_values(to_host(y), want, f"{fmt} gemm tile {tile}")
        same_values(to_host(qm.gemm(x, tile)), want, f"{fmt} gemm_ws tile {tile}")
    # few tokens: the K-split path, its partial sums added in split order
    for k0 in range(0, K, 7 * 9):
        ks = list(range(k0, min(K, k0 + 7)))
        for tile in (32, 64):
            same_values(to_host(qm.gemm(to_dev(one_hot(ks, K, xdt)), tile)), want[ks], f"{fmt} gemm N=7 tile {tile}")


@pytest.mark.parametrize("fmt", FORMATS)
def test_dequantize_pool(fmt):
    # the decode-only kernel on the same blocks: fp32 bits and the fp16 staging values
    K = K_of(fmt)
    blob = matrix(fmt)
    w = oracle.dequantize(fmt, blob, M, K)
    qm = q.QMatrix(to_dev(blob), fmt, M, K)
    same_values(to_host(qm.dequantize(0, torch.float32)), w, f"{fmt} dequantize fp32")
    same_values(to_host(qm.dequantize(0, torch.float16)), staged(w), f"{fmt} dequantize fp16")


def stack(fmt):
    blobs = [matrix(fmt, 13 * e) for e in range(E)]
    K = K_of(fmt)
    return np.concatenate(blobs), [oracle.dequantize(fmt, b, M, K) for b in blobs]


@pytest.mark.parametrize("xdt", [np.float32, np.float16])
@pytest.mark.parametrize("fmt", FORMATS)
def test_gemm_id_one_hot(fmt, xdt):
    K = K_of(fmt)
    blob, ws = stack(fmt)
    qm = q.QMatrix(to_dev(blob), fmt, M, K, E)
    want = np.stack([w.T for w in ws], axis=1)  # [K, E, M]: token k, slot s -> expert s column k
    ids = to_dev(np.tile(np.arange(E, dtype=np.int32), (32, 1)))
    got = []
    for k0 in range(0, K, 32):
        ks = list(range(k0, k0 + 32))
        x = np.repeat(one_hot(ks, K, xdt)[:, None, :], E, axis=1)       # one row per slot
        got.append(to_host(qm.gemm_id(to_dev(x), ids)))
    same_values(np.concatenate(got), want, f"{fmt} gemm_id")
    # shared activations ([N, K]) and a reversed slot order
    rev = to_dev(np.tile(np.arange(E - 1, -1, -1, dtype=np.int32), (32, 1)))
    got = [to_host(qm.gemm_id(to_dev(one_hot(list(range(k0, k0 + 32)), K, xdt)), rev)) for k0 in range(0, K, 32)]
    same_values(np.concatenate(got), want[:, ::-1], f"{fmt} gemm_id shared x")


@pytest.mark.parametrize("xdt", [np.float32, np.float16])
@pytest.mark.parametrize("fmt", FORMATS)
def test_gemm_id_tiled_one_hot(fmt, xdt):
    K = K_of(fmt)
    blob, ws = stack(fmt)
    qm = q.QMatrix(to_dev(blob), fmt, M, K, E)
    want = np.stack([staged(w).T for w in ws], axis=1)
    ids = to_dev(np.tile(np.arange(E, dtype=np.int32), (K, 1)))
    x = to_dev(np.repeat(one_hot(list(range(K)), K, xdt)[:, None, :], E, axis=1))
    for tile in ("auto", 32, 64):
        same_values(to_host(qm.gemm_id_tiled(x, ids, tile)), want, f"{fmt} gemm_id_tiled tile {tile}")
