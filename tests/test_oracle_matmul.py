"""Pins of the oracle's products (CPU only).

* exact rational arithmetic (fractions.Fraction) on small inputs: the fp64
  result is within fp64 rounding of the exact sum;
* closed forms: one-hot activations return a column of the dequantized
  matrix; an all-ones activation on a hand-built block returns the block sum;
* shape asymmetry (M != K != N) so a transposed operand cannot pass;
* the expert-indexed product against the dense one and against brute force,
  NaN rows for ids outside [0, E).
"""

from fractions import Fraction

import numpy as np

import oracle
from qmm_synth import quantize


def _exact_product(x, w):
    N, K = x.shape
    M = w.shape[0]
    xf = [[Fraction(float(v)) for v in row] for row in x]
    wf = [[Fraction(float(v)) for v in row] for row in w]
    return [[sum(xf[t][k] * wf[r][k] for k in range(K)) for r in range(M)] for t in range(N)]


def test_matmul_against_exact_rationals():
    g = np.random.default_rng(21)
    M, K, N = 3, 256, 2
    blob = quantize("q4_k", g.normal(0, 0.02, (M, K)).astype(np.float32))
    w = oracle.dequantize("q4_k", blob, M, K)
    x = g.standard_normal((N, K)).astype(np.float32)
    y = oracle.matmul_ref(x, w)
    s = oracle.tolerance_scale(x, w)
    exact = _exact_product(x, w)
    assert y.shape == (N, M)
    for t in range(N):
        for r in range(M):
            assert abs(Fraction(float(y[t, r])) - exact[t][r]) <= Fraction(1e-13) * Fraction(float(s[t, r]))
            s_exact = sum(abs(Fraction(float(x[t, k])) * Fraction(float(w[r, k]))) for k in range(K))
            assert abs(Fraction(float(s[t, r])) - s_exact) <= Fraction(1e-13) * s_exact


def test_matmul_fp16_activations_exact_rationals():
    g = np.random.default_rng(22)
    M, K, N = 2, 128, 3
    blob = quantize("a4g64", g.normal(0, 0.02, (M, K)).astype(np.float32))
    w = oracle.dequantize("a4g64", blob, M, K)
    x = g.standard_normal((N, K)).astype(np.float16)
    y = oracle.matmul_ref(x, w)
    exact = _exact_product(x, w)
    s = oracle.tolerance_scale(x, w)
    for t in range(N):
        for r in range(M):
            assert abs(Fraction(float(y[t, r])) - exact[t][r]) <= Fraction(1e-13) * Fraction(float(s[t, r]))


def test_one_hot_returns_columns():
    g = np.random.default_rng(23)
    M, K = 5, 96
    blob = quantize("q8_0", g.normal(0, 0.02, (M, K)).astype(np.float32))
    w = oracle.dequantize("q8_0", blob, M, K)
    ks = [0, 1, 31, 32, 63, 95]
    x = np.zeros((len(ks), K), np.float32)
    for t, k in enumerate(ks):
        x[t, k] = 1.0
    y = oracle.matmul_ref(x, w)
    for t, k in enumerate(ks):
        assert np.array_equal(y[t], w[:, k].astype(np.float64))


def test_all_ones_on_hand_block():
    # Q4_0 block with d=1, codes 0..15 then 15..0: weights -8..7 and 7..-8, sum -16.
    blk = np.frombuffer(bytes.fromhex("003c" "f0e1d2c3b4a5968778695a4b3c2d1e0f"), np.uint8)
    w = oracle.dequantize("q4_0", blk, 1, 32)
    y = oracle.matmul_ref(np.ones((1, 32), np.float32), w)
    assert y[0, 0] == -16.0
    # scaling x by 0.5 halves it exactly; x = index k gives sum k*w_k (closed form below)
    y2 = oracle.matmul_ref(np.arange(32, dtype=np.float32)[None, :], w)
    expect = sum(k * (k - 8) for k in range(16)) + sum((16 + i) * (7 - i) for i in range(16))
    assert y2[0, 0] == expect


def test_transposed_operand_fails():
    g = np.random.default_rng(24)
    M, K, N = 7, 64, 3
    w = oracle.dequantize("q4_0", quantize("q4_0", g.normal(0, 1, (M, K)).astype(np.float32)), M, K)
    x = g.standard_normal((N, K)).astype(np.float32)
    y = oracle.matmul_ref(x, w)
    assert y.shape == (N, M)
    # row r of y^T is w[r] . x[t] computed by hand for one element
    assert abs(y[2, 5] - float(np.dot(w[5].astype(np.float64), x[2].astype(np.float64)))) < 1e-12


def test_matmul_id_matches_dense_and_brute_force():
    g = np.random.default_rng(25)
    E, M, K, N, S = 5, 6, 64, 3, 2
    experts = [oracle.dequantize("q4_0", quantize("q4_0", g.normal(0, 0.02, (M, K)).astype(np.float32)), M, K)
               for _ in range(E)]
    x = g.standard_normal((N, S, K)).astype(np.float32)
    ids = np.array([[4, 0], [2, 2], [1, 3]], np.int32)
    y = oracle.matmul_id_ref(x, ids, experts)
    assert y.shape == (N, S, M)
    for t in range(N):
        for s in range(S):
            dense = oracle.matmul_ref(x[t, s][None, :], experts[ids[t, s]])[0]
            assert np.array_equal(y[t, s], dense)
            exact = _exact_product(x[t, s][None, :], experts[ids[t, s]])[0]
            for r in range(M):
                assert abs(Fraction(float(y[t, s, r])) - exact[r]) < Fraction(1, 10 ** 12)
    # shared activations: x [N, K] feeds every slot of its token
    xs = x[:, 0, :]
    ys = oracle.matmul_id_ref(xs, ids, experts)
    assert np.array_equal(ys[2, 1], oracle.matmul_ref(xs[2][None, :], experts[3])[0])


def test_matmul_id_invalid_ids_are_nan():
    g = np.random.default_rng(26)
    E, M, K = 2, 3, 32
    experts = [oracle.dequantize("q8_0", quantize("q8_0", g.normal(0, 1, (M, K)).astype(np.float32)), M, K)
               for _ in range(E)]
    x = g.standard_normal((2, 2, K)).astype(np.float32)
    ids = np.array([[0, -1], [2, 1]], np.int32)
    y = oracle.matmul_id_ref(x, ids, experts)
    assert np.all(np.isnan(y[0, 1])) and np.all(np.isnan(y[1, 0]))
    assert np.all(np.isfinite(y[0, 0])) and np.all(np.isfinite(y[1, 1]))
    s = oracle.tolerance_scale_id(x, ids, experts)
    assert np.all(np.isnan(s[0, 1])) and np.all(s[1, 1] >= 0)


def test_tolerance_scale_id_against_exact_rationals():
    """S[t, s, r] = sum_k |x_ts[k] * w_e[r, k]| with e = ids[t, s], as exact fractions.  The
    activations and weights take both signs, so a missing absolute value on either operand, a
    sum over the wrong expert, or the wrong slot's activations changes S by far more than fp64
    rounding."""
    g = np.random.default_rng(27)
    E, M, K, N, S = 3, 4, 64, 2, 3
    experts = [oracle.dequantize("q4_0", quantize("q4_0", g.normal(0, 0.02, (M, K)).astype(np.float32)), M, K)
               for _ in range(E)]
    assert all((w < 0).any() and (w > 0).any() for w in experts)
    ids = np.array([[2, 0, 2], [1, 5, 0]], np.int32)
    for per_slot in (True, False):
        x = g.standard_normal((N, S, K) if per_slot else (N, K)).astype(np.float32)
        got = oracle.tolerance_scale_id(x, ids, experts)
        assert got.shape == (N, S, M)
        for t in range(N):
            for s in range(S):
                e = int(ids[t, s])
                if not 0 <= e < E:
                    assert np.all(np.isnan(got[t, s]))
                    continue
                xs = x[t, s] if per_slot else x[t]
                for r in range(M):
                    exact = sum(abs(Fraction(float(xs[k])) * Fraction(float(experts[e][r, k]))) for k in range(K))
                    assert abs(Fraction(float(got[t, s, r])) - exact) <= Fraction(1e-14) * exact
                    # and it bounds the product itself
                    prod = sum(Fraction(float(xs[k])) * Fraction(float(experts[e][r, k])) for k in range(K))
                    assert abs(prod) <= exact
                    assert abs(prod) < exact  # both signs occur, so the bound is strict
