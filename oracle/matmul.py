"""The products the hot path computes, in fp64 -- CPU oracle (test infrastructure only).

Dense product.  All three pages compute y = x . W^T with W held as quantized
blocks that the kernel dequantizes itself: the candle pull request "Metal:
64-token tile for the quantized matrix-matrix kernel" (section "Why the tile
sets the weight reuse"), the llama.cpp pull request "metal : fix idle threads
in mul_mv_iq3_xxs for ne00 < 1024" (section "Overview": the matrix-vector
product over 32-weight chunks) and the tiny-llm pull request "perf: Optimize
quantized matmul for small decode batches" (section "Summary").  With W^ the
dequantized fp32 weights, the method reaches exactly (up to the order of the
floating-point additions) ``y[t, r] = sum_k x[t, k] * W^[r, k]``; this module
writes that definition out in fp64, where every product of an fp32 weight and
an fp32 or fp16 activation is exact.

Expert-indexed product.  The llama.cpp pull request (section "Additional
information") checks MUL_MAT_ID, the matrix-vector product whose weight matrix
is picked per (token, slot) by an expert id, against the CPU backend:
``y[t, s, r] = sum_k x[t, s, k] * W^_{ids[t, s]}[r, k]`` (one activation row per
slot, as for a down projection), or with ``x[t, k]`` shared by all slots of a
token.  An id outside [0, E) has no matrix; this library defines its output
row as all NaN.

Tolerance scale.  ``S[t, r] = sum_k |x[t, k] * W^[r, k]|`` in fp64, the
quantity the floating-point error of any summation order is proportional to.
"""

import numpy as np


def matmul_ref(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """x [N, K] (fp32 or fp16), w [M, K] fp32 dequantized weights -> y [N, M] fp64."""
    x64 = np.asarray(x).astype(np.float64)
    w64 = np.asarray(w).astype(np.float64)
    assert x64.ndim == 2 and w64.ndim == 2 and x64.shape[1] == w64.shape[1]
    return x64 @ w64.T


def tolerance_scale(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """S = |x| . |w|^T in fp64, [N, M]."""
    return np.abs(np.asarray(x).astype(np.float64)) @ np.abs(np.asarray(w).astype(np.float64)).T


def _slot_x(x: np.ndarray, t: int, s: int) -> np.ndarray:
    return x[t, s] if x.ndim == 3 else x[t]


def matmul_id_ref(x: np.ndarray, ids: np.ndarray, w_experts) -> np.ndarray:
    """Expert-indexed product.

    x          [N, S, K] (one row per slot) or [N, K] (shared by the token's slots)
    ids        [N, S] integer expert ids
    w_experts  sequence of E dequantized matrices [M, K] (or an [E, M, K] array)
    returns    y [N, S, M] fp64; rows whose id is outside [0, E) are NaN.
    """
    ids = np.asarray(ids)
    N, S = ids.shape
    E = len(w_experts)
    M = np.asarray(w_experts[0]).shape[0]
    y = np.full((N, S, M), np.nan, dtype=np.float64)
    for t in range(N):
        for s in range(S):
            e = int(ids[t, s])
            if 0 <= e < E:
                we = np.asarray(w_experts[e]).astype(np.float64)
                y[t, s] = we @ _slot_x(x, t, s).astype(np.float64)
    return y


def tolerance_scale_id(x: np.ndarray, ids: np.ndarray, w_experts) -> np.ndarray:
    """S for the expert-indexed product, [N, S, M]; NaN where the id is invalid."""
    ids = np.asarray(ids)
    N, S = ids.shape
    E = len(w_experts)
    M = np.asarray(w_experts[0]).shape[0]
    out = np.full((N, S, M), np.nan, dtype=np.float64)
    for t in range(N):
        for s in range(S):
            e = int(ids[t, s])
            if 0 <= e < E:
                we = np.abs(np.asarray(w_experts[e]).astype(np.float64))
                out[t, s] = we @ np.abs(_slot_x(x, t, s).astype(np.float64))
    return out
