"""Parity at the full benchmark sizes, in the launch configurations bench.py times.

The seeded workloads of the benchmark (the seven decode-layer projections, the
4-bit-group layer, the prefill GEMM at 7 .. 2048 tokens, the 128-expert matvec
and its prefill-sized tiled form) run through the same entry points and launch
shapes as bench.py; so do one-eighth row shards of three projections.  The oracle cannot take whole outputs at these sizes, so it
computes sampled outputs one by one: the sampled rows' blocks are dequantized by
the oracle and multiplied by the given activations in fp64.  Tolerances are
those of the smaller tests: 1e-5 * S on the fp32-accumulating matrix-vector
paths, 2e-3 * S on the fp16-staged matrix-core paths.  The two token tiles are
compared bit for bit over the whole output on the device.
"""

import functools

import numpy as np
import pytest
import torch

import block_quantized_weight_matmul_amd as q
from qmm_synth import workloads as W
from tests.gpu_helpers import assert_within, oracle, to_dev, to_host

pytestmark = pytest.mark.gpu

TOL_GEMV = 1e-5
TOL_GEMM = 2e-3


@functools.lru_cache(maxsize=None)
def decode_matrix(i):
    return W.decode_weights(i)


@functools.lru_cache(maxsize=None)
def small_matrix(i):
    return W.small_decode_weights(i)


@functools.lru_cache(maxsize=1)
def moe_stack():
    return W.moe_stack()


def sample_rows(M, seed, k=48):
    g = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, M - 1], g.choice(M, size=min(k, M), replace=False)]))


def rows_ref(m, rows):
    """Oracle weights of the sampled rows, [len(rows), K] fp32."""
    rb = oracle.row_bytes(m["fmt"], m["K"])
    blob = m["blob"]
    return np.concatenate([oracle.dequantize(m["fmt"], blob[r * rb:(r + 1) * rb], 1, m["K"]) for r in rows])


def check_rows(y, x, m, rows, tol, label):
    """y [N, M] (host) against the oracle on the sampled rows."""
    w = rows_ref(m, rows)
    assert_within(y[:, rows], oracle.matmul_ref(x, w), oracle.tolerance_scale(x, w), tol, label)


@pytest.mark.parametrize("j", range(len(W.DECODE_SHAPES)), ids=[s[0] for s in W.DECODE_SHAPES])
def test_decode_gemv_one_token(j):
    """The headline's launches: qmm_gemv of one fp32 token on each projection."""
    m = decode_matrix(j)
    x = W.decode_x(j)
    qm = q.QMatrix(to_dev(m["blob"]), m["fmt"], m["M"], m["K"])
    y = torch.empty((1, m["M"]), device="cuda")
    q.qmm_gemv(qm.handle, to_dev(x), 1, y)
    check_rows(to_host(y), x, m, sample_rows(m["M"], [80, j]), TOL_GEMV, f"decode {m['name']}")


@pytest.mark.parametrize("n", W.SMALL_DECODE_TOKENS)
def test_small_decode_layer(n):
    """The 4-bit-group layer at 1 .. 16 fp16 tokens, every projection."""
    for i in range(len(W.SMALL_DECODE_SHAPES)):
        m = small_matrix(i)
        x = W.small_decode_x(i, n)
        qm = q.QMatrix(to_dev(m["blob"]), m["fmt"], m["M"], m["K"])
        y = torch.empty((n, m["M"]), device="cuda")
        q.qmm_gemv(qm.handle, to_dev(x), n, y)
        check_rows(to_host(y), x.astype(np.float32), m, sample_rows(m["M"], [81, i, n]), TOL_GEMV,
                   f"a4g64 {m['name']} n={n}")


@pytest.mark.parametrize("n", W.PREFILL_TOKENS)
def test_prefill_gemm(n):
    """qmm_gemm_ws with the workspace the benchmark passes, both tiles and the
    rule's choice, on every projection: tiles bit-identical over the whole
    output, sampled outputs against the oracle."""
    for j in range(len(W.DECODE_SHAPES)):
        m = decode_matrix(j)
        x = W.prefill_x(j, n)
        qm = q.QMatrix(to_dev(m["blob"]), m["fmt"], m["M"], m["K"])
        nb = q.qmm_gemm_workspace_bytes(qm.handle, n)
        ws = torch.empty((nb + 15) // 16 * 4, device="cuda") if nb else None
        xd = to_dev(x)
        ys = {}
        for t in (32, 64):
            y = torch.empty((n, m["M"]), device="cuda")
            q.qmm_gemm_ws(qm.handle, xd, n, y, t, ws)
            ys[t] = y
        assert torch.equal(ys[32].view(torch.int32), ys[64].view(torch.int32)), f"{m['name']} n={n}: tiles differ"
        rows = sample_rows(m["M"], [82, j, n], k=24)
        check_rows(to_host(ys[64]), x.astype(np.float32), m, rows, TOL_GEMM, f"prefill {m['name']} n={n}")


SHARDS = 8  # row shards of one GPU's share when a layer is split over eight


@pytest.mark.parametrize("j", [0, 4, 6], ids=["attn_q", "ffn_gate", "ffn_down"])
@pytest.mark.parametrize("n", [1, 512])
def test_row_shard(j, n):
    """One GPU's row shard of a projection (rows [3M/8, 4M/8): 512x2560,
    1216x2560, 320x9728) is an ordinary matrix of M/8 rows: the one-token GEMV
    and the 512-token GEMM on it, sampled outputs against the oracle on the
    shard's own rows, tiles bit-identical."""
    m = decode_matrix(j)
    rb = oracle.row_bytes(m["fmt"], m["K"])
    Ms = m["M"] // SHARDS
    r0 = 3 * Ms
    shard = dict(m, M=Ms, blob=m["blob"][r0 * rb:(r0 + Ms) * rb])
    qm = q.QMatrix(to_dev(shard["blob"]), m["fmt"], Ms, m["K"])
    rows = sample_rows(Ms, [86, j, n], k=24)
    if n == 1:
        x = W.decode_x(j)
        y = torch.empty((1, Ms), device="cuda")
        q.qmm_gemv(qm.handle, to_dev(x), 1, y)
        check_rows(to_host(y), x, shard, rows, TOL_GEMV, f"shard {m['name']} n=1")
        return
    x = W.prefill_x(j, n)
    nb = q.qmm_gemm_workspace_bytes(qm.handle, n)
    ws = torch.empty((nb + 15) // 16 * 4, device="cuda") if nb else None
    xd = to_dev(x)
    ys = {}
    for t in (32, 64):
        ys[t] = torch.empty((n, Ms), device="cuda")
        q.qmm_gemm_ws(qm.handle, xd, n, ys[t], t, ws)
    assert torch.equal(ys[32].view(torch.int32), ys[64].view(torch.int32)), f"shard {m['name']}: tiles differ"
    check_rows(to_host(ys[64]), x.astype(np.float32), shard, rows, TOL_GEMM, f"shard {m['name']} n={n}")


def _moe_rows_check(y, x, ids, rows, tol, label):
    """y [N, S, M] (host) on the sampled rows of every (token, slot) pair."""
    stack = moe_stack()
    eb = stack.size // W.MOE_EXPERTS
    rb = oracle.row_bytes("q4_0", W.MOE_K)
    N, S = ids.shape
    for t in range(N):
        for s in range(S):
            e = int(ids[t, s])
            blob = stack[e * eb:(e + 1) * eb]
            w = np.concatenate([oracle.dequantize("q4_0", blob[r * rb:(r + 1) * rb], 1, W.MOE_K) for r in rows])
            xs = x[t, s][None, :].astype(np.float32)
            assert_within(y[t, s][None, rows], oracle.matmul_ref(xs, w), oracle.tolerance_scale(xs, w), tol,
                          f"{label} t={t} s={s} e={e}")


@pytest.mark.parametrize("n", W.MOE_TOKENS)
def test_expert_matvec(n):
    """qmm_gemm_id on the 128-expert stack with per-slot fp32 activations."""
    stack = moe_stack()
    qm = q.QMatrix(to_dev(stack), "q4_0", W.MOE_M, W.MOE_K, W.MOE_EXPERTS)
    ids = W.moe_ids(n, 0)
    x = W.moe_x(n)
    y = torch.empty((n, W.MOE_SLOTS, W.MOE_M), device="cuda")
    q.qmm_gemm_id(qm.handle, to_dev(x), n, W.MOE_SLOTS, 1, to_dev(ids), y)
    _moe_rows_check(to_host(y), x, ids, sample_rows(W.MOE_M, [83, n], k=16), TOL_GEMV, f"moe n={n}")


@pytest.mark.parametrize("n", W.MOE_PREFILL_TOKENS)
def test_expert_tiled(n):
    """qmm_gemm_id_tiled at prefill sizes (fp16 activations): sampled pairs."""
    stack = moe_stack()
    qm = q.QMatrix(to_dev(stack), "q4_0", W.MOE_M, W.MOE_K, W.MOE_EXPERTS)
    ids = W.moe_ids(n, 0)
    x = W.moe_prefill_x(n)
    y = torch.empty((n, W.MOE_SLOTS, W.MOE_M), device="cuda")
    q.qmm_gemm_id_tiled(qm.handle, to_dev(x), n, W.MOE_SLOTS, 1, to_dev(ids), y)
    yh = to_host(y)
    g = np.random.default_rng([84, n])
    toks = np.unique(np.concatenate([[0, n - 1], g.choice(n, size=min(6, n), replace=False)]))
    _moe_rows_check(yh[toks], x[toks], ids[toks], sample_rows(W.MOE_M, [85, n], k=16), TOL_GEMM,
                    f"moe tiled n={n}")


@pytest.mark.parametrize("group", [(0, 1), (4, 5), (0, 1, 2)], ids=["attn_q+attn_k", "ffn_gate+ffn_up", "attn_q+k+v"])
def test_decode_gemv_grouped(group):
    """The headline's grouped launches: qmm_gemv_group of one fp32 token on the layer's
    independent projections gives each the bits of its own qmm_gemv call."""
    ms = [decode_matrix(j) for j in group]
    xs = [W.decode_x(j) for j in group]
    qms = [q.QMatrix(to_dev(m["blob"]), m["fmt"], m["M"], m["K"]) for m in ms]
    xd = [to_dev(x) for x in xs]
    ys = [torch.empty((1, m["M"]), device="cuda") for m in ms]
    q.qmm_gemv_group([qm.handle for qm in qms], xd, 1, ys)
    for m, x, qm, y, xx in zip(ms, xd, qms, ys, xs):
        single = torch.empty((1, m["M"]), device="cuda")
        q.qmm_gemv(qm.handle, x, 1, single)
        got = to_host(y)
        assert np.array_equal(got.view(np.uint32), to_host(single).view(np.uint32)), m["name"]
        check_rows(got, xx, m, sample_rows(m["M"], [81, m["M"]]), TOL_GEMV, f"grouped {m['name']}")


@pytest.mark.parametrize("n", W.SMALL_DECODE_TOKENS)
def test_small_decode_layer_grouped(n):
    """The 4-bit-group layer's calls as the benchmark makes them: q+k+v and gate+up
    through qmm_gemv_group (one launch each), every output the bits of its own
    qmm_gemv call."""
    for grp in ([0, 1, 2], [4, 5]):
        ms = [small_matrix(i) for i in grp]
        xs = [W.small_decode_x(i, n) for i in grp]
        qms = [q.QMatrix(to_dev(m["blob"]), m["fmt"], m["M"], m["K"]) for m in ms]
        xd = [to_dev(x) for x in xs]
        ys = [torch.empty((n, m["M"]), device="cuda") for m in ms]
        q.qmm_gemv_group([qm.handle for qm in qms], xd, n, ys)
        for m, qm, x, y, xx in zip(ms, qms, xd, ys, xs):
            single = torch.empty((n, m["M"]), device="cuda")
            q.qmm_gemv(qm.handle, x, n, single)
            got = to_host(y)
            assert np.array_equal(got.view(np.uint32), to_host(single).view(np.uint32)), (m["name"], n)
            check_rows(got, xx.astype(np.float32), m, sample_rows(m["M"], [82, n]), TOL_GEMV,
                       f"a4g64 grouped {m['name']} n={n}")
