"""The library's launches captured into a HIP graph (via torch.cuda.graph on the
capture stream): every replay, with eager work and synchronisations between
replays, equals the eager result bit for bit.  The library records no memset
or allocation, only kernel launches."""

import numpy as np
import pytest
import torch

import block_quantized_weight_matmul_amd as q
from tests.gpu_helpers import count_differences, make_matrix, to_dev, to_host

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    M, K = 300, 2560
    dense = q.QMatrix(to_dev(make_matrix("q4_k", M, K, [81])), "q4_k", M, K)
    E, Me, Ke = 8, 128, 512
    stack = q.QMatrix(to_dev(np.concatenate([make_matrix("q4_0", Me, Ke, [82, e]) for e in range(E)])),
                      "q4_0", Me, Ke, E)
    g = np.random.default_rng(83)
    x1 = to_dev(g.standard_normal((1, K)).astype(np.float32))
    x5 = to_dev(g.standard_normal((5, K)).astype(np.float32))
    x70 = to_dev(g.standard_normal((70, K)).astype(np.float16))
    ids = to_dev(np.stack([g.choice(E, 4, replace=False) for _ in range(6)]).astype(np.int32))
    xid = to_dev(g.standard_normal((6, 4, Ke)).astype(np.float32))
    v6 = q.QMatrix(to_dev(make_matrix("q6_k", 200, K, [84])), "q6_k", 200, K)
    outs = [torch.empty((1, M), device="cuda"), torch.empty((5, M), device="cuda"),
            torch.empty((70, M), device="cuda"), torch.empty((6, 4, Me), device="cuda"),
            torch.empty((1, M), device="cuda"), torch.empty((1, 200), device="cuda"),
            torch.empty((5, M), device="cuda"), torch.empty((5, M), device="cuda")]

    def step():
        q.qmm_gemv(dense.handle, x1, 1, outs[0])
        q.qmm_gemv(dense.handle, x5, 5, outs[1])
        q.qmm_gemm(dense.handle, x70, 70, outs[2], 0)
        q.qmm_gemm_id(stack.handle, xid, 6, 4, 1, ids, outs[3])
        # grouped: a Q4_K + Q6_K one-token launch and a few-token launch of two Q4_K
        q.qmm_gemv_group([dense.handle, v6.handle], [x1, x1], 1, [outs[4], outs[5]])
        q.qmm_gemv_group([dense.handle, dense.handle], [x5, x5], 5, [outs[6], outs[7]])

    step()
    eager = [to_host(o).copy() for o in outs]
    for o in outs:
        o.fill_(-1.0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        got = [to_host(o) for o in outs]
        for a, b in zip(eager, got):
            assert count_differences(a, b) == 0, f"replay {rep}"
        # the grouped outputs are the single calls' bits
        assert count_differences(got[4], got[0]) == 0 and count_differences(got[6], got[1]) == 0
        assert count_differences(got[7], got[1]) == 0
        _ = (x5 * 2).sum().item()   # unrelated eager work between replays
