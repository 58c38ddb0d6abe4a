"""The library's calls inside a captured HIP graph.

Every entry point only launches kernels on the caller's stream (no allocation, no
memset, no synchronisation), so a sequence of calls can be captured once and
replayed.  Captured here: a dense bf16 GEMM with beta = 1, a split-K GEMM (its tile
counters must be back at zero after every replay), the 4:2 compressor followed by
the sparse GEMM, and a block-scaled fp8 GEMM.  The graph is replayed several times
with the program's own eager work and synchronisations in between (the inputs are
changed between replays), and every replay must give the eager call's bits.
"""
import numpy as np
import pytest
import torch

import sparse_matrix_multiply_amd as mm
from gpu_helpers import dev, pack_mx_scales
from oracle import BF16, E4M3, E5M2

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    d = dev()
    g = torch.Generator(device="cpu").manual_seed(3)
    M, N, K = 300, 520, 1024
    A = torch.randn(M, K, generator=g).to(d).to(torch.bfloat16)
    B = torch.randn(N, K, generator=g).to(d).to(torch.bfloat16)
    C = torch.randn(M, N, generator=g).to(d)
    Ms, Ns, Ks = 256, 256, 16384                       # small output, long K: split into ranges
    As = torch.randn(Ms, Ks, generator=g).to(d).to(torch.bfloat16)
    Bs = torch.randn(Ns, Ks, generator=g).to(d).to(torch.bfloat16)
    ws = mm.workspace(BF16, Ms, Ns, Ks, device=d)
    assert ws is not None
    A8 = torch.randn(M, K, generator=g).to(d).to(torch.float8_e4m3fn)
    A8[:, 1::4] = 0                                    # 4:2 pattern: positions {0, 2} of each group
    A8[:, 3::4] = 0
    B8 = torch.randn(N, K, generator=g).to(d).to(torch.float8_e5m2)
    Ac = torch.empty(M, K // 2, dtype=torch.float8_e4m3fn, device=d)
    idx = torch.empty(M, K // 32, dtype=torch.int32, device=d)
    SA = pack_mx_scales(np.random.default_rng(1).integers(120, 135, size=(M, K // 32)).astype(np.uint8))
    SB = pack_mx_scales(np.random.default_rng(2).integers(120, 135, size=(N, K // 32)).astype(np.uint8))
    outs = [torch.empty(M, N, device=d), torch.empty(Ms, Ns, device=d), torch.empty(M, N, device=d),
            torch.empty(M, N, device=d)]

    def calls(stream):
        mm.gemm_dense(A, B, outs[0], 1.0, 1.0, C, stream=stream)
        mm.gemm_dense(As, Bs, outs[1], stream=stream, workspace=ws)
        mm.sparse24_compress(A8, Ac, idx, a_type=E4M3, stream=stream)
        mm.gemm_sparse24(Ac, idx, B8, outs[2], K=K, a_type=E4M3, b_type=E5M2, stream=stream)
        mm.gemm_mx(A8, SA, B8, SB, outs[3], a_type=E4M3, b_type=E5M2, stream=stream)

    s = torch.cuda.Stream(device=d)
    s.wait_stream(torch.cuda.current_stream(d))
    with torch.cuda.stream(s):
        calls(s)                                       # warm-up outside the capture
    torch.cuda.current_stream(d).wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls(torch.cuda.current_stream(d))
    torch.cuda.synchronize()

    for rep in range(4):
        # new inputs (eager work on the default stream), then the eager result, then the replay
        A.copy_(torch.randn(M, K, generator=g).to(d).to(torch.bfloat16))
        Bs.copy_(torch.randn(Ns, Ks, generator=g).to(d).to(torch.bfloat16))
        B8.copy_(torch.randn(N, K, generator=g).to(d).to(torch.float8_e5m2))
        torch.cuda.synchronize()
        calls(torch.cuda.current_stream(d))
        torch.cuda.synchronize()
        want = [o.clone() for o in outs]
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(ws[:((Ms + 63) // 64) * ((Ns + 63) // 64) * 4]).item()) == 0, "counters"
        for k, (o, w) in enumerate(zip(outs, want)):
            assert torch.equal(o.view(torch.int32), w.view(torch.int32)), f"replay {rep}, output {k}"
