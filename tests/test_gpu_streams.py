"""Calls on several streams at once.

Every entry point keeps no state between calls except what the caller passes in (the split-K
workspace, owned by the caller; the allocation-free entry point's fixed array is documented as
shared and is not used here).  So calls on independent buffers, issued on three streams with
their launches interleaved and running concurrently, must give exactly the bits the same calls
give one after another on one stream.  Each stream runs a dense bf16 GEMM with beta = 1, a split-K
GEMM through a workspace of its own, the 4:2 compressor and the sparse fp8 GEMM after it.
"""
import pytest
import torch

import sparse_matrix_multiply_amd as mm
from gpu_helpers import dev
from oracle import BF16, E4M3, E5M2

pytestmark = pytest.mark.gpu


def _problem(g, d):
    M, N, K = 520, 300, 2048
    Ms, Ns, Ks = 256, 192, 16384
    p = {
        "A": torch.randn(M, K, generator=g).to(d).to(torch.bfloat16),
        "B": torch.randn(N, K, generator=g).to(d).to(torch.bfloat16),
        "C": torch.randn(M, N, generator=g).to(d),
        "As": torch.randn(Ms, Ks, generator=g).to(d).to(torch.bfloat16),
        "Bs": torch.randn(Ns, Ks, generator=g).to(d).to(torch.bfloat16),
        "ws": mm.workspace(BF16, Ms, Ns, Ks, device=d),
        "A8": torch.randn(M, K, generator=g).to(d).to(torch.float8_e4m3fn),
        "B8": torch.randn(N, K, generator=g).to(d).to(torch.float8_e5m2),
        "Ac": torch.empty(M, K // 2, dtype=torch.float8_e4m3fn, device=d),
        "idx": torch.empty(M, K // 32, dtype=torch.int32, device=d),
        "D": torch.empty(M, N, device=d),
        "Dsk": torch.empty(Ms, Ns, device=d),
        "Dsp": torch.empty(M, N, device=d),
    }
    assert p["ws"] is not None
    p["A8"][:, 1::4] = 0            # a 4:2 pattern: positions {0, 2} of each group of four
    p["A8"][:, 3::4] = 0
    return p


def _calls(p, stream):
    K = p["A8"].shape[1]
    return [
        lambda: mm.gemm_dense(p["A"], p["B"], p["D"], 1.0, 1.0, p["C"], stream=stream),
        lambda: mm.gemm_dense(p["As"], p["Bs"], p["Dsk"], stream=stream, workspace=p["ws"]),
        lambda: mm.sparse24_compress(p["A8"], p["Ac"], p["idx"], a_type=E4M3, stream=stream),
        lambda: mm.gemm_sparse24(p["Ac"], p["idx"], p["B8"], p["Dsp"], K=K, a_type=E4M3, b_type=E5M2, stream=stream),
    ]


def test_concurrent_streams_match_one_stream():
    d = dev()
    g = torch.Generator(device="cpu").manual_seed(11)
    probs = [_problem(g, d) for _ in range(3)]
    outs = ("D", "Dsk", "Ac", "idx", "Dsp")
    cur = torch.cuda.current_stream(d)
    # one after another on the current stream
    for p in probs:
        for c in _calls(p, cur):
            c()
    torch.cuda.synchronize()
    want = [{k: p[k].clone() for k in outs} for p in probs]
    for p in probs:
        for k in outs:
            if p[k].dtype == torch.int32:
                p[k].fill_(-1)
            else:
                p[k].view(torch.uint8).fill_(0xff)
    torch.cuda.synchronize()
    # three streams, launches interleaved, several rounds
    streams = [torch.cuda.Stream(device=d) for _ in probs]
    for s in streams:
        s.wait_stream(cur)
    for rnd in range(3):
        calls = [_calls(p, s) for p, s in zip(probs, streams)]
        for step in range(len(calls[0])):
            for cs in calls:
                cs[step]()
    for s in streams:
        cur.wait_stream(s)
    torch.cuda.synchronize()
    for i, (p, w) in enumerate(zip(probs, want)):
        for k in outs:
            assert torch.equal(p[k].view(torch.uint8), w[k].view(torch.uint8)), f"stream {i}, output {k}"
    # the split-K tile counters are back at zero in every workspace
    for p in probs:
        tiles = ((256 + 63) // 64) * ((192 + 63) // 64)
        assert int(torch.count_nonzero(p["ws"][:tiles * 4]).item()) == 0
