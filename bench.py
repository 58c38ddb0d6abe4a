"""Benchmark harness (being written)."""


def gemm_flops(M, N, K):
    """Work of one GEMM: 2*M*N*K operations (for a 4:2-sparse A, K is the dense K)."""
    return 2 * int(M) * int(N) * int(K)
