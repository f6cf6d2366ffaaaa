"""The entry points replayed from a captured HIP graph give the same bits as eager calls.

The graph is captured once and replayed several times, with eager calls, other torch work and
synchronisations between the replays; every replay is compared with the eager result of the
same call.  This covers the calls that bench.py replays from graphs (the reduction with and
without the fused cast, the chunked store product, ring attention); the kernels allocate
nothing and record no memset nodes."""
import numpy as np
import pytest
import torch

import pk_inputs
from _gpu import dev_bf16, log, require_gpu

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module")
def pk():
    return require_gpu()


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        fn()
    torch.cuda.synchronize()
    return g


def _unrelated_work():
    x = torch.randn(1 << 20, device="cuda")
    return float((x * x).sum())


def test_reduce_owner_with_cast_replays(pk):
    M, N, K = 600, 264, 136
    A = dev_bf16(pk_inputs.normal_bf16((M, K), 0.5, 9101))
    B = dev_bf16(pk_inputs.normal_bf16((K, N), 0.5, 9102))
    D0 = torch.randn(M, N, device="cuda")
    De, Dg = D0.clone(), D0.clone()
    Ce = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    Cg = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    call = lambda D, C: pk.gemm_reduce(A, B, list(D.split(256)), mode=pk.PK_REDUCE_OWNER,
                                       out_bf16=C)
    call(D0.clone(), torch.empty_like(Ce))   # first launch outside the capture
    g = _capture(lambda: call(Dg, Cg))       # captured, not run
    for r in range(REPLAYS):
        call(De, Ce)
        torch.cuda.synchronize()
        _unrelated_work()
        Cg.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        log("reduce replay %d" % r)
        assert torch.equal(Dg, De), r
        assert torch.equal(Cg.view(torch.int16), Ce.view(torch.int16)), r


def test_chunked_store_product_replays(pk):
    M, N, K = 512, 256, 320
    A = dev_bf16(pk_inputs.normal_bf16((M, K), 1.0, 9111))
    B = dev_bf16(pk_inputs.normal_bf16((K, N), 1.0, 9112))
    chunks = list(A.split(128))
    Ce = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    Cg = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    pk.gemm(chunks, B, Ce, first_chunk=2)
    g = _capture(lambda: pk.gemm(chunks, B, Cg, first_chunk=2))
    for r in range(REPLAYS):
        Cg.fill_(float("nan"))
        _unrelated_work()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Cg.view(torch.int16), Ce.view(torch.int16)), r


@pytest.mark.parametrize("chunk_len", [64, 128], ids=["64-key blocks", "128-key blocks"])
def test_ring_attention_replays(pk, chunk_len):
    BH, Sq, n, D = 2, 300, 3, 128
    Q = dev_bf16(pk_inputs.normal_bf16((BH, Sq, D), 1.0, 9121))
    K = [dev_bf16(pk_inputs.normal_bf16((BH, chunk_len, D), 1.0, 9122 + c)) for c in range(n)]
    V = [dev_bf16(pk_inputs.normal_bf16((BH, chunk_len, D), 1.0, 9132 + c)) for c in range(n)]
    Oe = torch.empty(BH, Sq, D, device="cuda")
    Le = torch.empty(BH, Sq, device="cuda")
    Og = torch.empty(BH, Sq, D, device="cuda")
    Lg = torch.empty(BH, Sq, device="cuda")
    pk.ring_attention(Q, K, V, Oe, Le, first_chunk=1)
    g = _capture(lambda: pk.ring_attention(Q, K, V, Og, Lg, first_chunk=1))
    for r in range(REPLAYS):
        Og.fill_(float("nan"))
        Lg.fill_(float("nan"))
        _unrelated_work()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Og, Oe) and torch.equal(Lg, Le), r
        assert not torch.isnan(Og).any()
