"""Seeded synthetic inputs shared by the HIP path's tests, the oracle's tests and the benchmark.

This module holds no arithmetic of the method itself (no products, sums over K, dispatch or
rounding of results): it only draws numbers and turns binary32 draws into bf16 bit patterns so
that both sides receive identical operands.  Random numbers are drawn with numpy's PCG64.

Workload shapes and value distributions follow the pages' workloads ("Loads and Loads of Fluffy
Kittens" summary, Results: AG+GEMM local N x N/8 x N, GEMM+RS local N x N x N/8, GEMM+AR, and
the MoE dispatch with top_k=8, 256 experts, D=7168, D_expert=2048).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Tuple

import numpy as np

__all__ = [
    "f32_to_bf16_bits", "normal_bf16", "small_int_bf16", "zipf_topk", "rs_prefill",
    "WORKLOADS", "Workload",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """binary32 -> bf16 bit patterns, round to nearest even (input preparation only).

    Works in 32-bit unsigned arithmetic, in chunks: adding 0x7FFF plus the kept bit's parity can
    only wrap around for NaN patterns, which are replaced by the quiet NaN 0x7FC0 anyway."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    flat = x.reshape(-1)
    u = flat.view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    step = 1 << 24
    for i in range(0, u.size, step):
        v = u[i:i + step]
        r = (v + np.uint32(0x7FFF) + ((v >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        o = r.astype(np.uint16)
        nan = np.isnan(flat[i:i + step])
        if nan.any():
            o[nan] = 0x7FC0
        out[i:i + step] = o
    return out.reshape(x.shape)


def normal_bf16(shape, std: float, seed: int) -> np.ndarray:
    """~N(0, std^2) drawn in binary32 with PCG64(seed), rounded to bf16 (uint16 bit patterns)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


def small_int_bf16(shape, lo: int, hi: int, seed: int) -> np.ndarray:
    """Uniform integers in [lo, hi] as bf16 bit patterns (exact for |v| <= 256)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    v = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    return f32_to_bf16_bits(v)


def zipf_topk(T: int, num_experts: int, top_k: int, s: float, seed: int) -> np.ndarray:
    """Route T tokens to top_k distinct experts each, drawn without replacement from a bounded
    Zipf law p_e proportional to (e+1)^-s (expert 0 hottest).  Sequential sampling without
    replacement is done with Gumbel keys (log p_e + Gumbel noise, keep the top_k largest).
    Returns int32 [T, top_k]; the k-order within a token is the sampling order."""
    rng = np.random.Generator(np.random.PCG64(seed))
    logp = -s * np.log(np.arange(1, num_experts + 1, dtype=np.float64))
    g = rng.gumbel(size=(T, num_experts))
    keys = logp[None, :] + g
    top = np.argsort(-keys, axis=1, kind="stable")[:, :top_k]
    return np.ascontiguousarray(top.astype(np.int32))


def rs_prefill(M: int, N: int, partials: int, std: float, seed0: int,
               row_block: int = 1024) -> np.ndarray:
    """Destination pre-filled with the sum of ``partials`` other producers' outputs, each drawn
    ~N(0, std^2) (seeds seed0 .. seed0+partials-1), summed in binary64 and rounded once to
    binary32.  Generated in row blocks to bound host memory."""
    out = np.empty((M, N), dtype=np.float32)
    rngs = [np.random.Generator(np.random.PCG64(seed0 + r)) for r in range(partials)]
    for r0 in range(0, M, row_block):
        r1 = min(M, r0 + row_block)
        acc = np.zeros((r1 - r0, N), dtype=np.float64)
        for g in rngs:
            acc += g.standard_normal(size=(r1 - r0, N), dtype=np.float32).astype(np.float64) * std
        out[r0:r1] = acc.astype(np.float32)
    return out


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: its kind, sizes and seeds (values only; no arithmetic)."""
    name: str
    kind: str                  # "reduce" | "gemm" | "grouped" | "combine" | "attention"
    M: int = 0
    N: int = 0
    K: int = 0
    std_a: float = 0.02
    std_b: float = 0.02
    seed_a: int = 0
    seed_b: int = 0
    producers: int = 1         # reduce: producers added by this call sequence
    shards: int = 1            # reduce: destination shards
    prefill_partials: int = 0  # reduce: other producers already summed into the destination
    prefill_std: float = 0.0
    prefill_seed: int = 0
    chunks: int = 1            # gemm: gathered row-chunks of A
    cast_bf16: bool = False    # reduce: bf16 cast pass after the reduction
    tokens: int = 0            # grouped
    top_k: int = 0
    num_experts: int = 0
    num_local: int = 0
    expert_begin: int = 0
    zipf_s: float = 0.0
    seed_route: int = 0
    seed_gates: int = 0        # combine: routing gate weights

    @property
    def flops(self) -> float:
        if self.kind in ("grouped", "combine"):
            raise ValueError("grouped flops depend on the routed row count")
        if self.kind == "attention":  # QK^T and PV over all keys of all chunks
            return 4.0 * self.M * self.N * self.chunks * self.tokens * self.K
        return 2.0 * self.M * self.N * self.K * self.producers


# The five workloads: a tiny 8-producer reduction, and the per-rank local shares at their real
# shapes (one GPU of eight).
WORKLOADS: Dict[str, Workload] = {
    "rs_tiny": Workload("rs_tiny", "reduce", M=512, N=512, K=64, std_a=1.0, std_b=1.0,
                        seed_a=1000, seed_b=2000, producers=8, shards=1),
    "ag_8192": Workload("ag_8192", "gemm", M=8192, N=1024, K=8192, seed_a=3001, seed_b=3002,
                        chunks=8),
    "rs_8192": Workload("rs_8192", "reduce", M=8192, N=8192, K=1024, seed_a=4001, seed_b=4002,
                        producers=1, shards=8, prefill_partials=7,
                        prefill_std=0.02 * 0.02 * 32.0, prefill_seed=4011),
    "ar_16384": Workload("ar_16384", "reduce", M=16384, N=16384, K=2048, seed_a=5001,
                         seed_b=5002, producers=1, shards=1, cast_bf16=True),
    "ring_attention": Workload("ring_attention", "attention", M=16 * 16, N=1024, K=128,
                               std_a=1.0, std_b=1.0, seed_a=8001, seed_b=8101, chunks=8,
                               tokens=1024),
    "moe_combine": Workload("moe_combine", "combine", K=2048, N=7168, std_a=1.0, std_b=0.02,
                            seed_a=7001, seed_b=7002, tokens=4096, top_k=8, num_experts=256,
                            num_local=32, expert_begin=0, zipf_s=1.1, seed_route=6003,
                            seed_gates=7004),
    "moe_dispatch": Workload("moe_dispatch", "grouped", K=7168, N=2048, std_a=1.0, std_b=0.02,
                             seed_a=6001, seed_b=6002, tokens=4096, top_k=8, num_experts=256,
                             num_local=32, expert_begin=0, zipf_s=1.1, seed_route=6003),
}


def producer_operands(w: Workload, p: int) -> Tuple[np.ndarray, np.ndarray]:
    """Operands of producer p of a reduce workload (A_p: M x K, B_p: K x N, bf16 bits)."""
    A = normal_bf16((w.M, w.K), w.std_a, w.seed_a + p)
    B = normal_bf16((w.K, w.N), w.std_b, w.seed_b + p)
    return A, B


def moe_inputs(w: Workload):
    """Routing and operands of the MoE workload: (topk_ids, X, W)."""
    ids = zipf_topk(w.tokens, w.num_experts, w.top_k, w.zipf_s, w.seed_route)
    X = normal_bf16((w.tokens, w.K), w.std_a, w.seed_a)
    W = normal_bf16((w.num_local, w.K, w.N), w.std_b, w.seed_b)
    return ids, X, W


def topk_gates(T: int, top_k: int, seed: int) -> np.ndarray:
    """Positive routing gate weights, T*top_k binary32 in slot order, each token's top_k weights
    summing to one (uniform draws divided by their token's sum)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    g = rng.random((T, top_k), dtype=np.float32) + np.float32(0.05)
    g /= g.sum(axis=1, keepdims=True)
    return np.ascontiguousarray(g.reshape(-1).astype(np.float32))


def combine_inputs(w: Workload):
    """Routing and operands of the MoE combine workload: (topk_ids, H, W, gates).  H has one row
    per routing slot (the capacity of the dispatched order); only the dispatched rows are read."""
    ids = zipf_topk(w.tokens, w.num_experts, w.top_k, w.zipf_s, w.seed_route)
    H = normal_bf16((w.tokens * w.top_k, w.K), w.std_a, w.seed_a)
    W = normal_bf16((w.num_local, w.K, w.N), w.std_b, w.seed_b)
    gates = topk_gates(w.tokens, w.top_k, w.seed_gates)
    return ids, H, W, gates


def attention_inputs(w: Workload):
    """Operands of the ring-attention local share: Q (BH x Sq x D) and the key / value chunks of
    every rank (lists of BH x chunk x D), all ~N(0, 1) bf16.  M = BH, N = local queries,
    K = head dimension, chunks = ranks, tokens = keys per chunk."""
    Q = normal_bf16((w.M, w.N, w.K), w.std_a, w.seed_a)
    Ks = [normal_bf16((w.M, w.tokens, w.K), w.std_a, w.seed_a + 1 + c) for c in range(w.chunks)]
    Vs = [normal_bf16((w.M, w.tokens, w.K), w.std_b, w.seed_b + c) for c in range(w.chunks)]
    return Q, Ks, Vs


def describe() -> List[str]:
    return ["%s: %s" % (k, v) for k, v in WORKLOADS.items()]
