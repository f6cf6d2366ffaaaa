"""Seeded input generators (CPU only): determinism, shapes, value classes, routing law."""
import numpy as np
import torch

import pk_inputs
from _parity import bf16_bits_to_f64


def test_normal_bf16_deterministic_and_rounded_like_torch():
    a = pk_inputs.normal_bf16((64, 33), 0.02, 5)
    b = pk_inputs.normal_bf16((64, 33), 0.02, 5)
    assert a.dtype == np.uint16 and np.array_equal(a, b)
    assert not np.array_equal(a, pk_inputs.normal_bf16((64, 33), 0.02, 6))
    rng = np.random.Generator(np.random.PCG64(5))
    x = rng.standard_normal(size=(64, 33), dtype=np.float32) * np.float32(0.02)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(a, want)
    v = bf16_bits_to_f64(pk_inputs.normal_bf16((256, 256), 0.02, 1))
    assert abs(v.std() - 0.02) < 0.001 and abs(v.mean()) < 0.001


def test_small_int_values_are_exact_integers():
    v = bf16_bits_to_f64(pk_inputs.small_int_bf16((100, 7), -4, 4, 3))
    assert np.all(v == np.round(v)) and v.min() >= -4 and v.max() <= 4


def test_zipf_topk_distinct_experts_and_law():
    ids = pk_inputs.zipf_topk(4096, 256, 8, 1.1, 6003)
    assert ids.shape == (4096, 8) and ids.dtype == np.int32
    assert np.all(np.sort(ids, axis=1)[:, 1:] != np.sort(ids, axis=1)[:, :-1])
    assert ids.min() >= 0 and ids.max() < 256
    counts = np.bincount(ids.reshape(-1), minlength=256)
    assert counts[0] == counts.max() and counts[0] > counts[31] > counts[255]
    # the local share of rank 0 (experts 0..31) under this law holds about two thirds of slots
    local = int(counts[:32].sum())
    assert 20000 < local < 23500
    assert np.array_equal(ids, pk_inputs.zipf_topk(4096, 256, 8, 1.1, 6003))


def test_rs_prefill_statistics():
    d = pk_inputs.rs_prefill(256, 512, 7, 0.0128, 4011, row_block=100)
    assert d.dtype == np.float32 and d.shape == (256, 512)
    assert abs(d.std() - 0.0128 * np.sqrt(7)) < 0.002
    assert np.array_equal(d, pk_inputs.rs_prefill(256, 512, 7, 0.0128, 4011, row_block=64))


def test_workload_table():
    w = pk_inputs.WORKLOADS
    assert set(w) == {"rs_tiny", "ag_8192", "rs_8192", "ar_16384", "moe_dispatch", "moe_combine",
                      "ring_attention"}
    a = w["ring_attention"]
    assert (a.M, a.N, a.K, a.chunks, a.tokens) == (256, 1024, 128, 8, 1024)
    assert a.flops == 4.0 * 256 * 1024 * 8192 * 128
    # the combine returns the dispatch workload's routing: same routing table, D 2048 -> 7168
    c, d = w["moe_combine"], w["moe_dispatch"]
    assert (c.tokens, c.top_k, c.num_experts, c.num_local, c.zipf_s, c.seed_route) == \
        (d.tokens, d.top_k, d.num_experts, d.num_local, d.zipf_s, d.seed_route)
    assert (c.K, c.N) == (d.N, d.K)
    assert (w["rs_8192"].M, w["rs_8192"].N, w["rs_8192"].K) == (8192, 8192, 1024)
    assert (w["ag_8192"].M, w["ag_8192"].N, w["ag_8192"].K) == (8192, 1024, 8192)
    assert w["rs_8192"].flops == 2.0 * 8192 * 8192 * 1024


def test_topk_gates_sum_to_one_per_token():
    g = pk_inputs.topk_gates(50, 8, 3).reshape(50, 8)
    assert g.dtype == np.float32 and np.all(g > 0)
    assert np.allclose(g.sum(axis=1), 1.0, atol=1e-6)
    assert np.array_equal(g.reshape(-1), pk_inputs.topk_gates(50, 8, 3))
