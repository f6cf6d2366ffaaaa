"""Pins of the oracle: each function checks one property that the pages or the mathematics fix,
against something other than the oracle itself (hand-worked fixtures, closed forms, exact
integer or rational arithmetic, an independent library routine, invariants).  Each takes an
``oracle.Oracle`` and raises AssertionError when the property fails, so the same checks can be
run against copies of the oracle with a planted mistake (tests/test_oracle_mutants.py).
"""
import os
from fractions import Fraction

import numpy as np
import torch

import pk_inputs
from _parity import bf16_bits_to_f64

GOLDEN_DIR = os.path.join(os.path.dirname(__file__), "golden")


def _bits(values):
    return pk_inputs.f32_to_bf16_bits(np.asarray(values, dtype=np.float32))


# ------------------------------------------------------------------------------------------- #
# bf16 rounding (store epilogue, cast pass)                                                     #
# ------------------------------------------------------------------------------------------- #

def golden_bf16_rows():
    rows = []
    for line in open(os.path.join(GOLDEN_DIR, "bf16_rne.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        parts = line.split()
        x = float(parts[0]) if parts[0] in ("inf", "-inf") else float.fromhex(parts[0])
        rows.append((x, int(parts[1], 16), " ".join(parts[2:])))
    return rows


def pin_bf16_golden(o):
    rows = golden_bf16_rows()
    assert len(rows) >= 20
    got = o.round_bf16(np.array([r[0] for r in rows]))
    for (x, want, why), g in zip(rows, got.tolist()):
        assert g == want, "%r: got %#06x want %#06x (%s)" % (x, g, want, why)


def pin_bf16_fixed_points(o):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bf16_bits_to_f64(bits)
    keep = np.isfinite(vals)
    assert np.array_equal(o.round_bf16(vals[keep]), bits[keep])


def pin_bf16_midpoints(o):
    """Between adjacent positive finite bf16 values: the exact midpoint goes to the neighbour
    with an even fraction; points a quarter-gap either side go to the nearer one."""
    pos = np.arange(0x0000, 0x7F7F, dtype=np.uint32).astype(np.uint16)
    lo = bf16_bits_to_f64(pos)
    hi = bf16_bits_to_f64(pos + 1)
    mid = (lo + hi) / 2.0
    q1 = lo + (hi - lo) / 4.0
    q3 = lo + 3.0 * (hi - lo) / 4.0
    even = np.where(pos % 2 == 0, pos, pos + 1).astype(np.int64)
    assert np.array_equal(o.round_bf16(mid).astype(np.int64), even)
    assert np.array_equal(o.round_bf16(q1).astype(np.int64), pos.astype(np.int64))
    assert np.array_equal(o.round_bf16(q3).astype(np.int64), pos.astype(np.int64) + 1)
    assert np.array_equal(o.round_bf16(-mid).astype(np.int64), even | 0x8000)


def pin_bf16_matches_torch(o):
    """Independent library: torch's binary32 -> bfloat16 conversion (round to nearest even)."""
    rng = np.random.Generator(np.random.PCG64(7))
    u = rng.integers(0, 2 ** 32, size=100000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(o.cast_f32_bf16(x), want)
    assert np.array_equal(o.round_bf16(x.astype(np.float64)), want)


def pin_bf16_decode(o):
    """Decode equals numpy's binary32 reinterpretation of (h << 16) on a spread of patterns."""
    sample = np.concatenate([np.arange(0, 65536, 97), [0x7F7F, 0x0001, 0x8001, 0xFF7F, 0x3F80]])
    sample = sample.astype(np.uint16)
    want = bf16_bits_to_f64(sample)
    got = o.bf16_to_f64(sample)
    fin = np.isfinite(want)
    assert np.array_equal(got[fin], want[fin])
    assert np.array_equal(np.isnan(got), np.isnan(want))


BF16_PINS = [pin_bf16_golden, pin_bf16_fixed_points, pin_bf16_midpoints, pin_bf16_matches_torch,
             pin_bf16_decode]


# ------------------------------------------------------------------------------------------- #
# products                                                                                      #
# ------------------------------------------------------------------------------------------- #

def pin_gemm_golden(o):
    rows = [l.split() for l in open(os.path.join(GOLDEN_DIR, "gemm_small.txt"))
            if l.strip() and not l.startswith("#")]
    A = np.array([[float(v) for v in r] for r in rows[0:2]])
    B = np.array([[float(v) for v in r] for r in rows[2:5]])
    R = np.array([[float(v) for v in r] for r in rows[5:7]])
    assert np.array_equal(o.gemm(_bits(A), _bits(B), nthreads=1), R)


def pin_gemm_all_ones(o):
    for M, N, K in [(5, 7, 64), (33, 17, 1024), (3, 130, 8192)]:
        got = o.gemm(_bits(np.ones((M, K))), _bits(np.ones((K, N))))
        assert np.array_equal(got, np.full((M, N), float(K))), (M, N, K)


def pin_gemm_identity(o):
    K, N = 96, 40
    B = pk_inputs.normal_bf16((K, N), 1.0, 11)
    got = o.gemm(_bits(np.eye(K)), B)
    assert np.array_equal(got, bf16_bits_to_f64(B))
    assert np.array_equal(o.round_bf16(got), B)


def pin_gemm_rank_one(o):
    """Only column 0 of A and row 0 of B are non-zero: R = u v^T exactly (distinct M, N, K)."""
    M, N, K = 37, 23, 48
    u = pk_inputs.normal_bf16((M,), 1.0, 3)
    v = pk_inputs.normal_bf16((N,), 1.0, 4)
    A = np.zeros((M, K), dtype=np.uint16); A[:, 0] = u
    B = np.zeros((K, N), dtype=np.uint16); B[0, :] = v
    want = np.outer(bf16_bits_to_f64(u), bf16_bits_to_f64(v))
    assert np.array_equal(o.gemm(A, B), want)


def pin_gemm_small_integers(o):
    """|a|,|b| <= 4, K = 512: every partial sum is an exact integer, so the binary64 result must
    equal numpy's int64 product."""
    M, N, K = 45, 61, 512
    A = pk_inputs.small_int_bf16((M, K), -4, 4, 21)
    B = pk_inputs.small_int_bf16((K, N), -4, 4, 22)
    Ai = bf16_bits_to_f64(A).astype(np.int64)
    Bi = bf16_bits_to_f64(B).astype(np.int64)
    assert np.array_equal(o.gemm(A, B), (Ai @ Bi).astype(np.float64))


def pin_gemm_brute_force_rational(o):
    """Exact rational brute force on tiny shapes: the binary64 sum lies within
    K * 2^-53 * sum|a b| of the exact value."""
    for M, N, K in [(1, 1, 1), (2, 3, 5), (4, 1, 7), (3, 4, 2)]:
        A = pk_inputs.normal_bf16((M, K), 1.0, 100 + M)
        B = pk_inputs.normal_bf16((K, N), 1.0, 200 + N)
        a = bf16_bits_to_f64(A); b = bf16_bits_to_f64(B)
        got = o.gemm(A, B, nthreads=1)
        for i in range(M):
            for j in range(N):
                exact = sum(Fraction(a[i, k]) * Fraction(b[k, j]) for k in range(K))
                absum = sum(abs(a[i, k] * b[k, j]) for k in range(K))
                assert abs(Fraction(got[i, j]) - exact) <= Fraction(K * 2.0 ** -53 * absum)


def pin_gemm_numpy(o):
    """Independent library product over the same decoded inputs (mid size)."""
    M, N, K = 96, 80, 1024
    A = pk_inputs.normal_bf16((M, K), 0.02, 31)
    B = pk_inputs.normal_bf16((K, N), 0.02, 32)
    a, b = bf16_bits_to_f64(A), bf16_bits_to_f64(B)
    got = o.gemm(A, B)
    assert np.all(np.abs(got - a @ b) <= 2 * K * 2.0 ** -53 * (np.abs(a) @ np.abs(b)))


GEMM_PINS = [pin_gemm_golden, pin_gemm_all_ones, pin_gemm_identity, pin_gemm_rank_one,
             pin_gemm_small_integers, pin_gemm_brute_force_rational, pin_gemm_numpy]


# ------------------------------------------------------------------------------------------- #
# reduction into the destination (GEMM+RS / GEMM+AR receiving side)                             #
# ------------------------------------------------------------------------------------------- #

def pin_reduce_integer_producers(o):
    """8 producers with small-integer operands and an integer D0: the sum is exact, so it must
    equal numpy's int64 arithmetic whatever the order."""
    M, N, K = 40, 56, 64
    prods = [(pk_inputs.small_int_bf16((M, K), -3, 3, 300 + p),
              pk_inputs.small_int_bf16((K, N), -3, 3, 400 + p)) for p in range(8)]
    D0 = np.random.Generator(np.random.PCG64(9)).integers(-100, 100, size=(M, N)).astype(np.float32)
    want = D0.astype(np.int64)
    for a, b in prods:
        want = want + bf16_bits_to_f64(a).astype(np.int64) @ bf16_bits_to_f64(b).astype(np.int64)
    assert np.array_equal(o.reduce(D0, prods), want.astype(np.float64))


def pin_reduce_all_ones(o):
    """8 all-ones producers with K = 64 into a zero destination give 512 everywhere."""
    M, N, K = 16, 24, 64
    one_a, one_b = _bits(np.ones((M, K))), _bits(np.ones((K, N)))
    assert np.array_equal(o.reduce(None, [(one_a, one_b)] * 8), np.full((M, N), 512.0))


def pin_reduce_concat_identity(o):
    """sum_p A_p B_p equals one product over the K-concatenated operands (library check)."""
    M, N, K = 32, 48, 64
    prods = [(pk_inputs.normal_bf16((M, K), 1.0, 500 + p),
              pk_inputs.normal_bf16((K, N), 1.0, 600 + p)) for p in range(8)]
    Acat = np.concatenate([bf16_bits_to_f64(a) for a, _ in prods], axis=1)
    Bcat = np.concatenate([bf16_bits_to_f64(b) for _, b in prods], axis=0)
    want = Acat @ Bcat
    got = o.reduce(None, prods)
    assert np.all(np.abs(got - want) <= 4 * 512 * 2.0 ** -53 * (np.abs(Acat) @ np.abs(Bcat)))


def pin_reduce_keeps_destination(o):
    """With one producer the result is D0 plus that product; with a zero product it is D0."""
    M, N, K = 12, 20, 32
    D0 = np.random.Generator(np.random.PCG64(10)).standard_normal((M, N)).astype(np.float32)
    zero_a = np.zeros((M, K), dtype=np.uint16)
    B = pk_inputs.normal_bf16((K, N), 1.0, 12)
    assert np.array_equal(o.reduce(D0, [(zero_a, B)]), D0.astype(np.float64))
    A = pk_inputs.small_int_bf16((M, K), -2, 2, 13)
    Bi = pk_inputs.small_int_bf16((K, N), -2, 2, 14)
    Di = np.round(D0 * 8).astype(np.float32)
    want = Di.astype(np.float64) + bf16_bits_to_f64(A) @ bf16_bits_to_f64(Bi)
    assert np.array_equal(o.reduce(Di, [(A, Bi)]), want)


REDUCE_PINS = [pin_reduce_integer_producers, pin_reduce_all_ones, pin_reduce_concat_identity,
               pin_reduce_keeps_destination]


# ------------------------------------------------------------------------------------------- #
# dispatch                                                                                      #
# ------------------------------------------------------------------------------------------- #

def golden_dispatch():
    vals = {}
    for line in open(os.path.join(GOLDEN_DIR, "dispatch_small.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        k, *v = line.split()
        vals[k] = [int(x) for x in v]
    return vals


def pin_dispatch_golden(o):
    g = golden_dispatch()
    ids = np.array(g["ids"], dtype=np.int32).reshape(g["T"][0], g["top_k"][0])
    counts, offsets, perm = o.dispatch(ids, g["num_experts"][0], g["expert_begin"][0],
                                       g["num_local"][0])
    assert counts.tolist() == g["counts"]
    assert offsets.tolist() == g["offsets"]
    assert perm.tolist() == g["perm"]


def library_dispatch(ids, num_experts, expert_begin, num_local):
    """Same result with numpy only: mask local slots, stable argsort by expert id."""
    flat = np.asarray(ids).reshape(-1).astype(np.int64)
    valid = (flat >= 0) & (flat < num_experts)
    local = valid & (flat >= expert_begin) & (flat < expert_begin + num_local)
    slots = np.nonzero(local)[0]
    e = flat[slots] - expert_begin
    order = np.argsort(e, kind="stable")
    counts = np.bincount(e, minlength=num_local)[:num_local]
    offsets = np.concatenate([[0], np.cumsum(counts)])
    return counts, offsets, slots[order]


def pin_dispatch_library(o):
    for seed, (T, top_k, E, begin, nl) in enumerate([(4096, 8, 256, 0, 32), (1000, 4, 64, 16, 16),
                                                       (333, 2, 8, 5, 3), (50, 6, 300, 290, 10)]):
        ids = pk_inputs.zipf_topk(T, E, top_k, 1.1, 70 + seed)
        c, off, perm = o.dispatch(ids, E, begin, nl)
        wc, woff, wperm = library_dispatch(ids, E, begin, nl)
        assert np.array_equal(c, wc) and np.array_equal(off, woff) and np.array_equal(perm, wperm)


def pin_dispatch_invariants(o):
    T, top_k, E, begin, nl = 777, 8, 64, 8, 24
    ids = pk_inputs.zipf_topk(T, E, top_k, 0.7, 81)
    c, off, perm = o.dispatch(ids, E, begin, nl)
    flat = ids.reshape(-1)
    assert off[0] == 0 and np.all(np.diff(off) >= 0) and np.array_equal(np.diff(off), c)
    local = np.nonzero((flat >= begin) & (flat < begin + nl))[0]
    assert off[-1] == local.size == perm.size
    assert np.array_equal(np.sort(perm), local)          # a bijection onto the local slots
    for e in range(nl):
        seg = perm[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)                   # stable: ascending slots
        assert np.all(flat[seg] == begin + e)             # every slot routed to this expert


def pin_dispatch_special_cases(o):
    # no local tokens
    ids = np.full((10, 2), 7, dtype=np.int32)
    c, off, perm = o.dispatch(ids, 8, 0, 4)
    assert c.tolist() == [0, 0, 0, 0] and off.tolist() == [0] * 5 and perm.size == 0
    # a single token
    c, off, perm = o.dispatch(np.array([[1, 3]], dtype=np.int32), 4, 0, 4)
    assert c.tolist() == [0, 1, 0, 1] and off.tolist() == [0, 0, 1, 1, 2] and perm.tolist() == [0, 1]
    # every token to one expert (top_k = 1)
    ids = np.full((9, 1), 2, dtype=np.int32)
    c, off, perm = o.dispatch(ids, 4, 0, 4)
    assert c.tolist() == [0, 0, 9, 0] and perm.tolist() == list(range(9))
    # ids outside [0, num_experts) are never local, even inside the local window
    ids = np.array([[4, 5], [2, -1], [3, 2]], dtype=np.int32)
    c, off, perm = o.dispatch(ids, 4, 2, 4)
    assert c.tolist() == [2, 1, 0, 0] and perm.tolist() == [2, 5, 4]


DISPATCH_PINS = [pin_dispatch_golden, pin_dispatch_library, pin_dispatch_invariants,
                 pin_dispatch_special_cases]


# ------------------------------------------------------------------------------------------- #
# grouped expert product                                                                        #
# ------------------------------------------------------------------------------------------- #

def pin_grouped_selection_weights(o):
    """W_e[k, n] = 2^(e mod 8 - 4) if k == n + c_e else 0, with X[t, k] = (t + 1) * 2^(k mod 8 - 4)
    (at most 6 significant bits, exact in bf16): Y[j, n] = 2^(e mod 8 - 4) * X[perm[j] // top_k,
    n + c_e] exactly.  Token, column shift and expert scale are all recoverable from Y, so this
    pins gather, offsets and the expert choice through the product."""
    T, top_k, E, nl, K, N = 40, 3, 12, 6, 64, 16
    ids = pk_inputs.zipf_topk(T, E, top_k, 0.5, 91)
    c, off, perm = o.dispatch(ids, E, 0, nl)
    tt = np.arange(T)[:, None].astype(np.float64)
    kk = np.arange(K)[None, :].astype(np.float64)
    Xv = (tt + 1.0) * 2.0 ** (kk % 8 - 4)
    X = _bits(Xv)
    assert np.array_equal(bf16_bits_to_f64(X), Xv)
    W = np.zeros((nl, K, N), dtype=np.float64)
    shift = [(3 * e) % (K - N + 1) for e in range(nl)]
    for e in range(nl):
        for n in range(N):
            W[e, n + shift[e], n] = 2.0 ** (e % 8 - 4)
    Y = o.grouped_gemm(off, perm, top_k, X, _bits(W))
    for e in range(nl):
        for j in range(off[e], off[e + 1]):
            t = perm[j] // top_k
            want = 2.0 ** (e % 8 - 4) * Xv[t, shift[e]:shift[e] + N]
            assert np.array_equal(Y[j], want), (e, j)


def pin_grouped_one_expert_is_gemm(o):
    """One local expert, top_k = 1, every token routed to it: the grouped product is the plain
    product of X with W_0 (rows in token order); checked with the library product."""
    T, K, N = 50, 96, 24
    ids = np.zeros((T, 1), dtype=np.int32)
    c, off, perm = o.dispatch(ids, 1, 0, 1)
    assert perm.tolist() == list(range(T))
    X = pk_inputs.normal_bf16((T, K), 1.0, 95)
    W = pk_inputs.normal_bf16((1, K, N), 0.02, 96)
    Y = o.grouped_gemm(off, perm, 1, X, W)
    x, w = bf16_bits_to_f64(X), bf16_bits_to_f64(W[0])
    assert np.all(np.abs(Y - x @ w) <= 2 * K * 2.0 ** -53 * (np.abs(x) @ np.abs(w)))


def pin_grouped_brute_force(o):
    """Tiny case against exact rationals, row by row, expert by expert."""
    T, top_k, E, nl, K, N = 6, 2, 5, 3, 5, 3
    ids = np.array([[0, 2], [1, 0], [2, 4], [0, 1], [3, 2], [1, 2]], dtype=np.int32)
    c, off, perm = o.dispatch(ids, E, 0, nl)
    X = pk_inputs.normal_bf16((T, K), 1.0, 97)
    W = pk_inputs.normal_bf16((nl, K, N), 1.0, 98)
    x, w = bf16_bits_to_f64(X), bf16_bits_to_f64(W)
    Y = o.grouped_gemm(off, perm, top_k, X, W)
    flat = ids.reshape(-1)
    j = 0
    for e in range(nl):
        for f in range(T * top_k):
            if flat[f] != e:
                continue
            t = f // top_k
            for n in range(N):
                exact = sum(Fraction(x[t, k]) * Fraction(w[e, k, n]) for k in range(K))
                absum = sum(abs(x[t, k] * w[e, k, n]) for k in range(K))
                assert abs(Fraction(Y[j, n]) - exact) <= Fraction(K * 2.0 ** -53 * absum)
            j += 1
    assert j == Y.shape[0]


GROUPED_PINS = [pin_grouped_selection_weights, pin_grouped_one_expert_is_gemm,
                pin_grouped_brute_force]

def _dispatched_row(ids, begin, nl):
    """Row index of every local routing slot in the stable expert-major order, counted directly
    from the routing table (independent of the oracle's dispatch): slots of lower experts first,
    then earlier slots of the same expert."""
    flat = np.asarray(ids).reshape(-1)
    local = (flat >= begin) & (flat < begin + nl)
    row = {}
    for f in range(flat.size):
        if not local[f]:
            continue
        e = flat[f] - begin
        lower = int(np.sum(local & (flat - begin < e)))
        earlier = int(np.sum(local[:f] & (flat[:f] == flat[f])))
        row[f] = lower + earlier
    return row


def pin_combine_selection_weights(o):
    """Combine with selection weights: W_e[k, n] = 2^(e mod 8 - 4) if k == n + c_e, H[j, k] =
    (j + 1) * 2^(k mod 8 - 4), gates 2^-(f mod 4).  Every term and every sum is exact, so
    out[t, n] = sum over the local slots f of t of gate_f * 2^(e mod 8 - 4) * H[row(f), n + c_e]
    exactly, with row(f) counted from the routing table.  Pins the token each row goes back to, the
    gate it is weighted by, the expert weight and the destination term."""
    T, top_k, E, begin, nl, K, N = 30, 3, 10, 2, 5, 48, 12
    ids = pk_inputs.zipf_topk(T, E, top_k, 0.3, 131)
    c, off, perm = o.dispatch(ids, E, begin, nl)
    rows = int(off[-1])
    jj = np.arange(rows)[:, None].astype(np.float64)
    kk = np.arange(K)[None, :].astype(np.float64)
    Hv = (jj + 1.0) * 2.0 ** (kk % 8 - 4)
    H = _bits(Hv)
    assert np.array_equal(bf16_bits_to_f64(H), Hv)
    W = np.zeros((nl, K, N), dtype=np.float64)
    shift = [(5 * e) % (K - N + 1) for e in range(nl)]
    for e in range(nl):
        for n in range(N):
            W[e, n + shift[e], n] = 2.0 ** (e % 8 - 4)
    gates = (2.0 ** -(np.arange(T * top_k) % 4)).astype(np.float32)
    out0 = np.arange(T * N, dtype=np.float64).reshape(T, N) * 0.25
    got = o.combine(T, top_k, off, perm, H, _bits(W), gates, out0=out0)
    want = out0.copy()
    row = _dispatched_row(ids, begin, nl)
    flat = ids.reshape(-1)
    for f, j in row.items():
        e = flat[f] - begin
        want[f // top_k] += float(gates[f]) * 2.0 ** (e % 8 - 4) * Hv[j, shift[e]:shift[e] + N]
    assert np.array_equal(got, want)


def pin_combine_brute_force(o):
    """Tiny combine against exact rationals, slot by slot from the routing table."""
    T, top_k, E, begin, nl, K, N = 5, 2, 4, 1, 3, 4, 3
    ids = np.array([[1, 3], [2, 1], [0, 3], [3, 2], [1, 0]], dtype=np.int32)
    c, off, perm = o.dispatch(ids, E, begin, nl)
    rows = int(off[-1])
    H = pk_inputs.normal_bf16((rows, K), 1.0, 141)
    W = pk_inputs.normal_bf16((nl, K, N), 1.0, 142)
    gates = np.random.Generator(np.random.PCG64(143)).random(T * top_k).astype(np.float32)
    h, w = bf16_bits_to_f64(H), bf16_bits_to_f64(W)
    got = o.combine(T, top_k, off, perm, H, W, gates)
    row = _dispatched_row(ids, begin, nl)
    flat = ids.reshape(-1)
    for t in range(T):
        for n in range(N):
            exact, bound = Fraction(0), Fraction(0)
            for k in range(top_k):
                f = t * top_k + k
                if f not in row:
                    continue
                e, j = flat[f] - begin, row[f]
                g = Fraction(float(gates[f]))
                exact += g * sum(Fraction(h[j, q]) * Fraction(w[e, q, n]) for q in range(K))
                bound += abs(g) * sum(abs(Fraction(h[j, q]) * Fraction(w[e, q, n])) for q in range(K))
            assert abs(Fraction(got[t, n]) - exact) <= bound * Fraction(2 * (K + top_k) * 2.0 ** -53)


def pin_combine_token_subset(o):
    """Computing only some tokens gives exactly those rows of the full result (the rest is the
    initial value)."""
    T, top_k, E, nl, K, N = 24, 4, 8, 8, 32, 16
    ids = pk_inputs.zipf_topk(T, E, top_k, 1.0, 151)
    c, off, perm = o.dispatch(ids, E, 0, nl)
    H = pk_inputs.normal_bf16((int(off[-1]), K), 1.0, 152)
    W = pk_inputs.normal_bf16((nl, K, N), 0.1, 153)
    gates = np.random.Generator(np.random.PCG64(154)).random(T * top_k).astype(np.float32)
    full = o.combine(T, top_k, off, perm, H, W, gates)
    sub = [1, 7, 19]
    part = o.combine(T, top_k, off, perm, H, W, gates, tokens=sub)
    assert np.array_equal(part[sub], full[sub])
    others = [t for t in range(T) if t not in sub]
    assert np.all(part[others] == 0.0)


COMBINE_PINS = [pin_combine_selection_weights, pin_combine_brute_force, pin_combine_token_subset]

def pin_attention_uniform_scores(o):
    """Q = 0 makes every score 0: the softmax is uniform over all keys of all chunks, so O is the
    exact mean of the value rows and lse = log(number of keys)."""
    Sq, D, Sk, n = 4, 16, 6, 3
    Q = np.zeros((Sq, D), dtype=np.uint16)
    Ks = [pk_inputs.normal_bf16((Sk, D), 1.0, 201 + c) for c in range(n)]
    Vs = [pk_inputs.normal_bf16((Sk, D), 1.0, 211 + c) for c in range(n)]
    O, lse = o.ring_attention(Q, Ks, Vs, 0.125)
    allv = np.concatenate([bf16_bits_to_f64(v) for v in Vs])
    for d in range(D):
        mean = sum(Fraction(x) for x in allv[:, d]) / (Sk * n)
        for i in range(Sq):
            assert abs(Fraction(O[i, d]) - mean) <= Fraction(2.0 ** -48) * (1 + abs(mean))
    assert np.allclose(lse, np.log(Sk * n), rtol=0, atol=1e-15)


def pin_attention_one_hot(o):
    """Query i points at exactly one key (one-hot rows, a huge scale): every other weight
    underflows to zero, so O[i] is that key's value row bit for bit and lse is its score."""
    D, Sk, n = 16, 5, 4
    keys = [(c, j) for c in range(n) for j in range(Sk)]
    K = np.zeros((n * Sk, D))
    for idx in range(n * Sk):
        K[idx, idx % D] = 1.0 + (idx // D)          # distinct (column, magnitude) per key
    picks = [0, 7, 13, 19, 11]
    Q = np.zeros((len(picks), D))
    for i, idx in enumerate(picks):
        Q[i, idx % D] = 1.0
    scale = 4096.0
    Kb, Qb = _bits(K), _bits(Q)
    Vs = [pk_inputs.normal_bf16((Sk, D), 1.0, 221 + c) for c in range(n)]
    O, lse = o.ring_attention(Qb, [Kb[c * Sk:(c + 1) * Sk] for c in range(n)], Vs, scale)
    allv = np.concatenate([bf16_bits_to_f64(v) for v in Vs])
    for i, idx in enumerate(picks):
        col, mag = idx % D, 1.0 + idx // D
        best = max(range(n * Sk), key=lambda j: K[j, col])  # the strongest key in that column
        assert np.array_equal(O[i], allv[best]), (i, idx, best)
        assert lse[i] == scale * K[best, col]
    del keys


def pin_attention_two_keys_logistic(o):
    """Two keys in two chunks: the weights are the logistic function of the score difference,
    p = 1 / (1 + exp(s2 - s1)), so O = p V1 + (1 - p) V2 and lse = s1 + log1p(exp(s2 - s1))."""
    D = 8
    Q = pk_inputs.normal_bf16((3, D), 1.0, 231)
    K1, K2 = pk_inputs.normal_bf16((1, D), 1.0, 232), pk_inputs.normal_bf16((1, D), 1.0, 233)
    V1, V2 = pk_inputs.normal_bf16((1, D), 1.0, 234), pk_inputs.normal_bf16((1, D), 1.0, 235)
    scale = 0.5
    O, lse = o.ring_attention(Q, [K1, K2], [V1, V2], scale)
    q, k1, k2 = bf16_bits_to_f64(Q), bf16_bits_to_f64(K1)[0], bf16_bits_to_f64(K2)[0]
    v1, v2 = bf16_bits_to_f64(V1)[0], bf16_bits_to_f64(V2)[0]
    for i in range(3):
        s1 = scale * float(sum(Fraction(a) * Fraction(b) for a, b in zip(q[i], k1)))
        s2 = scale * float(sum(Fraction(a) * Fraction(b) for a, b in zip(q[i], k2)))
        p = 1.0 / (1.0 + np.exp(s2 - s1))
        assert np.allclose(O[i], p * v1 + (1.0 - p) * v2, rtol=1e-14, atol=1e-15)
        assert abs(lse[i] - (s1 + np.log1p(np.exp(s2 - s1)))) <= 1e-14 * (1 + abs(lse[i]))


def pin_attention_chunking_invariance(o):
    """The log-sum-exp merge is exact up to rounding: splitting the keys into chunks differently
    or visiting the chunks in another order gives the same O and lse (binary64 rounding only)."""
    Sq, D, S = 6, 32, 24
    Q = pk_inputs.normal_bf16((Sq, D), 1.0, 241)
    K = pk_inputs.normal_bf16((S, D), 1.0, 242)
    V = pk_inputs.normal_bf16((S, D), 1.0, 243)
    one = o.ring_attention(Q, [K], [V], 0.3)
    for parts in ([8, 8, 8], [12, 12], [4, 4, 4, 4, 4, 4]):
        edges = np.cumsum([0] + parts)
        Ks = [K[edges[c]:edges[c + 1]] for c in range(len(parts))]
        Vs = [V[edges[c]:edges[c + 1]] for c in range(len(parts))]
        for order in (list(range(len(parts))), list(reversed(range(len(parts))))):
            O, lse = o.ring_attention(Q, [Ks[c] for c in order], [Vs[c] for c in order], 0.3)
            assert np.allclose(O, one[0], rtol=0, atol=1e-13)
            assert np.allclose(lse, one[1], rtol=0, atol=1e-13)


ATTENTION_PINS = [pin_attention_uniform_scores, pin_attention_one_hot,
                  pin_attention_two_keys_logistic, pin_attention_chunking_invariance]

ALL_PINS = (BF16_PINS + GEMM_PINS + REDUCE_PINS + DISPATCH_PINS + GROUPED_PINS + COMBINE_PINS
            + ATTENTION_PINS)
