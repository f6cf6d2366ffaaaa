"""pk_ring_attention (one rank's share of ring attention) against the oracle on the GPU, through
the C ABI."""
import numpy as np
import pytest
import torch

import pk_inputs
from _gpu import dev_bf16, host_bits, host_f32, log, require_gpu
from _parity import bf16_bits_to_f64, check_bf16, check_f32

pytestmark = pytest.mark.gpu

D = 128

# Gates per probability mode, derived from the arithmetic.  Scores, the softmax and the row sums
# are fp32; a probability p enters the product with V either rounded to bf16 ("bf16": relative
# error at most the bf16 unit roundoff 2^-8, rms 2^-8/sqrt(6) ~ 1.6e-3 for significands spread
# over [1, 2)) or as a bf16 pair ("split": ~16 significant bits).  Per output element the error
# is then within eps * sum_j p_j |V_j| (exact weights p), with a 2^-14 allowance for the fp32
# parts; the global gates are relF and maxabs / RMS(reference).
MODES = {
    "bf16": dict(eps=2.0 ** -8 + 2.0 ** -14, rel=4e-3, maxabs=4e-2),
    "split": dict(eps=2.0 ** -14, rel=1e-3, maxabs=1e-2),
}


@pytest.fixture(scope="module")
def pk():
    return require_gpu()


def _inputs(BH, Sq, n, Lc, seed, std=1.0):
    Q = pk_inputs.normal_bf16((BH, Sq, D), std, seed)
    K = [pk_inputs.normal_bf16((BH, Lc, D), std, seed + 1 + c) for c in range(n)]
    V = [pk_inputs.normal_bf16((BH, Lc, D), 1.0, seed + 101 + c) for c in range(n)]
    return Q, K, V


def _run(pk, Q, K, V, scale, first=0, dtype=torch.float32, want_lse=True, probs="bf16"):
    BH, Sq, _ = Q.shape
    O = torch.full((BH, Sq, D), float("nan"), dtype=dtype, device="cuda")
    lse = torch.full((BH, Sq), float("nan"), device="cuda") if want_lse else None
    pk.ring_attention(dev_bf16(Q), [dev_bf16(k) for k in K], [dev_bf16(v) for v in V], O, lse,
                      scale=scale, first_chunk=first, probs=probs)
    torch.cuda.synchronize()
    return O, lse


def _weights_bound(Q, K, V, scale, b, rows):
    """Per output element: sum_j p_j |V_j| with the exact softmax weights (numpy, binary64), the
    natural scale of the attention output's rounding error."""
    q = bf16_bits_to_f64(Q[b][rows])
    k = np.concatenate([bf16_bits_to_f64(x[b]) for x in K])
    v = np.abs(np.concatenate([bf16_bits_to_f64(x[b]) for x in V]))
    s = scale * (q @ k.T)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return p @ v


def _check(o, Q, K, V, scale, O, lse, rows_of=None, what="", probs="bf16"):
    g = MODES[probs]
    BH, Sq, _ = Q.shape
    On = host_f32(O.float()) if O.dtype == torch.float32 else None
    Ob = host_bits(O) if O.dtype == torch.bfloat16 else None
    L = host_f32(lse) if lse is not None else None
    for b in range(BH):
        rows = list(range(Sq)) if rows_of is None else rows_of(b)
        R, Rl = o.ring_attention(np.ascontiguousarray(Q[b][rows]), [x[b] for x in K],
                                 [x[b] for x in V], scale)
        bound = g["eps"] * _weights_bound(Q, K, V, scale, b, rows) + 1e-7
        if On is not None:
            check_f32(On[b][rows], R, None, None, "%s b=%d" % (what, b), rel_tol=g["rel"],
                      maxabs_tol=g["maxabs"])
            assert np.all(np.abs(On[b][rows] - R) <= bound), "%s b=%d elementwise" % (what, b)
        else:
            check_bf16(Ob[b][rows], R, o.round_bf16(R), what="%s b=%d" % (what, b), bound=bound,
                       rel_tol=g["rel"])
        if L is not None:
            assert np.max(np.abs(L[b][rows] - Rl)) <= 1e-4, "%s b=%d lse" % (what, b)


@pytest.mark.parametrize("probs", sorted(MODES))
@pytest.mark.parametrize("shape", [(3, 300, 4, 128), (2, 64, 1, 64), (1, 513, 3, 192)],
                         ids=["ragged", "one-chunk", "odd-rows"])
def test_attention_parity_fp32(pk, oracle_mod, shape, probs):
    BH, Sq, n, Lc = shape
    Q, K, V = _inputs(BH, Sq, n, Lc, 301)
    scale = 1.0 / np.sqrt(D)
    log("attention %s probs=%s" % (shape, probs))
    O, lse = _run(pk, Q, K, V, scale, probs=probs)
    _check(oracle_mod.default(), Q, K, V, scale, O, lse, what="fp32 %s %s" % (shape, probs),
           probs=probs)


@pytest.mark.parametrize("probs", sorted(MODES))
def test_attention_parity_bf16_output_and_rotation(pk, oracle_mod, probs):
    """bf16 output (faithfully rounded up to the mode's bound); visiting the chunks from another
    starting chunk gives the same result up to reassociation -- within fp32 rounding for split
    probabilities, within twice the mode's bound for bf16 ones (the running max, and with it each
    probability's rounding, depends on the visiting order)."""
    BH, Sq, n, Lc = 2, 256, 4, 128
    Q, K, V = _inputs(BH, Sq, n, Lc, 311, std=1.5)
    scale = 1.0 / np.sqrt(D)
    O, lse = _run(pk, Q, K, V, scale, dtype=torch.bfloat16, probs=probs)
    _check(oracle_mod.default(), Q, K, V, scale, O, lse, what="bf16 " + probs, probs=probs)
    O1, _ = _run(pk, Q, K, V, scale, first=0, probs=probs)
    O2, _ = _run(pk, Q, K, V, scale, first=3, probs=probs)
    a, b = host_f32(O1), host_f32(O2)
    if probs == "split":
        assert np.max(np.abs(a - b)) <= 1e-5 * max(1.0, np.max(np.abs(a)))
    else:
        for bh in range(BH):
            bound = 2 * MODES[probs]["eps"] * _weights_bound(Q, K, V, scale, bh, list(range(Sq)))
            assert np.all(np.abs(a[bh] - b[bh]) <= bound + 1e-7), bh


@pytest.mark.parametrize("probs", sorted(MODES))
def test_attention_uniform_and_one_hot(pk, oracle_mod, probs):
    """Q = 0: every key weighs the same, O is the mean of the values (checked against the
    oracle) and lse = log(#keys).  One-hot queries with a huge scale: O is exactly the value row
    of the strongest key."""
    BH, Sq, n, Lc = 1, 64, 2, 64
    _, K, V = _inputs(BH, Sq, n, Lc, 321)
    Q0 = np.zeros((BH, Sq, D), dtype=np.uint16)
    O, lse = _run(pk, Q0, K, V, 0.1, probs=probs)
    _check(oracle_mod.default(), Q0, K, V, 0.1, O, lse, what="uniform", probs=probs)
    assert np.allclose(host_f32(lse), np.log(n * Lc), atol=1e-5)
    # one-hot: key j has a single non-zero entry 1 + j // D in column j % D
    Kh = np.zeros((n * Lc, D))
    for j in range(n * Lc):
        Kh[j, j % D] = 1.0 + j // D
    Kb = pk_inputs.f32_to_bf16_bits(Kh.astype(np.float32))
    Kc = [Kb[c * Lc:(c + 1) * Lc][None] for c in range(n)]
    Qh = np.zeros((Sq, D))
    for i in range(Sq):
        Qh[i, (5 * i) % D] = 1.0
    Qb = pk_inputs.f32_to_bf16_bits(Qh.astype(np.float32))[None]
    # scale 4096: every other weight underflows to exactly 0 (the MFMA adds with truncation, so
    # even tiny non-zero terms could move the exact result by an ulp)
    O, _ = _run(pk, Qb, Kc, V, 4096.0, probs=probs)
    got = host_f32(O)[0]
    allv = np.concatenate([bf16_bits_to_f64(v[0]) for v in V])
    for i in range(Sq):
        col = (5 * i) % D
        best = int(np.argmax(Kh[:, col]))
        assert np.array_equal(got[i].astype(np.float64), allv[best]), i


def test_attention_local_share_workload_sampled(pk, oracle_mod):
    """The ring-attention workload's local share: B=16, H=16 (256 batch*head rows), a 8192-token
    sequence over 8 ranks (1024 local queries, 8 chunks of 1024 keys), D=128, bf16 output, both
    probability modes; sampled (batch*head, query) rows against the oracle."""
    w = pk_inputs.WORKLOADS["ring_attention"]
    log("ring attention: generating inputs")
    Q, K, V = pk_inputs.attention_inputs(w)
    scale = 1.0 / np.sqrt(D)
    results = {}
    for probs in sorted(MODES):
        log("ring attention: running, probs=%s" % probs)
        O, lse = _run(pk, Q, K, V, scale, dtype=torch.bfloat16, probs=probs)
        results[probs] = host_bits(O), host_f32(lse)
        del O, lse
    rng = np.random.Generator(np.random.PCG64(331))
    bhs = sorted(set([0, w.M - 1]) | set(int(x) for x in rng.integers(0, w.M, 3)))
    o = oracle_mod.default()
    for b in bhs:
        rows = sorted(set([0, w.N - 1]) | set(int(x) for x in rng.integers(0, w.N, 6)))
        R, Rl = o.ring_attention(np.ascontiguousarray(Q[b][rows]), [x[b] for x in K],
                                 [x[b] for x in V], scale)
        wb = _weights_bound(Q, K, V, scale, b, rows)
        for probs, (Ob, L) in results.items():
            g = MODES[probs]
            check_bf16(Ob[b][rows], R, o.round_bf16(R), what="ring %s b=%d" % (probs, b),
                       bound=g["eps"] * wb + 1e-7, rel_tol=g["rel"])
            assert np.max(np.abs(L[b][rows] - Rl)) <= 1e-4


def test_attention_single_query_sixteen_chunks_from_the_last(pk, oracle_mod):
    """One query row per (batch, head), the most chunks a call takes (16 of 64 keys), visited
    from the last one; fp32 output against the oracle, both probability modes."""
    BH, Sq, n, Lc = 5, 1, 16, 64
    Q, K, V = _inputs(BH, Sq, n, Lc, 341)
    scale = 1.0 / np.sqrt(D)
    for probs in sorted(MODES):
        O, lse = _run(pk, Q, K, V, scale, first=n - 1, probs=probs)
        _check(oracle_mod.default(), Q, K, V, scale, O, lse, what="Sq=1 " + probs, probs=probs)


def test_attention_padded_rows_and_empty_queries(pk, oracle_mod):
    """Row strides beyond the head dimension (Q, K, V and an fp32 O inside wider buffers, and a
    batch*head stride with a gap): only the addressed elements are read and written.  No query
    rows: the call returns without touching O."""
    BH, Sq, n, Lc = 2, 96, 3, 128
    Q, K, V = _inputs(BH, Sq, n, Lc, 351)
    scale = 0.09

    def padded(bits, width, extra_rows=0):
        b, s, _ = bits.shape
        full = np.zeros((b, s + extra_rows, width), dtype=np.uint16)
        full[:, :s, :D] = bits
        return dev_bf16(full)[:, :s, :D]

    Qd = padded(Q, 136, extra_rows=5)
    Kd = [padded(k, 192) for k in K]
    Vd = [padded(v, 144, extra_rows=3) for v in V]
    Ofull = torch.full((BH, Sq, 140), 7.0, device="cuda")
    O = Ofull[:, :, :D]
    lse = torch.full((BH, Sq), float("nan"), device="cuda")
    pk.ring_attention(Qd, Kd, Vd, O, lse, scale=scale)
    torch.cuda.synchronize()
    assert torch.all(Ofull[:, :, D:] == 7.0)   # the padding is never written
    _check(oracle_mod.default(), Q, K, V, scale, O, lse, what="padded")
    # no query rows: nothing happens
    Oe = torch.full((BH, 0, D), 1.0, device="cuda")
    pk.ring_attention(Qd[:, :0], Kd, Vd, Oe, scale=scale)
    torch.cuda.synchronize()
