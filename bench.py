#!/usr/bin/env python3
"""Benchmark of the one-GPU GEMM+RS local share at N=8192 on MI355X.

One step = one pass of the hot path over the workload: pk_gemm_reduce of A (8192 x 1024 bf16)
times B (1024 x 8192 bf16) into an 8192 x 8192 fp32 destination held as 8 row shards of 1024
rows, pre-filled with 7 other producers' partials (tile schedule, operand staging, MFMA loop and
the reduction epilogue, all in the HIP kernels).  Inputs are seeded synthetic data resident in
HBM before the timed region.

Prints ONE JSON line (rank 0): TFLOP/s and the fraction of the bf16 dense MFMA peak, the
roofline of the dominant kernel (timed with HIP events on the stream it runs on), the atomic
reduction mode measured beside the owner mode, and the oracle's CPU time on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--mode owner|atomic] [--workload rs_8192|...]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# The sources each workload's dominant kernel is built from: a counter record stays valid until
# one of them changes.
KERNEL_SOURCES = {
    "gemm": ("pk_gemm.hip", "pk_device.h", "pk_internal.h"),
    "attention": ("pk_attention.hip", "pk_device.h", "pk_attention.h"),
}
WORKLOAD_TITLES = {
    "rs_8192": "GEMM+RS local share N=8192",
    "ag_8192": "AG+GEMM local share N=8192",
    "ar_16384": "GEMM+AR local share N=16384",
    "moe_dispatch": "token dispatch + expert GEMM (MoE local share)",
    "moe_combine": "MoE combine (expert down-projection + gated scatter)",
    "ring_attention": "ring attention local share B=16 H=16 D=128",
    "rs_tiny": "GEMM+RS tiny (8 producers of 512x512x64)",
}


def kernel_family(workload: str) -> str:
    return "attention" if workload == "ring_attention" else "gemm"


def _code_only(text: str) -> str:
    """Source text without comments and with whitespace collapsed: what the compiler sees."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(family: str = "gemm") -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[family]:
        text = open(os.path.join(ROOT, "gemm_tile_granular_bf16_amd", "csrc", f)).read()
        h.update(_code_only(text).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, mode: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they were taken on the
    current source of the workload's kernel (null otherwise)."""
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    rec = data.get("%s/%s" % (workload, mode))
    if not rec or rec.get("source_hash") != kernel_source_hash(kernel_family(workload)):
        return None
    return rec.get("bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="rs_8192",
                    choices=["rs_8192", "ag_8192", "ar_16384", "moe_dispatch", "moe_combine",
                             "ring_attention", "rs_tiny"])
    ap.add_argument("--mode", default="owner", choices=["owner", "atomic"])
    ap.add_argument("--no-variant", action="store_true", help="skip the other reduce mode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="launch every step from Python instead of replaying a captured HIP graph")
    ap.add_argument("--no-detail", action="store_true",
                    help="skip the per-call, flushed and store-epilogue timings after the timed steps")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--sweep", action="store_true",
                    help="the pages' N sweep of the AG and RS local shares (context, several lines)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 256 MiB device copy (reference for the HBM byte counters)")
    return ap.parse_args()


def sweep(torch, pk, calls):
    """The pages' shape sweep as context (not the headline): the GEMM+RS local share
    N x N x N/8 (owner and atomic reduction into 8 row shards of an fp32 destination) and the
    AG+GEMM local share N x N/8 x N (A as 8 row-chunks, bf16 output), for N = 2048 .. 16384.
    Inputs are seeded normals drawn on the device; one JSON line per point, median per call."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(9001)
    rnd = lambda r, c: (torch.randn(r, c, generator=gen, device="cuda") * 0.02).to(torch.bfloat16)
    stream = torch.cuda.current_stream()
    for n in (2048, 4096, 8192, 16384):
        k = n // 8
        A, B = rnd(n, k), rnd(k, n)
        D = torch.zeros(n, n, device="cuda")
        shards = list(D.split(n // 8))
        flops = 2.0 * n * n * k
        for mode, mid in (("owner", pk.PK_REDUCE_OWNER), ("atomic", pk.PK_REDUCE_ATOMIC)):
            fn = lambda: pk.gemm_reduce(A, B, shards, mode=mid)
            for _ in range(3):
                fn()
            ms = float(np.median(per_call_ms(fn, torch, stream, calls)))
            print(json.dumps({"sweep": "gemm_rs", "N": n, "reduce": mode, "M": n, "N_cols": n, "K": k,
                              "median_ms": round(ms, 5), "tflops": round(flops / ms / 1e9, 1)}), flush=True)
        del A, B, D, shards
        A = rnd(n, n)
        chunks = list(A.split(n // 8))
        B = rnd(n, k)
        C = torch.empty(n, k, dtype=torch.bfloat16, device="cuda")
        fn = lambda: pk.gemm(chunks, B, C)
        for _ in range(3):
            fn()
        ms = float(np.median(per_call_ms(fn, torch, stream, calls)))
        print(json.dumps({"sweep": "ag_gemm", "N": n, "M": n, "N_cols": k, "K": n,
                          "median_ms": round(ms, 5), "tflops": round(flops / ms / 1e9, 1)}), flush=True)
        del A, chunks, B, C
        torch.cuda.empty_cache()


def calibrate_copy(torch):
    """A plain device-to-device copy of a known size: the HBM byte counters of a profiler run of
    this mode give the scale factor between counter readings and bytes moved."""
    n = 64 * 1024 * 1024  # 256 MiB of fp32
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes_read": 4 * n, "calibrate_copy_bytes_written": 4 * n,
                      "launches": 5}), flush=True)


class Timer:
    """HIP events recorded on the stream the kernels are launched on: one before the first timed
    step and one after the last, so the average device time per step carries no per-step event
    overhead (back-to-back launches on one stream)."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream
        self.start = torch.cuda.Event(enable_timing=True)
        self.end = torch.cuda.Event(enable_timing=True)
        self.steps = 0

    def begin(self):
        self.start.record(self.stream)

    def step(self, fn, count=1):
        fn()
        self.steps += count

    def finish(self):
        self.end.record(self.stream)

    def kernel_ms(self):
        return self.start.elapsed_time(self.end) / max(self.steps, 1)


def setup_workload(name, mode, torch, pk):
    """Returns (step_fn, flops, algorithmic bytes per launch, bound, description)."""
    import pk_inputs
    w = pk_inputs.WORKLOADS[name]
    dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)
    mode_id = pk.PK_REDUCE_OWNER if mode == "owner" else pk.PK_REDUCE_ATOMIC
    if w.kind == "reduce":
        prods = [pk_inputs.producer_operands(w, p) for p in range(w.producers)]
        if w.prefill_partials:
            D0 = pk_inputs.rs_prefill(w.M, w.N, w.prefill_partials, w.prefill_std, w.prefill_seed)
            D = torch.from_numpy(D0).cuda()
            del D0
        else:
            D = torch.zeros((w.M, w.N), device="cuda")
        shards = list(D.split(w.M // w.shards))
        ops = [(dev(a), dev(b)) for a, b in prods]
        out = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda") if w.cast_bf16 else None

        def step():
            for i, (a, b) in enumerate(ops):
                pk.gemm_reduce(a, b, shards, mode=mode_id,
                               out_bf16=out if (out is not None and i == len(ops) - 1) else None)
        flops = w.flops
        # A and B once, destination read + written once per producer; the bf16 output is written
        # by the owner epilogue (2 B per element) or by a cast pass that re-reads the destination
        nbytes = sum(2 * (w.M * w.K + w.K * w.N) + 8 * w.M * w.N for _ in prods)
        if w.cast_bf16:
            nbytes += (2 if mode == "owner" else 6) * w.M * w.N
        desc = {"M": w.M, "N": w.N, "K": w.K, "producers": w.producers, "shards": w.shards,
                "prefill_partials": w.prefill_partials, "reduce": mode,
                "cast_bf16": w.cast_bf16}
        if w.producers == 1:
            # the same product with a plain store epilogue (bf16 C): the reference point for how
            # much of the reduction stays exposed
            a0, b0 = ops[0]
            c_store = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
            desc["_gemm_only"] = lambda: pk.gemm(a0, b0, c_store)
            return step, flops, nbytes, desc, (D, ops, out, c_store)
        return step, flops, nbytes, desc, (D, ops, out)
    if w.kind == "gemm":
        A = pk_inputs.normal_bf16((w.M, w.K), w.std_a, w.seed_a)
        B = pk_inputs.normal_bf16((w.K, w.N), w.std_b, w.seed_b)
        rows = w.M // w.chunks
        chunks = [dev(A[i * rows:(i + 1) * rows]) for i in range(w.chunks)]
        Bd = dev(B)
        C = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")

        def step():
            pk.gemm(chunks, Bd, C, first_chunk=0)
        nbytes = 2 * (w.M * w.K + w.K * w.N + w.M * w.N)
        desc = {"M": w.M, "N": w.N, "K": w.K, "chunks": w.chunks, "out": "bf16"}
        return step, w.flops, nbytes, desc, (chunks, Bd, C)
    if w.kind == "attention":
        Q, Ks, Vs = pk_inputs.attention_inputs(w)
        Qd = dev(Q)
        Kd = [dev(k) for k in Ks]
        Vd = [dev(v) for v in Vs]
        del Q, Ks, Vs
        O = torch.empty((w.M, w.N, w.K), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((w.M, w.N), device="cuda")

        def step():
            pk.ring_attention(Qd, Kd, Vd, O, lse, first_chunk=0, probs="bf16")
        keys = w.chunks * w.tokens
        # Q, every key and value once, O and lse written once
        nbytes = 2 * w.M * w.N * w.K * 2 + 2 * 2 * w.M * keys * w.K + 4 * w.M * w.N
        desc = {"batch_heads": w.M, "local_queries": w.N, "head_dim": w.K, "chunks": w.chunks,
                "keys_per_chunk": w.tokens, "out": "bf16", "probs": "bf16"}
        return step, w.flops, nbytes, desc, (Qd, Kd, Vd, O, lse)
    if w.kind == "combine":
        ids, H, W, gates = pk_inputs.combine_inputs(w)
        ids_d = torch.from_numpy(ids).cuda()
        Hd, Wd, gd = dev(H), dev(W), torch.from_numpy(gates).cuda()
        offsets = torch.empty(w.num_local + 1, dtype=torch.int32, device="cuda")
        perm = torch.empty(w.tokens * w.top_k, dtype=torch.int32, device="cuda")
        # the dispatch tables come from the library's own dispatch (a product with N = 8 that
        # is not timed); the combine consumes them as the step after the expert FFN would
        Xs = torch.zeros((w.tokens, 8), dtype=torch.bfloat16, device="cuda")
        Ws = torch.zeros((w.num_local, 8, 8), dtype=torch.bfloat16, device="cuda")
        Ys = torch.empty((w.tokens * w.top_k, 8), dtype=torch.bfloat16, device="cuda")
        gws = torch.empty(pk.grouped_gemm_workspace_size(w.tokens, w.top_k, w.num_local),
                          dtype=torch.uint8, device="cuda")
        pk.grouped_gemm(ids_d, Xs, Ws, w.num_experts, w.expert_begin, offsets, perm, Ys, gws)
        torch.cuda.synchronize()
        del Xs, Ws, Ys, gws
        rows = int(offsets[-1].item())
        out = torch.zeros((w.tokens, w.N), device="cuda")
        ws = torch.empty(pk.grouped_combine_workspace_size(w.num_local), dtype=torch.uint8,
                         device="cuda")

        def step():
            pk.grouped_combine(w.tokens, w.top_k, offsets, perm, Hd, Wd, gd, out, ws)
        flops = 2.0 * rows * w.K * w.N
        # weights and dispatched rows once, output rows read and written once
        nbytes = 2 * (w.num_local * w.K * w.N + rows * w.K) + 8 * w.tokens * w.N
        desc = {"tokens": w.tokens, "D_expert": w.K, "D": w.N, "top_k": w.top_k,
                "experts": w.num_experts, "local_experts": w.num_local, "local_rows": rows,
                "atomic_payload_bytes": 4 * rows * w.N}
        return step, flops, nbytes, desc, (ids_d, Hd, Wd, gd, offsets, perm, out, ws)
    # grouped
    ids, X, W = pk_inputs.moe_inputs(w)
    ids_d = torch.from_numpy(ids).cuda()
    Xd, Wd = dev(X), dev(W)
    offsets = torch.empty(w.num_local + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(w.tokens * w.top_k, dtype=torch.int32, device="cuda")
    Y = torch.empty((w.tokens * w.top_k, w.N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(pk.grouped_gemm_workspace_size(w.tokens, w.top_k, w.num_local),
                     dtype=torch.uint8, device="cuda")

    def step():
        pk.grouped_gemm(ids_d, Xd, Wd, w.num_experts, w.expert_begin, offsets, perm, Y, ws)
    step()  # the routed row count (device result) prices the step
    torch.cuda.synchronize()
    rows = int(offsets[-1].item())
    flops = 2.0 * rows * w.K * w.N
    nbytes = 2 * (w.num_local * w.K * w.N + w.tokens * w.K + rows * w.N)
    desc = {"tokens": w.tokens, "D": w.K, "D_expert": w.N, "top_k": w.top_k,
            "experts": w.num_experts, "local_experts": w.num_local, "local_rows": rows}
    return step, flops, nbytes, desc, (ids_d, Xd, Wd, offsets, perm, Y, ws)


def per_call_ms(fn, torch, stream, calls, flush=None):
    """Device time of each call between its own pair of events (outside the timed region);
    `flush` runs before each call, outside the pair."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(calls)]
    for a, b in ev:
        if flush is not None:
            flush()
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def detail_timing(step, gemm_only, torch, stream, calls):
    """Median and mean per call, the same with L2 and the 256 MB memory-side cache flushed by a
    512 MiB write before each call, and for a reduction the same product with a plain store
    epilogue: (t_reduce - t_store) / t_reduce is the part of the reduction left exposed."""
    warm = per_call_ms(step, torch, stream, calls)
    scratch = torch.empty(128 << 20, device="cuda")  # 512 MiB
    cold = per_call_ms(step, torch, stream, calls, flush=lambda: scratch.fill_(1.0))
    del scratch
    out = {"calls": calls, "median_ms": round(float(np.median(warm)), 5),
           "mean_ms": round(float(np.mean(warm)), 5),
           "flushed_median_ms": round(float(np.median(cold)), 5)}
    if gemm_only is not None:
        for _ in range(3):
            gemm_only()
        g = float(np.median(per_call_ms(gemm_only, torch, stream, calls)))
        out["store_epilogue_median_ms"] = round(g, 5)
        out["reduction_exposed_frac"] = round((out["median_ms"] - g) / out["median_ms"], 4)
    return out


def device_peak(torch):
    """bf16 dense MFMA peak from the device: CUs x highest shader clock x 4096 flop/clk/CU (the
    clock from the driver's DPM table; None where it cannot be read)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    mhz = None
    import glob
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            levels = [int(l.split(":")[1].strip().lower().replace("mhz", "").strip("* "))
                      for l in open(f) if ":" in l]
        except (OSError, ValueError, IndexError):
            continue
        if levels:
            mhz = max(levels)
            break
    if mhz is None:
        return {"cus": cus, "max_sclk_mhz": None, "tflops": None}
    return {"cus": cus, "max_sclk_mhz": mhz, "tflops": round(cus * mhz * 1e6 * 4096 / 1e12, 1)}


# Workloads whose step is replayed from a captured HIP graph: their kernels allocate nothing,
# clear nothing with memset nodes and give the same bits on every replay (tests/test_gpu_graph.py).
# The grouped workloads (dispatch counters, split-tail partial sums) run eagerly.
GRAPH_KINDS = ("reduce", "gemm", "attention")


def graph_batch(steps: int) -> int:
    """Steps per captured graph: the largest divisor of `steps` up to 10."""
    if steps < 1:
        return 1
    return max(d for d in range(1, min(steps, 10) + 1) if steps % d == 0)


def capture_steps(step, per, torch):
    """`per` steps captured into one graph on a side stream (the stream the binding sees as
    current while capturing)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for _ in range(per):
            step()
    torch.cuda.synchronize()
    return g


def wall_ms_per_step(fn, steps, torch):
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def run_gpu(name, mode, steps, warmup, torch, pk, detail=False, graph=False):
    import pk_inputs
    step, flops, nbytes, desc, keep = setup_workload(name, mode, torch, pk)
    gemm_only = desc.pop("_gemm_only", None)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    graph = graph and pk_inputs.WORKLOADS[name].kind in GRAPH_KINDS
    eager_ms, g, per = None, None, 1
    if graph:
        eager_ms = wall_ms_per_step(step, min(steps, 20), torch)
        per = graph_batch(steps)
        g = capture_steps(step, per, torch)
        g.replay()  # untimed
        torch.cuda.synchronize()
    desc["launch"] = "hip graph of %d steps" % per if graph else "eager"
    timer = Timer(torch, stream)
    t0 = time.perf_counter()
    timer.begin()
    if graph:
        for _ in range(steps // per):
            timer.step(g.replay, per)
    else:
        for _ in range(steps):
            timer.step(step)
    timer.finish()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kms = timer.kernel_ms()
    det = detail_timing(step, gemm_only, torch, stream, min(steps, 50)) if detail else None
    del keep, gemm_only, g
    torch.cuda.empty_cache()
    return {"ms_per_step": wall * 1e3 / steps, "kernel_ms": kms, "flops": flops,
            "bytes": nbytes, "desc": desc, "detail": det, "eager_ms_per_step": eager_ms}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(name, target_s):
    """The oracle as it stands, on a bounded row sample of the same workload."""
    import oracle
    import pk_inputs
    w = pk_inputs.WORKLOADS[name]
    threads = oracle.default_threads()
    o = oracle.default()
    if w.kind == "attention":
        # the oracle on the first batch*head, for a growing prefix of its query rows
        Q, Ks, Vs = pk_inputs.attention_inputs(w)
        scale = 1.0 / np.sqrt(w.K)
        K0, V0 = [k[0] for k in Ks], [v[0] for v in Vs]

        def timed_a(n):
            t = time.perf_counter()
            o.ring_attention(np.ascontiguousarray(Q[0][:n]), K0, V0, scale, nthreads=threads)
            return time.perf_counter() - t

        n = 16
        dt = timed_a(n)
        if dt < target_s:
            n = int(min(w.N, max(n, n * target_s / max(dt, 1e-3))))
            dt = timed_a(n)
        flops = 4.0 * n * w.chunks * w.tokens * w.K
        return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                "sample": "query rows 0..%d of batch*head 0 (of %d x %d), %d keys (%.1f s)"
                          % (n - 1, w.M, w.N, w.chunks * w.tokens, dt)}
    if w.kind == "combine":
        # the oracle's dispatch, then its combine for a growing prefix of tokens
        ids, H, W, gates = pk_inputs.combine_inputs(w)
        _, offsets, perm = o.dispatch(ids, w.num_experts, w.expert_begin, w.num_local)
        tok_of_row = perm // w.top_k

        def timed_c(n):
            t = time.perf_counter()
            o.combine(w.tokens, w.top_k, offsets, perm, H, W, gates, tokens=range(n),
                      nthreads=threads)
            return time.perf_counter() - t, int(np.sum(tok_of_row < n))

        n = 16
        dt, rows = timed_c(n)
        if dt < target_s:
            n = int(min(w.tokens, max(n, n * target_s / max(dt, 1e-3))))
            dt, rows = timed_c(n)
        flops = 2.0 * rows * w.K * w.N
        return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                "sample": "tokens 0..%d of %d (%d dispatched rows), K=%d, N=%d (%.1f s)"
                          % (n - 1, w.tokens, rows, w.K, w.N, dt)}
    if w.kind == "grouped":
        # the oracle's dispatch, then its grouped product over the rows of the last experts
        # (a suffix of the expert list, grown until it takes about target_s)
        ids, X, W = pk_inputs.moe_inputs(w)
        _, offsets, perm = o.dispatch(ids, w.num_experts, w.expert_begin, w.num_local)
        total = int(offsets[-1])

        def timed_g(e0):
            sub_off = (offsets[e0:] - offsets[e0]).astype(np.int32)
            sub_perm = perm[offsets[e0]:]
            t = time.perf_counter()
            o.grouped_gemm(sub_off, sub_perm, w.top_k, X, W[e0:], nthreads=threads)
            return time.perf_counter() - t, int(sub_off[-1])

        e0 = w.num_local - 1
        dt, rows = timed_g(e0)
        while e0 > 0 and dt < target_s:
            per_row = dt / max(rows, 1)
            want = target_s / per_row
            while e0 > 0 and int(offsets[-1] - offsets[e0]) < want:
                e0 -= 1
            dt, rows = timed_g(e0)
        flops = 2.0 * rows * w.N * w.K
        return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                "sample": "%d of %d dispatched rows (experts %d..%d of %d), K=%d, N=%d (%.1f s)"
                          % (rows, total, e0, w.num_local - 1, w.num_local, w.K, w.N, dt)}
    A = pk_inputs.normal_bf16((w.M, w.K), w.std_a, w.seed_a)
    B = pk_inputs.normal_bf16((w.K, w.N), w.std_b, w.seed_b)
    D0 = np.zeros((1, w.N), np.float32)

    def timed(rows):
        a = np.ascontiguousarray(A[:rows])
        t = time.perf_counter()
        if w.kind == "reduce":
            o.reduce(np.zeros((rows, w.N), np.float32), [(a, B)], nthreads=threads)
        else:
            o.gemm(a, B, nthreads=threads)
        return time.perf_counter() - t

    probe = min(w.M, 64)
    dt = timed(probe)
    rows = int(min(w.M, max(probe, probe * target_s / max(dt, 1e-3))))
    dt = timed(rows)
    flops = 2.0 * rows * w.N * w.K
    del D0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d output rows x all %d columns, K=%d, one producer (%.1f s)"
                      % (rows, w.M, w.N, w.K, dt)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus %d refused)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import gemm_tile_granular_bf16_amd as pk
    pk.library()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy(torch)
        return
    if args.sweep:
        sweep(torch, pk, max(args.steps, 10))
        return
    name = args.workload
    res = run_gpu(name, args.mode, args.steps, args.warmup, torch, pk, detail=not args.no_detail,
                  graph=not args.eager)
    tflops = res["flops"] / (res["ms_per_step"] * 1e-3) / 1e12
    ktflops = res["flops"] / (res["kernel_ms"] * 1e-3) / 1e12
    intensity = res["flops"] / res["bytes"]
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if intensity < ridge:
        achieved = res["bytes"] / (res["kernel_ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(ktflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ktflops / MFMA_BF16_PEAK_TFLOPS, 4)}
    roof["traffic"] = measured_traffic(name, args.mode)
    roof["algorithmic_bytes"] = res["bytes"]
    roof["kernel_ms"] = round(res["kernel_ms"], 5)
    line = {
        "metric": "TFLOP/s + % bf16 MFMA peak, " + WORKLOAD_TITLES[name] + " (1 GPU)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "mfma_peak_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "config": dict({"workload": name}, **res["desc"]),
        "roofline": roof,
    }
    if res["detail"] is not None:
        line["timing"] = res["detail"]
    if res["eager_ms_per_step"] is not None:
        line["eager_ms_per_step"] = round(res["eager_ms_per_step"], 5)
    line["peak_from_device"] = device_peak(torch)
    if name.startswith("rs") or name.startswith("ar"):
        if not args.no_variant:
            other = "atomic" if args.mode == "owner" else "owner"
            v = run_gpu(name, other, max(5, args.steps // 2), min(args.warmup, 3), torch, pk)
            line["variant"] = {"reduce": other, "ms_per_step": round(v["ms_per_step"], 5),
                               "tflops": round(v["flops"] / (v["ms_per_step"] * 1e-3) / 1e12, 2),
                               "kernel_ms": round(v["kernel_ms"], 5)}
    if not args.no_cpu_baseline:
        cb = cpu_baseline(name, args.cpu_seconds)
        if cb is not None:
            cb["cpu_model"] = cpu_model()
            line["cpu_baseline"] = cb
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
