"""Benchmark: mixed continuous-batch paged attention on one MI355X.

One step = one pass of the whole hot path over the mixed Llama-3-8B-shaped batch (32 q / 8 kv
heads, head_dim 128, block 16): for each of its three scheduler iterations — slot mapping and
cache write (one fused launch), the varlen plan upload and one paged_attention_varlen call
(decode rows on the VALU path, chunked-prefill / prefix-hit rows on MFMA, then the split-KV
reduce).  The 330 query tokens of the pass give the headline attention tokens/s per layer.  Inputs are synthetic (seeded N(0,1)
bf16) and resident in HBM before timing starts.

Also reported: the dominant kernel's roofline (algorithmic bytes / HIP-event-timed launch
duration against 8 TB/s).  Its headline is taken with cold caches: a 1 GiB write before each
timed launch evicts the L2s and the 256 MB MALL; the warm figure (launches back to back) is
context.  Every kernel time is given as mean, median and p10/p90 over at least 20 launches.
Beside it: the decode-only batch's HBM GB/s (bf16 and fp8 pools), the speculative-verify batch,
the tiny batched prefill, the graph-replayed decode step, the MFMA-bound passes (the cascade
shared-prefix pass and the long chunked prefill, each as TFLOP/s against the 2.5 PFLOP/s bf16
peak, with the cascade suffix pass, merge and the cascade-vs-single-pass ratio), and the CPU fp64
oracle timed on a bounded sample of the same workload (``cpu_baseline``).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-decode] [--no-graph] [--no-mfma]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def stats(ms):
    """mean, median and p10/p90 (ms) of per-launch durations."""
    a = np.asarray(ms, dtype=np.float64)
    return {
        "mean_ms": float(a.mean()),
        "median_ms": float(np.median(a)),
        "p10_ms": float(np.percentile(a, 10)),
        "p90_ms": float(np.percentile(a, 90)),
        "launches": int(a.size),
    }


def timed_launches(P, fn, reps, flush=None):
    """Per-launch attention-kernel milliseconds (library HIP events on the launch's stream) over
    `reps` calls of fn; with `flush`, a 1 GiB write precedes every call (outside the events)."""
    P.timing_begin()
    for _ in range(reps):
        if flush is not None:
            flush()
        fn()
    P.timing_end()
    return P.timing_durations()


def kv_bytes(seq_lens, num_kv_heads, head_dim):
    return int(np.sum(seq_lens, dtype=np.int64)) * num_kv_heads * head_dim * 2 * 2


def step_bytes(st, wl):
    """Algorithmic HBM bytes of one varlen launch: each K/V byte once per kv head, plus Q, O
    and the block-table entries read."""
    kv = kv_bytes(st.seq_lens, wl.num_kv_heads, wl.head_dim)
    qo = 2 * st.num_tokens * wl.num_q_heads * wl.head_dim * 2
    bt = int(np.sum(-(-st.seq_lens // wl.block_size))) * 4
    return kv + qo + bt


def step_flops(st, wl):
    """4*D flops per unmasked (q head, key) pair."""
    ql = st.query_lens.astype(np.int64)
    ctx = st.context_lens.astype(np.int64)
    pairs = np.sum(ql * ctx + ql * (ql + 1) // 2)
    return int(pairs) * wl.num_q_heads * 4 * wl.head_dim


class Runner:
    """Device-resident copy of a workload plus the calls of one pass."""

    def __init__(self, wl, torch, P):
        self.wl, self.torch, self.P = wl, torch, P
        d16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()  # noqa: E731
        d32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()  # noqa: E731
        self.k_cache = d16(wl.k_cache)
        self.v_cache = d16(wl.v_cache)
        self.shape = P.make_shape(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_blocks, wl.bt_stride, block_size=wl.block_size)
        self.steps = []
        for st in wl.steps:
            self.steps.append(
                dict(
                    st=st,
                    q=d16(st.q),
                    k=d16(st.k),
                    v=d16(st.v),
                    bt=d32(st.block_tables),
                    qsl=d32(st.query_start_loc),
                    ctx=d32(st.context_lens),
                    seq=d32(st.seq_lens),
                    slots=torch.empty(st.num_tokens, dtype=torch.int64, device="cuda"),
                    out=torch.empty((st.num_tokens, wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda"),
                )
            )
        max_seq = max(int(s.seq_lens.max()) for s in wl.steps)
        self.ws = P.alloc_workspace(
            P.varlen_workspace_size(
                max(s.num_seqs for s in wl.steps), max(s.num_tokens for s in wl.steps), max_seq, self.shape
            )
        )

    def run_pass(self, events=None, flush=None):
        P = self.P
        for i, s in enumerate(self.steps):
            st = s["st"]
            # slot mapping + cache write (one launch), plan upload, attention (one launch)
            P.append_kv(s["k"], s["v"], self.k_cache, self.v_cache, s["bt"], s["qsl"], s["ctx"], self.shape,
                        slot_mapping=s["slots"])
            plan = P.plan_varlen(self.ws, st.query_start_loc, st.context_lens, st.seq_lens, self.shape)
            if flush is not None:
                flush()
            if events is not None:
                events[i][0].record()
            P.paged_attention_varlen(
                s["q"], self.k_cache, self.v_cache, s["bt"], s["qsl"], s["ctx"], s["seq"], self.shape, plan, self.ws,
                out=s["out"],
            )
            if events is not None:
                events[i][1].record()


def time_passes(runner, torch, steps, warmup):
    """Time `steps` passes bracketed by device syncs, then `steps` more with the library's
    launch timing on, which brackets each varlen attention kernel with a pair of HIP events on
    its stream.  The events add GPU time between launches (about 7 us per launch here), so the
    step time comes from the first loop and the kernel times from the second.  Returns (total ms
    of the first loop, per-launch kernel ms of the second)."""
    import gc

    P = runner.P
    for _ in range(warmup):
        runner.run_pass()
    torch.cuda.synchronize()
    gc.collect()
    gc.disable()  # no collector pauses inside the timed regions
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        runner.run_pass()
    stop.record()
    torch.cuda.synchronize()
    P.timing_begin()
    for _ in range(steps):
        runner.run_pass()
    torch.cuda.synchronize()
    P.timing_end()
    gc.enable()
    return start.elapsed_time(stop), P.timing_durations()


class Flusher:
    """Writes a 1 GiB scratch buffer: evicts the L2s and the 256 MB MALL before a timed launch."""

    def __init__(self, torch):
        self.buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        self.n = 0

    def __call__(self):
        self.n += 1
        self.buf.fill_(self.n & 255)


def time_flushed(runner, torch, passes):
    """Per-launch kernel ms of the varlen launches when every launch starts with cold caches (a
    1 GiB write before it, outside the kernel's HIP events)."""
    P = runner.P
    fl = Flusher(torch)
    runner.run_pass(flush=fl)
    torch.cuda.synchronize()
    P.timing_begin()
    for _ in range(passes):
        runner.run_pass(flush=fl)
    P.timing_end()
    d = P.timing_durations()
    del fl
    torch.cuda.empty_cache()
    return d


HERE = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(HERE, "profiles", "varlen_kernel_mixed_llama8b_hbm_traffic.json")


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE runs (scaled by a
    plain-copy calibration), or None when the kernel sources changed since they were taken."""
    import hashlib

    try:
        with open(TRAFFIC_FILE) as f:
            doc = json.load(f)
        h = hashlib.sha256()
        for p in doc["kernel_sources"]:
            with open(os.path.join(HERE, p), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != doc["kernel_sources_sha256"]:
            return None
        return float(doc["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(wl, budget_s=10.0):
    """The fp64 oracle over whole passes of the same workload (every scheduler iteration: slot
    mapping, cache write, attention), repeated from the initial pools until ~budget_s."""
    import oracle as O

    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    toks = 0
    passes = 0
    t0 = time.perf_counter()
    while True:
        kp, vp = wl.k_cache, wl.v_cache
        for st in wl.steps:
            slots = O.slot_mapping(st.block_tables, st.query_start_loc, st.context_lens, wl.block_size)
            kp, vp = O.reshape_and_cache(st.k, st.v, kp, vp, slots, wl.block_size)
            O.paged_attention(st.q, kp, vp, st.block_tables, st.query_start_loc, st.context_lens, st.seq_lens,
                              wl.block_size)
            toks += st.num_tokens
        passes += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {
        "value": toks / dt,
        "unit": "tokens/s/layer",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{passes} full passes of the bench step ({len(wl.steps)} scheduler iterations, {toks} query tokens "
        f"in all) over the same mixed batch, numpy float64 with BLAS threads = cores, {dt:.2f} s",
    }


def decode_hbm(torch, P, reps=20, warmup=5):
    """Decode-only batch (256 rows, context 1024..8192): varlen kernel GB/s against 8 TB/s, with
    cold caches (headline) and warm."""
    import workloads as W

    wl = W.decode_only(seed=0)
    r = Runner(wl, torch, P)
    st = wl.steps[0]
    s = r.steps[0]
    P.append_kv(s["k"], s["v"], r.k_cache, r.v_cache, s["bt"], s["qsl"], s["ctx"], r.shape)
    plan = P.plan_varlen(r.ws, st.query_start_loc, st.context_lens, st.seq_lens, r.shape)

    def call():
        P.paged_attention_varlen(
            s["q"], r.k_cache, r.v_cache, s["bt"], s["qsl"], s["ctx"], s["seq"], r.shape, plan, r.ws, out=s["out"]
        )

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    warm = stats(timed_launches(P, call, reps))
    fl = Flusher(torch)
    cold = stats(timed_launches(P, call, reps, flush=fl))
    del fl
    nbytes = step_bytes(st, wl)
    gbs = nbytes / (cold["mean_ms"] * 1e-3) / 1e9
    res = {
        "workload": "decode_only: 256 seqs, ctx U[1024,8192], 32q/8kv, D128, bs16",
        "algorithmic_bytes": nbytes,
        "GB/s": gbs,
        "frac_of_peak": gbs / HBM_PEAK_GBS,
        "tokens/s/layer": st.num_tokens / (cold["mean_ms"] * 1e-3),
        "kernel_ms_flushed": cold,
        "kernel_ms_warm": warm,
        "warm_frac_of_peak": nbytes / (warm["mean_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "blocks_per_split": plan.blocks_per_split,
        "items": plan.num_items,
    }
    del r
    torch.cuda.empty_cache()
    return res


def fp8_decode_hbm(torch, P, reps=20, warmup=5, bf16_ms=None):
    """The decode-only batch over FP8 (e4m3) pools with per-(block, kv head) scales: varlen
    kernel GB/s (K/V at one byte per element, plus the scales read) against 8 TB/s, cold caches
    (headline) and warm."""
    import workloads as W

    wl = W.decode_only(seed=0)
    c = W.fp8_cache(wl, seed=0)
    st = wl.steps[0]
    shape = P.make_shape(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_blocks, wl.bt_stride, block_size=wl.block_size)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    kc, vc, ks, vs = dev(c.k_cache), dev(c.v_cache), dev(c.k_scale), dev(c.v_scale)
    del c
    i16 = lambda a: dev(a.view(np.int16))  # noqa: E731
    q, k, v = i16(st.q), i16(st.k), i16(st.v)
    bt, qsl, ctx, seq = (dev(x.astype(np.int32)) for x in (st.block_tables, st.query_start_loc, st.context_lens,
                                                           st.seq_lens))
    ws = P.alloc_workspace(P.varlen_workspace_size(st.num_seqs, st.num_tokens, int(st.seq_lens.max()), shape))
    out = torch.empty((st.num_tokens, wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    P.append_kv_fp8(k, v, kc, vc, ks, vs, bt, qsl, ctx, shape)
    plan = P.plan_varlen(ws, st.query_start_loc, st.context_lens, st.seq_lens, shape)

    def call():
        P.paged_attention_varlen_fp8(q, kc, vc, ks, vs, bt, qsl, ctx, seq, shape, plan, ws, out=out)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    warm = stats(timed_launches(P, call, reps))
    fl = Flusher(torch)
    cold = stats(timed_launches(P, call, reps, flush=fl))
    del fl
    kvb = kv_bytes(st.seq_lens, wl.num_kv_heads, wl.head_dim) // 2
    blocks = int(np.sum(-(-st.seq_lens // wl.block_size)))
    nbytes = kvb + 2 * blocks * wl.num_kv_heads * 4 + 2 * st.num_tokens * wl.num_q_heads * wl.head_dim * 2 + blocks * 4
    gbs = nbytes / (cold["mean_ms"] * 1e-3) / 1e9
    res = {
        "workload": "decode_only over fp8 e4m3 pools: 256 seqs, ctx U[1024,8192], 32q/8kv, D128, bs16",
        "algorithmic_bytes": nbytes,
        "GB/s": gbs,
        "frac_of_peak": gbs / HBM_PEAK_GBS,
        "tokens/s/layer": st.num_tokens / (cold["mean_ms"] * 1e-3),
        "kernel_ms_flushed": cold,
        "kernel_ms_warm": warm,
        "warm_frac_of_peak": nbytes / (warm["mean_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
    }
    if bf16_ms:
        res["speedup_vs_bf16_pools"] = bf16_ms / cold["mean_ms"]
    del kc, vc
    torch.cuda.empty_cache()
    return res


def decode_graph_step(torch, P, reps=50):
    """A small decode step (16 rows, context 512..2048: fused cache write + device-split decode +
    reduce) issued eagerly vs replayed from a HIP graph captured once: per-step time back to
    back, and the median latency of one step issued and waited for."""
    import time

    import workloads as W

    wl = W.decode_only(seed=7, num_seqs=16, ctx_range=(512, 2048))
    st = wl.steps[0]
    r = Runner(wl, torch, P)
    s = r.steps[0]
    max_seq = wl.bt_stride * wl.block_size
    ws = P.alloc_workspace(P.decode_workspace_size(st.num_seqs, max_seq, r.shape))
    lse = torch.empty(st.q.shape[:2], dtype=torch.float32, device="cuda")

    def step():
        P.append_kv(s["k"], s["v"], r.k_cache, r.v_cache, s["bt"], s["qsl"], s["ctx"], r.shape)
        P.paged_attention_decode(s["q"], r.k_cache, r.v_cache, s["bt"], s["qsl"], s["seq"], r.shape, max_seq,
                                 workspace=ws, out=s["out"], lse=lse)

    def timed(fn):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        b2b = (time.perf_counter() - t0) / reps * 1e6
        lat = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            lat.append(time.perf_counter() - t0)
        return b2b, float(np.median(lat)) * 1e6

    eager = timed(step)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.synchronize()
    graph = timed(g.replay)
    out = {
        "workload": "decode step, 16 rows, ctx U[512,2048], 32q/8kv, D128: append_kv + paged_attention_decode",
        "eager_us_back_to_back": eager[0],
        "graph_us_back_to_back": graph[0],
        "eager_us_latency": eager[1],
        "graph_us_latency": graph[1],
    }
    del r, g
    torch.cuda.empty_cache()
    return out


def spec_verify_hbm(torch, P, reps=20):
    """Speculative-verify batch (64 rows of 1 + 4 tokens, context 1024..4096): varlen launch
    GB/s against 8 TB/s (the five query tokens of a row share every K/V byte), cold caches
    (headline) and warm."""
    import workloads as W

    wl = W.spec_verify(seed=0)
    r = Runner(wl, torch, P)
    st, s = wl.steps[0], r.steps[0]
    P.append_kv(s["k"], s["v"], r.k_cache, r.v_cache, s["bt"], s["qsl"], s["ctx"], r.shape)
    plan = P.plan_varlen(r.ws, st.query_start_loc, st.context_lens, st.seq_lens, r.shape)

    def call():
        P.paged_attention_varlen(s["q"], r.k_cache, r.v_cache, s["bt"], s["qsl"], s["ctx"], s["seq"], r.shape, plan,
                                 r.ws, out=s["out"])

    for _ in range(5):
        call()
    torch.cuda.synchronize()
    warm = stats(timed_launches(P, call, reps))
    fl = Flusher(torch)
    cold = stats(timed_launches(P, call, reps, flush=fl))
    del fl
    byts = step_bytes(st, wl)
    out = {
        "workload": "spec_verify: 64 rows x (1 + 4 drafted) tokens, ctx U[1024,4096], 32q/8kv, D128",
        "algorithmic_bytes": byts,
        "GB/s": byts / (cold["mean_ms"] * 1e-3) / 1e9,
        "frac_of_peak": byts / (cold["mean_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "warm_frac_of_peak": byts / (warm["mean_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "tokens/s/layer": st.num_tokens / (cold["mean_ms"] * 1e-3),
        "kernel_ms_flushed": cold,
        "kernel_ms_warm": warm,
    }
    del r
    torch.cuda.empty_cache()
    return out


def tiny_prefill_latency(torch, P, reps=20):
    """The 31 + 29 + 30 batched prefill (4 q / 2 kv heads, D64): a latency-bound single launch."""
    import workloads as W

    wl = W.tiny_prefill(seed=0)
    r = Runner(wl, torch, P)
    st, s = wl.steps[0], r.steps[0]
    P.append_kv(s["k"], s["v"], r.k_cache, r.v_cache, s["bt"], s["qsl"], s["ctx"], r.shape)
    plan = P.plan_varlen(r.ws, st.query_start_loc, st.context_lens, st.seq_lens, r.shape)

    def call():
        P.paged_attention_varlen(s["q"], r.k_cache, r.v_cache, s["bt"], s["qsl"], s["ctx"], s["seq"], r.shape, plan,
                                 r.ws, out=s["out"])

    call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        call()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / reps * 1e3
    return {"workload": "tiny_prefill: prompts of 31, 29 and 30 tokens, 4 q / 2 kv heads, D64", "us_per_call": us,
            "tokens/s": st.num_tokens / (us * 1e-6)}


def mfma_roofline(kernel, flops, cold, warm):
    """Roofline block of an MFMA-bound pass: flops per launch over the mean cold-cache launch
    time against the 2.5 PFLOP/s dense bf16 peak (warm launches as context)."""
    tf = flops / (cold["mean_ms"] * 1e-3) / 1e12
    return {
        "kernel": kernel,
        "bound": "mfma",
        "achieved": tf,
        "peak": MFMA_BF16_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": tf / MFMA_BF16_PEAK_TFLOPS,
        "flops_per_launch": flops,
        "kernel_ms_flushed": cold,
        "kernel_ms_warm": warm,
        "warm_frac": flops / (warm["mean_ms"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
    }


def mfma_paths(torch, P, reps=20):
    """MFMA-bound passes: the cascade shared-prefix pass (512 queries x 64 q heads over a
    16384-token prefix, with its suffix pass, merge and the cascade-vs-single-pass ratio) and
    the long chunked prefill (one 32768-token prompt in 16 chunks of 2048, alone and beside 128
    decode rows), as TFLOP/s against the 2.5 PFLOP/s dense bf16 peak."""
    import workloads as W

    out = {}
    wl = W.cascade_shared_prefix(seed=0)
    r = Runner(wl, torch, P)
    st, s, cv = wl.steps[0], r.steps[0], wl.cascade
    P.append_kv(s["k"], s["v"], r.k_cache, r.v_cache, s["bt"], s["qsl"], s["ctx"], r.shape)
    pbt = torch.from_numpy(cv.prefix_block_table).cuda()
    cws = P.alloc_workspace(P.cascade_workspace_size(st.num_tokens, cv.prefix_len, r.shape))
    o = torch.empty(st.q.shape, dtype=torch.float32, device="cuda")
    l = torch.empty(st.q.shape[:2], dtype=torch.float32, device="cuda")
    pb = cv.prefix_len // wl.block_size
    sbt = torch.from_numpy(np.ascontiguousarray(st.block_tables[:, pb:])).cuda()
    sshape = P.make_shape(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_blocks, sbt.shape[1], block_size=wl.block_size)
    sctx, sseq = torch.from_numpy(cv.suffix_context_lens).cuda(), torch.from_numpy(cv.suffix_seq_lens).cuda()
    splan = P.plan_varlen(r.ws, st.query_start_loc, cv.suffix_context_lens, cv.suffix_seq_lens, sshape)
    os_, ls_ = torch.empty_like(o), torch.empty_like(l)
    merged = torch.empty(st.q.shape, dtype=torch.bfloat16, device="cuda")

    def prefix():
        P.cascade_prefix_attention(s["q"], r.k_cache, r.v_cache, pbt, cv.prefix_len, r.shape, cws, out=o, lse=l)

    def suffix():
        P.paged_attention_varlen(s["q"], r.k_cache, r.v_cache, sbt, s["qsl"], sctx, sseq, sshape, splan, r.ws,
                                 out=os_, lse=ls_)

    def cascade():
        prefix()
        suffix()
        P.merge_attn_states(o, l, os_, ls_, out=merged)

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    fl = Flusher(torch)
    for _ in range(5):
        prefix()
    pre_warm = stats(timed_launches(P, prefix, reps))
    pre_cold = stats(timed_launches(P, prefix, reps, flush=fl))
    # Sustained: whole calls (the kernel and the merge of its key segments) back to back, one
    # event pair around all of them.
    pre_sustained = timed(prefix, 4 * reps)
    suffix()
    suf_warm = stats(timed_launches(P, suffix, reps))
    suf_cold = stats(timed_launches(P, suffix, reps, flush=fl))
    cascade_ms = timed(cascade, 10)
    merge_ms = timed(lambda: P.merge_attn_states(o, l, os_, ls_, out=merged), 10)
    # suffix keys once per kv head + bf16 Q + fp32 O and LSE + block-table entries
    suffix_bytes = (kv_bytes(cv.suffix_seq_lens, wl.num_kv_heads, wl.head_dim)
                    + st.num_tokens * wl.num_q_heads * (wl.head_dim * 2 + wl.head_dim * 4 + 4)
                    + int(np.sum(-(-cv.suffix_seq_lens // wl.block_size))) * 4)
    fplan = P.plan_varlen(r.ws, st.query_start_loc, st.context_lens, st.seq_lens, r.shape)
    single_ms = timed(lambda: P.paged_attention_varlen(s["q"], r.k_cache, r.v_cache, s["bt"], s["qsl"], s["ctx"],
                                                       s["seq"], r.shape, fplan, r.ws, out=s["out"]), 5)
    flops = st.num_tokens * wl.num_q_heads * cv.prefix_len * 4 * wl.head_dim
    res = mfma_roofline("cascade_kernel (pkv_cascade_prefix_attention)", flops, pre_cold, pre_warm)
    res.update({
        "sustained_call_ms": pre_sustained,
        "sustained_frac": flops / (pre_sustained * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "sustained_timing": "whole pkv_cascade_prefix_attention calls (kernel + segment merge) back to back",
        "workload": "cascade_shared_prefix: 512 queries, 64 q / 8 kv heads, D128, shared 16384-token prefix",
        "suffix_pass": {
            "kernel_ms_flushed": suf_cold,
            "kernel_ms_warm": suf_warm,
            "algorithmic_bytes": suffix_bytes,
            "GB/s": suffix_bytes / (suf_cold["mean_ms"] * 1e-3) / 1e9,
            "frac_of_peak": suffix_bytes / (suf_cold["mean_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
        },
        "merge_ms": merge_ms,
        "cascade_total_ms": cascade_ms,
        "single_pass_ms": single_ms,
        "cascade_speedup": single_ms / cascade_ms,
        "cascade_speedup_pages_h100_context": "up to 31x on H100 SXM 80GB, workload not stated",
    })
    out["cascade_prefix"] = res
    del r
    torch.cuda.empty_cache()

    wl = W.long_chunked_prefill(seed=0, num_decode=0)
    r = Runner(wl, torch, P)
    warm_all, cold_all, tot_fl = [], [], 0
    chunk_reps = 3
    calls = []
    for s in r.steps:
        st = s["st"]
        P.append_kv(s["k"], s["v"], r.k_cache, r.v_cache, s["bt"], s["qsl"], s["ctx"], r.shape)
        ws_c = P.alloc_workspace(
            P.varlen_workspace_size(st.num_seqs, st.num_tokens, int(st.seq_lens.max()), r.shape))
        plan = P.plan_varlen(ws_c, st.query_start_loc, st.context_lens, st.seq_lens, r.shape)

        def call(s=s, plan=plan, ws_c=ws_c):
            P.paged_attention_varlen(s["q"], r.k_cache, r.v_cache, s["bt"], s["qsl"], s["ctx"], s["seq"], r.shape,
                                     plan, ws_c, out=s["out"])

        call()
        warm_all.append(timed_launches(P, call, chunk_reps))
        cold_all.append(timed_launches(P, call, chunk_reps, flush=fl))
        tot_fl += step_flops(st, wl)
        calls.append(call)
    # Sustained: the 16 chunk calls in order, back to back, one event pair around two passes.
    sustained_ms = timed(lambda: [c() for c in calls], 2)
    # Whole-prompt time: the 16 chunks' launches, each chunk's launch repeated chunk_reps times;
    # stats over the chunk_reps sums of one launch per chunk.
    warm_tot = stats(np.sum(np.stack(warm_all), axis=0))
    cold_tot = stats(np.sum(np.stack(cold_all), axis=0))
    res = mfma_roofline("prefill_wide_kernel (pkv_paged_attention_varlen, 16 launches)", tot_fl, cold_tot, warm_tot)
    res["workload"] = ("long_chunked_prefill: one 32768-token prompt in 16 chunks of 2048 against its growing paged "
                       "context, 32 q / 8 kv heads, D128; times are of all 16 chunk launches together")
    res["last_chunk_ms_flushed"] = stats(cold_all[-1])
    res["sustained_all_chunks_ms"] = sustained_ms
    res["sustained_frac"] = tot_fl / (sustained_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS
    res["sustained_timing"] = "the 16 chunk calls in order, back to back (two passes)"
    out["long_chunked_prefill"] = res
    del r
    torch.cuda.empty_cache()

    # The same prompt beside 128 decode rows at context 2048 (+1 per chunk): whole steps.
    wl2 = W.long_chunked_prefill(seed=0)
    r2 = Runner(wl2, torch, P)
    mixed_ms = 0.0
    for s2 in r2.steps:
        st2 = s2["st"]
        P.append_kv(s2["k"], s2["v"], r2.k_cache, r2.v_cache, s2["bt"], s2["qsl"], s2["ctx"], r2.shape)
        plan2 = P.plan_varlen(r2.ws, st2.query_start_loc, st2.context_lens, st2.seq_lens, r2.shape)
        mixed_ms += timed(lambda: P.paged_attention_varlen(s2["q"], r2.k_cache, r2.v_cache, s2["bt"], s2["qsl"],
                                                           s2["ctx"], s2["seq"], r2.shape, plan2, r2.ws,
                                                           out=s2["out"]), 2)
    out["long_chunked_prefill_with_decode"] = {
        "workload": "the same 16 chunks, each step beside 128 decode rows at context 2048 + chunk index",
        "ms_all_steps": mixed_ms,
        "tokens/s/layer": sum(s2["st"].num_tokens for s2 in r2.steps) / (mixed_ms * 1e-3),
    }
    del r2, fl
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replayed decode step")
    ap.add_argument("--no-mfma", action="store_true", help="skip the MFMA-bound cascade prefix and long prefill")
    ap.add_argument(
        "--only",
        choices=["decode", "fp8_decode", "spec_verify", "mfma", "graph"],
        help="run just one measured section (e.g. under a profiler) and print its JSON",
    )
    ap.add_argument("--reps", type=int, default=20, help="timed repetitions per section")
    ap.add_argument(
        "--copy-calibration",
        type=int,
        default=0,
        metavar="BYTES",
        help="only run one plain device-to-device copy of BYTES (to scale rocprofv3 FETCH_SIZE/WRITE_SIZE)",
    )
    args = ap.parse_args()
    if args.gpus != 1:
        print(
            "bench.py measures one GPU only: this build has no multi-GPU path (the attention shards "
            "by request or kv head with no exchange between GPUs). Run with --gpus 1.",
            file=sys.stderr,
        )
        sys.exit(2)

    import torch

    if args.copy_calibration:
        n = args.copy_calibration // 2
        src = torch.ones(n, dtype=torch.int16, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 2 * n}), flush=True)
        return

    import paged_kv_cache_285_amd as P
    import workloads as W

    if args.only:
        sections = {
            "decode": lambda: decode_hbm(torch, P, reps=args.reps),
            "fp8_decode": lambda: fp8_decode_hbm(torch, P, reps=args.reps),
            "spec_verify": lambda: spec_verify_hbm(torch, P, reps=args.reps),
            "mfma": lambda: mfma_paths(torch, P, reps=args.reps),
            "graph": lambda: decode_graph_step(torch, P, reps=args.reps),
        }
        log(f"bench: section {args.only} only, {args.reps} reps")
        print(json.dumps({"only": args.only, args.only: sections[args.only]()}), flush=True)
        return

    log("bench: building mixed_llama8b workload (seed 0)")
    wl = W.mixed_llama8b(seed=0)
    runner = Runner(wl, torch, P)
    log(f"bench: timing {args.steps} steps after {args.warmup} warmup")
    total_ms, warm_each = time_passes(runner, torch, args.steps, args.warmup)
    ms_per_step = total_ms / args.steps
    tokens = sum(st.num_tokens for st in wl.steps)
    value = tokens / (ms_per_step * 1e-3)

    bytes_per_launch = [step_bytes(st, wl) for st in wl.steps]
    flops_per_launch = [step_flops(st, wl) for st in wl.steps]
    mean_bytes = float(np.mean(bytes_per_launch))
    log("bench: the same launches with cold caches")
    cold_each = time_flushed(runner, torch, passes=max(7, -(-20 // len(wl.steps))))
    warm, cold = stats(warm_each), stats(cold_each)
    achieved = mean_bytes / (cold["mean_ms"] * 1e-3) / 1e9
    traffic = measured_traffic()
    line = {
        "metric": "paged-attn decode HBM GB/s (% peak) + mixed-batch attn tokens/s per layer",
        "value": value,
        "unit": "tokens/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) bf16 Q/K/V, random block tables over a 1.2x permuted pool",
        "config": {
            "workload": "mixed_llama8b: one layer, 32 q / 8 kv heads, head_dim 128, block 16; "
            "3 scheduler iterations: 48-token prompt in chunks of 16, 31-token prompt as 16+15, "
            "107-token prompt with 48 prefix-cached, 64 decode rows ctx U[128,4096]",
            "query_tokens_per_step": tokens,
            "launches_per_step": len(wl.steps),
        },
        "roofline": {
            "kernel": "varlen_kernel (paged_attention_varlen)",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "timing": "achieved = algorithmic bytes / mean launch time with cold caches (1 GiB write before "
                      "each launch); warm = the K timed steps' launches back to back",
            "algorithmic_bytes_per_launch": mean_bytes,
            "flops_per_launch": float(np.mean(flops_per_launch)),
            "kernel_ms_flushed": cold,
            "kernel_ms_warm": warm,
            "warm_achieved": mean_bytes / (warm["mean_ms"] * 1e-3) / 1e9,
            "warm_frac": mean_bytes / (warm["mean_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
        },
    }
    props = torch.cuda.get_device_properties(0)
    line["device"] = {
        "name": props.name,
        "arch": getattr(props, "gcnArchName", None),
        "compute_units": props.multi_processor_count,
        "memory_GiB": round(props.total_memory / 2**30, 1),
        "peaks": "published MI355X figures: HBM 8 TB/s; dense bf16 MFMA 2.5 PFLOP/s (256 CUs at 2.4 GHz)",
    }
    if not args.no_decode:
        log("bench: decode-only batch")
        line["decode_hbm"] = decode_hbm(torch, P)
        log("bench: decode-only batch over fp8 pools")
        line["fp8_decode_hbm"] = fp8_decode_hbm(torch, P, bf16_ms=line["decode_hbm"]["kernel_ms_flushed"]["mean_ms"])
    if not args.no_decode:
        log("bench: speculative-verify batch, tiny prefill")
        line["spec_verify_hbm"] = spec_verify_hbm(torch, P)
        line["tiny_prefill"] = tiny_prefill_latency(torch, P)
        if not args.no_graph:
            line["decode_graph_step"] = decode_graph_step(torch, P)
    if not args.no_mfma:
        log("bench: MFMA paths (cascade prefix, long chunked prefill)")
        line["mfma_paths"] = mfma_paths(torch, P)
    if not args.no_cpu:
        log("bench: cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
