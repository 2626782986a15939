"""Benchmark: one KIVI decode step over a 2-bit KV cache, Llama-2-7B shape.

Workload (the default): batch 16, 32 heads (MHA), d_h 128, 4096 cached tokens,
G 32, R 128, int2; the step appends token 4096 and attends 4097 tokens.  A
step is the whole path: the new key/value rows go into the fp16 residuals,
the value that leaves the 128-token window is quantized and appended, and
decode attention runs over [quantized | residual] keys and values -- one
kvq_kivi_step call, which at this shape is one launch (the append runs in
the attention kernel's last wave of each stream).

Timing: the cache is built (prefill, on the GPU) in several independent
copies whose total exceeds twice the 256 MB Infinity Cache, and each timed
step uses the next copy, so the reads come from HBM.  A HIP graph holds
`rounds` passes over the copies, one step per copy per pass (a step repeated
on a copy rewrites the same rows and reads the same state, so every step does
identical work on identical data); W warm-up and then K timed steps are
replayed, with a synchronize on both sides, after about a second of untimed
replays that lets the clocks settle.  The host integers of every copy are
restored before each capture.

Prints one JSON line.  `value` is the effective bandwidth of the step
(algorithmic bytes / step time); `roofline` covers the decode-attention
kernels (split + merge) timed live the same way; `cpu_baseline` times the
CPU oracle's decode step on a sample of streams on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0


def step_bytes(w: workloads.Workload, state):
    """Algorithmic HBM bytes of decode attention and of the whole step."""
    n_kq, r_k, n_vq, r_v = state
    streams = w.batch * w.n_kv_heads
    d, b, G = w.d_h, w.bits, w.group
    k_codes = n_kq * d * b / 8
    k_meta = n_kq // G * d * 4
    v_codes = n_vq * d * b / 8
    v_meta = n_vq * (d // G) * 4
    res = (r_k + r_v) * d * 2
    attn = streams * (k_codes + k_meta + v_codes + v_meta + res) + w.batch * w.n_q_heads * d * (2 + 4)
    # append: read 2 new rows, write 2 rows; quantize 1 value row: read it, write codes + meta
    extra = streams * (4 * d * 2 + d * 2 + d * b / 8 + (d // G) * 4)
    return attn, attn + extra


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "decode_kernel_llama2_7b_int2_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "decode_attention_kivi_amd", "csrc", f)
                  for f in ("decode.hip", "kvq_device.h", "kvq_internal.h", "kvq_quant.h")]


def measured_traffic(workload: str):
    """HBM bytes per decode launch from the committed FETCH_SIZE/WRITE_SIZE
    summary, or None when it does not cover this workload or the kernel
    sources have changed since the counters were taken."""
    import hashlib
    if workload != "llama2_7b" or not os.path.exists(TRAFFIC_PROFILE):
        return None
    fields = {}
    for line in open(TRAFFIC_PROFILE):
        if ":" in line and line.strip().split(":")[0] in ("traffic_bytes_per_launch", "kernel_sources_sha256"):
            k, v = line.strip().split(":", 1)
            fields[k] = v.strip()
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    if fields.get("kernel_sources_sha256") != h.hexdigest():
        return None
    return int(fields["traffic_bytes_per_launch"])


def _cpu_worker(job):
    """One CPU-baseline worker (its own process, single-threaded BLAS): for
    each of its streams, the oracle's prefill (quantize + pack, timed apart)
    and `reps` decode steps (append + float64 attention) on identical copies
    of the state, until `budget_s` of timed work has accumulated."""
    name, units, reps, budget_s = job
    import copy
    from threadpoolctl import threadpool_limits
    from oracle.kivi import KiviStream
    w = workloads.get(name)
    q = workloads.queries(w)
    L, g = w.context, w.gqa
    t_step = t_quant = 0.0
    n_steps = n_streams = 0
    last = None
    with threadpool_limits(limits=1):
        for i, (b, h) in enumerate(units):
            k, v = workloads.unit_kv(w, b, h)
            st = KiviStream(w.d_h, w.bits, w.group, w.residual)
            t0 = time.perf_counter()
            st.prefill(k[:L], v[:L])
            dt = time.perf_counter() - t0
            if i > 0:                                          # the first call pays library set-up
                t_quant += dt
            copies = [copy.deepcopy(st) for _ in range(reps)]
            if i == 0:
                st.decode_append(k[L], v[L])
                st.attend(q[b, h * g:(h + 1) * g], w.sm_scale)
            for c in copies:
                t0 = time.perf_counter()
                c.decode_append(k[L], v[L])
                c.attend(q[b, h * g:(h + 1) * g], w.sm_scale)
                t_step += time.perf_counter() - t0
                n_steps += 1
            last = copies[0].lengths
            n_streams += 1
            if t_step + t_quant > budget_s:
                break
    return {"t_step": t_step, "n_steps": n_steps, "t_quant": t_quant, "n_quant": max(n_streams - 1, 0),
            "n_streams": n_streams, "lengths": last}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w: workloads.Workload, budget_s: float = 8.0, reps: int = 16, max_workers: int = 16):
    """The oracle's decode step on this host's cores: one single-threaded
    worker process per core this process may run on (at most 16, the CPU
    share of one GPU), each taking its own streams of the workload in a
    seeded random order until about `budget_s` of timed work.  The rate is
    the sum of the workers' rates (they run at once).  The oracle's
    quantizer (the prefill of a stream: keys and values quantized and
    packed) is timed apart and reported beside it."""
    import multiprocessing as mp
    cores = max(1, min(len(os.sched_getaffinity(0)), max_workers))
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"                          # inherited by the workers
    units = workloads.sample_units(w, w.batch * w.n_kv_heads, seed=99)
    jobs = [(w.name, units[i::cores], reps, budget_s) for i in range(cores)]
    t_wall = time.perf_counter()
    with mp.get_context("spawn").Pool(cores) as pool:
        res = pool.map(_cpu_worker, jobs)
    t_wall = time.perf_counter() - t_wall
    lengths = next(r["lengths"] for r in res if r["lengths"] is not None)
    _, step_b = step_bytes(w, lengths)
    per_stream = step_b / (w.batch * w.n_kv_heads)
    rate = sum(per_stream * r["n_steps"] / r["t_step"] for r in res if r["t_step"] > 0)
    n_steps = sum(r["n_steps"] for r in res)
    n_streams = sum(r["n_streams"] for r in res)
    qb = 2 * w.context * w.d_h * 2                     # fp16 keys + values of one stream's prefill
    q_rate = sum(qb * r["n_quant"] / r["t_quant"] for r in res if r["t_quant"] > 0)
    return {"value": round(rate / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "us_per_step": round(w.batch * w.n_kv_heads * per_stream / rate * 1e6, 1),
            "quantize_GBs": round(q_rate / 1e9, 4),
            "sample": f"{n_streams} of {w.batch * w.n_kv_heads} (batch, kv-head) streams of the same "
                      f"workload over {cores} single-threaded worker processes, {reps} identical decode "
                      f"steps each (append + float64 attention), {n_steps} steps, {t_wall:.1f} s wall; "
                      f"quantize_GBs: the oracle's prefill quantizer (keys and values of a stream, "
                      f"{w.context} tokens) in fp16 input bytes per second"}


def component_times(w, cache, k_new, v_new, q, out, stream, reps: int = 50):
    """Mean microseconds of each library call of a decode step, one call at a
    time between events (launch gaps included): the fused append, the key
    flush of R tokens (every R steps), the value-window compaction (R rows,
    every R + 2 steps), the attention, and the whole step as one
    kvq_kivi_step call.  The cache state is restored after each call."""
    import torch
    from decode_attention_kivi_amd import KVQ_KEYS, kvq_quantize_append, kvq_residual_append
    saved = (cache.n_kq, cache.r_k, cache.n_vq, cache.r_v, cache.v_start)

    def restore():
        cache.n_kq, cache.r_k, cache.n_vq, cache.r_v, cache.v_start = saved

    # the flush writes into scratch arenas of R tokens (the cache's own key run
    # has no room past its current length)
    kc = torch.empty(cache.n_streams, cache.R * cache.d * cache.bits // 8, dtype=torch.uint8,
                     device=q.device)
    km = torch.empty(cache.n_streams, cache.R // cache.G * cache.d * 4, dtype=torch.uint8, device=q.device)

    def flush():
        kvq_quantize_append(KVQ_KEYS, cache.bits, cache.G, cache.n_streams, cache.d, cache.R,
                            cache.k_res, cache.k_res.stride(0), cache.d, None, kc, kc.stride(0),
                            km, km.stride(0), 0, stream)

    def compaction():
        # the value window's R rows move back to row 0 (every R + 2 steps)
        kvq_residual_append(cache.n_streams, cache.d, cache.R, cache.v_res[:, cache.R + 2:], cache.v_res.stride(0),
                            cache.d, cache.v_res, cache.v_res.stride(0), 0, stream)

    calls = {
        "decode_append": lambda: cache.append(k_new, v_new, stream=stream),
        "key_flush_R_tokens": flush,
        "window_compaction_R_rows": compaction,
        "attention": lambda: cache.attend(q, w.sm_scale, out=out, stream=stream),
        "kivi_step_one_call": lambda: cache.step(k_new, v_new, q, w.sm_scale, out=out, stream=stream),
    }
    res = {}
    for name, fn in calls.items():
        total = 0.0
        for i in range(reps + 5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            restore()
            torch.cuda.synchronize()
            if i >= 5:
                total += e0.elapsed_time(e1)
        res[name] = round(total / reps * 1e3, 2)
    return res


def host_call_us(cache, q, out, sm_scale, stream, calls: int = 200):
    """Host microseconds per eager call (argument marshalling in the binding,
    the library's checks and launch plan, the launch itself), for
    kvq_decode_attn with the arguments built once and for the cache helper
    that builds them per call (its workspace query plans a second time)."""
    import torch
    import decode_attention_kivi_amd as kvq
    a = cache.decode_args(q, out, sm_scale)
    res = {}
    for name, fn in (("kvq_decode_attn", lambda: kvq.kvq_decode_attn(a, stream)),
                     ("cache_attend", lambda: cache.attend(q, sm_scale, out=out, stream=stream))):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(calls):
            fn()
        res[name] = round((time.perf_counter() - t0) / calls * 1e6, 2)
        torch.cuda.synchronize()
    return res


def device_kv(w: workloads.Workload, dev, seed: int = 0):
    """Keys and values fp16 [B][Hkv][N][d] of a workload drawn on the device
    with the workload's distribution (N(0, 1), the same outlier key channels
    scaled in fp32 before the cast); only the timing uses these, so they come
    from torch's device generator rather than the host streams."""
    import torch
    g = torch.Generator(device=dev).manual_seed(seed)
    shape = (w.batch, w.n_kv_heads, w.n_tokens, w.d_h)
    k = torch.randn(shape, generator=g, device=dev)
    for h in range(w.n_kv_heads):
        oc = workloads.outlier_channels(w, h)
        if oc.size:
            k[:, h, :, torch.from_numpy(oc).to(dev)] *= w.outlier_factor
    k = k.half()
    v = torch.randn(shape, generator=g, device=dev).half()
    return k, v


def graph_time_us(stream, calls_per_graph: int, record, reps: int = 40, warm: int = 3):
    """Mean microseconds per call of `record()` (which enqueues
    calls_per_graph calls) captured in one HIP graph and replayed `reps`
    times between events on `stream`."""
    import torch
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            record()
        for _ in range(warm):
            graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            graph.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * calls_per_graph) * 1e3


def flush_rate(dev, stream, copies: int = 16, streams: int = 512, d: int = 128, R: int = 128,
               G: int = 32, bits: int = 2):
    """The two calls a KIVI cache makes besides the step, at the Llama-2-7B
    decode shape (16 sequences x 32 heads = 512 streams, d128, G32, R128,
    int2): the key flush (kvq_quantize_append of the R residual keys, every R
    steps) and the value-window compaction (kvq_residual_append of R rows back
    to row 0, every R + 2 steps).  Each call reads the next of `copies`
    residual copies (16 x 16.8 MB, more than the 256 MB Infinity Cache), one
    HIP graph per kind.  Algorithmic bytes: the flush reads R fp16 rows and
    writes their codes and R / G (scale, zero) rows per stream; the
    compaction reads and writes R fp16 rows per stream."""
    import torch
    import decode_attention_kivi_amd as kvq
    g = torch.Generator(device=dev).manual_seed(7)
    res = [torch.randn(streams, 2 * R + 2, d, generator=g, device=dev).half() for _ in range(copies)]
    kc = [torch.empty(streams, R * d * bits // 8, dtype=torch.uint8, device=dev) for _ in range(copies)]
    km = [torch.empty(streams, R // G * d * 4, dtype=torch.uint8, device=dev) for _ in range(copies)]
    row = (2 * R + 2) * d

    def flushes():
        for r, c, m in zip(res, kc, km):
            kvq.kvq_quantize_append(kvq.KVQ_KEYS, bits, G, streams, d, R, r, row, d, None, c, c.stride(0),
                                    m, m.stride(0), 0, stream)

    def compactions():
        for r in res:
            kvq.kvq_residual_append(streams, d, R, r[:, R + 2:], row, d, r, row, 0, stream)
    flush_us = graph_time_us(stream, copies, flushes)
    comp_us = graph_time_us(stream, copies, compactions)
    fb = streams * (R * d * 2 + R * d * bits // 8 + R // G * d * 4)
    cb = streams * R * d * 2 * 2
    del res, kc, km
    return {"config": f"{streams} streams (16 x 32 heads), d{d}, G{G}, R{R}, int{bits}; "
                      f"{copies} rotating residual copies",
            "key_flush": {"us_per_call": round(flush_us, 2), "algorithmic_bytes": fb,
                          "GBs": round(fb / (flush_us * 1e-6) / 1e9, 1)},
            "window_compaction": {"us_per_call": round(comp_us, 2), "algorithmic_bytes": cb,
                                  "GBs": round(cb / (comp_us * 1e-6) / 1e9, 1)}}


def config_rate(name: str, dev, stream, min_copies: int = 2):
    """kvq_decode_attn at one of the uniform KIVI workloads' full sizes, in
    the state after prefill and one decode step, over rotating cache copies
    (at least two and more than twice the 256 MB Infinity Cache, so the
    reads come from HBM; a cache smaller than that is simply repeated)."""
    import torch
    from decode_attention_kivi_amd.cache import KiviCache
    w = workloads.get(name)
    k, v = device_kv(w, dev)
    q = torch.randn(w.batch, w.n_q_heads, w.d_h, generator=torch.Generator(device=dev).manual_seed(1),
                    device=dev).half()
    L = w.context
    caches = []
    while True:
        c = KiviCache(w.batch, w.n_kv_heads, w.d_h, w.bits, w.group, w.residual, w.n_tokens, dev)
        c.prefill(k[:, :, :L], v[:, :, :L])
        c.append(k[:, :, L:L + 1], v[:, :, L:L + 1])
        caches.append(c)
        attn_b, _ = step_bytes(w, c.lengths)
        if len(caches) >= min_copies and (len(caches) * attn_b > 2 * 256e6 or len(caches) >= 32):
            break
    del k, v
    outs = [torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in caches]
    for c, o in zip(caches, outs):
        c.attend(q, w.sm_scale, out=o)              # workspaces outside capture
    rounds = max(1, 16 // len(caches))

    def record():
        for _ in range(rounds):
            for c, o in zip(caches, outs):
                c.attend(q, w.sm_scale, out=o)
    us = graph_time_us(stream, rounds * len(caches), record)
    a = caches[0].decode_args(q, outs[0], w.sm_scale)
    import decode_attention_kivi_amd as kvq
    merge = kvq.kvq_decode_attn_workspace(a) > 0
    n_copies = len(caches)
    del caches, a
    torch.cuda.synchronize()
    return {"us_per_launch": round(us, 2), "algorithmic_bytes": int(attn_b),
            "GBs": round(attn_b / (us * 1e-6) / 1e9, 1), "frac": round(attn_b / (us * 1e-6) / 8e12, 4),
            "cache_copies": n_copies, "merge_kernel": merge,
            "tokens_context_per_s": round(w.batch * w.n_tokens / (us * 1e-6), 1)}


def window_search_rate(dev, stream, reps: int = 30, copies: int = 3):
    """The WindowQuant window-level search (kvq_window_search) at the size
    of the pages' video workloads: one request, a 64-token prompt and 128
    windows of 256 visual tokens, encoder dim 3584.  It reads every token
    once: (64 + 32768) * 3584 * 2 bytes.  Consecutive calls use different
    copies of the tokens (3 x 235 MB, more than twice the 256 MB Infinity
    Cache), so the rate is that of HBM reads."""
    import torch
    import decode_attention_kivi_amd as kvq
    B, N, W, S, D = 1, 64, 128, 256, 3584
    M = W * S
    g = torch.Generator(device=dev).manual_seed(0)
    inputs = [(torch.randn(B, N, D, generator=g, device=dev).half(),
               torch.randn(B, M, D, generator=g, device=dev).half()) for _ in range(copies)]
    bits = torch.empty(W, dtype=torch.uint8, device=dev)
    nbytes = kvq.kvq_window_search_workspace(B, N, M, D, S)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    t_low, t_high = kvq.kvq_window_thresholds(0.5, 2.0)

    def call(i):
        text, vis = inputs[i % copies]
        kvq.kvq_window_search(B, N, M, D, text, N * D, D, vis, M * D, D, S, t_low, t_high, 1, None,
                              bits, ws, nbytes, stream)
    for i in range(2 * copies):
        call(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps):
        call(i)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    read = (N + M) * D * 2 * B
    del inputs
    return {"config": "B1 prompt 64 tokens, 128 windows x 256 tokens, dim 3584, 3 rotating input copies",
            "us_per_call": round(us, 2), "bytes_read": read, "GBs": round(read / (us * 1e-6) / 1e9, 1)}


def paged_ragged_rate(dev, stream, n_seq: int = 32, page_tokens: int = 256, copies: int = 2,
                      reps: int = 40):
    """kvq_decode_attn_paged on a ragged batch in pages: 32 sequences x 32
    heads (Llama-2-7B attention), d128, G32, R128, int2, page 256 tokens,
    contexts from workloads.ragged_contexts (log-uniform in [512, 8192]);
    each sequence is in the state after its prefill and one decode step.
    Consecutive calls use different cache copies (> 2 x 256 MB in total)."""
    import torch
    from decode_attention_kivi_amd.cache import PagedKiviCache, kivi_step_lengths
    H, d, G, R, bits = 32, 128, 32, 128, 2
    ctx = workloads.ragged_contexts(n_seq)
    g = torch.Generator(device=dev).manual_seed(5)
    caches = []
    for c in range(copies):
        cache = PagedKiviCache(n_seq, H, d, bits, G, R, page_tokens, max(ctx) + 1, device=dev, seed=c)
        for b, L in enumerate(ctx):
            k = torch.randn(H, L + 1, d, generator=g, device=dev).half()
            v = torch.randn(H, L + 1, d, generator=g, device=dev).half()
            cache.fill_step(b, k, v)
            del k, v
        caches.append(cache)
    q = torch.randn(n_seq, H, d, generator=g, device=dev).half()
    outs = [torch.empty(n_seq, H, d, dtype=torch.float32, device=dev) for _ in caches]
    sm = 1.0 / d ** 0.5
    for c, o in zip(caches, outs):
        c.attend(q, sm, out=o)                      # workspace allocated outside capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            for _ in range(4):
                for c, o in zip(caches, outs):
                    c.attend(q, sm, out=o)
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            graph.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / (reps * 4 * copies) * 1e3
    rb = d * bits // 8
    nbytes = 0
    for L in ctx:
        n_kq, r_k, n_vq, r_v = kivi_step_lengths(L, R)
        nbytes += H * (n_kq * (rb + d * 4 // G) + n_vq * (rb + (d // G) * 4) + (r_k + r_v) * d * 2)
    nbytes += n_seq * H * d * (2 + 4)
    wg = caches[0].args(q, sm, outs[0])
    import decode_attention_kivi_amd as kvq
    ws = kvq.kvq_decode_attn_paged_workspace(wg)
    del caches
    return {"config": f"{n_seq} sequences, 32 heads, d128, G32, R128, int2, page {page_tokens} tokens, "
                      f"contexts log-uniform in [512, 8192] (total {sum(ctx) + n_seq} tokens), "
                      f"{copies} rotating cache copies",
            "us_per_call": round(us, 2), "algorithmic_bytes": int(nbytes),
            "GBs": round(nbytes / (us * 1e-6) / 1e9, 1), "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / 8e12, 4),
            "merge_kernel": ws > 0}


def windows_decode_rate(dev, stream, copies: int = 32):
    """kvq_decode_attn on the mixed-precision window cache (qwen2_7b_windows:
    28 q / 4 kv heads, 128 windows x 256 tokens at 8/4/2 bits after the
    reorder + 65 fp16 tokens).  The cache is 17.7 MB, so `copies` copies
    (566 MB, more than twice the 256 MB Infinity Cache) are read in turn and
    every call reads HBM."""
    import torch
    from decode_attention_kivi_amd.cache import WindowCache
    w = workloads.get("qwen2_7b_windows")
    k, v = workloads.full_kv(w)
    bits = workloads.window_bits(w, k)
    q = torch.from_numpy(workloads.queries(w)).to(dev)
    kt, vt, bt = torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev), torch.from_numpy(bits).to(dev)
    caches = [WindowCache(kt, vt, bt, w.window_tokens, w.group) for _ in range(copies)]
    outs = [torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in caches]
    for c, o in zip(caches, outs):
        c.attend(q, w.sm_scale, out=o)              # workspace outside capture

    def record():
        for c, o in zip(caches, outs):
            c.attend(q, w.sm_scale, out=o)
    us = graph_time_us(stream, copies, record)
    cache = caches[0]
    d, G, H = w.d_h, w.group, w.n_kv_heads
    nbytes = 0
    for sg in cache.segs:
        b, n = sg[0], sg[2]
        if b == 16:
            nbytes += 2 * n * d * 2
        else:
            nbytes += n * d * b // 8 + n // G * d * 4 + n * d * b // 8 + n * (d // G) * 4
    nbytes = H * (nbytes + 2 * cache.n_res * d * 2) + w.batch * w.n_q_heads * d * 6
    n_res = cache.n_res
    del caches, cache
    return {"config": "qwen2_7b_windows: B1, 28 q / 4 kv heads, 128 windows x 256 tokens "
                      f"({int((bits == 8).sum())} int8 / {int((bits == 4).sum())} int4 / "
                      f"{int((bits == 2).sum())} int2, reordered) + {n_res} fp16 tokens; "
                      f"{copies} rotating cache copies",
            "us_per_launch": round(us, 2), "algorithmic_bytes": int(nbytes),
            "GBs": round(nbytes / (us * 1e-6) / 1e9, 1), "frac": round(nbytes / (us * 1e-6) / 8e12, 4)}


def pq_search_rate(dev, stream, reps: int = 50, B: int = 4, n: int = 32769):
    """kvq_pq_search (PQCache's decode-time PQ search) at the GQA long-context
    shape: B sequences x 32 query heads over 8 kv heads, n tokens (32769, or
    the page's 128K context), m = 2 sub-spaces of 256 centroids (8-bit
    codes), Top-k = 1/10 of the tokens.  One kernel per call (a head's 32769 scores fit in LDS): each
    query head's workgroup reads its kv head's codes and centroids and q,
    writes the fp32 scores and the Top-k indices.  Algorithmic bytes count
    the codes and centroids once per kv head."""
    import torch
    import decode_attention_kivi_amd as kvq
    Hq, Hkv, d, m, bits = 32, 8, 128, 2, 8
    k = (n + 9) // 10
    w = workloads.Workload(name="pq", batch=B, n_q_heads=Hq, n_kv_heads=Hkv, d_h=d, context=n,
                           group=32, residual=32, bits=2)
    c, codes = workloads.pq_inputs(B, Hkv, n, d, m, bits)
    stride = (n * m + 15) // 16 * 16
    padded = np.zeros((B * Hkv, stride), np.uint8)
    padded[:, :n * m] = codes.reshape(B * Hkv, -1)
    qt = torch.from_numpy(workloads.queries(w)).to(dev)
    ct = torch.from_numpy(c).to(dev)
    kt = torch.from_numpy(padded).to(dev)
    sc = torch.empty(B, Hq, n, dtype=torch.float32, device=dev)
    idx = torch.empty(B, Hq, k, dtype=torch.int32, device=dev)

    def call():
        kvq.kvq_pq_search(B, Hq, Hkv, d, m, bits, n, k, qt, ct, kt, stride, sc, idx, stream)
    with torch.cuda.stream(stream):
        for _ in range(5):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    nbytes = B * Hkv * (n * m + m * (1 << bits) * (d // m) * 2) + B * Hq * (d * 2 + n * 4 + k * 4)
    return {"config": f"B{B}, {Hq} q / {Hkv} kv heads, d{d}, {n} tokens, m {m}, {1 << bits} centroids, "
                      f"Top-k {k}", "us_per_call": round(us, 2), "algorithmic_bytes": int(nbytes),
            "tokens_scored_per_s": round(B * Hq * n / (us * 1e-6), 1)}


def vq_decode_rate(dev, stream, rounds: int, reps: int = 30, copies: int = 2):
    """kvq_vq_decode_attn (decode attention over a vector-quantized cache,
    4-channel codebooks of 256 entries; rounds = 1 is CQ-2, 2 is CQ-4) at the
    Llama-2-7B decode shape: 16 sequences x 32 heads, d128, 4097 tokens.
    Consecutive calls read different copies of the codes (2 x 134 MB for
    CQ-2), so they come from HBM.  Algorithmic bytes: the key and value codes
    once, both codebooks of every kv head once, q and out."""
    import torch
    import decode_attention_kivi_amd as kvq
    B, H, d, n = 16, 32, 128, 4097
    tb = rounds * d // 4
    stride = (n * tb + 15) // 16 * 16
    g = torch.Generator(device=dev).manual_seed(0)
    codes = [(torch.randint(0, 256, (B * H, stride), generator=g, device=dev, dtype=torch.uint8),
              torch.randint(0, 256, (B * H, stride), generator=g, device=dev, dtype=torch.uint8))
             for _ in range(copies)]
    kb = torch.randn(H, rounds, d // 4, 256, 4, generator=g, device=dev).half()
    vb = torch.randn(H, rounds, d // 4, 256, 4, generator=g, device=dev).half()
    q = torch.randn(B, H, d, generator=g, device=dev).half()
    out = torch.empty(B, H, d, dtype=torch.float32, device=dev)
    ws_bytes = kvq.kvq_vq_decode_attn_workspace(B, H, H, d, rounds, n)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

    def call(i):
        kc, vc = codes[i % copies]
        kvq.kvq_vq_decode_attn(B, H, H, d, rounds, n, 1.0 / d ** 0.5, q, kc, vc, stride, kb, vb, out,
                               ws if ws_bytes else None, ws_bytes, stream)
    with torch.cuda.stream(stream):
        for i in range(4):
            call(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            call(i)
        e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    nbytes = 2 * B * H * n * tb + 2 * H * rounds * (d // 4) * 256 * 4 * 2 + B * H * d * 6
    return {"config": f"CQ-{2 * rounds}: 16 x 32 heads, d128, 4097 tokens, 4-channel codebooks of 256 entries, "
                      f"{rounds} round(s)", "us_per_call": round(us, 2), "algorithmic_bytes": int(nbytes),
            "GBs": round(nbytes / (us * 1e-6) / 1e9, 1), "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / 8e12, 4)}


def streaming_read_ceiling(dev, stream, gib: float = 1.0, reps: int = 20) -> float:
    """GB/s of a plain streaming read on this GPU: torch's sum over a 1 GiB
    buffer (well past the 256 MB Infinity Cache), the practical ceiling the
    decode kernel is compared with (its roofline fraction stays against the
    8 TB/s peak)."""
    import torch
    x = torch.ones(int(gib * (1 << 30)) // 8, dtype=torch.int64, device=dev)
    for _ in range(3):
        x.sum()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        x.sum()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del x
    return round(x_bytes(gib) / (ms * 1e-3) / 1e9, 1)


def x_bytes(gib: float) -> int:
    return int(gib * (1 << 30)) // 8 * 8


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama2_7b")
    ap.add_argument("--copies", type=int, default=0, help="cache copies (0 = enough for 2x 256 MB)")
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--rounds", type=int, default=4, help="passes over the cache copies per graph")
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="seconds of untimed replays before timing (clock ramp-up)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--part", choices=("all", "attention", "step", "paged", "pq", "search", "windows", "vq",
                                       "config", "flush"),
                    default="all",
                    help="profiling runs: time only the attention graph, only the step graph, the paged "
                         "ragged batch, the PQ search, the window search, the mixed-precision "
                         "window cache, the VQ-cache decode, one workload's attention (--workload) "
                         "or the key flush and window compaction (and skip the rest)")
    ap.add_argument("--page-tokens", type=int, default=256, help="page size of the paged ragged batch")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one fp16 row copy of this many MiB first (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "one GPU only: --gpus must be 1 "
                                   "(sharding the streams or the context across GPUs is not built)"}))
        sys.exit(2)

    import torch
    from decode_attention_kivi_amd.cache import KiviCache
    lib = os.path.join(ROOT, "decode_attention_kivi_amd", "libkvq.so")
    if not os.path.exists(lib):
        import __graft_entry__
        __graft_entry__.build()
    if args.copy_probe_mib:
        # a plain copy of known size through the library's row-copy kernel:
        # its FETCH_SIZE / WRITE_SIZE per byte calibrate the traffic counters
        import decode_attention_kivi_amd as kvq
        rows = args.copy_probe_mib * (1 << 20) // 256
        src = torch.ones(rows, 128, dtype=torch.float16, device="cuda:0")
        dst = torch.empty_like(src)
        kvq.kvq_residual_append(1, 128, rows, src, 0, 128, dst, 0, 0)
        torch.cuda.synchronize()
        del src, dst
    if args.part == "vq":
        dev, st = torch.device("cuda:0"), torch.cuda.Stream()
        for rounds in (1, 2):
            print(json.dumps({"part": "vq", **vq_decode_rate(dev, st, rounds)}), flush=True)
        return
    if args.part in ("paged", "pq", "search", "windows", "config", "flush"):
        dev, st = torch.device("cuda:0"), torch.cuda.Stream()
        if args.part == "flush":
            r = flush_rate(dev, st)
        elif args.part == "config":
            r = {"workload": args.workload, **config_rate(args.workload, dev, st)}
        elif args.part == "paged":
            r = paged_ragged_rate(dev, st, page_tokens=args.page_tokens)
        elif args.part == "pq":
            r = pq_search_rate(dev, st)
            r["context_128k"] = pq_search_rate(dev, st, reps=20, B=1, n=131072)
        elif args.part == "search":
            r = window_search_rate(dev, st)
        else:
            r = windows_decode_rate(dev, st)
        print(json.dumps({"part": args.part, **r}), flush=True)
        return

    w = workloads.get(args.workload)
    assert not w.mixed, "bench runs the uniform KIVI workloads"
    dev = torch.device("cuda:0")
    L = w.context
    k, v = workloads.full_kv(w)
    q = torch.from_numpy(workloads.queries(w)).to(dev)
    kt = torch.from_numpy(k).to(dev)
    vt = torch.from_numpy(v).to(dev)
    del k, v

    attn_probe = None
    caches = []
    copies = args.copies
    t_build = time.perf_counter()
    while True:
        c = KiviCache(w.batch, w.n_kv_heads, w.d_h, w.bits, w.group, w.residual, w.n_tokens, dev)
        c.prefill(kt[:, :, :L], vt[:, :, :L])
        caches.append(c)
        if attn_probe is None:
            st0 = c.lengths, c.v_start
            c.append(kt[:, :, L:L + 1], vt[:, :, L:L + 1])
            attn_probe = c.lengths
            (c.n_kq, c.r_k, c.n_vq, c.r_v), c.v_start = st0
        attn_b, total_b = step_bytes(w, attn_probe)
        if copies and len(caches) >= copies:
            break
        if not copies and len(caches) >= 4 and len(caches) * attn_b > 2 * 256e6:
            break
    torch.cuda.synchronize()
    t_build = time.perf_counter() - t_build
    n_caches = len(caches)
    saved = [(c.n_kq, c.r_k, c.n_vq, c.r_v, c.v_start) for c in caches]
    outs = [torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in caches]
    k_new, v_new = kt[:, :, L:L + 1], vt[:, :, L:L + 1]

    def restore():
        for c, s in zip(caches, saved):
            c.n_kq, c.r_k, c.n_vq, c.r_v, c.v_start = s

    # a decode step is one kvq_kivi_step call (append + attention; fused into
    # one launch at this shape) unless a split size is forced, then the two
    # separate calls; workspaces are prepared outside capture
    def one_step(c, o):
        if args.split_tokens:
            c.append(k_new, v_new)
            c.attend(q, w.sm_scale, out=o, split_tokens=args.split_tokens)
        else:
            c.step(k_new, v_new, q, w.sm_scale, out=o)
    for c, o in zip(caches, outs):
        one_step(c, o)
    step_launches = caches[0].last_launches if not args.split_tokens else None
    restore()
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()
    step_graph = torch.cuda.CUDAGraph() if args.part in ("all", "step") else None
    attn_graph = torch.cuda.CUDAGraph() if args.part in ("all", "attention") else None
    with torch.cuda.stream(stream):
        if step_graph is not None:
            with torch.cuda.graph(step_graph, stream=stream):
                for _ in range(args.rounds):
                    restore()
                    for c, o in zip(caches, outs):
                        one_step(c, o)
        restore()
        for c in caches:           # attention-only graph on the post-step state
            c.append(k_new, v_new)
        torch.cuda.synchronize()
        if attn_graph is not None:
            with torch.cuda.graph(attn_graph, stream=stream):
                for _ in range(args.rounds):
                    for c, o in zip(caches, outs):
                        c.attend(q, w.sm_scale, out=o, split_tokens=args.split_tokens)
    restore()
    torch.cuda.synchronize()
    n_copies = len(caches) * args.rounds       # steps per graph replay
    # the steps a whole number of replays leaves over: one more graph of that
    # many steps (the first copies of a pass), so exactly --steps are timed
    tail_n = args.steps % n_copies
    step_tail = attn_tail = None
    if tail_n:
        with torch.cuda.stream(stream):
            if step_graph is not None:
                step_tail = torch.cuda.CUDAGraph()
                with torch.cuda.graph(step_tail, stream=stream):
                    restore()
                    for c, o in list(zip(caches, outs))[:tail_n]:
                        one_step(c, o)
            restore()
            for c in caches:
                c.append(k_new, v_new)
            torch.cuda.synchronize()
            if attn_graph is not None:
                attn_tail = torch.cuda.CUDAGraph()
                with torch.cuda.graph(attn_tail, stream=stream):
                    for c, o in list(zip(caches, outs))[:tail_n]:
                        c.attend(q, w.sm_scale, out=o, split_tokens=args.split_tokens)
        restore()
        torch.cuda.synchronize()

    def timed(graph, tail, steps, warmup):
        """Mean ms per step over exactly `steps` timed steps (whole replays,
        then the tail graph), the step count, and the (p10, p50, p90) of the
        per-replay means of the whole replays (events between replays)."""
        reps_w = max(1, -(-warmup // n_copies))
        reps = steps // n_copies
        for _ in range(reps_w):
            graph.replay()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 2)]
        ev[0].record(stream)
        for i in range(reps):
            graph.replay()
            ev[i + 1].record(stream)
        if steps % n_copies:
            tail.replay()
        ev[reps + 1].record(stream)
        torch.cuda.synchronize()
        per = sorted(ev[i].elapsed_time(ev[i + 1]) / n_copies for i in range(reps)) or \
            [ev[0].elapsed_time(ev[1]) / max(steps, 1)]
        pct = lambda f: per[min(len(per) - 1, int(round(f * (len(per) - 1))))]
        return ev[0].elapsed_time(ev[reps + 1]) / steps, steps, (pct(.1), pct(.5), pct(.9))

    with torch.cuda.stream(stream):
        # let the clocks settle (both graphs, untimed) before either is timed
        t_settle = time.perf_counter()
        while time.perf_counter() - t_settle < args.settle_s:
            for g in (step_graph, attn_graph):
                if g is not None:
                    g.replay()
            torch.cuda.synchronize()
        attn_ms = step_ms = None
        attn_pct = step_pct = (float("nan"),) * 3
        n_steps = 0
        components = ceiling = search_rate = paged_rate = windows_rate = pq_rate = vq_rates = None
        configs = host_us = flush = None
        if attn_graph is not None:
            attn_ms, n_steps, attn_pct = timed(attn_graph, attn_tail, args.steps, args.warmup)
        if step_graph is not None:
            step_ms, n_steps, step_pct = timed(step_graph, step_tail, args.steps, args.warmup)
        if args.part == "all":
            components = component_times(w, caches[0], k_new, v_new, q, outs[0], stream)
            host_us = host_call_us(caches[0], q, outs[0], w.sm_scale, stream)
            restore()
            flush = flush_rate(dev, stream)
            ceiling = streaming_read_ceiling(dev, stream)
            search_rate = window_search_rate(dev, stream)
            paged_rate = paged_ragged_rate(dev, stream, page_tokens=args.page_tokens)
            windows_rate = windows_decode_rate(dev, stream)
            del caches, outs, kt, vt
            configs = {"llama2_7b": None}
            for name in ("tiny", "llama2_7b_b64_int2", "llama2_7b_b64_int4", "llama31_8b_gqa"):
                configs[name] = config_rate(name, dev, stream)
            configs["qwen2_7b_windows"] = windows_rate
            pq_rate = pq_search_rate(dev, stream)
            pq_rate["context_128k"] = pq_search_rate(dev, stream, reps=20, B=1, n=131072)
            vq_rates = {f"cq{2 * r}": vq_decode_rate(dev, stream, r) for r in (1, 2)}
    torch.cuda.synchronize()

    if args.part != "all":
        print(json.dumps({"part": args.part, "workload": w.name, "steps": n_steps,
                          "us_per_launch": round(attn_ms * 1e3, 2) if attn_ms else None,
                          "us_per_step": round(step_ms * 1e3, 2) if step_ms else None,
                          "launches_per_step": step_launches}), flush=True)
        return
    achieved = attn_b / (attn_ms * 1e-3) / 1e9
    value = total_b / (step_ms * 1e-3) / 1e9
    configs["llama2_7b"] = {"us_per_launch": round(attn_ms * 1e3, 2), "algorithmic_bytes": int(attn_b),
                            "GBs": round(achieved, 1), "frac": round(achieved / HBM_PEAK_GBS, 4),
                            "cache_copies": n_caches, "merge_kernel": False,
                            "tokens_context_per_s": round(w.batch * w.n_tokens / (attn_ms * 1e-3), 1)}
    # a step that also flushes the key residual (every R steps) or compacts
    # the value window (every R + 2 steps) costs those calls on top
    amortized = step_ms * 1e3 + flush["key_flush"]["us_per_call"] / w.residual + \
        flush["window_compaction"]["us_per_call"] / (w.residual + 2)
    result = {
        "metric": "decode-attn effective KV GB/s (% of HBM peak) + us/step, int2 Llama-2-7B shape",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": n_steps,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 5), "us_per_step": round(step_ms * 1e3, 2),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_context_per_s": round(w.batch * w.n_tokens / (step_ms * 1e-3), 1),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u2/f16/f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.n_q_heads,
                   "kv_heads": w.n_kv_heads, "d_h": w.d_h, "context": w.context,
                   "attended_tokens": w.n_tokens, "group": w.group, "residual": w.residual,
                   "bits": w.bits, "cache_copies": n_caches, "steps_per_graph": n_copies,
                   "cache_state_nKq_rK_nVq_rV": list(attn_probe),
                   "launches_per_step": step_launches,
                   "algorithmic_bytes_step": int(total_b), "algorithmic_bytes_attention": int(attn_b)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(w.name),
                     "traffic_note": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated), "
                                     "null if the kernel changed since the counters were taken",
                     "algorithmic_bytes_per_launch": int(attn_b),
                     "kernel": "decode_kernel: one kvq_decode_attn call (one workgroup per stream here, so no merge kernel)",
                     "us_per_launch": round(attn_ms * 1e3, 2),
                     "us_per_launch_p10_p50_p90": [round(x * 1e3, 2) for x in attn_pct],
                     "streaming_read_ceiling_GBs": ceiling,
                     "frac_by_workload": {k: c["frac"] for k, c in configs.items()}},
        "configs": configs,
        "configs_note": "kvq_decode_attn per workload at full size, graph-replayed over rotating cache "
                        "copies (HBM reads); algorithmic bytes / us per launch (split + merge kernels)",
        "us_per_step_p10_p50_p90": [round(x * 1e3, 2) for x in step_pct],
        "components_us": components,
        "components_note": "each library call timed alone between events with a synchronize after it "
                           "(launch latency included); us_per_step is the graph-replayed step",
        "us_per_step_amortized": round(amortized, 2),
        "us_per_step_amortized_note": "us_per_step + key flush / R + window compaction / (R + 2), the "
                                      "last two graph-replayed over rotating copies (flush_and_compaction)",
        "flush_and_compaction": flush,
        "host_us_per_call": host_us,
        "window_search": search_rate,
        "paged_ragged": paged_rate,
        "pq_search": pq_rate,
        "vq_decode": vq_rates,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
