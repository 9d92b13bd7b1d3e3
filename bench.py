#!/usr/bin/env python3
"""Benchmark of the paged-KV attention hot path on one MI355X.

Headline: one decode layer-step of the batch-64 decode workload (batch 64, context_lens U[512,4096], block_size 256, bf16,
16 q / 8 kv heads, head_dim 128): slot_mapping, the store of each sequence's new token and the paged decode
attention, in one attn_decode_paged_store call (the same results as kv_slot_mapping -> kv_store ->
attn_decode_paged, which is measured too, under ``secondary``).  ``value`` is the KV-cache bytes the decode
must read (sum(context_lens) * 2 * Hkv * hd * 2 B) divided by the whole step's time.  Steps rotate over
``--layers`` independent caches (different layers of the model), so the 256 MB Infinity Cache cannot hold
the working set between steps.

The same JSON line carries:
  roofline      the step's call (split + combine kernels) timed with two HIP events on the stream it runs
                on around K back-to-back calls over the same rotated caches (an event record per call would
                make the GPU drain before each one), against MI355X's 8 TB/s HBM peak; ``traffic`` from
                rocprofv3 counters kept in profiles/ (null if the kernel source changed since they were
                taken); ``kernel_ms_spread`` gives the median and the minimum ms per call over chunks of 50
                calls of a second pass (events at chunk boundaries only), as the decode, prefill and store
                entries do;
  cpu_baseline  the CPU oracle on the host's cores (a pool of worker processes, one BLAS thread each, run
                before the GPU is touched): decode attention of the whole batch-64 decode workload, with the
                varlen prefill (TFLOP/s) and the store sweep (GB/s) beside it;
  secondary     the unfused decode step and call, varlen prefill TFLOP/s (8 sequences of 128-2048), prefix-cache
                prefill TFLOP/s (16 sequences), chunked prefill on 16k/32k-token cached prefixes (with and without
                the splitting of long key ranges), the platform BLAS's bf16 GEMM rate (the practical matrix-core
                rate under full load), the store sweep GB/s (N=16384), the long padded decode GB/s (batch 256)
                and the fused QK-Norm + RoPE + store GB/s (the 8 prefill sequences' tokens); the bandwidth-bound
                ones rotate enough independent inputs (``sets_rotated``) that each call reads from HBM, not from
                rows the last-level cache kept from an earlier call.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--headline-only] [--no-cpu]
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
PROFILES = os.path.join(ROOT, "profiles")
METRIC = "paged decode attn KV GB/s (% HBM peak); varlen prefill TFLOP/s; store GB/s"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "paged_kv_cache_300_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(name, src_hash):
    """Bytes per launch from committed rocprofv3 counter runs, if they were taken on the current source."""
    path = os.path.join(PROFILES, f"{name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


# ------------------------------------------------------------------------------------------------ GPU side

def run_steps(torch, step, steps, warmup):
    """W untimed steps, then exactly K timed steps between device synchronisations; returns ms per step."""
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def time_kernel(torch, call, n):
    """HIP events on the current stream around ``n`` back-to-back calls (no event between them: an event
    record waits for the GPU to drain, which would add its own gap to every call); returns ms per call."""
    for i in range(2):
        call(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(n):
        call(i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / n


def time_kernel_spread(torch, call, n, per_chunk=50):
    """The same back-to-back calls as time_kernel, in chunks of ``per_chunk`` with an event at each chunk boundary
    only: the median and the minimum over chunks of the ms per call (a separate pass, so the events between chunks
    do not touch the mean the line reports)."""
    chunks = max(1, n // per_chunk)
    for i in range(2):
        call(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(chunks + 1)]
    ev[0].record()
    for c in range(chunks):
        for i in range(per_chunk):
            call(c * per_chunk + i)
        ev[c + 1].record()
    torch.cuda.synchronize()
    per_call = sorted(ev[c].elapsed_time(ev[c + 1]) / per_chunk for c in range(chunks))
    return {"median_ms": round(per_call[len(per_call) // 2], 5), "min_ms": round(per_call[0], 5),
            "chunks": chunks, "calls_per_chunk": per_chunk}


def dev_case_layers(make, layers, torch):
    """``layers`` independent draws of one workload's tensors (same metadata, different data and caches)."""
    import workloads
    out = []
    for layer in range(layers):
        case = make(device="cuda")
        if layer:
            gen = torch.Generator(device="cuda")
            gen.manual_seed(1000 + layer)
            for name in ("q", "k", "v", "hist_k", "hist_v"):
                t = getattr(case, name)
                setattr(case, name, torch.randn(t.shape, generator=gen, device="cuda").to(t.dtype))
        out.append(case)
    return out, workloads


def build_caches(pkv, torch, case):
    import workloads
    shape = (case.num_blocks, case.block_size, case.num_kv_heads, case.head_dim)
    kc = torch.full(shape, workloads.NAN_BITS["bf16"], dtype=torch.int16, device="cuda").view(torch.bfloat16)
    vc = kc.clone()
    n_hist = int(case.cu_hist[-1])
    if n_hist:
        hist = torch.from_numpy(case.cu_hist).cuda()
        bt = torch.from_numpy(case.block_tables).cuda()
        sm = pkv.kv_slot_mapping(bt, case.block_size, n_hist, cu_seqlens_q=hist, cu_seqlens_k=hist)
        pkv.kv_store(case.hist_k, case.hist_v, kc, vc, sm)
        case.hist_k = case.hist_v = None  # the history now lives in the cache only
    return kc, vc


def bench_decode(pkv, torch, make, steps, warmup, layers, fused=False):
    cases, _ = dev_case_layers(make, layers, torch)
    c0 = cases[0]
    meta = {
        "bt": torch.from_numpy(c0.block_tables).cuda(),
        "ctx": torch.from_numpy(c0.context_lens).cuda(),
    }
    caches = [build_caches(pkv, torch, c) for c in cases]
    ws_bytes = pkv.attn_decode_workspace_bytes(c0.batch, c0.num_q_heads, c0.num_kv_heads, c0.head_dim,
                                               c0.max_blocks, c0.block_size)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    sm = torch.empty(c0.batch, dtype=torch.int32, device="cuda")
    outs = [torch.empty_like(c.q) for c in cases]
    torch.cuda.synchronize()

    def store(L):
        c, (kc, vc) = cases[L], caches[L]
        pkv.kv_slot_mapping(meta["bt"], c0.block_size, c0.batch, context_lens=meta["ctx"], out=sm)
        pkv.kv_store(c.k, c.v, kc, vc, sm)

    def attend(L):
        c, (kc, vc) = cases[L], caches[L]
        pkv.attn_decode_paged(c.q, kc, vc, meta["ctx"], meta["bt"], c0.scale, out=outs[L], workspace=ws)

    def fused_step(L):
        c, (kc, vc) = cases[L], caches[L]
        pkv.attn_decode_paged_store(c.q, c.k, c.v, kc, vc, meta["ctx"], meta["bt"], c0.scale, out=outs[L],
                                    workspace=ws, slot_mapping_out=sm)

    def step(i):
        if fused:
            fused_step(i % layers)
        else:
            store(i % layers)
            attend(i % layers)

    wall_ms = run_steps(torch, step, steps, warmup)
    kern_ms = time_kernel(torch, lambda i: (fused_step if fused else attend)(i % layers), steps)
    spread = time_kernel_spread(torch, lambda i: (fused_step if fused else attend)(i % layers), steps)
    kv_bytes = int(c0.Lk.astype(int).sum()) * 2 * c0.num_kv_heads * c0.head_dim * 2
    del caches, cases
    torch.cuda.empty_cache()
    return {"wall_ms": wall_ms, "kernel_ms": kern_ms, "spread": spread, "kv_bytes": kv_bytes, "batch": c0.batch,
            "sum_ctx": int(c0.Lk.astype(int).sum())}


def prefill_flops(case):
    lq = case.Lq.astype(int)
    lk = case.Lk.astype(int)
    pairs = int(sum(q * (k - q) + q * (q + 1) // 2 for q, k in zip(lq, lk)))
    return 4 * case.head_dim * case.num_q_heads * pairs


CHUNKED_SHAPES = (("chunked_prefill_1x512_on_32k", [512], [32768]),
                  ("chunked_prefill_4x256_on_16k", [256] * 4, [16384] * 4))


def bench_chunked_prefill(pkv, torch, steps):
    """New-token chunks on long cached prefixes (few query tiles over long key ranges): the call as the library
    runs it (the planner cuts the long key ranges into pieces merged by a second kernel) and, for reference, the
    same call without a workspace (each query tile walks its whole key range in one work-group)."""
    import workloads
    out = {}
    for name, chunks, prefixes in CHUNKED_SHAPES:
        c = workloads.chunked_prefill(chunks, prefixes, device="cuda")
        kc, vc = build_caches(pkv, torch, c)
        bt = torch.from_numpy(c.block_tables).cuda()
        cu_q = torch.from_numpy(c.cu_seqlens_q).cuda()
        cu_k = torch.from_numpy(c.cu_seqlens_k).cuda()
        n = int(c.cu_seqlens_q[-1])
        sm = pkv.kv_slot_mapping(bt, c.block_size, n, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k)
        pkv.kv_store(c.k, c.v, kc, vc, sm)
        res = torch.empty_like(c.q)
        mq, mk = int(c.Lq.max()), int(c.Lk.max())
        ws = torch.empty(pkv.attn_prefill_workspace_bytes(c.batch, n, mq, 16, 8, 128), dtype=torch.uint8,
                         device="cuda")
        split_ms = time_kernel(torch, lambda i: pkv.attn_prefill_varlen(
            c.q, kc, vc, cu_q, cu_k, mq, mk, c.scale, block_table=bt, out=res, workspace=ws), max(steps // 4, 10))
        whole_ms = time_kernel(torch, lambda i: pkv.attn_prefill_varlen(
            c.q, kc, vc, cu_q, cu_k, mq, mk, c.scale, block_table=bt, out=res, order=False), max(steps // 4, 10))
        flops = prefill_flops(c)
        out[name] = {"value": round(flops / (split_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                     "kernel_ms": round(split_ms, 4), "flops": flops,
                     "without_split_TFLOPs": round(flops / (whole_ms * 1e-3) / 1e12, 2),
                     "without_split_kernel_ms": round(whole_ms, 4),
                     "shape": f"{len(chunks)} x {chunks[0]} new tokens on {prefixes[0]}-token cached prefixes"}
        del kc, vc, ws, res, c
        torch.cuda.empty_cache()
    return out


def bench_gemm_reference(torch, n=8192, reps=20):
    """The platform BLAS (hipBLASLt through torch.matmul) on an n^3 bf16 product: the dense matrix-core rate this GPU
    sustains under full load, where its clock is held well below the 2.4 GHz the 2.5 PFLOP/s figure assumes."""
    a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    c = torch.empty_like(a)
    for _ in range(5):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b, c
    torch.cuda.empty_cache()
    return 2 * n ** 3 / (ms * 1e-3) / 1e12


def bench_prefill(pkv, torch, make, steps, warmup, layers, paged):
    cases, _ = dev_case_layers(make, layers, torch)
    c0 = cases[0]
    bt = torch.from_numpy(c0.block_tables).cuda()
    cu_q = torch.from_numpy(c0.cu_seqlens_q).cuda()
    cu_k = torch.from_numpy(c0.cu_seqlens_k).cuda()
    caches = [build_caches(pkv, torch, c) for c in cases]
    n = int(c0.cu_seqlens_q[-1])
    sm = torch.empty(n, dtype=torch.int32, device="cuda")
    outs = [torch.empty_like(c.q) for c in cases]
    mq, mk = int(c0.Lq.max()), int(c0.Lk.max())
    torch.cuda.synchronize()

    def attn(c, kc, vc, L):
        if paged:
            pkv.attn_prefill_varlen(c.q, kc, vc, cu_q, cu_k, mq, mk, c0.scale, block_table=bt, out=outs[L])
        else:
            pkv.attn_prefill_varlen(c.q, c.k, c.v, cu_q, cu_k, mq, mk, c0.scale, out=outs[L])

    def step(i):
        L = i % layers
        c, (kc, vc) = cases[L], caches[L]
        pkv.kv_slot_mapping(bt, c0.block_size, n, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k, out=sm)
        pkv.kv_store(c.k, c.v, kc, vc, sm)
        attn(c, kc, vc, L)

    wall_ms = run_steps(torch, step, steps, warmup)
    kern_ms = time_kernel(torch, lambda i: attn(cases[i % layers], *caches[i % layers], i % layers), steps)
    spread = time_kernel_spread(torch, lambda i: attn(cases[i % layers], *caches[i % layers], i % layers), steps)
    flops = prefill_flops(c0)
    del caches, cases
    torch.cuda.empty_cache()
    return {"wall_ms": wall_ms, "kernel_ms": kern_ms, "spread": spread, "flops": flops, "tokens": n}


def bench_store(pkv, torch, steps, warmup):
    import workloads
    sw = workloads.store_sweep(device="cuda")
    shape = (sw.num_blocks, sw.block_size, sw.num_kv_heads, sw.head_dim)
    kc = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    slots = [torch.from_numpy(s).cuda() for s in sw.slots]
    torch.cuda.synchronize()

    def step(i):
        s = i % len(slots)
        pkv.kv_store(sw.key[s], sw.value[s], kc, vc, slots[s])

    wall_ms = run_steps(torch, step, steps, warmup)
    kern_ms = time_kernel(torch, step, steps)
    spread = time_kernel_spread(torch, step, steps)
    n = len(sw.slots[0])
    row = sw.num_kv_heads * sw.head_dim * 2
    moved = 2 * n * row * 2 + 4 * n  # read + write of K and V rows, plus the slots

    # References for the same bytes and rotation, by the framework's own kernels (not this library's): its
    # scatter with the same slots (contiguous row reads, random distinct 2 KiB row writes), and a contiguous
    # device copy of the same rows (the read + write pattern with no scatter at all).
    d = sw.num_kv_heads * sw.head_dim
    idx64 = [s.long() for s in slots]
    kflat, vflat = kc.view(-1, d), vc.view(-1, d)

    def torch_scatter(i):
        s = i % len(slots)
        kflat.index_copy_(0, idx64[s], sw.key[s].view(-1, d))
        vflat.index_copy_(0, idx64[s], sw.value[s].view(-1, d))

    dst_k = torch.empty((n, d), dtype=torch.bfloat16, device="cuda")
    dst_v = torch.empty_like(dst_k)

    def torch_copy(i):
        s = i % len(slots)
        dst_k.copy_(sw.key[s].view(-1, d))
        dst_v.copy_(sw.value[s].view(-1, d))

    # The same kernel with each set's rows stored to consecutive slots (its own region of the cache): the same
    # bytes and launch, the destination contiguous -- what placing 2 KiB rows at random slots costs.
    seq = [torch.arange(s * n, (s + 1) * n, dtype=torch.int32, device="cuda") for s in range(len(slots))]

    def store_sequential(i):
        s = i % len(slots)
        pkv.kv_store(sw.key[s], sw.value[s], kc, vc, seq[s])

    scatter_ms = time_kernel(torch, torch_scatter, steps)
    copy_ms = time_kernel(torch, torch_copy, steps)
    seq_ms = time_kernel(torch, store_sequential, steps)
    del kc, vc, kflat, vflat, dst_k, dst_v
    torch.cuda.empty_cache()
    return {"wall_ms": wall_ms, "kernel_ms": kern_ms, "spread": spread, "bytes": moved, "tokens": n, "sets": len(slots),
            "torch_scatter_ms": scatter_ms, "torch_copy_ms": copy_ms, "copy_bytes": 2 * n * row * 2,
            "sequential_slots_ms": seq_ms}


LAYERS_PER_GRAPH = 8


def bench_decode_latency(pkv, torch, reps):
    """The decode step (attn_decode_paged_store) at fixed batch sizes, the batch padded up to each with rows of
    context 0 (slot -1), launched eagerly and replayed from a HIP graph captured once per size: time per step
    back to back, and one step's latency from launch to completion as the host sees it."""
    import numpy as np
    import workloads
    res = {}
    for real, bucket in ((1, 1), (5, 8), (24, 32), (64, 64), (200, 256)):
        rng = np.random.default_rng(40 + bucket)
        ctx = np.concatenate([rng.integers(512, 4096, size=real, endpoint=True), np.zeros(bucket - real, np.int64)])
        case = workloads.decode_case(ctx, num_blocks=int(sum(math.ceil(int(c) / 256) for c in ctx)) + 2,
                                     seed=41 + bucket, device="cuda", max_blocks=16, rng=rng)
        kc, vc = build_caches(pkv, torch, case)
        bt = torch.from_numpy(case.block_tables).cuda()
        cl = torch.from_numpy(case.context_lens).cuda()
        ws = torch.empty(max(pkv.attn_decode_workspace_bytes(bucket, 16, 8, 128, 16, 256), 1), dtype=torch.uint8,
                         device="cuda")
        o = torch.empty_like(case.q)
        sm = torch.empty(bucket, dtype=torch.int32, device="cuda")

        def step():
            pkv.attn_decode_paged_store(case.q, case.k, case.v, kc, vc, cl, bt, case.scale, out=o, workspace=ws,
                                        slot_mapping_out=sm)

        def single(fn):
            times = []
            for _ in range(reps):
                t0 = time.perf_counter()
                fn()
                torch.cuda.synchronize()
                times.append(time.perf_counter() - t0)
            return sorted(times)[len(times) // 2] * 1e6

        step()
        torch.cuda.synchronize()
        eager = run_steps(torch, lambda i: step(), reps, 5) * 1e3
        eager_one = single(step)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize()
        graph = run_steps(torch, lambda i: g.replay(), reps, 5) * 1e3
        graph_one = single(g.replay)
        # A model step holds one such call per layer: the same step captured LAYERS_PER_GRAPH times in one graph
        # (as a serving loop captures a whole forward pass), replayed back to back, time per decode step.
        g8 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g8):
            for _ in range(LAYERS_PER_GRAPH):
                step()
        torch.cuda.synchronize()
        graph8 = run_steps(torch, lambda i: g8.replay(), max(reps // LAYERS_PER_GRAPH, 5), 3) * 1e3 / LAYERS_PER_GRAPH
        res[str(bucket)] = {"real_rows": real, "kv_MB": round(int(ctx.sum()) * 4096 / 1e6, 1),
                            "eager_us_per_step": round(eager, 1), "graph_us_per_step": round(graph, 1),
                            "graph_%d_layers_us_per_step" % LAYERS_PER_GRAPH: round(graph8, 1),
                            "eager_us_one_step": round(eager_one, 1), "graph_us_one_step": round(graph_one, 1)}
        del g, g8, kc, vc, case
        torch.cuda.empty_cache()
    return res


def bench_prefill_data(pkv, torch, steps):
    """The same prefill call on the same shapes with different K/V values: N(0,1) (as every workload), all zero,
    all 1.0, then N(0,1) again.  The kernels run the same instructions either way; a rate that moves with the
    values shows the chip's power limit (operands that switch fewer bits draw less power, so the clock stays
    higher), not the instruction stream, setting the pace.  Dense rows: 32 sequences of 2048 tokens, non-causal,
    contiguous K/V."""
    B, L = 32, 2048
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2048)
    q = torch.randn(B * L, 16, 128, device="cuda", generator=gen).to(torch.bfloat16)
    k = torch.randn(B * L, 8, 128, device="cuda", generator=gen).to(torch.bfloat16)
    v = torch.randn(B * L, 8, 128, device="cuda", generator=gen).to(torch.bfloat16)
    cu = torch.arange(0, (B + 1) * L, L, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    flops = 4 * 128 * 16 * B * L * L
    res = {"shape": "32 x 2048 tokens, non-causal, bf16 16/8/128, contiguous K/V", "flops": flops}
    for name, kk, vv in (("randn", k, v), ("zero", torch.zeros_like(k), torch.zeros_like(v)),
                         ("ones", torch.ones_like(k), torch.ones_like(v)), ("randn_again", k, v)):
        ms = time_kernel(torch, lambda i: pkv.attn_prefill_varlen(q, kk, vv, cu, cu, L, L, 128 ** -0.5,
                                                                  causal=False, out=out), max(steps // 10, 20))
        res[f"kv_{name}_TFLOPs"] = round(flops / (ms * 1e-3) / 1e12, 1)
    return res


def bench_sublayer(pkv, torch, steps, warmup):
    """The synthetic-weight attention sub-layer (qkv GEMM, QK-Norm + RoPE + store, paged attention, o GEMM):
    a prefill step over the 8 varlen prefill sequences and a decode step over the batch-64 decode workload."""
    import numpy as np
    import workloads
    sub = pkv.AttentionSublayer(seed=11)
    res = {}
    # Prefill: the 8 varlen prefill sequences' lengths, keys read back from the paged cache.
    c3 = workloads.varlen_prefill_8seq(device="cuda")
    n = int(c3.cu_seqlens_q[-1])
    shape = (c3.num_blocks, c3.block_size, c3.num_kv_heads, c3.head_dim)
    kc = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(12)
    x = torch.randn(n, sub.hidden, generator=gen, device="cuda").to(torch.bfloat16)
    cu = torch.from_numpy(c3.cu_seqlens_q).cuda()
    pos = torch.from_numpy(np.concatenate([np.arange(int(L)) for L in c3.Lq]).astype(np.int32)).cuda()
    bt = torch.from_numpy(c3.block_tables).cuda()
    mq = int(c3.Lq.max())
    sm = pkv.kv_slot_mapping(bt, c3.block_size, n, cu_seqlens_q=cu, cu_seqlens_k=cu)
    pre_ms = run_steps(torch, lambda i: sub.prefill(x, pos, cu, cu, mq, mq, bt, kc, vc, slot_mapping=sm), steps, warmup)
    res["prefill_varlen_8seq"] = {"tokens": n, "ms_per_step": round(pre_ms, 4),
                                "tokens_per_s": round(n / (pre_ms * 1e-3), 0)}
    del kc, vc, c3
    # Decode: the batch-64 workload's batch and contexts over caches holding (random) history.
    c2 = workloads.decode_batch64(device="cuda")
    kc, vc = build_caches(pkv, torch, c2)
    bt = torch.from_numpy(c2.block_tables).cuda()
    cl = torch.from_numpy(c2.context_lens).cuda()
    xd = torch.randn(c2.batch, sub.hidden, generator=gen, device="cuda").to(torch.bfloat16)
    ws = torch.empty(max(pkv.attn_decode_workspace_bytes(c2.batch, 16, 8, 128, c2.max_blocks, 256), 1),
                     dtype=torch.uint8, device="cuda")
    dec_ms = run_steps(torch, lambda i: sub.decode(xd, cl, bt, kc, vc, workspace=ws), steps, warmup)
    res["decode_batch64"] = {"batch": c2.batch, "ms_per_step": round(dec_ms, 4),
                               "kv_GBps": round(int(c2.Lk.astype(int).sum()) * 4096 / (dec_ms * 1e-3) / 1e9, 1)}
    del kc, vc, c2
    torch.cuda.empty_cache()
    return res


def bench_qknorm_rope_store(pkv, torch, make, steps, warmup, layers):
    """The fused QK-Norm + RoPE + store over one prefill step's new tokens (the 8 varlen prefill sequences' q, k, v)."""
    cases, _ = dev_case_layers(make, layers, torch)
    c0 = cases[0]
    n, hq, hkv, hd = int(c0.cu_seqlens_q[-1]), c0.num_q_heads, c0.num_kv_heads, c0.head_dim
    bt = torch.from_numpy(c0.block_tables).cuda()
    cu_q = torch.from_numpy(c0.cu_seqlens_q).cuda()
    cu_k = torch.from_numpy(c0.cu_seqlens_k).cuda()
    sm = pkv.kv_slot_mapping(bt, c0.block_size, n, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k)
    pos = torch.cat([torch.arange(int(lk) - int(lq), int(lk), dtype=torch.int32) for lq, lk in zip(c0.Lq, c0.Lk)])
    pos = pos.cuda()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    wq = (1 + 0.1 * torch.randn(hd, generator=gen, device="cuda")).to(torch.bfloat16)
    wk = (1 + 0.1 * torch.randn(hd, generator=gen, device="cuda")).to(torch.bfloat16)
    shape = (c0.num_blocks, c0.block_size, hkv, hd)
    caches = [(torch.zeros(shape, dtype=torch.bfloat16, device="cuda"),
               torch.zeros(shape, dtype=torch.bfloat16, device="cuda")) for _ in cases]
    outs = [torch.empty_like(c.q) for c in cases]
    torch.cuda.synchronize()

    def step(i):
        L = i % layers
        c, (kc, vc) = cases[L], caches[L]
        pkv.kv_store_qk_norm_rope(c.q, c.k, c.v, pos, wq, wk, kc, vc, sm, q_out=outs[L])

    wall_ms = run_steps(torch, step, steps, warmup)
    kern_ms = time_kernel(torch, step, steps)
    moved = 2 * n * (hq + 2 * hkv) * hd * 2 + 8 * n  # q, k, v read and written once, plus positions and slots
    del caches, cases
    torch.cuda.empty_cache()
    return {"wall_ms": wall_ms, "kernel_ms": kern_ms, "bytes": moved, "tokens": n}


# ------------------------------------------------------------------------------------------------ CPU side
#
# The oracle as it stands (float64 NumPy, test infrastructure), timed on the host's cores: independent oracle
# calls -- one per sequence (decode) or per (sequence, kv head) (prefill) -- run on a pool of worker processes
# forked before this process touches the GPU, one BLAS thread each.  Processes, not threads: the oracle's
# per-row loop holds the interpreter lock.

_CPU = {}  # host data the forked workers inherit


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_workers():
    """The CPUs this process may run on, at most 16 (one GPU's share of the host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _one_blas_thread():
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)


def _decode_task(b):
    """The oracle's decode of sequence b over the blocks its table names (a compact copy of them, table
    renumbered 0..n-1: the same logical keys and values), widened to float64 as the oracle consumes them."""
    import numpy as np
    import oracle
    d = _CPU["decode"]
    n = int(-(-int(d["ctx"][b]) // 256))
    blocks = d["bt"][b, :n]
    kc = oracle.as_f64(d["kc"][blocks], "bf16")
    vc = oracle.as_f64(d["vc"][blocks], "bf16")
    table = np.arange(n, dtype=np.int32)[None]
    return oracle.decode_ref(d["q"][b:b + 1], kc, vc, d["ctx"][b:b + 1], table, 256, d["scale"])


def _prefill_task(bg):
    """The oracle's causal attention of sequence b for the query heads of kv head g."""
    import oracle
    b, g = bg
    p = _CPU["prefill"]
    q0, q1 = int(p["cu"][b]), int(p["cu"][b + 1])
    grp = p["group"]
    return oracle.attention_ref(p["q"][q0:q1, g * grp:(g + 1) * grp], p["k"][q0:q1, g:g + 1],
                                p["v"][q0:q1, g:g + 1], [0, q1 - q0], [0, q1 - q0], p["scale"], causal=True)


def _time_pool(pool, fn, tasks, min_seconds):
    reps, t0 = 0, time.perf_counter()
    while True:
        list(pool.map(fn, tasks, chunksize=1))
        reps += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    return reps, (time.perf_counter() - t0) / reps


def cpu_baseline(min_seconds=8.0):
    """The oracle on the host: decode attention of the whole batch-64 decode workload (KV GB/s), causal
    attention of the whole 8-sequence varlen prefill workload (TFLOP/s), and the store of an eighth of the store
    sweep (GB/s).  Must run before the GPU is initialised (the pool is forked)."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    import numpy as np
    import oracle
    import workloads
    _one_blas_thread()
    workers = cpu_workers()
    # decode: the cache after the oracle's slot_mapping + store of every sequence's history and new token
    c2 = workloads.decode_batch64(device="cpu")
    cache = workloads.nan_cache_host(c2.num_blocks, 256, 8, 128, "bf16")
    hist_sm = oracle.slot_mapping_ref(c2.block_tables, 256, int(c2.cu_hist[-1]), cu_seqlens_q=c2.cu_hist,
                                      cu_seqlens_k=c2.cu_hist)
    kc, vc = oracle.store_ref(c2.hist_k, c2.hist_v, cache, cache, hist_sm)
    del cache
    sm = oracle.slot_mapping_ref(c2.block_tables, 256, c2.batch, context_lens=c2.context_lens)
    kc, vc = oracle.store_ref(c2.k, c2.v, kc, vc, sm)
    _CPU["decode"] = {"kc": kc, "vc": vc, "bt": c2.block_tables, "ctx": c2.context_lens,
                      "q": oracle.as_f64(c2.q, "bf16"), "scale": c2.scale}
    # prefill: the new tokens' q, k, v widened once (the attention reads this step's rows)
    c3 = workloads.varlen_prefill_8seq(device="cpu")
    _CPU["prefill"] = {"q": oracle.as_f64(c3.q, "bf16"), "k": oracle.as_f64(c3.k, "bf16"),
                       "v": oracle.as_f64(c3.v, "bf16"), "cu": c3.cu_seqlens_q, "scale": c3.scale,
                       "group": c3.num_q_heads // c3.num_kv_heads}
    with ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("fork"),
                             initializer=_one_blas_thread) as pool:
        list(pool.map(time.sleep, [0.05] * workers))  # every worker started before the clock runs
        d_reps, d_secs = _time_pool(pool, _decode_task, range(c2.batch), min_seconds)
        tasks = sorted(((b, g) for b in range(c3.batch) for g in range(c3.num_kv_heads)),
                       key=lambda bg: -int(c3.Lq[bg[0]]))  # longest first
        p_reps, p_secs = _time_pool(pool, _prefill_task, tasks, min_seconds / 2)
    _CPU.clear()
    del kc, vc
    # store: one sequential scatter into one cache (the oracle copies the cache, then writes the rows); an
    # eighth of the sweep -- 2048 tokens into a 512-block cache, the same tokens per cache slot
    sw = workloads.store_sweep(2048, n_sets=1, num_blocks=512, device="cpu")
    sc = workloads.nan_cache_host(sw.num_blocks, sw.block_size, sw.num_kv_heads, sw.head_dim, "bf16")
    s_reps, t0 = 0, time.perf_counter()
    while s_reps < 1 or time.perf_counter() - t0 < min_seconds / 4:
        oracle.store_ref(sw.key[0], sw.value[0], sc, sc, sw.slots[0])
        s_reps += 1
    s_secs = (time.perf_counter() - t0) / s_reps
    sw_slots = sw.slots[0]
    del sc, sw

    kv_bytes = int(c2.Lk.astype(int).sum()) * 2 * 8 * 128 * 2
    flops = 4 * c3.head_dim * c3.num_q_heads * int(sum(int(L) * (int(L) + 1) // 2 for L in c3.Lq))
    n_store = len(sw_slots)
    store_bytes = 2 * n_store * 1024 * 2 * 2 + 4 * n_store
    model = cpu_model()
    return {
        "value": round(kv_bytes / d_secs / 1e9, 4), "unit": "GB/s", "cores": workers, "kind": "oracle",
        "cpu_model": model, "cpus_visible": len(os.sched_getaffinity(0)),
        "sample": f"decode attention of the whole batch-64 decode workload (64 sequences, sum ctx "
                  f"{int(c2.Lk.sum())}, float64), one oracle call per sequence over {workers} worker processes "
                  f"(one BLAS thread each), {d_reps} repetitions of {d_secs:.3f} s",
        "prefill": {"value": round(flops / p_secs / 1e12, 6), "unit": "TFLOP/s", "cores": workers,
                    "sample": f"causal attention of the whole 8-sequence varlen prefill workload "
                              f"({int(c3.Lq.sum())} tokens, {flops / 1e9:.1f} GFLOP of causal pairs, float64), "
                              f"one oracle call per (sequence, kv head), {p_reps} repetitions of {p_secs:.3f} s"},
        "store": {"value": round(store_bytes / s_secs / 1e9, 4), "unit": "GB/s", "cores": 1,
                  "sample": f"an eighth of the store sweep: {n_store} tokens into a 512-block cache (the same "
                            f"tokens per slot; the oracle copies both 256 MiB caches, then writes the rows; one "
                            f"process), {s_reps} repetitions of {s_secs:.3f} s"},
    }


# ------------------------------------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # 1000 steps of the decode step take about 0.1 s: enough that the first launch and the final synchronisation
    # no longer weigh on the per-step figure (at 50 steps they added about 6 us to each 110 us step).
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--layers", type=int, default=4, help="independent caches rotated over the steps")
    ap.add_argument("--headline-only", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--only", choices=["prefill", "prefix", "chunked", "store", "long_decode", "qknorm_rope",
                                       "unfused_decode", "decode_latency", "sublayer", "prefill_data"],
                    default=None,
                    help="run just one secondary workload (after the headline), e.g. for a profiler")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    cpu = None
    if not args.no_cpu:
        # before anything touches the GPU: the oracle's worker processes are forked from this one
        log(f"cpu oracle baseline ({cpu_workers()} worker processes)")
        cpu = cpu_baseline()

    import torch
    import paged_kv_cache_300_amd as pkv
    import workloads
    pkv.lib()
    torch.cuda.set_device(0)

    log("decode step (fused store + decode), batch 64")
    dec = bench_decode(pkv, torch, workloads.decode_batch64, args.steps, args.warmup, args.layers, fused=True)
    achieved = dec["kv_bytes"] / (dec["kernel_ms"] * 1e-3) / 1e9
    value = dec["kv_bytes"] / (dec["wall_ms"] * 1e-3) / 1e9
    dec_hash = source_hash("attn_decode.hip", "common.h")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic("attn_decode_paged_store_decode_batch64", dec_hash),
                "kernel": "attn_decode_paged_store (decode_lean_kernel<2, store> + decode_combine_kernel)",
                "kernel_ms": round(dec["kernel_ms"], 5), "kernel_ms_spread": dec["spread"],
                "algorithmic_bytes": dec["kv_bytes"], "source_hash": dec_hash}

    secondary = {}
    if not args.headline_only:
        want = lambda name: args.only in (None, name)
        p3 = p4 = st = d5 = qr = fd = dl = sb = ch = pdv = None
        if want("unfused_decode"):
            log("unfused decode step (slot_mapping, store, decode), batch 64")
            fd = bench_decode(pkv, torch, workloads.decode_batch64, args.steps, args.warmup, args.layers)
        if want("prefill"):
            log("varlen prefill, 8 sequences")
            p3 = bench_prefill(pkv, torch, workloads.varlen_prefill_8seq, args.steps, args.warmup, args.layers, paged=False)
        if want("prefix"):
            log("prefix prefill, 16 sequences")
            p4 = bench_prefill(pkv, torch, workloads.prefix_prefill_16seq, args.steps, args.warmup, args.layers, paged=True)
        if want("chunked"):
            log("chunked prefill on long cached prefixes")
            ch = bench_chunked_prefill(pkv, torch, args.steps)
        if want("store"):
            log("store sweep, 16384 tokens")
            st = bench_store(pkv, torch, args.steps, args.warmup)
        if want("qknorm_rope"):
            log("QK-Norm + RoPE + store, the 8 prefill sequences' tokens")
            # at least 8 input sets (8 x 67 MB of q, k, v rows, twice the last-level cache): rows are read from HBM
            qr = bench_qknorm_rope_store(pkv, torch, workloads.varlen_prefill_8seq, args.steps, args.warmup,
                                         max(args.layers, 8))
        if want("decode_latency"):
            log("decode step latency at padded fixed batch sizes, eager and graph")
            dl = bench_decode_latency(pkv, torch, max(args.steps, 20))
        if want("sublayer"):
            log("synthetic-weight attention sub-layer, workloads 3 (prefill) and 2 (decode)")
            sb = bench_sublayer(pkv, torch, args.steps, args.warmup)
        if args.only == "prefill_data":  # on request only: it does not measure a workload
            log("prefill rate against the K/V values (same shapes and instructions)")
            pdv = bench_prefill_data(pkv, torch, args.steps)
        if want("long_decode"):
            log("long padded decode, batch 256")
            d5 = bench_decode(pkv, torch, workloads.long_decode_batch256, max(args.steps // 5, 3), 2, 2)
        gemm = None
        if p3 is not None or p4 is not None:
            log("bf16 GEMM 8192^3 through the platform BLAS (practical matrix-core rate)")
            gemm = bench_gemm_reference(torch)
            secondary["bf16_gemm_8192_reference"] = {
                "value": round(gemm, 1), "unit": "TFLOP/s", "frac_bf16_mfma_peak": round(gemm / BF16_MFMA_PEAK_TFLOPS, 4),
                "what": "torch.matmul of two 8192x8192 bf16 matrices (hipBLASLt): not part of this library; the "
                        "dense matrix-core rate the GPU sustains under full load"}
        for name, r in (("varlen_prefill_8seq", p3), ("prefix_prefill_16seq", p4)):
            if r is None:
                continue
            tf = r["flops"] / (r["kernel_ms"] * 1e-3) / 1e12
            secondary[name] = {"value": round(tf, 2), "unit": "TFLOP/s", "frac_bf16_mfma_peak":
                               round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                               "frac_of_bf16_gemm_reference": round(tf / gemm, 4),
                               "kernel_ms": round(r["kernel_ms"], 4), "kernel_ms_spread": r["spread"],
                               "step_ms": round(r["wall_ms"], 4), "flops": r["flops"], "tokens": r["tokens"]}
        if st is not None:
            gbs = st["bytes"] / (st["kernel_ms"] * 1e-3) / 1e9
            secondary["store_sweep_16k"] = {"value": round(gbs, 1), "unit": "GB/s",
                                                 "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                                                 "kernel_ms": round(st["kernel_ms"], 5),
                                                 "kernel_ms_spread": st["spread"], "bytes": st["bytes"],
                                                 "tokens": st["tokens"], "sets_rotated": st["sets"],
                                                 "reference_torch_index_copy_GBps":
                                                     round(st["copy_bytes"] / (st["torch_scatter_ms"] * 1e-3) / 1e9, 1),
                                                 "reference_contiguous_copy_GBps":
                                                     round(st["copy_bytes"] / (st["torch_copy_ms"] * 1e-3) / 1e9, 1),
                                                 "same_kernel_sequential_slots_GBps":
                                                     round(st["bytes"] / (st["sequential_slots_ms"] * 1e-3) / 1e9, 1)}
        if fd is not None:
            gbk = fd["kv_bytes"] / (fd["kernel_ms"] * 1e-3) / 1e9
            secondary["decode_step_unfused_batch64"] = {
                "value": round(fd["kv_bytes"] / (fd["wall_ms"] * 1e-3) / 1e9, 1), "unit": "GB/s",
                "step_ms": round(fd["wall_ms"], 5), "call_ms": round(fd["kernel_ms"], 5),
                "call_GBps": round(gbk, 1), "call_frac_hbm_peak": round(gbk / HBM_PEAK_GBS, 4),
                "step": "kv_slot_mapping + kv_store + attn_decode_paged (call = attn_decode_paged alone)"}
        if qr is not None:
            gbq = qr["bytes"] / (qr["kernel_ms"] * 1e-3) / 1e9
            secondary["qknorm_rope_store_8seq_tokens"] = {"value": round(gbq, 1), "unit": "GB/s",
                                                       "frac_hbm_peak": round(gbq / HBM_PEAK_GBS, 4),
                                                       "kernel_ms": round(qr["kernel_ms"], 5), "bytes": qr["bytes"],
                                                       "tokens": qr["tokens"], "sets_rotated": max(args.layers, 8)}
        if ch is not None:
            secondary.update(ch)
        if dl is not None:
            secondary["decode_step_latency_padded_batches"] = dl
        if sb is not None:
            secondary["attention_sublayer"] = sb
        if pdv is not None:
            secondary["prefill_rate_vs_kv_values"] = pdv
        if d5 is not None:
            gbs5 = d5["kv_bytes"] / (d5["kernel_ms"] * 1e-3) / 1e9
            secondary["long_decode_batch256"] = {"value": round(gbs5, 1), "unit": "GB/s",
                                                 "frac_hbm_peak": round(gbs5 / HBM_PEAK_GBS, 4),
                                                 "kernel_ms": round(d5["kernel_ms"], 4), "kv_bytes": d5["kv_bytes"],
                                                 "step_ms": round(d5["wall_ms"], 4)}

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["wall_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workloads.WORKLOADS["decode_batch64"], "batch": dec["batch"], "sum_context_lens": dec["sum_ctx"],
                   "heads": "16 q / 8 kv", "head_dim": 128, "block_size": 256, "layers_rotated": args.layers,
                   "step": "attn_decode_paged_store (slot_mapping + store of the new token + paged decode)"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
