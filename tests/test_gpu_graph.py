"""HIP-graph capture of the hot path: a decode step (kv_slot_mapping + kv_store + attn_decode_paged) and a
prefix-cache prefill call captured once and replayed several times, with eager work and synchronisations
between the replays; every replay must equal the eager result bit for bit, and the eager result matches the
oracle."""

import math

import numpy as np
import pytest
import torch

import workloads
from gpu_util import gpu_slot_mapping, gpu_store_history, i32, log, max_abs_err, nan_cache, oracle_attention, to_dev, to_host
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_300_amd as m
    m.lib()
    return m


def _graph(fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def test_decode_step_graph_replays(pkv):
    ctx = np.array([700, 1, 0, 2049, 300, 4096, 0, 77])  # padding rows (context 0, slot -1) included
    case = workloads.decode_case(ctx, num_blocks=int(sum(math.ceil(c / 256) for c in ctx)) + 2, seed=91,
                                 max_blocks=16)
    kc, vc = nan_cache(case), nan_cache(case)
    gpu_store_history(case, kc, vc)
    k, v, q = (to_dev(x, "bf16") for x in (case.k, case.v, case.q))
    bt, cl = i32(case.block_tables), i32(case.context_lens)
    sm = torch.empty(case.batch, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(pkv.attn_decode_workspace_bytes(case.batch, 16, 8, 128, 16, 256), 1), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(q)

    def step():
        pkv.kv_slot_mapping(bt, 256, case.batch, context_lens=cl, out=sm)
        pkv.kv_store(k, v, kc, vc, sm)
        pkv.attn_decode_paged(q, kc, vc, cl, bt, case.scale, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    want = oracle_attention(case)
    got = oracle.as_f64(to_host(eager), "bf16")
    err = max(max_abs_err(got[b:b + 1], w) for b, w in want.items())
    log(f"eager decode max-abs {err:.3e}")
    assert err <= 2e-2
    g = _graph(step)
    for rep in range(4):
        out.fill_(7.0)                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs"
        scratch = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager kernels on the same stream
        torch.cuda.synchronize()
        del scratch


@pytest.mark.parametrize("lq,prefix", [([200, 64, 1], [1000, 0, 3000]), ([64], [20000])])
def test_prefix_prefill_graph_replays(pkv, lq, prefix):
    """A prefix-cache prefill with the planner's workspace, captured once and replayed: both cases have too few
    query tiles to fill the GPU, so the captured launches are the planner, the key-range pieces and their merge."""
    lk = [a + b for a, b in zip(lq, prefix)]
    case = workloads.make_case(lq, lk, num_q_heads=16, num_kv_heads=8, head_dim=128, block_size=256,
                               num_blocks=sum(math.ceil(c / 256) for c in lk) + 2, dtype="bf16", seed=92)
    kc, vc = nan_cache(case), nan_cache(case)
    gpu_store_history(case, kc, vc)
    pkv.kv_store(to_dev(case.k, "bf16"), to_dev(case.v, "bf16"), kc, vc, gpu_slot_mapping(case))
    q = to_dev(case.q, "bf16")
    cu_q, cu_k, bt = i32(case.cu_seqlens_q), i32(case.cu_seqlens_k), i32(case.block_tables)
    ws = torch.empty(pkv.attn_prefill_workspace_bytes(len(lq), sum(lq), max(lq), 16, 8, 128), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(q)

    def call():
        pkv.attn_prefill_varlen(q, kc, vc, cu_q, cu_k, max(lq), max(lk), case.scale, block_table=bt, out=out,
                                workspace=ws)

    call()
    torch.cuda.synchronize()
    eager = out.clone()
    g = _graph(call)
    for rep in range(4):
        out.zero_()
        ws.fill_(0xEE)                      # the planner's workspace needs no clearing
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs"
    want = oracle_attention(case)
    got = oracle.as_f64(to_host(eager), "bf16")
    err = max(max_abs_err(got[int(case.cu_seqlens_q[b]):int(case.cu_seqlens_q[b + 1])], w) for b, w in want.items())
    log(f"prefill eager max-abs {err:.3e}")
    assert err <= 2e-2


@pytest.mark.parametrize("real,bucket", [(5, 8), (64, 64), (200, 256)])
def test_padded_fixed_batch_decode_loop_in_a_graph(pkv, real, bucket):
    """The serving pattern the -1 slot exists for: one decode step (attn_decode_paged_store) captured at a fixed
    batch size, the batch padded up to it with rows of context 0 (slot -1), then replayed for several steps while
    the static inputs change in place (context lengths grow by one, new q / k / v rows).  Every replay's output,
    caches and slot_mapping equal those of the same steps run eagerly on a copy of the caches, bit for bit."""
    rng = np.random.default_rng(93 + real)
    ctx0 = np.concatenate([rng.integers(512, 4090, size=real), np.zeros(bucket - real, np.int64)])
    steps = 3
    case = workloads.decode_case(ctx0 + steps, num_blocks=int(sum(math.ceil((c + steps) / 256) for c in ctx0)) + 2,
                                 seed=94 + real, max_blocks=16)
    kc, vc = nan_cache(case), nan_cache(case)
    gpu_store_history(case, kc, vc)  # history up to the last step's context: every step reads only its own part
    kc2, vc2 = kc.clone(), vc.clone()
    bt = i32(case.block_tables)
    live = torch.from_numpy((ctx0 > 0).astype(np.int32)).cuda()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(95)
    draws = [tuple(torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16)
                   for shape in ((bucket, 16, 128), (bucket, 8, 128), (bucket, 8, 128))) for _ in range(steps)]
    ws = torch.empty(max(pkv.attn_decode_workspace_bytes(bucket, 16, 8, 128, 16, 256), 1), dtype=torch.uint8,
                     device="cuda")
    # Static buffers of the captured step.
    q_s, k_s, v_s = (torch.empty_like(x) for x in draws[0])
    cl_s = i32(ctx0.astype(np.int32))
    out_s = torch.empty_like(q_s)
    sm_s = torch.empty(bucket, dtype=torch.int32, device="cuda")

    def captured():
        pkv.attn_decode_paged_store(q_s, k_s, v_s, kc2, vc2, cl_s, bt, case.scale, out=out_s, workspace=ws,
                                    slot_mapping_out=sm_s)

    # One eager call first (on throwaway copies of the caches), so nothing is set up during the capture.
    warm_k, warm_v = kc.clone(), vc.clone()
    pkv.attn_decode_paged_store(draws[0][0], draws[0][1], draws[0][2], warm_k, warm_v, i32(ctx0.astype(np.int32) + 1),
                                bt, case.scale, workspace=ws)
    torch.cuda.synchronize()
    del warm_k, warm_v
    # Capture with the first step's inputs in place (capturing launches nothing).
    q_s.copy_(draws[0][0]); k_s.copy_(draws[0][1]); v_s.copy_(draws[0][2])
    cl_s.add_(live)
    torch.cuda.synchronize()
    g = _graph(captured)
    cl_s.sub_(live)
    cl = i32(ctx0.astype(np.int32))
    for step in range(steps):
        q, k, v = draws[step]
        cl.add_(live)                        # eager: each real row's context grows by its new token
        want = pkv.attn_decode_paged_store(q, k, v, kc, vc, cl, bt, case.scale)
        want_sm = pkv.kv_slot_mapping(bt, 256, bucket, context_lens=cl)
        q_s.copy_(q); k_s.copy_(k); v_s.copy_(v)
        cl_s.add_(live)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_s, want), f"step {step}: replayed output differs"
        assert torch.equal(sm_s, want_sm), f"step {step}: slot_mapping differs"
        assert torch.equal(kc2.view(torch.int16), kc.view(torch.int16)), f"step {step}: k cache differs"
        assert torch.equal(vc2.view(torch.int16), vc.view(torch.int16)), f"step {step}: v cache differs"
        assert bool((out_s[real:] == 0).all()), "padding rows must be zero"
        assert bool((sm_s[real:] == -1).all()), "padding rows have no slot"
    log(f"graph decode loop: {real} rows padded to {bucket}, {steps} replays equal the eager steps")
