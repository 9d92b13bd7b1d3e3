"""Seeded random GPU parity cases: shapes, GQA groups, block sizes, cached prefixes, empty sequences, causal and
non-causal prefill, plain and fused decode, each drawn from its own seed so a failing case can be rerun alone.
Every result is checked against the float64 oracle (bf16 2e-2 max-abs); the fused decode step's caches and
slot_mapping must equal the unfused step's bit for bit."""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import (BF16_TOL, gpu_store_history, i32, log, logical_kv, max_abs_err, nan_cache,
                      oracle_slot_mapping, to_dev, to_host)

pytestmark = pytest.mark.gpu

# (query heads, kv heads): groups of 2, 1, 4, 4 and 4 with two kv heads.
HEADS = [(16, 8), (8, 8), (16, 4), (32, 8), (8, 2)]
# Powers of two from 64 up take the tile-per-block loads; the others the per-row block-table lookup.
BLOCK_SIZES = [1, 7, 16, 64, 128, 256, 512]


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_300_amd as m
    m.lib()
    return m


def _bits(t):
    return t.detach().contiguous().view(torch.int16)


def _oracle(case, causal, rows):
    """float64 attention of every listed sequence over its logical keys (the last Lq of Lk are the queries)."""
    outs = {}
    for b in rows:
        lk = int(case.Lk[b])
        q0, q1 = int(case.cu_seqlens_q[b]), int(case.cu_seqlens_q[b + 1])
        q = oracle.as_f64(case.q[q0:q1], case.dtype)
        if lk == 0 or q1 == q0:
            outs[b] = np.zeros_like(q)
            continue
        k = oracle.as_f64(logical_kv(case, b, "k"), case.dtype)
        v = oracle.as_f64(logical_kv(case, b, "v"), case.dtype)
        outs[b] = oracle.attention_ref(q, k, v, [0, q1 - q0], [0, lk], case.scale, causal=causal)
    return outs


def _prefill_params(idx):
    rng = np.random.default_rng([2026, idx])
    hq, hkv = HEADS[rng.integers(len(HEADS))]
    paged = bool(rng.random() < 0.6)
    bs = int(BLOCK_SIZES[rng.integers(len(BLOCK_SIZES))]) if paged else 256
    batch = int(rng.integers(1, 6))
    lq = rng.integers(1, 300, size=batch)
    lq[rng.random(batch) < 0.15] = 0
    prefix = rng.integers(0, 800, size=batch) if paged else np.zeros(batch, np.int64)
    causal = bool(rng.random() < 0.75)
    order = bool(rng.random() < 0.7)
    return dict(hq=int(hq), hkv=int(hkv), paged=paged, bs=bs, lq=[int(x) for x in lq],
                prefix=[int(x) for x in prefix], causal=causal, order=order, seed=3000 + idx)


@pytest.mark.parametrize("idx", range(24))
def test_random_prefill(pkv, idx):
    c = _prefill_params(idx)
    lk = [a + b for a, b in zip(c["lq"], c["prefix"])]
    bs = c["bs"]
    case = workloads.make_case(c["lq"], lk, num_q_heads=c["hq"], num_kv_heads=c["hkv"], head_dim=128,
                               block_size=bs, num_blocks=sum(math.ceil(x / bs) for x in lk) + 3, dtype="bf16",
                               seed=c["seed"], max_blocks=max(max(math.ceil(x / bs) for x in lk), 1) + 1)
    log(f"random prefill {idx}: {c}")
    kc, vc = nan_cache(case), nan_cache(case)
    gpu_store_history(case, kc, vc)
    n = int(case.cu_seqlens_q[-1])
    bt = i32(case.block_tables)
    cu_q, cu_k = i32(case.cu_seqlens_q), i32(case.cu_seqlens_k)
    sm = pkv.kv_slot_mapping(bt, bs, n, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k)
    k, v, q = to_dev(case.k, "bf16"), to_dev(case.v, "bf16"), to_dev(case.q, "bf16")
    pkv.kv_store(k, v, kc, vc, sm)
    max_q, max_k = max(int(case.Lq.max()), 1), max(int(case.Lk.max()), 1)
    if c["paged"]:
        out = pkv.attn_prefill_varlen(q, kc, vc, cu_q, cu_k, max_q, max_k, case.scale, causal=c["causal"],
                                      block_table=bt, order=c["order"])
    else:
        out = pkv.attn_prefill_varlen(q, k, v, cu_q, cu_k, max_q, max_k, case.scale, causal=c["causal"],
                                      order=c["order"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(sm), oracle_slot_mapping(case))
    want = _oracle(case, c["causal"], range(case.batch))
    got = oracle.as_f64(to_host(out), "bf16")
    worst = 0.0
    for b, w in want.items():
        q0 = int(case.cu_seqlens_q[b])
        worst = max(worst, max_abs_err(got[q0:q0 + w.shape[0]], w))
    log(f"  max-abs error {worst:.3e}")
    assert worst <= BF16_TOL


def _decode_params(idx):
    rng = np.random.default_rng([2027, idx])
    hq, hkv = HEADS[rng.integers(len(HEADS))]
    bs = int(BLOCK_SIZES[rng.integers(len(BLOCK_SIZES))])
    batch = int(rng.integers(1, 41))
    kind = rng.random(batch)
    ctx = np.where(kind < 0.1, 0, np.where(kind < 0.4, rng.integers(1, 65, size=batch),
                                           rng.integers(65, 3000, size=batch)))
    return dict(hq=int(hq), hkv=int(hkv), bs=bs, ctx=[int(x) for x in ctx], fused=bool(rng.random() < 0.6),
                seed=4000 + idx)


@pytest.mark.parametrize("idx", range(16))
def test_random_decode(pkv, idx):
    c = _decode_params(idx)
    bs, ctx = c["bs"], c["ctx"]
    case = workloads.decode_case(ctx, num_q_heads=c["hq"], num_kv_heads=c["hkv"], head_dim=128, block_size=bs,
                                 num_blocks=sum(math.ceil(x / bs) for x in ctx) + 3, seed=c["seed"],
                                 max_blocks=max(max(math.ceil(x / bs) for x in ctx), 1) + 1)
    log(f"random decode {idx}: {dict(c, ctx=f'{len(ctx)} rows, max {max(ctx)}, sum {sum(ctx)}')}")
    kc, vc = nan_cache(case), nan_cache(case)
    gpu_store_history(case, kc, vc)
    bt, cl = i32(case.block_tables), i32(case.context_lens)
    q, k, v = to_dev(case.q, "bf16"), to_dev(case.k, "bf16"), to_dev(case.v, "bf16")
    if c["fused"]:
        kc2, vc2 = kc.clone(), vc.clone()
        sm = pkv.kv_slot_mapping(bt, bs, case.batch, context_lens=cl)
        pkv.kv_store(k, v, kc2, vc2, sm)
        sm_fused = torch.full((case.batch,), -7, dtype=torch.int32, device="cuda")
        out = pkv.attn_decode_paged_store(q, k, v, kc, vc, cl, bt, case.scale, slot_mapping_out=sm_fused)
        torch.cuda.synchronize()
        assert torch.equal(_bits(kc), _bits(kc2)) and torch.equal(_bits(vc), _bits(vc2)), "caches differ"
        assert torch.equal(sm_fused, sm), "slot_mapping differs"
    else:
        sm = pkv.kv_slot_mapping(bt, bs, case.batch, context_lens=cl)
        pkv.kv_store(k, v, kc, vc, sm)
        out = pkv.attn_decode_paged(q, kc, vc, cl, bt, case.scale)
        torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(sm), oracle_slot_mapping(case))
    want = _oracle(case, True, range(case.batch))
    got = oracle.as_f64(to_host(out), "bf16")
    worst = max(max_abs_err(got[b:b + 1], w) for b, w in want.items())
    log(f"  max-abs error {worst:.3e}")
    assert worst <= BF16_TOL
    for b in np.where(np.asarray(ctx) == 0)[0]:
        assert bool((out[int(b)] == 0).all()), "padding rows must be zero"
