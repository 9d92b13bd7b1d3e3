"""The allocation-free fused decode step (attn_decode_paged_store_noalloc, workspace in the library's static
device scratch) against attn_decode_paged_store with a caller workspace: the same caches and slot_mapping bit for
bit and the same output, on two calls in a row, the second with a smaller batch (the scratch keeps the first
call's contents)."""

import math

import numpy as np
import pytest
import torch

import workloads
from gpu_util import BF16_TOL, gpu_store_history, i32, log, nan_cache, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_300_amd as m
    m.lib()
    return m


def _bits(t):
    return t.detach().contiguous().view(torch.int16)


def _compare(pkv, case):
    kc, vc = nan_cache(case), nan_cache(case)
    gpu_store_history(case, kc, vc)
    kc2, vc2 = kc.clone(), vc.clone()
    bt, ctx = i32(case.block_tables), i32(case.context_lens)
    q, k, v = (to_dev(x, case.dtype) for x in (case.q, case.k, case.v))
    sm = torch.full((case.batch,), -7, dtype=torch.int32, device="cuda")
    sm2 = sm.clone()
    out2 = torch.empty_like(q)
    torch.cuda.synchronize()
    out = pkv.attn_decode_paged_store(q, k, v, kc, vc, ctx, bt, case.scale, slot_mapping_out=sm)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    pkv.attn_decode_paged_store_noalloc(q, k, v, kc2, vc2, ctx, bt, case.scale, out2, slot_mapping_out=sm2)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before, "the allocation-free call allocated through torch"
    assert torch.equal(_bits(kc), _bits(kc2)) and torch.equal(_bits(vc), _bits(vc2)), "caches differ"
    assert torch.equal(sm, sm2), "slot_mapping differs"
    diff = float((out.float() - out2.float()).abs().max())
    log(f"  batch {case.batch}: output max-abs difference {diff:.3e}, bit-equal {torch.equal(_bits(out), _bits(out2))}")
    assert diff <= BF16_TOL


def test_noalloc_matches_workspace_call_twice(pkv):
    """The batch-64 decode workload, then a smaller batch (24 rows, two of them padding) on the same scratch."""
    log("no-alloc decode: batch 64 workload")
    _compare(pkv, workloads.decode_batch64(device="cuda"))
    rng = np.random.default_rng(77)
    ctx = np.concatenate([rng.integers(1, 3000, 22), [0, 0]])
    case = workloads.decode_case(ctx, num_blocks=int(sum(math.ceil(c / 256) for c in ctx)) + 3, seed=78,
                                 device="cuda", max_blocks=12, rng=rng)
    log("no-alloc decode: 24 rows after it")
    _compare(pkv, case)


def test_noalloc_refuses_oversized_batch(pkv):
    """A batch whose workspace exceeds the static scratch is refused (nothing launched)."""
    b = 4000  # about 40 MiB of workspace
    case_q = torch.zeros((b, 16, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((b, 8, 128), dtype=torch.bfloat16, device="cuda")
    cache = torch.zeros((4, 256, 8, 128), dtype=torch.bfloat16, device="cuda")
    ctx = torch.ones(b, dtype=torch.int32, device="cuda")
    bt = torch.zeros((b, 1), dtype=torch.int32, device="cuda")
    out = torch.empty_like(case_q)
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.attn_decode_paged_store_noalloc(case_q, kv, kv, cache, cache.clone(), ctx, bt, 0.088, out)
    assert e.value.code == -3
