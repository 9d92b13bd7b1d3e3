"""GPU parity of the fused QK-Norm + RoPE + store (kv_store_qk_norm_rope) against the float64 oracle: q_out
and the cache's k rows within the bf16 (2e-2) / float32 (1e-5) max-abs bars, the cache's v rows bit-exact,
every other cache byte untouched (NaN-poisoned), padding tokens (slot -1) writing nothing."""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import BF16_TOL, F32_TOL, log, nan_cache, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_300_amd as m
    m.lib()
    return m


def _weights(rng, hd, dtype):
    w = rng.uniform(0.8, 1.2, size=hd).astype(np.float32)
    return workloads.f32_to_bf16_bits(w) if dtype == "bf16" else w


def _positions(case):
    """Absolute position of every new token: the last Lq of each sequence's Lk positions."""
    return np.concatenate([np.arange(int(lk) - int(lq), int(lk)) for lq, lk in zip(case.Lq, case.Lk)]).astype(np.int32)


def _check(pkv, case, positions, sm, *, eps=1e-6, theta=1e6, seed=0, q=None, k=None, v=None):
    dtype, hd, hq, hkv = case.dtype, case.head_dim, case.num_q_heads, case.num_kv_heads
    rng = np.random.default_rng(seed)
    wq, wk = _weights(rng, hd, dtype), _weights(rng, hd, dtype)
    kc, vc = nan_cache(case), nan_cache(case)
    before_k, before_v = to_host(kc).copy(), to_host(vc).copy()
    q = to_dev(case.q, dtype) if q is None else q
    k = to_dev(case.k, dtype) if k is None else k
    v = to_dev(case.v, dtype) if v is None else v
    q_out = pkv.kv_store_qk_norm_rope(q, k, v, torch.from_numpy(positions).cuda(), to_dev(wq, dtype), to_dev(wk, dtype),
                                      kc, vc, torch.from_numpy(sm).cuda(), eps=eps, rope_theta=theta)
    torch.cuda.synchronize()
    want_q, want_k = oracle.qk_norm_rope_ref(oracle.as_f64(case.q, dtype), oracle.as_f64(case.k, dtype), positions,
                                             oracle.as_f64(wq, dtype), oracle.as_f64(wk, dtype), eps, theta)
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    err_q = float(np.max(np.abs(oracle.as_f64(to_host(q_out), dtype) - want_q)))
    got_k, got_v = to_host(kc), to_host(vc)
    flat = lambda a: a.reshape(-1, hkv, hd)
    err_k = 0.0
    written = np.zeros(flat(got_k).shape[0], dtype=bool)
    for i, s in enumerate(sm):
        if s < 0:
            continue
        written[s] = True
        err_k = max(err_k, float(np.max(np.abs(oracle.as_f64(flat(got_k)[s], dtype) - want_k[i]))))
        assert np.array_equal(flat(got_v)[s], np.asarray(case.v)[i]), f"v row of token {i} differs"
    bits = np.uint16 if dtype == "bf16" else np.uint32
    assert np.array_equal(flat(got_k)[~written].view(bits), flat(before_k)[~written].view(bits))
    assert np.array_equal(flat(got_v)[~written].view(bits), flat(before_v)[~written].view(bits))
    log(f"  q_out max-abs {err_q:.3e}, cache k max-abs {err_k:.3e} (tol {tol:.0e})")
    assert err_q <= tol and err_k <= tol


@pytest.mark.parametrize("dtype,hq,hkv,hd,lq,prefix,bs,seed", [
    ("bf16", 16, 8, 128, [130, 1, 64, 200], [0, 5, 300, 1000], 256, 101),
    ("bf16", 16, 8, 64, [70, 9], [0, 40], 16, 102),
    ("bf16", 8, 4, 256, [33, 40], [3, 0], 64, 103),
    ("bf16", 4, 2, 32, [17], [100], 8, 104),
    ("f32", 4, 2, 16, [6, 3], [0, 0], 4, 105),   # the tiny fp32 layer's shape
    ("f32", 16, 8, 128, [50], [20], 256, 106),
    ("bf16", 6, 3, 128, [45, 2], [7, 0], 16, 111),   # 12 rows a token: a short last chunk of rows
    ("bf16", 4, 2, 16, [300], [0], 32, 112),          # two lanes a row
    ("f32", 32, 8, 256, [20, 5], [0, 9], 16, 113),    # 48 rows a token: more chunks than lane groups
    ("f32", 6, 3, 64, [31], [2], 8, 114),
])
def test_prefill_tokens(pkv, dtype, hq, hkv, hd, lq, prefix, bs, seed):
    lk = [a + b for a, b in zip(lq, prefix)]
    case = workloads.make_case(lq, lk, num_q_heads=hq, num_kv_heads=hkv, head_dim=hd, block_size=bs,
                               num_blocks=sum(math.ceil(c / bs) for c in lk) + 2, dtype=dtype, seed=seed)
    sm = oracle.slot_mapping_ref(case.block_tables, bs, int(case.Lq.sum()), cu_seqlens_q=case.cu_seqlens_q,
                                 cu_seqlens_k=case.cu_seqlens_k)
    log(f"qk-norm+rope+store {dtype} {hq}/{hkv}/{hd} lq={lq} prefix={prefix}")
    _check(pkv, case, _positions(case), sm, seed=seed)


def test_decode_tokens_with_padding(pkv):
    ctx = np.array([700, 1, 0, 4096, 33, 0])  # two padding rows: slot -1, position -1 (unused)
    case = workloads.decode_case(ctx, num_blocks=int(sum(math.ceil(c / 256) for c in ctx)) + 2, seed=107,
                                 max_blocks=16)
    sm = oracle.slot_mapping_ref(case.block_tables, 256, case.batch, context_lens=case.context_lens)
    assert (sm[ctx == 0] == -1).all()
    _check(pkv, case, (ctx - 1).astype(np.int32), sm, seed=107)


def test_large_positions_and_theta(pkv):
    """Angles up to 131072 rad: formed in float64 and reduced modulo 2 pi before the float32 sine/cosine."""
    lq = [8, 8]
    lk = [131072, 70000]
    case = workloads.make_case(lq, [8, 8], num_q_heads=16, num_kv_heads=8, head_dim=128, block_size=256,
                               num_blocks=4, dtype="bf16", seed=108)
    pos = np.concatenate([np.arange(l - 8, l) for l in lk]).astype(np.int32)
    sm = np.arange(16, dtype=np.int32)
    _check(pkv, case, pos, sm, theta=1e4, seed=108)
    _check(pkv, case, pos, sm, theta=1e6, seed=109)


def test_rows_of_a_merged_qkv_projection(pkv):
    """q, k, v sliced out of one [N, (Hq + 2 Hkv) hd] buffer, as the pages' qkv split."""
    case = workloads.make_case([90, 40], [90, 40], num_q_heads=16, num_kv_heads=8, head_dim=128, block_size=256,
                               num_blocks=3, dtype="bf16", seed=110)
    n = 130
    merged = np.concatenate([case.q.reshape(n, -1), case.k.reshape(n, -1), case.v.reshape(n, -1)], axis=1)
    dev = to_dev(merged, "bf16")
    q = dev[:, :2048].view(n, 16, 128)
    k = dev[:, 2048:3072].view(n, 8, 128)
    v = dev[:, 3072:].view(n, 8, 128)
    sm = oracle.slot_mapping_ref(case.block_tables, 256, n, cu_seqlens_q=case.cu_seqlens_q,
                                 cu_seqlens_k=case.cu_seqlens_k)
    _check(pkv, case, _positions(case), sm, seed=110, q=q, k=k, v=v)


def test_unaligned_rows_take_the_elementwise_kernel(pkv):
    """q, k and v starting 2 bytes past a 16-byte boundary: the element-wise kernel, same results."""
    case = workloads.make_case([37, 12], [40, 12], num_q_heads=16, num_kv_heads=8, head_dim=128, block_size=16,
                               num_blocks=8, dtype="bf16", seed=115)
    n = 49

    def shifted(x, heads):
        buf = torch.empty(n * heads * 128 + 1, dtype=torch.bfloat16, device="cuda")
        view = buf[1:].view(n, heads, 128)
        view.copy_(to_dev(x, "bf16"))
        assert view.data_ptr() % 16 == 2
        return view

    sm = oracle.slot_mapping_ref(case.block_tables, 16, n, cu_seqlens_q=case.cu_seqlens_q,
                                 cu_seqlens_k=case.cu_seqlens_k)
    _check(pkv, case, _positions(case), sm, seed=115, q=shifted(case.q, 16), k=shifted(case.k, 8),
           v=shifted(case.v, 8))
