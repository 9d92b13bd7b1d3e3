"""GPU parity of kv_slot_mapping and kv_store against the oracle: bit-exact."""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from conftest import load_golden
from gpu_util import i32, log, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_300_amd as m
    m.lib()
    return m


def _random_tables(rng, lk, bs, num_blocks, extra_cols=2):
    need = [math.ceil(n / bs) for n in lk]
    perm = rng.permutation(num_blocks)
    bt = np.full((len(lk), max(need + [1]) + extra_cols), -1, np.int32)
    pos = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    return bt


@pytest.mark.parametrize("seed", range(6))
def test_slot_mapping_prefill_random(pkv, seed):
    rng = np.random.default_rng(1000 + seed)
    bs = int(rng.choice([1, 3, 4, 16, 256]))
    batch = int(rng.integers(1, 9))
    lq = rng.integers(0, 40, batch)
    lk = lq + rng.integers(0, 60, batch) * int(rng.integers(0, 2))  # sometimes a cached prefix
    bt = _random_tables(rng, lk, bs, int(sum(math.ceil(n / bs) for n in lk)) + 5)
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    n = int(cu_q[-1]) + int(rng.integers(0, 5))  # padding rows past the last token
    log(f"slot_mapping prefill seed={seed} bs={bs} batch={batch} n={n}")
    want = oracle.slot_mapping_ref(bt, bs, n, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k)
    got = pkv.kv_slot_mapping(i32(bt), bs, n, cu_seqlens_q=i32(cu_q), cu_seqlens_k=i32(cu_k))
    np.testing.assert_array_equal(to_host(got), want)
    if np.array_equal(lq, lk):  # cu_seqlens_k omitted means "nothing cached"
        got2 = pkv.kv_slot_mapping(i32(bt), bs, n, cu_seqlens_q=i32(cu_q))
        np.testing.assert_array_equal(to_host(got2), want)


@pytest.mark.parametrize("seed", range(4))
def test_slot_mapping_decode_random_with_padding(pkv, seed):
    rng = np.random.default_rng(2000 + seed)
    bs = int(rng.choice([1, 4, 256]))
    ctx = rng.integers(1, 700, 37)
    ctx[-5:] = 0  # padding rows
    bt = _random_tables(rng, ctx, bs, int(sum(math.ceil(n / bs) for n in ctx)) + 1)
    want = oracle.slot_mapping_ref(bt, bs, 40, context_lens=ctx)
    got = pkv.kv_slot_mapping(i32(bt), bs, 40, context_lens=i32(ctx))
    np.testing.assert_array_equal(to_host(got), want)
    assert np.all(want[-8:] == -1)


def test_slot_mapping_exercise_a_on_gpu(pkv):
    g = load_golden("slot_mapping_exercise_a.json")
    bt = i32(np.array([g["block_table"]]))
    for c in g["cases"]:
        got = pkv.kv_slot_mapping(bt, g["block_size"], c["new"], cu_seqlens_q=i32([0, c["new"]]),
                                  cu_seqlens_k=i32([0, c["cached"] + c["new"]]))
        assert to_host(got).tolist() == c["slots_expected"]


def test_store_4token_example_on_gpu(pkv):
    g = load_golden("store_4tok.json")
    nkv, hd = g["num_kv_heads"], g["head_dim"]
    n = len(g["slot_mapping"])
    base = torch.arange(nkv * hd).reshape(1, nkv, hd)
    key = (torch.arange(n).reshape(n, 1, 1) * 10 + base).float().cuda()
    value = key + 100
    kc = torch.zeros(g["num_blocks"], g["block_size"], nkv, hd, device="cuda")
    vc = torch.zeros_like(kc)
    pkv.kv_store(key, value, kc, vc, i32(g["slot_mapping"]))
    assert kc.view(-1, nkv * hd).cpu().tolist() == g["k_cache_expected"]
    assert vc.view(-1, nkv * hd)[0].cpu().tolist() == g["v_cache_slot0_expected"]


def test_scatter_skeleton_example_on_gpu(pkv):
    g = load_golden("scatter_n3_d4.json")
    src = torch.tensor(g["src"], dtype=torch.float32, device="cuda").view(3, 1, 4)
    dst = torch.zeros(1, 3, 1, 4, device="cuda")
    other = torch.zeros_like(dst)
    pkv.kv_store(src, src, dst, other, i32(g["slot"]))
    assert dst.view(3, 4).cpu().tolist() == g["dst_expected"]


@pytest.mark.parametrize("dtype,hkv,hd,strided,seed", [
    ("bf16", 8, 128, False, 0), ("bf16", 8, 128, True, 1), ("bf16", 2, 16, False, 2), ("f32", 2, 16, True, 3),
    ("bf16", 3, 5, False, 4), ("f32", 1, 3, True, 5), ("bf16", 4, 64, True, 6),
])
def test_store_random_bit_exact(pkv, dtype, hkv, hd, strided, seed):
    rng = np.random.default_rng(3000 + seed)
    num_blocks, bs = 6, 16
    num_slots = num_blocks * bs
    n = 70
    slots = rng.choice(num_slots, n, replace=False).astype(np.int32)
    slots[rng.choice(n, 9, replace=False)] = -1                 # padding tokens
    slots[rng.choice(np.where(slots >= 0)[0], 2)] = num_slots + 7  # out of range: skipped, never written
    d = hkv * hd
    width = 3 * d + (8 if strided else 0) if strided else d
    if dtype == "bf16":
        buf = rng.integers(0, 2**16, size=(n, width), dtype=np.uint16)
        buf[(buf & 0x7F80) == 0x7F80] = 0x1234  # no NaN/inf patterns in the data, so byte compare is exact
        cache = rng.integers(0, 2**16, size=(num_blocks, bs, hkv, hd), dtype=np.uint16)
    else:
        buf = rng.standard_normal((n, width)).astype(np.float32)
        cache = rng.standard_normal((num_blocks, bs, hkv, hd)).astype(np.float32)
    kslice = (slice(None), slice(d, 2 * d)) if strided else (slice(None), slice(0, d))
    vslice = (slice(None), slice(2 * d, 3 * d)) if strided else (slice(None), slice(0, d))
    buf_v = buf if strided else (buf[:, ::-1].copy() if dtype == "f32" else buf ^ np.uint16(0x0101))
    key_h = buf[kslice].reshape(n, hkv, hd)
    val_h = buf_v[vslice].reshape(n, hkv, hd)
    want_k, want_v = oracle.store_ref(key_h, val_h, cache, cache, slots)
    dev_buf = to_dev(buf, dtype)
    dev_buf_v = dev_buf if strided else to_dev(buf_v, dtype)
    key = dev_buf[kslice].view(n, hkv, hd)
    value = dev_buf_v[vslice].view(n, hkv, hd)
    kc, vc = to_dev(cache, dtype), to_dev(cache, dtype)
    log(f"store dtype={dtype} hkv={hkv} hd={hd} strided={strided} key_stride={key.stride(0)}")
    pkv.kv_store(key, value, kc, vc, i32(slots))
    assert np.array_equal(to_host(kc).view(np.uint8), np.asarray(want_k).view(np.uint8))
    assert np.array_equal(to_host(vc).view(np.uint8), np.asarray(want_v).view(np.uint8))


def test_store_zero_tokens_is_a_noop(pkv):
    kc = torch.ones(2, 4, 1, 8, device="cuda")
    vc = torch.ones_like(kc)
    empty = torch.empty(0, 1, 8, device="cuda")
    pkv.kv_store(empty, empty, kc, vc, torch.empty(0, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert bool((kc == 1).all()) and bool((vc == 1).all())


def test_binding_rejects_short_metadata(pkv):
    """The kernels read cu_seqlens [batch + 1] and context_lens [batch]; shorter tensors are refused before any
    launch (the C ABI cannot see their lengths)."""
    bt = i32(np.arange(6).reshape(3, 2))
    with pytest.raises(ValueError):
        pkv.kv_slot_mapping(bt, 4, 8, cu_seqlens_q=i32([0, 3, 8]))            # 3 entries for batch 3
    with pytest.raises(ValueError):
        pkv.kv_slot_mapping(bt, 4, 8, cu_seqlens_q=i32([0, 3, 5, 8]), cu_seqlens_k=i32([0, 4]))
    with pytest.raises(ValueError):
        pkv.kv_slot_mapping(bt, 4, 3, context_lens=i32([1, 2]))
    with pytest.raises(ValueError):
        pkv.kv_slot_mapping(bt, 4, 3)                                          # neither mode
    got = pkv.kv_slot_mapping(bt, 4, 3, context_lens=i32([1, 5, 0]))
    assert to_host(got).tolist() == [0, 3 * 4 + 0, -1]   # row 1: position 4 is cell 0 of block bt[1][1] = 3


def test_slot_beyond_int32_is_none(pkv):
    """A block id whose slot does not fit an int32 gives -1 (formed in 64 bits, never wrapped into range)."""
    big = (2 ** 31) // 256 + 5                      # big * 256 > INT32_MAX
    bt = i32([[big], [3]])
    got = pkv.kv_slot_mapping(bt, 256, 2, context_lens=i32([10, 10]))
    assert to_host(got).tolist() == [-1, 3 * 256 + 9]
