"""GPU parity of attention (prefill contiguous / paged, decode) against the float64 oracle at small sizes that
still span several tiles, splits and ragged tails; float32 path to 1e-5, bf16 path to 2e-2 (max-abs)."""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import (BF16_TOL, F32_TOL, f64, gpu_slot_mapping, gpu_store_history, host_of, i32, log, logical_kv,
                      max_abs_err, nan_cache, oracle_attention, oracle_slot_mapping, to_dev, to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import paged_kv_cache_300_amd as m
    m.lib()
    return m


def _tol(dtype):
    return BF16_TOL if dtype == "bf16" else F32_TOL


def _run_step(pkv, case, paged, order=True):
    """Store history + new tokens through the HIP path, then attention; returns (out, kc, vc, slot_mapping)."""
    kc, vc = nan_cache(case), nan_cache(case)
    gpu_store_history(case, kc, vc)
    sm = gpu_slot_mapping(case)
    k, v, q = to_dev(case.k, case.dtype), to_dev(case.v, case.dtype), to_dev(case.q, case.dtype)
    pkv.kv_store(k, v, kc, vc, sm)
    bt = i32(case.block_tables)
    if case.decode:
        out = pkv.attn_decode_paged(q, kc, vc, i32(case.context_lens), bt, case.scale)
    elif paged:
        out = pkv.attn_prefill_varlen(q, kc, vc, i32(case.cu_seqlens_q), i32(case.cu_seqlens_k), int(case.Lq.max()),
                                      int(case.Lk.max()), case.scale, causal=True, block_table=bt, order=order)
    else:
        out = pkv.attn_prefill_varlen(q, k, v, i32(case.cu_seqlens_q), i32(case.cu_seqlens_k), int(case.Lq.max()),
                                      int(case.Lk.max()), case.scale, causal=True, order=order)
    torch.cuda.synchronize()
    return out, kc, vc, sm


def _check_attention(case, out, rows=None):
    want = oracle_attention(case, rows)
    got = oracle.as_f64(to_host(out), case.dtype)
    worst = 0.0
    for b, w in want.items():
        q0 = int(case.cu_seqlens_q[b])
        worst = max(worst, max_abs_err(got[q0:q0 + w.shape[0]], w))
    log(f"  max-abs error {worst:.3e} (tol {_tol(case.dtype):.0e})")
    assert worst <= _tol(case.dtype)
    return worst


def test_tiny_fp32_layer_end_to_end(pkv):
    """Tiny fp32 layer: store + causal prefill (contiguous and paged), then one decode step per sequence."""
    pre = workloads.tiny_fp32_prefill()
    log(f"tiny fp32 layer block_tables={pre.block_tables.tolist()}")
    for paged in (False, True):
        out, kc, vc, sm = _run_step(pkv, pre, paged)
        np.testing.assert_array_equal(to_host(sm), oracle_slot_mapping(pre))
        _check_attention(pre, out)
    # cache bytes after the prefill store equal the oracle's store, NaN-poisoned slots included
    cache = workloads.nan_cache_host(pre.num_blocks, pre.block_size, 2, 16, "f32")
    want_k, want_v = oracle.store_ref(pre.k, pre.v, cache, cache, oracle_slot_mapping(pre))
    assert np.array_equal(to_host(kc).view(np.uint32), want_k.view(np.uint32))
    assert np.array_equal(to_host(vc).view(np.uint32), want_v.view(np.uint32))
    # decode step on top of the same cache
    dec = workloads.tiny_fp32_decode(pre)
    sm_d = gpu_slot_mapping(dec)
    want_sm = oracle_slot_mapping(dec)
    np.testing.assert_array_equal(to_host(sm_d), want_sm)
    assert want_sm.tolist() == [int(pre.block_tables[0, 1]) * 4 + 2, int(pre.block_tables[1, 0]) * 4 + 3]
    pkv.kv_store(to_dev(dec.k, "f32"), to_dev(dec.v, "f32"), kc, vc, sm_d)
    out = pkv.attn_decode_paged(to_dev(dec.q, "f32"), kc, vc, i32(dec.context_lens), i32(dec.block_tables), dec.scale)
    torch.cuda.synchronize()
    _check_attention(dec, out)


DECODE_CASES = [
    # (dtype, hq, hkv, hd, bs, context lengths, seed)
    ("bf16", 16, 8, 128, 256, [1, 2, 255, 256, 257, 600, 1000, 1300], 11),
    ("bf16", 16, 8, 128, 16, [5, 100, 1029, 31, 0, 300], 12),
    ("bf16", 8, 8, 128, 3, [7, 64, 300, 1], 13),
    ("bf16", 16, 4, 128, 1, [65, 200, 3], 14),
    ("bf16", 16, 2, 128, 32, [700, 33], 15),  # group of 8: generic path
    ("bf16", 8, 4, 64, 8, [100, 9, 513], 16),   # head_dim 64: generic path
    ("bf16", 4, 2, 128, 16, [40, 0, 3, 77], 19),  # two kv heads: small work-groups
    ("bf16", 16, 8, 128, 256, [0, 0, 0], 20),      # all padding: no key anywhere
    ("bf16", 16, 8, 128, 4, [1, 2, 0], 30),        # fewer keys than work-groups: empty ranges
    ("f32", 4, 2, 16, 4, [1, 7, 30, 100], 17),
    ("f32", 16, 8, 128, 256, [300, 1], 18),
]


@pytest.mark.parametrize("dtype,hq,hkv,hd,bs,ctx,seed", DECODE_CASES)
def test_decode_small(pkv, dtype, hq, hkv, hd, bs, ctx, seed):
    num_blocks = sum(math.ceil(c / bs) for c in ctx) + 3
    case = workloads.decode_case(ctx, num_q_heads=hq, num_kv_heads=hkv, head_dim=hd, block_size=bs,
                                 num_blocks=num_blocks, dtype=dtype, seed=seed,
                                 max_blocks=max(math.ceil(c / bs) for c in ctx) + 1)
    log(f"decode {dtype} {hq}/{hkv}/{hd} bs={bs} ctx={ctx}")
    out, kc, vc, sm = _run_step(pkv, case, paged=True)
    np.testing.assert_array_equal(to_host(sm), oracle_slot_mapping(case))
    _check_attention(case, out)
    if 0 in ctx:
        assert bool((out[ctx.index(0)] == 0).all())


def test_decode_batch_beyond_lds_prefix_staging(pkv):
    """2100 sequences (more than the 2048 prefix sums the decode stages in LDS, more than one 1024-wide scan)."""
    rng = np.random.default_rng(61)
    ctx = rng.integers(0, 40, 2100)
    case = workloads.decode_case(ctx, num_q_heads=16, num_kv_heads=8, head_dim=128, block_size=16,
                                 num_blocks=int(sum(math.ceil(c / 16) for c in ctx)) + 1, seed=61, max_blocks=3)
    log(f"decode batch {case.batch}, sum ctx {int(ctx.sum())}")
    out, kc, vc, sm = _run_step(pkv, case, paged=True)
    np.testing.assert_array_equal(to_host(sm), oracle_slot_mapping(case))
    _check_attention(case, out, rows=list(range(0, 2100, 7)) + [2099])
    zeros = np.where(ctx == 0)[0]
    assert bool((out[torch.from_numpy(zeros).cuda()] == 0).all())


@pytest.mark.parametrize("ctx", [[20000], [127, 1, 3], [129]])
def test_decode_one_long_sequence_many_pieces(pkv, ctx):
    """One sequence cut into as many ranges as the launch has workers (hundreds of partial states merged), and
    batches with fewer keys than a worker's minimum (one worker takes everything)."""
    case = workloads.decode_case(ctx, num_blocks=sum(math.ceil(c / 256) for c in ctx) + 2, seed=71,
                                 max_blocks=max(math.ceil(c / 256) for c in ctx))
    log(f"decode ctx={ctx}")
    out, kc, vc, sm = _run_step(pkv, case, paged=True)
    _check_attention(case, out)


@pytest.mark.parametrize("batch,paged", [(3000, False), (3000, True), (4100, True)])
def test_prefill_many_short_sequences(pkv, batch, paged):
    """Thousands of short sequences (0-5 new tokens, paged: after cached prefixes of 0-99): the longest-first
    planner up to its 4096-sequence limit, and the grid order beyond it (no workspace is asked for there)."""
    rng = np.random.default_rng(81 + batch)
    lq = rng.integers(0, 6, batch)
    prefix = rng.integers(0, 100, batch) if paged else np.zeros(batch, np.int64)
    lk = lq + prefix
    bs = 16
    case = workloads.make_case(lq, lk, num_q_heads=16, num_kv_heads=8, head_dim=128, block_size=bs,
                               num_blocks=int(sum(math.ceil(c / bs) for c in lk)) + 2, dtype="bf16", seed=81 + batch)
    assert (pkv.attn_prefill_workspace_bytes(batch, int(lq.sum()), int(lq.max()), 16, 8, 128) > 0) == (batch <= 4096)
    log(f"prefill batch {batch} paged={paged}, {int(lq.sum())} new tokens")
    out, kc, vc, sm = _run_step(pkv, case, paged)
    np.testing.assert_array_equal(to_host(sm), oracle_slot_mapping(case))
    _check_attention(case, out, rows=list(range(0, batch, 13)) + [batch - 1])


PREFILL_CASES = [
    # (dtype, hq, hkv, hd, bs, new lengths, cached prefix lengths, seed)
    ("bf16", 16, 8, 128, 256, [1, 63, 64, 65, 200, 333], [0] * 6, 21),
    ("bf16", 16, 8, 128, 256, [130, 17, 64, 1], [300, 0, 511, 1000], 22),
    ("bf16", 16, 8, 128, 16, [77, 5], [40, 3], 23),
    ("bf16", 8, 8, 128, 7, [50, 129], [0, 20], 24),
    ("bf16", 16, 4, 128, 64, [96, 3], [10, 0], 25),
    ("bf16", 16, 2, 128, 32, [40], [30], 26),       # group of 8: generic path
    ("bf16", 4, 2, 32, 4, [33, 8], [5, 0], 27),       # head_dim 32: generic path
    ("f32", 4, 2, 16, 4, [6, 3, 17], [0, 0, 9], 28),
    ("f32", 16, 8, 128, 256, [70, 1], [0, 300], 29),
]


# Contiguous K/V (paged=False) only for cases without a cached prefix: a prefix is only readable through the
# block tables.
PREFILL_RUNS = [(*c, paged, order) for c in PREFILL_CASES for paged in (False, True) for order in (True, False)
                if paged or not any(c[6])]


@pytest.mark.parametrize("dtype,hq,hkv,hd,bs,lq,prefix,seed,paged,order", PREFILL_RUNS)
def test_prefill_small(pkv, dtype, hq, hkv, hd, bs, lq, prefix, seed, paged, order):
    lk = [a + b for a, b in zip(lq, prefix)]
    num_blocks = sum(math.ceil(c / bs) for c in lk) + 2
    case = workloads.make_case(lq, lk, num_q_heads=hq, num_kv_heads=hkv, head_dim=hd, block_size=bs,
                               num_blocks=num_blocks, dtype=dtype, seed=seed)
    log(f"prefill {dtype} {hq}/{hkv}/{hd} bs={bs} lq={lq} prefix={prefix} paged={paged} order={order}")
    out, kc, vc, sm = _run_step(pkv, case, paged, order)
    np.testing.assert_array_equal(to_host(sm), oracle_slot_mapping(case))
    _check_attention(case, out)


ORDER_CASES = [
    # (hq, hkv, new lengths, cached prefix lengths, block size, seed): prefixes of very different lengths,
    # empty sequences between full ones, a single tile, GQA groups 1 / 2 / 4, block sizes 64 .. 256 and 7.
    (16, 8, [90, 513, 64, 300], [3000, 100, 4100, 0], 256, 71),
    (16, 8, [0, 700, 0, 333, 1], [0, 20, 5, 900, 4000], 256, 72),
    (16, 8, [64], [130], 256, 73),
    (8, 8, [200, 900], [1200, 0], 64, 74),
    (32, 8, [400, 129], [2000, 77], 128, 75),
    (16, 8, [100, 37], [500, 900], 7, 76),
    # keys that fill the block-table row exactly (the pipelined paged loop looks a tile past the last one)
    (16, 8, [256, 64], [768, 0], 256, 77),
    (32, 8, [128, 1], [128, 63], 64, 78),
    (8, 8, [64], [0], 64, 79),
]


@pytest.mark.parametrize("hq,hkv,lq,prefix,bs,seed", ORDER_CASES)
def test_prefill_longest_first_order(pkv, hq, hkv, lq, prefix, bs, seed):
    """Query tiles listed longest first by the planner (for GQA groups of 2 also cut into key-range pieces
    merged afterwards): within tolerance of the oracle, as is the latest-tile-first grid, and the two differ
    only by rounding (a split tile sums its keys in pieces; a tile's arithmetic does not depend on when it
    runs)."""
    lk = [a + b for a, b in zip(lq, prefix)]
    case = workloads.make_case(lq, lk, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, block_size=bs,
                               num_blocks=sum(math.ceil(c / bs) for c in lk) + 2, dtype="bf16", seed=seed)
    log(f"longest-first {hq}/{hkv} lq={lq} prefix={prefix} bs={bs}")
    out, *_ = _run_step(pkv, case, paged=True, order=True)
    _check_attention(case, out)
    ref, *_ = _run_step(pkv, case, paged=True, order=False)
    _check_attention(case, ref)
    # one bf16 rounding step of the value (2^-8 relative) plus float32 summation noise
    torch.testing.assert_close(out.float(), ref.float(), rtol=2.0 ** -7, atol=1e-3)


SPLIT_CASES = [
    # (lq, prefix, paged, block_size): too few query tiles to fill the GPU, over key ranges far longer than the
    # work each resident work-group gets, so the planner cuts them into pieces (causal diagonal tiles in the last
    # piece, cached prefixes spanning many pieces, short rows beside them)
    ([2000, 5, 64], [0, 0, 0], False, 256),
    ([700, 130, 1], [5000, 3000, 7000], True, 256),
    ([1100, 64, 65], [2300, 4100, 0], True, 64),
    ([64], [20000], True, 256),  # one chunk of new tokens on a long cached prefix
]


@pytest.mark.parametrize("lq,prefix,paged,bs", SPLIT_CASES)
def test_prefill_split_long_rows(pkv, lq, prefix, paged, bs):
    """Long rows cut into key-range pieces whose partial states a second kernel merges [P2 §5.2 ②]: every row
    against the oracle, and within one bf16 rounding of the unplanned (unsplit) launch."""
    lk = [a + b for a, b in zip(lq, prefix)]
    case = workloads.make_case(lq, lk, num_q_heads=16, num_kv_heads=8, head_dim=128, block_size=bs,
                               num_blocks=sum(math.ceil(c / bs) for c in lk) + 2, dtype="bf16", seed=sum(lk))
    log(f"split pieces lq={lq} prefix={prefix} paged={paged} bs={bs}")
    out, *_ = _run_step(pkv, case, paged=paged, order=True)
    _check_attention(case, out)
    ref, *_ = _run_step(pkv, case, paged=paged, order=False)
    torch.testing.assert_close(out.float(), ref.float(), rtol=2.0 ** -7, atol=1e-3)


SPLIT_HEAD_CASES = [
    # (lq, prefix, paged, block_size, hq, hkv): the same cut at other head counts (GQA groups of 2), so the
    # workspace's per-kv-head partial slots and the merge's (unit, kv head) grid are exercised beyond 8 kv heads:
    # 19 query tiles x 16 kv heads of one 1200-token sequence, and chunks on long prefixes with 4 kv heads
    ([1200], [0], False, 256, 32, 16),
    ([64, 128], [9000, 3000], True, 128, 8, 4),
]


@pytest.mark.parametrize("lq,prefix,paged,bs,hq,hkv", SPLIT_HEAD_CASES)
def test_prefill_split_other_head_counts(pkv, lq, prefix, paged, bs, hq, hkv):
    lk = [a + b for a, b in zip(lq, prefix)]
    case = workloads.make_case(lq, lk, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, block_size=bs,
                               num_blocks=sum(math.ceil(c / bs) for c in lk) + 2, dtype="bf16", seed=7 + sum(lk))
    log(f"split pieces lq={lq} prefix={prefix} paged={paged} bs={bs} heads {hq}/{hkv}")
    out, *_ = _run_step(pkv, case, paged=paged, order=True)
    _check_attention(case, out)
    ref, *_ = _run_step(pkv, case, paged=paged, order=False)
    torch.testing.assert_close(out.float(), ref.float(), rtol=2.0 ** -7, atol=1e-3)


def test_prefill_one_long_sequence_sampled_rows(pkv):
    """One 6000-token causal sequence from contiguous rows: 94 query tiles, the last over 94 key tiles (the 32x32
    kernel in grid order).  Sampled rows against the oracle, row i as its own problem: one query at position i over
    keys 0..i [P2 §5.3, causal varlen call], which is what the causal mask leaves of the whole sequence."""
    L = 6000
    case = workloads.make_case([L], [L], num_q_heads=16, num_kv_heads=8, head_dim=128, block_size=256,
                               num_blocks=math.ceil(L / 256) + 2, dtype="bf16", seed=6000)
    out, *_ = _run_step(pkv, case, paged=False, order=True)
    got = oracle.as_f64(to_host(out), "bf16")
    q = f64(case.q, "bf16")
    k = oracle.as_f64(logical_kv(case, 0, "k"), "bf16")
    v = oracle.as_f64(logical_kv(case, 0, "v"), "bf16")
    rng = np.random.default_rng(6000)
    rows = sorted(set(rng.integers(0, L, 48).tolist()) | {0, 1, 63, 64, 4095, 4096, L - 65, L - 1})
    worst = 0.0
    for i in rows:
        want = oracle.attention_ref(q[i:i + 1], k[:i + 1], v[:i + 1], [0, 1], [0, i + 1], case.scale, causal=True)
        worst = max(worst, max_abs_err(got[i:i + 1], want))
    log(f"  {len(rows)} sampled rows, max-abs error {worst:.3e} (tol {BF16_TOL:.0e})")
    assert worst <= BF16_TOL


def test_prefill_order_workspace(pkv):
    """The planner's workspace needs no clearing (garbage in, same result) and an undersized one is refused."""
    lq, prefix = [300, 70, 129], [2000, 10, 600]
    lk = [a + b for a, b in zip(lq, prefix)]
    case = workloads.make_case(lq, lk, num_q_heads=16, num_kv_heads=8, head_dim=128, block_size=256,
                               num_blocks=sum(math.ceil(c / 256) for c in lk) + 2, dtype="bf16", seed=77)
    kc, vc = nan_cache(case), nan_cache(case)
    gpu_store_history(case, kc, vc)
    pkv.kv_store(to_dev(case.k, "bf16"), to_dev(case.v, "bf16"), kc, vc, gpu_slot_mapping(case))
    q, bt = to_dev(case.q, "bf16"), i32(case.block_tables)
    args = (q, kc, vc, i32(case.cu_seqlens_q), i32(case.cu_seqlens_k), 300, 2600, case.scale)
    need = pkv.attn_prefill_workspace_bytes(3, sum(lq), 300, 16, 8, 128)
    assert need > 0
    ws = torch.full((need,), 0xAB, dtype=torch.uint8, device="cuda")
    first = pkv.attn_prefill_varlen(*args, block_table=bt, workspace=ws)
    torch.cuda.synchronize()
    _check_attention(case, first)
    ws.fill_(0x7F)
    again = pkv.attn_prefill_varlen(*args, block_table=bt, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(first, again)
    with pytest.raises(pkv.PagedKVError):
        pkv.attn_prefill_varlen(*args, block_table=bt, workspace=ws[: need - 1])


def test_prefill_strided_qkv_from_merged_projection(pkv):
    """q, k, v sliced out of one merged [N, (Hq + 2 Hkv) * hd] buffer, as the pages' split of qkv_proj."""
    rng = np.random.default_rng(31)
    lens, hq, hkv, hd = [70, 129], 16, 8, 128
    n = sum(lens)
    qkv = workloads.f32_to_bf16_bits(rng.standard_normal((n, (hq + 2 * hkv) * hd)).astype(np.float32))
    dev = to_dev(qkv, "bf16")
    q = dev[:, : hq * hd].view(n, hq, hd)
    k = dev[:, hq * hd: (hq + hkv) * hd].view(n, hkv, hd)
    v = dev[:, (hq + hkv) * hd:].view(n, hkv, hd)
    cu = np.array([0, lens[0], n], np.int32)
    out = pkv.attn_prefill_varlen(q, k, v, i32(cu), i32(cu), max(lens), max(lens), 1 / math.sqrt(hd))
    torch.cuda.synchronize()
    qf = oracle.as_f64(qkv[:, : hq * hd].reshape(n, hq, hd), "bf16")
    kf = oracle.as_f64(qkv[:, hq * hd: (hq + hkv) * hd].reshape(n, hkv, hd), "bf16")
    vf = oracle.as_f64(qkv[:, (hq + hkv) * hd:].reshape(n, hkv, hd), "bf16")
    want = oracle.attention_ref(qf, kf, vf, cu, cu, 1 / math.sqrt(hd))
    err = max_abs_err(oracle.as_f64(to_host(out), "bf16"), want)
    log(f"  strided max-abs {err:.3e}")
    assert err <= BF16_TOL


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_non_causal(pkv, dtype):
    hd = 128 if dtype == "bf16" else 16
    case = workloads.make_case([40, 90], [40, 90], num_q_heads=16, num_kv_heads=8, head_dim=hd, block_size=256,
                               num_blocks=4, dtype=dtype, seed=41)
    q, k, v = (to_dev(x, dtype) for x in (case.q, case.k, case.v))
    out = pkv.attn_prefill_varlen(q, k, v, i32(case.cu_seqlens_q), i32(case.cu_seqlens_k), 90, 90, case.scale,
                                  causal=False)
    torch.cuda.synchronize()
    want = oracle.attention_ref(f64(case.q, dtype), f64(case.k, dtype), f64(case.v, dtype), case.cu_seqlens_q,
                                case.cu_seqlens_k, case.scale, causal=False)
    assert max_abs_err(oracle.as_f64(to_host(out), dtype), want) <= _tol(dtype)


def test_single_key_is_exact_in_bf16(pkv):
    """Closed form: a row that sees one key returns that key's V exactly, even in bf16."""
    case = workloads.decode_case([1, 1, 1], num_blocks=4, seed=51)
    out, *_ = _run_step(pkv, case, paged=True)
    v_new = to_dev(case.v, "bf16")
    for b in range(3):
        for h in range(16):
            assert torch.equal(out[b, h], v_new[b, h // 2])
    pre = workloads.make_case([1, 1], [1, 1], num_q_heads=16, num_kv_heads=8, head_dim=128, block_size=256,
                              num_blocks=2, dtype="bf16", seed=52)
    for paged in (False, True):
        out, *_ = _run_step(pkv, pre, paged)
        v_new = to_dev(pre.v, "bf16")
        for h in range(16):
            assert torch.equal(out[:, h], v_new[:, h // 2])


def test_zero_query_gives_prefix_means(pkv):
    """Closed form: q = 0 makes every visible key equally weighted (causal prefix means of V)."""
    case = workloads.make_case([150], [150], num_q_heads=16, num_kv_heads=8, head_dim=128, block_size=256,
                               num_blocks=2, dtype="bf16", seed=53)
    case.q = np.zeros_like(case.q)
    out, *_ = _run_step(pkv, case, paged=False)
    v = f64(case.v, "bf16")
    means = np.cumsum(v, axis=0) / np.arange(1, 151)[:, None, None]
    got = oracle.as_f64(to_host(out), "bf16")
    for h in range(16):
        assert np.max(np.abs(got[:, h] - means[:, h // 2])) <= BF16_TOL


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("scale", [-0.0883883, 1e-30, 0.0883883])
def test_prefill_scale_signs(pkv, paged, scale):
    """GQA groups of 2 with a negative scale (served by the 16x16 kernels), a tiny positive one (every weight 1 to
    within rounding; the 32x32 kernel) and the usual 1/sqrt(128), against the oracle [P2 §5.3 softmax_scale]."""
    case = workloads.make_case([130, 70], [400, 70] if paged else [130, 70], num_q_heads=16, num_kv_heads=8,
                               head_dim=128, block_size=256, num_blocks=6, dtype="bf16", seed=61, scale=scale)
    log(f"prefill scale={scale} paged={paged}")
    out, *_ = _run_step(pkv, case, paged)
    _check_attention(case, out)


def test_prefill_paged_block_size_1024(pkv):
    """Paged prefill with 1024-token blocks: sixteen 64-key tiles per block, prefixes ending mid-block."""
    case = workloads.make_case([300, 70, 5], [1800, 2270, 1029], num_q_heads=16, num_kv_heads=8, head_dim=128,
                               block_size=1024, num_blocks=9, dtype="bf16", seed=62)
    log("prefill bs=1024 lq=[300, 70, 5] prefix=[1500, 2200, 1024]")
    out, *_ = _run_step(pkv, case, paged=True)
    _check_attention(case, out)


def test_prefill_grid_order_several_chunks(pkv):
    """Causal self-attention launched in grid order (no planner) over nine sequences: two full chunks of four
    sequences and a last chunk of one, with empty, single-token and multi-tile sequences."""
    lq = [700, 64, 0, 513, 1, 130, 260, 65, 390]
    case = workloads.make_case(lq, lq, num_q_heads=16, num_kv_heads=8, head_dim=128, block_size=256, num_blocks=16,
                               dtype="bf16", seed=63)
    log(f"prefill grid order lq={lq}")
    out, *_ = _run_step(pkv, case, paged=False, order=False)
    _check_attention(case, out)
