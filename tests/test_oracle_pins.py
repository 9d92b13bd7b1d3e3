"""Pins of the CPU oracle against values the pages print and against closed forms (no GPU)."""

import math

import numpy as np
import pytest

import oracle
from conftest import load_golden


# ---------------------------------------------------------------- worked examples printed on the pages

def test_scatter_skeleton_example():
    g = load_golden("scatter_n3_d4.json")
    src = np.array(g["src"], dtype=np.float32)
    dst = oracle.scatter_rows_ref(src, g["slot"], np.zeros_like(src))
    assert dst.tolist() == g["dst_expected"]


def test_store_4token_example_bit_exact():
    g = load_golden("store_4tok.json")
    nkv, hd = g["num_kv_heads"], g["head_dim"]
    n = len(g["slot_mapping"])
    base = np.arange(nkv * hd).reshape(1, nkv, hd)
    key = (np.arange(n).reshape(n, 1, 1) * 10 + base).astype(np.float32)
    value = key + 100
    shape = (g["num_blocks"], g["block_size"], nkv, hd)
    kc, vc = oracle.store_ref(key, value, np.zeros(shape, np.float32), np.zeros(shape, np.float32),
                              np.array(g["slot_mapping"], np.int32))
    assert kc.reshape(-1, nkv * hd).tolist() == g["k_cache_expected"]
    assert vc.reshape(-1, nkv * hd)[0].tolist() == g["v_cache_slot0_expected"]
    # the padding token (slot -1) wrote nothing anywhere: its key prefix 20 is absent from both caches
    assert not np.any((kc >= 20) & (kc < 30)) and not np.any((vc >= 120) & (vc < 130))


def test_store_keeps_untouched_bytes_of_bf16_cache():
    rng = np.random.default_rng(0)
    cache = rng.integers(0, 2**16, size=(3, 4, 2, 8), dtype=np.uint16)
    key = rng.integers(0, 2**16, size=(5, 2, 8), dtype=np.uint16)
    value = rng.integers(0, 2**16, size=(5, 2, 8), dtype=np.uint16)
    slots = np.array([7, -1, 0, 11, 3], np.int32)
    kc, vc = oracle.store_ref(key, value, cache, cache, slots)
    flat_k, flat_v, flat_c = kc.reshape(12, 16), vc.reshape(12, 16), cache.reshape(12, 16)
    for idx, s in enumerate(slots):
        if s >= 0:
            assert np.array_equal(flat_k[s], key[idx].reshape(-1))
            assert np.array_equal(flat_v[s], value[idx].reshape(-1))
    untouched = [s for s in range(12) if s not in set(slots.tolist())]
    assert np.array_equal(flat_k[untouched], flat_c[untouched])
    assert np.array_equal(flat_v[untouched], flat_c[untouched])


def test_store_honours_token_stride():
    # rows of a wider buffer (e.g. k sliced out of a merged qkv row): the copy is by value
    rng = np.random.default_rng(1)
    qkv = rng.standard_normal((4, 3 * 8)).astype(np.float32)
    key = qkv[:, 8:16].reshape(4, 2, 4)
    value = qkv[:, 16:24].reshape(4, 2, 4)
    kc, vc = oracle.store_ref(key, value, np.zeros((2, 2, 2, 4), np.float32), np.zeros((2, 2, 2, 4), np.float32),
                              np.array([3, 0, 2, 1], np.int32))
    assert np.array_equal(kc.reshape(4, 8)[3], qkv[0, 8:16])
    assert np.array_equal(vc.reshape(4, 8)[1], qkv[3, 16:24])


def test_slot_mapping_exercise_a():
    g = load_golden("slot_mapping_exercise_a.json")
    bs, bt = g["block_size"], np.array([g["block_table"]], np.int32)
    for c in g["cases"]:
        cached, new = c["cached"], c["new"]
        walk = oracle.slot_mapping_block_walk(bt[0], cached, cached + new, bs)
        assert walk == c["slots_expected"]
        ref = oracle.slot_mapping_ref(bt, bs, new, cu_seqlens_q=[0, new], cu_seqlens_k=[0, cached + new])
        assert ref.tolist() == c["slots_expected"]


def test_integration_layer0_slots_and_decode_formula():
    g = load_golden("integration_layer0.json")
    bs = g["block_size"]
    p = g["prefill"]
    ref = oracle.slot_mapping_ref(np.array([p["block_table"]]), bs, p["new"], cu_seqlens_q=[0, p["new"]])
    assert ref.tolist() == p["slots_expected"]
    d = g["decode"]
    assert oracle.decode_slot_ref(d["block_table"], d["context_len"], bs) == d["slot_expected"]
    ref = oracle.slot_mapping_ref(np.array([d["block_table"]]), bs, 1, context_lens=[d["context_len"]])
    assert ref.tolist() == [d["slot_expected"]]


def test_decode_last_block_formula_matches_closed_form():
    rng = np.random.default_rng(2)
    for _ in range(200):
        bs = int(rng.integers(1, 9))
        ctx = int(rng.integers(1, 40))
        nblk = math.ceil(ctx / bs)
        row = rng.permutation(64)[:nblk]
        via_last = oracle.decode_slot_ref(row, ctx, bs)
        padded = np.full((1, nblk + 3), -1, np.int32)
        padded[0, :nblk] = row
        closed = oracle.slot_mapping_ref(padded, bs, 1, context_lens=[ctx])
        assert closed.tolist() == [via_last]


def test_online_softmax_worked_example():
    g = load_golden("online_softmax_example.json")
    s = np.array(g["scores"], float)
    v = np.array(g["values"], float)
    r = lambda x: round(float(x), g["decimals"])
    # whole row, by the definition
    out = oracle.attention_ref(np.ones((1, 1, 1)), s.reshape(4, 1, 1), v.reshape(4, 1, 1), [0, 1], [0, 4],
                               1.0, causal=False)
    assert r(out[0, 0, 0]) == g["whole_row"]["o"]
    w = np.exp(s - s.max())
    assert r(w.sum()) == g["whole_row"]["l"]
    assert [r(x) for x in w / w.sum()] == g["whole_row"]["weights"]
    # blocked, by the accumulators
    o, traj = oracle.online_softmax_blocks(s, v, g["blocks"])
    assert r(traj[0]["l"]) == g["after_A"]["l"] and r(traj[0]["o"]) == g["after_A"]["o_bar"]
    assert r(traj[1]["rescale"]) == g["rescale_factor"]
    assert r(traj[1]["l_rescaled"]) == g["A_rescaled"]["l"]
    assert r(traj[1]["o_rescaled"]) == g["A_rescaled"]["o_bar"]
    assert r(traj[1]["l"]) == g["after_B"]["l"] and r(traj[1]["o"]) == g["after_B"]["o_bar"]
    assert r(o) == g["final_o"]
    # the rescaled sums are exactly the whole-row contributions of the first two keys
    assert traj[1]["l_rescaled"] == pytest.approx(w[:2].sum(), rel=1e-14)
    assert traj[1]["o_rescaled"] == pytest.approx((w[:2] * v[:2]).sum(), rel=1e-14)
    assert r(w[:2].sum()) == g["first_two_terms"]["l"]


def test_online_softmax_example_embedded_in_paged_decode():
    # the same row as a paged decode: head_dim 16, q = e0, k_j = s_j e0, v_j = v_j e0, scale 1,
    # block_size 2 so blocks A and B are two physical blocks, stored in swapped physical order
    g = load_golden("online_softmax_example.json")
    s = np.array(g["scores"], float)
    v = np.array(g["values"], float)
    hd, bs = 16, 2
    q = np.zeros((1, 1, hd)); q[0, 0, 0] = 1.0
    kc = np.full((4, bs, 1, hd), np.nan); vc = np.full((4, bs, 1, hd), np.nan)
    table = np.array([[3, 1]], np.int32)
    for j in range(4):
        blk, off = table[0, j // bs], j % bs
        kc[blk, off, 0] = 0.0; kc[blk, off, 0, 0] = s[j]
        vc[blk, off, 0] = 0.0; vc[blk, off, 0, 0] = v[j]
    out = oracle.decode_ref(q, kc, vc, [4], table, bs, 1.0)
    assert round(out[0, 0, 0], 3) == g["final_o"]
    assert np.all(out[0, 0, 1:] == 0.0)


def test_gqa_group_map_on_the_pages_shapes():
    # 16 q heads in 8 groups of 2 share 8 kv heads (q_size 2048 = 16 x 128, kv_size 1024 = 8 x 128)
    groups = [oracle.kv_head_of(h, 16, 8) for h in range(16)]
    assert groups == [h // 2 for h in range(16)]
    assert 16 * 128 == 2048 and 8 * 128 == 1024


def test_bf16_widening_exact():
    bits = np.array([0x0000, 0x3F80, 0xBF80, 0x4049, 0x7F80, 0x0001], np.uint16)
    vals = oracle.bf16_bits_to_f64(bits)
    assert vals[0] == 0.0 and vals[1] == 1.0 and vals[2] == -1.0
    assert vals[3] == 3.140625 and np.isinf(vals[4])
    assert vals[5] == 2.0 ** -133


# ---------------------------------------------------------------- closed forms and special cases

def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_single_key_returns_its_value_exactly():
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 3, 4, 8), _rand(rng, 3, 2, 8), _rand(rng, 3, 2, 8)
    # three sequences of one token each: every row sees only its own key
    out = oracle.attention_ref(q, k, v, [0, 1, 2, 3], [0, 1, 2, 3], 0.3)
    for b in range(3):
        for h in range(4):
            assert np.array_equal(out[b, h], v[b, h // 2])


def test_zero_query_gives_causal_prefix_means():
    rng = np.random.default_rng(4)
    L = 7
    q, k, v = np.zeros((L, 2, 4)), _rand(rng, L, 1, 4), _rand(rng, L, 1, 4)
    out = oracle.attention_ref(q, k, v, [0, L], [0, L], 1.0)
    for i in range(L):
        np.testing.assert_allclose(out[i, 0], v[: i + 1, 0].mean(axis=0), rtol=1e-13, atol=1e-14)


def test_empty_context_rows_are_zero():
    rng = np.random.default_rng(5)
    q = _rand(rng, 2, 2, 4)
    kc = np.full((2, 4, 1, 4), np.nan); vc = np.full((2, 4, 1, 4), np.nan)
    kc[1, :3] = _rand(rng, 3, 1, 4); vc[1, :3] = _rand(rng, 3, 1, 4)
    bt = np.array([[1], [-1]], np.int32)
    out = oracle.decode_ref(q, kc, vc, [3, 0], bt, 4, 0.5)
    assert np.all(out[1] == 0.0) and np.all(np.isfinite(out[0]))


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(6)
    L, hd = 9, 8
    q = np.zeros((1, 1, hd)); q[0, 0, 0] = 1.0
    k = _rand(rng, L, 1, hd) * 0.1
    k[4, 0, 0] = 1000.0  # score gap of ~1000: every other weight underflows to 0
    v = _rand(rng, L, 1, hd)
    out = oracle.attention_ref(q, k, v, [0, 1], [0, L], 1.0)
    assert np.array_equal(out[0, 0], v[4, 0])


def test_uniform_scores_give_mean_over_any_split():
    rng = np.random.default_rng(7)
    v = _rand(rng, 10, 3)
    o, _ = oracle.online_softmax_blocks(np.full(10, 2.5), v, [3, 3, 4])
    np.testing.assert_allclose(o, v.mean(axis=0), rtol=1e-13)


def test_generator_rounding_is_nearest_even():
    """The seeded generator's float32 -> bf16 rounding (shared input preparation, not method arithmetic) is
    round-to-nearest-even: it agrees with torch's CPU conversion on ties, carries into the exponent, signed
    zeros, infinities and random patterns."""
    import torch
    import workloads
    rng = np.random.default_rng(9)
    pats = np.concatenate([
        rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32),
        np.array([0x3F808000, 0x3F818000, 0x3F807FFF, 0x3F808001, 0x3FFF8000, 0x7F7F8000, 0x7F7FFFFF,
                  0x80000000, 0x00000000, 0x7F800000, 0xFF800000, 0x00008000, 0x80018000], dtype=np.uint32)])
    x = pats.view(np.float32)
    finite = np.isfinite(x)
    got = workloads.f32_to_bf16_bits(x[finite])
    want = torch.from_numpy(x[finite].copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, want)
    inf = workloads.f32_to_bf16_bits(np.array([np.inf, -np.inf], np.float32))
    assert inf.tolist() == [0x7F80, 0xFF80]
