"""Pins of the CPU oracle by invariants, a textbook routine and brute force (no GPU).

Each invariant relates two different uses of the oracle whose equality the pages' method implies; the
mutation tests at the end plant plausible mistakes in a copy of the oracle's logic and show that these
pins catch them.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oatt
from oracle import slots as oslots
import workloads


def _paged_from_logical(rng, k_seqs, v_seqs, block_size, num_blocks):
    """Place logical per-sequence K/V rows in a NaN-filled paged cache under a random block permutation,
    using the oracle's own slot_mapping and store."""
    hkv, hd = k_seqs[0].shape[1:]
    need = [math.ceil(len(k) / block_size) for k in k_seqs]
    perm = rng.permutation(num_blocks)
    bt = np.full((len(k_seqs), max(max(need), 1) + 1), -1, np.int32)
    pos = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    lens = [len(k) for k in k_seqs]
    cu = np.concatenate([[0], np.cumsum(lens)])
    slots = oracle.slot_mapping_ref(bt, block_size, int(cu[-1]), cu_seqlens_q=cu)
    kc = np.full((num_blocks, block_size, hkv, hd), np.nan)
    vc = np.full((num_blocks, block_size, hkv, hd), np.nan)
    kc, vc = oracle.store_ref(np.concatenate(k_seqs), np.concatenate(v_seqs), kc, vc, slots)
    return kc, vc, bt, cu


def _random_seqs(rng, lens, hkv, hd):
    return ([rng.standard_normal((n, hkv, hd)) for n in lens], [rng.standard_normal((n, hkv, hd)) for n in lens])


# ---------------------------------------------------------------- brute force and a textbook routine

def _brute_force(q, kc, vc, bt, lq, lk, bs, scale, causal):
    """Direct evaluation with scalar loops: walk each sequence's block table cell by cell."""
    hq, hd = q.shape[1], q.shape[2]
    hkv = kc.shape[2]
    out = np.zeros_like(q)
    row0 = 0
    for b in range(len(lq)):
        keys = []
        for blk_idx in range(math.ceil(lk[b] / bs)):
            for cell in range(bs):
                if blk_idx * bs + cell < lk[b]:
                    keys.append((int(bt[b][blk_idx]), cell))
        for i in range(lq[b]):
            last = lk[b] - lq[b] + i if causal else lk[b] - 1
            for h in range(hq):
                g = h * hkv // hq
                scores = []
                for j, (blk, cell) in enumerate(keys[: last + 1]):
                    scores.append(scale * sum(q[row0 + i, h, d] * kc[blk, cell, g, d] for d in range(hd)))
                if not scores:
                    continue
                top = max(scores)
                ws = [math.exp(s - top) for s in scores]
                tot = sum(ws)
                for d in range(hd):
                    out[row0 + i, h, d] = sum(w * vc[blk, cell, g, d] for w, (blk, cell) in zip(ws, keys)) / tot
        row0 += lq[b]
    return out


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_tiny_random(seed):
    rng = np.random.default_rng(100 + seed)
    bs = int(rng.integers(1, 5))
    hkv = int(rng.integers(1, 3))
    hq = hkv * int(rng.integers(1, 3))
    hd = int(rng.choice([1, 2, 16]))
    nb = int(rng.integers(1, 4))
    lk = [int(x) for x in rng.integers(0, 10, nb)]
    lq = [int(rng.integers(0, n + 1)) for n in lk]
    causal = bool(rng.integers(0, 2))
    k_seqs, v_seqs = _random_seqs(rng, lk, hkv, hd)
    kc, vc, bt, _ = _paged_from_logical(rng, k_seqs, v_seqs, bs, sum(math.ceil(n / bs) for n in lk) + 2)
    q = rng.standard_normal((sum(lq), hq, hd))
    scale = float(rng.uniform(0.1, 1.0))
    cu_q = np.concatenate([[0], np.cumsum(lq)])
    cu_k = np.concatenate([[0], np.cumsum(lk)])
    got = oracle.attention_ref(q, kc, vc, cu_q, cu_k, scale, causal=causal, block_tables=bt, block_size=bs)
    want = _brute_force(q, kc, vc, bt, lq, lk, bs, scale, causal)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("seed", range(4))
def test_matches_textbook_sdpa_with_bottom_right_mask(seed):
    rng = np.random.default_rng(200 + seed)
    lq, lk, hq, hkv, hd = 5, 11, 4, 2, 16
    q = rng.standard_normal((lq, hq, hd))
    k = rng.standard_normal((lk, hkv, hd))
    v = rng.standard_normal((lk, hkv, hd))
    scale = 1 / math.sqrt(hd)
    got = oracle.attention_ref(q, k, v, [0, lq], [0, lk], scale)
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(np.repeat(k, hq // hkv, axis=1)).permute(1, 0, 2)
    vt = torch.from_numpy(np.repeat(v, hq // hkv, axis=1)).permute(1, 0, 2)
    mask = torch.ones(lq, lk, dtype=torch.bool).tril(diagonal=lk - lq)
    want = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    np.testing.assert_allclose(got, want.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("bs", [1, 3, 4, 16])
def test_paged_equals_contiguous(bs):
    rng = np.random.default_rng(bs)
    lens = [13, 1, 30, 7]
    k_seqs, v_seqs = _random_seqs(rng, lens, 2, 8)
    kc, vc, bt, cu = _paged_from_logical(rng, k_seqs, v_seqs, bs, sum(math.ceil(n / bs) for n in lens) + 3)
    q = rng.standard_normal((int(cu[-1]), 4, 8))
    contiguous = oracle.attention_ref(q, np.concatenate(k_seqs), np.concatenate(v_seqs), cu, cu, 0.35)
    paged = oracle.attention_ref(q, kc, vc, cu, cu, 0.35, block_tables=bt, block_size=bs)
    np.testing.assert_allclose(paged, contiguous, rtol=1e-13, atol=1e-14)
    assert np.all(np.isfinite(paged))  # no poisoned cell was read


def test_decode_equals_last_prefill_row():
    rng = np.random.default_rng(11)
    lens, bs = [9, 17, 4], 4
    k_seqs, v_seqs = _random_seqs(rng, lens, 2, 8)
    kc, vc, bt, cu = _paged_from_logical(rng, k_seqs, v_seqs, bs, 16)
    q = rng.standard_normal((int(cu[-1]), 4, 8))
    full = oracle.attention_ref(q, kc, vc, cu, cu, 0.4, block_tables=bt, block_size=bs)
    last_rows = cu[1:] - 1
    dec = oracle.decode_ref(q[last_rows], kc, vc, lens, bt, bs, 0.4)
    np.testing.assert_allclose(dec, full[last_rows], rtol=1e-13, atol=1e-14)


def test_chunked_prefill_rows_equal_full_prefill_rows():
    rng = np.random.default_rng(12)
    lens, chunks, bs = [20, 9, 33], [5, 9, 1], 8
    k_seqs, v_seqs = _random_seqs(rng, lens, 2, 8)
    kc, vc, bt, cu = _paged_from_logical(rng, k_seqs, v_seqs, bs, 16)
    q = rng.standard_normal((int(cu[-1]), 4, 8))
    full = oracle.attention_ref(q, kc, vc, cu, cu, 0.3, block_tables=bt, block_size=bs)
    rows = np.concatenate([np.arange(cu[b + 1] - c, cu[b + 1]) for b, c in enumerate(chunks)])
    cu_q = np.concatenate([[0], np.cumsum(chunks)])
    part = oracle.attention_ref(q[rows], kc, vc, cu_q, cu, 0.3, block_tables=bt, block_size=bs)
    np.testing.assert_allclose(part, full[rows], rtol=1e-13, atol=1e-14)


def test_moving_physical_blocks_leaves_output_unchanged():
    rng = np.random.default_rng(13)
    lens, bs = [10, 6], 4
    k_seqs, v_seqs = _random_seqs(rng, lens, 1, 4)
    kc, vc, bt, cu = _paged_from_logical(rng, k_seqs, v_seqs, bs, 8)
    q = rng.standard_normal((int(cu[-1]), 2, 4))
    base = oracle.attention_ref(q, kc, vc, cu, cu, 0.5, block_tables=bt, block_size=bs)
    perm = rng.permutation(8)  # block b moves to perm[b]
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1)
    moved = oracle.attention_ref(q, kc2, vc2, cu, cu, 0.5, block_tables=bt2, block_size=bs)
    np.testing.assert_array_equal(moved, base)


def test_gqa_equals_mha_with_replicated_kv():
    rng = np.random.default_rng(14)
    hq, hkv, L = 8, 2, 12
    q = rng.standard_normal((L, hq, 8))
    k = rng.standard_normal((L, hkv, 8))
    v = rng.standard_normal((L, hkv, 8))
    gqa = oracle.attention_ref(q, k, v, [0, L], [0, L], 0.3)
    rep = [h // (hq // hkv) for h in range(hq)]  # consecutive groups share a kv head
    mha = oracle.attention_ref(q, k[:, rep], v[:, rep], [0, L], [0, L], 0.3)
    np.testing.assert_array_equal(gqa, mha)


def test_slot_mapping_forms_agree_random():
    rng = np.random.default_rng(15)
    for _ in range(300):
        bs = int(rng.integers(1, 9))
        lk = int(rng.integers(1, 50))
        cached = int(rng.integers(0, lk))
        row = rng.permutation(100)[: math.ceil(lk / bs)]
        walk = oracle.slot_mapping_block_walk(row, cached, lk, bs)
        closed = [oslots._slot_of_position(row, p, bs) for p in range(cached, lk)]
        assert walk == closed
        assert len(set(walk)) == len(walk)


def test_slot_mapping_padding_rows_and_decode_padding():
    bt = np.array([[3, 5], [-1, -1]], np.int32)
    sm = oracle.slot_mapping_ref(bt, 4, 6, cu_seqlens_q=[0, 3, 3])
    assert sm.tolist() == [12, 13, 14, -1, -1, -1]
    sm = oracle.slot_mapping_ref(bt, 4, 3, context_lens=[6, 0])
    assert sm.tolist() == [21, -1, -1]


@pytest.mark.parametrize("seed", range(5))
def test_split_merge_equals_whole(seed):
    rng = np.random.default_rng(300 + seed)
    n = int(rng.integers(1, 200))
    s = rng.standard_normal(n) * 4
    v = rng.standard_normal((n, 16))
    cuts = np.sort(rng.choice(np.arange(1, n), size=min(5, n - 1), replace=False)) if n > 1 else []
    parts = np.split(np.arange(n), cuts)
    partials = []
    for p in parts:
        m = s[p].max()
        w = np.exp(s[p] - m)
        partials.append((m, w.sum(), w @ v[p]))
    partials.append((-np.inf, 0.0, np.zeros(16)))  # an empty split
    m, l, o = oracle.merge_partials(partials)
    w = np.exp(s - s.max())
    np.testing.assert_allclose(o / l, (w @ v) / w.sum(), rtol=1e-12, atol=1e-14)
    lens = [len(p) for p in parts]
    o2, _ = oracle.online_softmax_blocks(s, v, lens)
    np.testing.assert_allclose(o2, (w @ v) / w.sum(), rtol=1e-12, atol=1e-14)


def test_tiny_fp32_layer_end_to_end_consistency():
    """The tiny fp32 layer through the oracle: store, prefill and decode agree with the contiguous definition."""
    pre = workloads.tiny_fp32_prefill()
    dec = workloads.tiny_fp32_decode(pre)
    cache = workloads.nan_cache_host(pre.num_blocks, pre.block_size, 2, 16, "f32")
    sm = oracle.slot_mapping_ref(pre.block_tables, pre.block_size, 9, cu_seqlens_q=pre.cu_seqlens_q)
    kc, vc = oracle.store_ref(pre.k, pre.v, cache, cache, sm)
    f = lambda x: oracle.as_f64(x, "f32")
    cont = oracle.attention_ref(f(pre.q), f(pre.k), f(pre.v), pre.cu_seqlens_q, pre.cu_seqlens_k, pre.scale)
    paged = oracle.attention_ref(f(pre.q), f(kc), f(vc), pre.cu_seqlens_q, pre.cu_seqlens_k, pre.scale,
                                 block_tables=pre.block_tables, block_size=pre.block_size)
    np.testing.assert_allclose(paged, cont, rtol=1e-13, atol=1e-14)
    sm_d = oracle.slot_mapping_ref(dec.block_tables, dec.block_size, 2, context_lens=dec.context_lens)
    bt = pre.block_tables
    assert sm_d.tolist() == [int(bt[0, 1]) * 4 + 2, int(bt[1, 0]) * 4 + 3]
    kc2, vc2 = oracle.store_ref(dec.k, dec.v, kc, vc, sm_d)
    out = oracle.decode_ref(f(dec.q), f(kc2), f(vc2), dec.context_lens, dec.block_tables, 4, dec.scale)
    # decode == full causal prefill over the 7 + 4 tokens, last row of each sequence
    kk = [np.concatenate([pre.k[0:6], dec.k[0:1]]), np.concatenate([pre.k[6:9], dec.k[1:2]])]
    vv = [np.concatenate([pre.v[0:6], dec.v[0:1]]), np.concatenate([pre.v[6:9], dec.v[1:2]])]
    for b in range(2):
        L = len(kk[b])
        qq = np.zeros((L, 4, 16)); qq[-1] = f(dec.q[b])
        full = oracle.attention_ref(qq, f(kk[b]), f(vv[b]), [0, L], [0, L], dec.scale)
        np.testing.assert_allclose(out[b], full[-1], rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- planted mistakes are caught

def _sdpa_pin_passes():
    try:
        test_matches_textbook_sdpa_with_bottom_right_mask(0)
        test_single_key_pin()
        return True
    except AssertionError:
        return False


def test_single_key_pin():
    rng = np.random.default_rng(3)
    q, k, v = rng.standard_normal((3, 4, 8)), rng.standard_normal((3, 2, 8)), rng.standard_normal((3, 2, 8))
    out = oracle.attention_ref(q, k, v, [0, 1, 2, 3], [0, 1, 2, 3], 0.3)
    for b in range(3):
        for h in range(4):
            assert np.array_equal(out[b, h], v[b, h // 2])


def test_planted_mistakes_are_caught(monkeypatch):
    good = oatt._attend_one_head

    def off_by_one_causal(q_rows, k_rows, v_rows, scale, causal, first_pos):
        return good(q_rows, k_rows, v_rows, scale, causal, first_pos - 1)

    def top_left_alignment(q_rows, k_rows, v_rows, scale, causal, first_pos):
        return good(q_rows, k_rows, v_rows, scale, causal, 0)

    def scale_dropped(q_rows, k_rows, v_rows, scale, causal, first_pos):
        return good(q_rows, k_rows, v_rows, 1.0, causal, first_pos)

    def transposed_kv(q_rows, k_rows, v_rows, scale, causal, first_pos):
        return good(q_rows, v_rows, k_rows, scale, causal, first_pos)

    for bad in (off_by_one_causal, top_left_alignment, scale_dropped, transposed_kv):
        monkeypatch.setattr(oatt, "_attend_one_head", bad)
        assert not _sdpa_pin_passes(), bad.__name__
    monkeypatch.setattr(oatt, "_attend_one_head", good)
    assert _sdpa_pin_passes()

    # an interleaved head map instead of consecutive groups
    monkeypatch.setattr(oatt, "kv_head_of", lambda h, hq, hkv: h % hkv)
    with pytest.raises(AssertionError):
        test_gqa_equals_mha_with_replicated_kv()
    monkeypatch.undo()

    # a slot formula that drops the in-block offset of the first block
    orig = oslots._slot_of_position
    monkeypatch.setattr(oslots, "_slot_of_position", lambda row, p, bs: orig(row, p - p % bs, bs))
    from conftest import load_golden
    g = load_golden("slot_mapping_exercise_a.json")
    with pytest.raises(AssertionError):
        sm = oracle.slot_mapping_ref(np.array([g["block_table"]]), 4, 6, cu_seqlens_q=[0, 6])
        assert sm.tolist() == g["cases"][0]["slots_expected"]
