"""Pins of the attention sub-layer oracle (CPU only): a prompt run in one prefill step equals the same tokens run
one decode step at a time; identity weights reduce it to attention over the normalised, rotated inputs; and
planted mistakes in the composition fail."""

import numpy as np
import pytest

import oracle
import oracle.sublayer
from oracle.sublayer import sublayer_step_ref

HQ, HKV, HD = 4, 2, 16
HIDDEN = 24


def _weights(rng, hidden=HIDDEN):
    w_qkv = rng.standard_normal(((HQ + 2 * HKV) * HD, hidden)) / np.sqrt(hidden)
    wq = rng.uniform(0.8, 1.2, HD)
    wk = rng.uniform(0.8, 1.2, HD)
    w_o = rng.standard_normal((hidden, HQ * HD)) / np.sqrt(HQ * HD)
    return w_qkv, wq, wk, w_o


def _step(x, pos, hk, hv, w, scale=0.25):
    return sublayer_step_ref(x, pos, hk, hv, *w, HQ, HKV, HD, 1e-6, 1e4, scale)


def test_prefill_equals_token_by_token_decode():
    rng = np.random.default_rng(0)
    w = _weights(rng)
    x = rng.standard_normal((7, HIDDEN))
    empty = np.zeros((0, HKV, HD))
    y_prefill, k_all, v_all = _step(x, np.arange(7), empty, empty, w)
    hk, hv = empty, empty
    for t in range(7):
        y_t, hk, hv = _step(x[t:t + 1], [t], hk, hv, w)
        np.testing.assert_allclose(y_t[0], y_prefill[t], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(hk, k_all, atol=0)
    np.testing.assert_allclose(hv, v_all, atol=0)
    # chunked: 4 tokens, then 3 with the first 4 as history
    y_a, hk, hv = _step(x[:4], np.arange(4), empty, empty, w)
    y_b, _, _ = _step(x[4:], np.arange(4, 7), hk, hv, w)
    np.testing.assert_allclose(np.concatenate([y_a, y_b]), y_prefill, rtol=1e-12, atol=1e-12)


def test_identity_weights_reduce_to_attention_of_normalised_inputs():
    """hidden = Hq*hd and selection matrices: q = x, k = v = the first Hkv*hd columns; W_o = I."""
    rng = np.random.default_rng(1)
    hidden = HQ * HD
    x = rng.standard_normal((5, hidden))
    sel_q = np.eye(hidden)
    sel_kv = np.eye(HKV * HD, hidden)
    w_qkv = np.concatenate([sel_q, sel_kv, sel_kv])
    w = (w_qkv, np.ones(HD), np.ones(HD), np.eye(hidden))
    empty = np.zeros((0, HKV, HD))
    y, _, _ = sublayer_step_ref(x, np.arange(5), empty, empty, *w, HQ, HKV, HD, 0.0, 1e4, 0.25)
    q = x.reshape(5, HQ, HD)
    kv = x[:, :HKV * HD].reshape(5, HKV, HD)
    qn, kn = oracle.qk_norm_rope_ref(q, kv, np.arange(5), np.ones(HD), np.ones(HD), 0.0, 1e4)
    want = oracle.attention_ref(qn, kn, kv, [0, 5], [0, 5], 0.25).reshape(5, hidden)
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-12)
    # the first token sees only itself: its output rows are its own v
    np.testing.assert_allclose(want[0].reshape(HQ, HD)[0], kv[0, 0], atol=1e-12)


def test_planted_composition_mistakes_fail():
    rng = np.random.default_rng(2)
    w = _weights(rng)
    x = rng.standard_normal((6, HIDDEN))
    empty = np.zeros((0, HKV, HD))
    good, _, _ = _step(x, np.arange(6), empty, empty, w)
    # one token at the wrong position (a uniform shift would not show: RoPE only sees position differences)
    bad_pos, _, _ = _step(x, [0, 1, 2, 2, 4, 5], empty, empty, w)
    assert not np.allclose(bad_pos, good, atol=1e-6)
    shifted, _, _ = _step(x, np.arange(100, 106), empty, empty, w)
    np.testing.assert_allclose(shifted, good, rtol=1e-9, atol=1e-9)
    # q and k weights swapped
    swapped = (w[0], w[2], w[1], w[3])
    bad_w, _, _ = _step(x, np.arange(6), empty, empty, swapped)
    assert not np.allclose(bad_w, good, atol=1e-6)
    # k and v blocks of the merged projection swapped
    nq, nk = HQ * HD, HKV * HD
    w_kv = np.concatenate([w[0][:nq], w[0][nq + nk:], w[0][nq:nq + nk]])
    bad_split, _, _ = _step(x, np.arange(6), empty, empty, (w_kv,) + w[1:])
    assert not np.allclose(bad_split, good, atol=1e-6)


def _check_distinct_kv_split():
    """Identity weights in which q, k and v select different columns of x: q = x, k = x[:, :Hkv*hd],
    v = x[:, Hkv*hd:2*Hkv*hd], W_o = I.  The merged projection's rows are ordered [q | k | v] [P2 §3, the
    QKV split into q_size, kv_size, kv_size in that order], so the output must be attention over the
    normalised, rotated first block with the plain second block as values; in particular the first token,
    which sees only itself, returns exactly its own second block for every query head of the group."""
    rng = np.random.default_rng(3)
    hidden = HQ * HD
    nk = HKV * HD
    x = rng.standard_normal((5, hidden))
    sel_q = np.eye(hidden)
    sel_k = np.eye(nk, hidden)                      # columns 0 .. nk-1
    sel_v = np.eye(nk, hidden, k=nk)                # columns nk .. 2nk-1
    w_qkv = np.concatenate([sel_q, sel_k, sel_v])
    w = (w_qkv, np.ones(HD), np.ones(HD), np.eye(hidden))
    empty = np.zeros((0, HKV, HD))
    y, k_all, v_all = oracle.sublayer.sublayer_step_ref(x, np.arange(5), empty, empty, *w, HQ, HKV, HD, 0.0,
                                                        1e4, 0.25)
    k_in = x[:, :nk].reshape(5, HKV, HD)
    v_in = x[:, nk:2 * nk].reshape(5, HKV, HD)
    # the values the step leaves in the cache are the plain second block, bit for bit
    np.testing.assert_array_equal(v_all, v_in)
    # closed form: token 0 sees one key, so its output for q head h is v of kv head h // (Hq/Hkv)
    y0 = y[0].reshape(HQ, HD)
    for h in range(HQ):
        np.testing.assert_allclose(y0[h], v_in[0, h // (HQ // HKV)], rtol=0, atol=1e-12)
    # all rows: attention over the normalised, rotated first block, values the second block
    qn, kn = oracle.qk_norm_rope_ref(x.reshape(5, HQ, HD), k_in, np.arange(5), np.ones(HD), np.ones(HD), 0.0, 1e4)
    np.testing.assert_allclose(k_all, kn, rtol=0, atol=1e-12)
    want = oracle.attention_ref(qn, kn, v_in, [0, 5], [0, 5], 0.25).reshape(5, hidden)
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-12)


def test_identity_weights_distinct_k_and_v_blocks():
    _check_distinct_kv_split()


def test_planted_kv_split_swap_fails(monkeypatch):
    """The split order is pinned: an oracle that took the v block as k and the k block as v fails the pin."""
    good = oracle.sublayer.project_split_ref

    def swapped(*args, **kw):
        q, k, v = good(*args, **kw)
        return q, v, k

    monkeypatch.setattr(oracle.sublayer, "project_split_ref", swapped)
    with pytest.raises(AssertionError):
        _check_distinct_kv_split()
