"""Attention over contiguous or paged K/V: varlen causal prefill and paged decode (oracle; test infrastructure only).

Definition [P2 §5.2, first paragraph]: for one query row and one head, ``o = softmax(scale * q . K^T) V``
over the keys the row may see.  The row maximum is subtracted before exponentiating, which leaves the
weights unchanged (shift invariance) and keeps every exponent <= 0 [P2 §5.2 ②].

Which keys a row sees:

* varlen prefill: sequence ``b`` owns query rows ``[cu_q[b], cu_q[b+1])`` and key rows
  ``[cu_k[b], cu_k[b+1])``; attention never crosses sequences (block-diagonal) and is causal inside a
  sequence [P2 §5.3; P1 Q6 §3];
* prefix-cache / chunked prefill: keys are read from the paged cache through the block table and the key
  length exceeds the query length [P2 §5.3 prefix branch; P3 §4 point 3];
* decode: one query per sequence reads ``context_lens[b]`` keys from the paged cache through the block
  table [P2 §5.3; P3 §4 point 2].

Readings (where the pages are silent or loose):

* causal alignment is bottom-right: the ``Lq`` queries are the last ``Lq`` of the ``Lk`` positions, so
  query ``i`` sits at absolute position ``Lk - Lq + i`` and sees keys ``0 .. Lk - Lq + i``.  This is the
  only alignment under which the new tokens are the newest positions [P2 §5.3 prefix branch] and decode
  step ``t`` sees position ``t`` itself [P3 §4 note];
* query head ``h`` reads kv head ``h // (num_q_heads // num_kv_heads)`` (consecutive groups) [P2 §3];
* a row that sees no key (``Lk == 0``, or a query placed before position 0) is all zeros.

Arrays are float64; callers widen stored bf16/f32 data with ``oracle.bf16.as_f64`` first.
"""

import numpy as np


def kv_head_of(h, num_q_heads, num_kv_heads):
    """The kv head that query head ``h`` shares with its group [P2 §3: groups of Hq/Hkv consecutive heads]."""
    assert num_q_heads % num_kv_heads == 0
    group = num_q_heads // num_kv_heads
    return h // group


def gather_logical_kv(cache, block_table_row, length, block_size):
    """Logical rows ``0 .. length-1`` of one sequence from a paged cache ``[num_blocks, bs, ...]``.

    Position ``j`` lives in cell ``j % block_size`` of physical block ``block_table_row[j // block_size]``
    [P3 §2; P2 §5.3 decode call].
    """
    rows = []
    for j in range(length):
        blk = int(block_table_row[j // block_size])
        rows.append(cache[blk, j % block_size])
    if not rows:
        return np.zeros((0,) + cache.shape[2:], dtype=cache.dtype)
    return np.stack(rows)


def _attend_one_head(q_rows, k_rows, v_rows, scale, causal, first_pos):
    """Softmax attention for one head of one sequence.

    ``q_rows [Lq, d]``, ``k_rows [Lk, d]``, ``v_rows [Lk, dv]``; query ``i`` is at position ``first_pos + i``.
    """
    lq, lk = q_rows.shape[0], k_rows.shape[0]
    out = np.zeros((lq, v_rows.shape[1]), dtype=np.float64)
    if lq == 0 or lk == 0:
        return out
    s = scale * (q_rows @ k_rows.T)  # [Lq, Lk] scores
    for i in range(lq):
        visible = lk if not causal else min(lk, first_pos + i + 1)
        if visible <= 0:
            continue
        row = s[i, :visible]
        m = row.max()
        w = np.exp(row - m)
        out[i] = (w @ v_rows[:visible]) / w.sum()
    return out


def attention_ref(q, k, v, cu_seqlens_q, cu_seqlens_k, scale, causal=True, block_tables=None,
                  block_size=None):
    """Varlen attention; returns float64 ``[Nq, Hq, head_dim]``.

    ``q``: ``[Nq, Hq, d]``.  Contiguous mode (``block_tables is None``): ``k``, ``v`` are ``[Nk, Hkv, d]``
    indexed by ``cu_seqlens_k``.  Paged mode: ``k``, ``v`` are caches ``[num_blocks, bs, Hkv, d]`` and only
    the per-sequence key lengths ``cu_k[b+1] - cu_k[b]`` matter.
    """
    q = np.asarray(q, dtype=np.float64)
    cq = np.asarray(cu_seqlens_q, dtype=np.int64)
    ck = np.asarray(cu_seqlens_k, dtype=np.int64)
    num_q_heads = q.shape[1]
    num_kv_heads = k.shape[-2]
    out = np.zeros((q.shape[0], num_q_heads, v.shape[-1]), dtype=np.float64)
    for b in range(len(cq) - 1):
        q0, q1 = int(cq[b]), int(cq[b + 1])
        lq, lk = q1 - q0, int(ck[b + 1] - ck[b])
        if block_tables is None:
            kb = np.asarray(k[int(ck[b]):int(ck[b]) + lk], dtype=np.float64)
            vb = np.asarray(v[int(ck[b]):int(ck[b]) + lk], dtype=np.float64)
        else:
            kb = np.asarray(gather_logical_kv(k, block_tables[b], lk, block_size), dtype=np.float64)
            vb = np.asarray(gather_logical_kv(v, block_tables[b], lk, block_size), dtype=np.float64)
        for h in range(num_q_heads):
            g = kv_head_of(h, num_q_heads, num_kv_heads)
            out[q0:q1, h] = _attend_one_head(q[q0:q1, h], kb[:, g] if lk else np.zeros((0, q.shape[2])),
                                             vb[:, g] if lk else np.zeros((0, v.shape[-1])),
                                             scale, causal, lk - lq)
    return out


def decode_ref(q, k_cache, v_cache, context_lens, block_tables, block_size, scale):
    """Paged single-token decode; ``q [B, Hq, d]`` -> float64 ``[B, Hq, d]``.

    Equivalent to a paged prefill with one query per sequence and ``Lk = context_lens[b]``; the query is at
    position ``Lk - 1`` and sees every cached key, itself included [P3 §4 note].
    """
    ctx = np.maximum(np.asarray(context_lens, dtype=np.int64), 0)
    batch = q.shape[0]
    cu_q = np.arange(batch + 1, dtype=np.int64)
    cu_k = np.concatenate([[0], np.cumsum(ctx)])
    return attention_ref(q, k_cache, v_cache, cu_q, cu_k, scale, causal=True, block_tables=block_tables,
                         block_size=block_size)


def online_softmax_blocks(scores, values, block_lengths):
    """Run the three accumulators (m, l, O-bar) over consecutive key blocks of one row [P2 §5.2 ②].

    ``scores [L]`` are already scaled; ``values [L]`` or ``[L, dv]``.  For each block the running maximum is
    raised to cover it, the old sums are multiplied by ``exp(m_old - m_new)`` (exact, because
    ``exp(a - c) = exp(a - b) * exp(b - c)``), and the block's own terms are added.  Returns
    ``(O, trajectory)`` with ``O = O-bar / l`` and one dict per block holding the rescale factor, the
    rescaled sums and the updated sums.
    """
    s = np.asarray(scores, dtype=np.float64)
    v = np.asarray(values, dtype=np.float64)
    m = -np.inf
    l = 0.0
    o = np.zeros(v.shape[1:], dtype=np.float64)
    traj = []
    start = 0
    for n in block_lengths:
        blk_s, blk_v = s[start:start + n], v[start:start + n]
        start += n
        m_new = max(m, float(blk_s.max()))
        alpha = 0.0 if m == -np.inf else float(np.exp(m - m_new))
        l_rescaled, o_rescaled = l * alpha, o * alpha
        w = np.exp(blk_s - m_new)
        l = l_rescaled + w.sum()
        o = o_rescaled + np.tensordot(w, blk_v, axes=(0, 0))
        m = m_new
        traj.append({"m": m, "rescale": alpha, "l_rescaled": l_rescaled, "o_rescaled": o_rescaled,
                     "l": l, "o": o.copy()})
    assert start == len(s)
    return o / l, traj


def merge_partials(partials):
    """Merge partial softmax states ``(m_i, l_i, O-bar_i)`` taken over disjoint key sets.

    The same factorisation as the online update [P2 §5.2 ②]: bring every partial to the common maximum
    ``m = max m_i`` by ``exp(m_i - m)``, then add.  Partials over no keys (``l_i == 0``) contribute nothing.
    Returns ``(m, l, O-bar)``; the output is ``O-bar / l``.
    """
    live = [(m_i, l_i, np.asarray(o_i, dtype=np.float64)) for m_i, l_i, o_i in partials if l_i > 0]
    if not live:
        return -np.inf, 0.0, None
    m = max(p[0] for p in live)
    l = sum(l_i * np.exp(m_i - m) for m_i, l_i, _ in live)
    o = sum(o_i * np.exp(m_i - m) for m_i, _, o_i in live)
    return m, l, o
