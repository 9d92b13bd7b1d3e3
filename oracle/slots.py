"""slot_mapping: where each new token's K/V row goes in the paged cache (oracle; test infrastructure only).

The paged cache is one flat array of slots; slot ``blk * block_size + j`` is cell ``j`` of physical block
``blk`` [P3 "课程 04 · KV 到底写到了哪一格", §2].  A sequence's block table lists its physical blocks in
logical order, and slot_mapping is that table unrolled over the positions computed in this step, in batch
order [P3 §1 table; §2].  A padding entry is -1 [P2 §5.1; P1 Q6 §3].

Two independent forms are kept and cross-checked on every call:

* ``slot_mapping_block_walk`` walks the logical blocks a position range touches, where the first block may
  be entered mid-block and the last may be left mid-block [P3 §2];
* the per-position closed form ``block_table[p // block_size] * block_size + p % block_size``.

Readings where the pages are silent (all produce -1, i.e. "no slot"): a position below 0, a logical block
past the end of the table row, a negative block-table entry, and output rows past the last real token.
"""

import numpy as np


def slot_mapping_block_walk(block_table_row, start, end, block_size):
    """Slots for positions ``start .. end-1`` of one sequence, by walking its logical blocks [P3 §2].

    Positions ``[start, end)`` are new this step; ``start`` tokens are already cached.  Each logical block
    ``i`` that the range touches contributes the contiguous run of cells it covers, offset by that block's
    physical base ``block_table_row[i] * block_size``.
    """
    out = []
    if end <= start:
        return out
    first_block = start // block_size
    last_block = (end - 1) // block_size
    for i in range(first_block, last_block + 1):
        block_lo = i * block_size
        lo = max(start, block_lo)  # the first block may be entered mid-block
        hi = min(end, block_lo + block_size)  # the last block may be left mid-block
        base = int(block_table_row[i]) * block_size
        out.extend(range(base + (lo - block_lo), base + (hi - block_lo)))
    return out


def _slot_of_position(block_table_row, p, block_size):
    """Closed form for one position; -1 where no slot exists (see module docstring)."""
    if p < 0:
        return -1
    i = p // block_size
    if i >= len(block_table_row):
        return -1
    blk = int(block_table_row[i])
    if blk < 0:
        return -1
    return blk * block_size + p % block_size


def slot_mapping_ref(block_tables, block_size, num_tokens, cu_seqlens_q=None, cu_seqlens_k=None,
                     context_lens=None):
    """slot_mapping for one step, as int32 ``[num_tokens]``.

    Prefill (``context_lens is None``): sequence ``b`` owns query rows ``[cu_q[b], cu_q[b+1])``; its key
    length is ``cu_k[b+1] - cu_k[b]`` (equal to the query length when ``cu_seqlens_k`` is None).  Its new
    tokens are the last ``Lq`` of its ``Lk`` positions, so they sit at positions ``Lk - Lq .. Lk - 1``
    [P2 §5.3 prefix-cache branch; P1 Q6 §3; P3 §7 chunked second pass].

    Decode (``context_lens`` given): one token per sequence at position ``context_lens[b] - 1``; the
    context length already counts the token being written [P3 §4 note; §9 exercise C].

    Rows ``>= `` the number of real tokens are padding and get -1.
    """
    bt = np.asarray(block_tables)
    out = np.full(num_tokens, -1, dtype=np.int64)
    if context_lens is not None:
        ctx = np.asarray(context_lens)
        ranges = [(int(c) - 1, int(c)) for c in ctx]
    else:
        cq = np.asarray(cu_seqlens_q)
        ck = cq if cu_seqlens_k is None else np.asarray(cu_seqlens_k)
        ranges = []
        for b in range(len(cq) - 1):
            lq = int(cq[b + 1] - cq[b])
            lk = int(ck[b + 1] - ck[b])
            ranges.append((lk - lq, lk))
    row = 0
    for b, (start, end) in enumerate(ranges):
        closed = [_slot_of_position(bt[b], p, block_size) for p in range(start, end)]
        # Cross-check with the block walk wherever every position has a slot.
        if start >= 0 and all(s >= 0 for s in closed):
            walk = slot_mapping_block_walk(bt[b], start, end, block_size)
            assert walk == closed, (b, walk, closed)
        for s in closed:
            if row < num_tokens:
                out[row] = s
            row += 1
    return out.astype(np.int32)


def decode_slot_ref(block_table_row, context_len, block_size):
    """Decode slot by the last-block formula [P3 §9 exercise C, question 1].

    The sequence owns exactly ``ceil(context_len / block_size)`` blocks, listed in ``block_table_row``;
    the new token is the last of the ``last_block_num_tokens`` tokens held by the last block, so its slot
    is ``last_block * block_size + last_block_num_tokens - 1``.
    """
    row = list(block_table_row)
    n_blocks = len(row)
    last_block_num_tokens = context_len - (n_blocks - 1) * block_size
    assert 1 <= last_block_num_tokens <= block_size, "table must hold exactly the blocks in use"
    return int(row[-1]) * block_size + last_block_num_tokens - 1
