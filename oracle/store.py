"""store_kvcache: scatter each new token's K/V row into the paged cache (oracle; test infrastructure only).

Token ``idx`` owns one row of ``D = num_kv_heads * head_dim`` elements in ``key`` and in ``value``; the
row is copied unchanged to cache slot ``slot_mapping[idx]``, whose elements are ``[slot * D, slot * D + D)``
of the flat cache, for K and for V with the same slot [P2 §5.1, the three changes from the skeleton;
P3 §3].  A slot of -1 marks a padding token and writes nothing [P2 §5.1 ②; P1 attention.py walkthrough].
Slots that nobody writes keep their previous bytes [P2 §5.1 4-token example].

Readings: every negative slot is skipped (only -1 ever occurs on the pages), a slot at or past the end of
the cache is skipped too, and if two tokens name the same slot the later token wins (the pages never
produce duplicates).
"""

import numpy as np


def scatter_rows_ref(src, slot, dst):
    """Row ``idx`` of ``src`` goes to row ``slot[idx]`` of ``dst`` (the teaching skeleton of P2 §5.1)."""
    out = np.array(dst, copy=True)
    for idx in range(len(slot)):
        out[int(slot[idx])] = src[idx]
    return out


def store_ref(key, value, k_cache, v_cache, slot_mapping):
    """Return ``(k_cache', v_cache')`` after storing ``key``/``value`` rows at ``slot_mapping``.

    ``key``/``value``: ``[N, num_kv_heads, head_dim]`` arrays (any row stride; the copy is by value).
    Caches: ``[num_blocks, block_size, num_kv_heads, head_dim]`` of the same element type (bf16 caches
    are handled as raw ``uint16`` patterns, so the copy is bit-exact).
    """
    key = np.asarray(key)
    value = np.asarray(value)
    n = key.shape[0]
    assert len(slot_mapping) == n
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    num_slots = kc.shape[0] * kc.shape[1]
    d = int(np.prod(kc.shape[2:]))
    kflat = kc.reshape(num_slots, d)
    vflat = vc.reshape(num_slots, d)
    for idx in range(n):
        slot = int(slot_mapping[idx])
        if slot < 0 or slot >= num_slots:
            continue
        kflat[slot] = key[idx].reshape(d)
        vflat[slot] = value[idx].reshape(d)
    return kc, vc
