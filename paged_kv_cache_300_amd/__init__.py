"""Paged-KV attention hot path for AMD Instinct MI355X (gfx950): Python binding of ``libpagedkv.so``.

The binding only marshals arguments: it checks tensor shapes and strides, allocates outputs with torch
(device memory) and passes raw pointers plus torch's current stream to the C ABI declared in
``include/pagedkv.h``.  Every step of the path runs in the library's HIP kernels; there is no fallback,
and a missing or unloadable library raises ``RuntimeError``.

Function names and argument order follow the calls described for nano-vLLM's attention layer:
``kv_store(key, value, k_cache, v_cache, slot_mapping)`` is store_kvcache [P2 §5.1],
``attn_prefill_varlen`` mirrors the varlen prefill call and ``attn_decode_paged`` the paged decode call
[P2 §5.3; P3 §4].  (Pages: [P2] www.yeyulingfeng.com/a/738130.html, [P3]
diomchen.github.io/lessons/0004-attention-slot-mapping.html.)
"""

from ._lib import (
    PKV_F32,
    PKV_BF16,
    PagedKVError,
    lib,
    library_path,
    kv_slot_mapping,
    kv_store,
    kv_store_qk_norm_rope,
    attn_prefill_varlen,
    attn_prefill_workspace_bytes,
    attn_decode_workspace_bytes,
    attn_decode_paged,
    attn_decode_paged_store,
    attn_decode_paged_store_noalloc,
)
from .sublayer import AttentionSublayer

__all__ = [
    "PKV_F32",
    "PKV_BF16",
    "PagedKVError",
    "lib",
    "library_path",
    "kv_slot_mapping",
    "kv_store",
    "kv_store_qk_norm_rope",
    "attn_prefill_varlen",
    "attn_prefill_workspace_bytes",
    "attn_decode_workspace_bytes",
    "attn_decode_paged",
    "attn_decode_paged_store",
    "attn_decode_paged_store_noalloc",
    "AttentionSublayer",
]
