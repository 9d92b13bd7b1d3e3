"""The Qwen3 attention sub-layer around the hot path, with synthetic (seeded random) weights.

The seven steps of the sub-layer [P2 §2; P1 attention.py walkthrough]: the merged qkv projection, the split into
q / k / v views, QK-Norm and RoPE, the store into the paged cache, attention (varlen causal prefill or paged
decode), and the output projection after flattening the heads [P2 §6].  The two projections are plain dense
GEMMs, run by the platform BLAS (hipBLASLt through torch); everything between them runs in this library's
kernels: ``kv_store_qk_norm_rope`` (steps 4-6a, one pass), then ``attn_prefill_varlen`` over the paged cache or
``attn_decode_paged``.  The page's trained Qwen3-0.6B weights are not used: the weights are drawn from a seeded
generator, scaled by 1/sqrt(fan-in) so activations stay of unit size.

(Page: [P2] www.yeyulingfeng.com/a/738130.html; [P1] m.demingchina.com/news/18656.)
"""

import math

import torch

from . import _lib as L


class AttentionSublayer:
    """One attention sub-layer: ``prefill`` for a varlen batch of new tokens, ``decode`` for one token per row.

    The caches are ``[num_blocks, block_size, num_kv_heads, head_dim]`` bf16, shared with the caller; keys are
    stored normalised and rotated, as the attention reads them.
    """

    def __init__(self, hidden_size=1024, num_q_heads=16, num_kv_heads=8, head_dim=128, eps=1e-6, rope_theta=1e6,
                 seed=0, device="cuda"):
        self.hidden, self.hq, self.hkv, self.hd = hidden_size, num_q_heads, num_kv_heads, head_dim
        self.eps, self.theta = float(eps), float(rope_theta)
        self.scale = head_dim ** -0.5
        gen = torch.Generator(device=device)
        gen.manual_seed(seed)
        qkv_out = (num_q_heads + 2 * num_kv_heads) * head_dim
        bf = torch.bfloat16

        def draw(*shape, std):
            return (torch.randn(shape, generator=gen, device=device) * std).to(bf)

        self.w_qkv = draw(qkv_out, hidden_size, std=1.0 / math.sqrt(hidden_size))
        self.q_norm_weight = (1.0 + draw(head_dim, std=0.1).float()).to(bf)
        self.k_norm_weight = (1.0 + draw(head_dim, std=0.1).float()).to(bf)
        self.w_o = draw(hidden_size, num_q_heads * head_dim, std=1.0 / math.sqrt(num_q_heads * head_dim))

    def _project(self, x):
        """qkv projection and the split into q, k, v views of the one [N, (Hq + 2 Hkv) hd] result (no copy)."""
        n = x.shape[0]
        qkv = torch.nn.functional.linear(x, self.w_qkv)
        nq, nk = self.hq * self.hd, self.hkv * self.hd
        q = qkv[:, :nq].view(n, self.hq, self.hd)
        k = qkv[:, nq:nq + nk].view(n, self.hkv, self.hd)
        v = qkv[:, nq + nk:].view(n, self.hkv, self.hd)
        return q, k, v

    def prefill(self, x, positions, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, block_tables, k_cache,
                v_cache, slot_mapping=None):
        """``x [N, hidden]`` bf16: the new tokens of a varlen batch, ``positions [N]`` int32 their positions in
        their sequences (the last ``Lq`` of each sequence's ``Lk``).  Keys are read back from the paged cache,
        so cached prefixes (``cu_seqlens_k != cu_seqlens_q``) work as they are."""
        n = x.shape[0]
        q, k, v = self._project(x)
        bs = k_cache.shape[1]
        if slot_mapping is None:
            slot_mapping = L.kv_slot_mapping(block_tables, bs, n, cu_seqlens_q=cu_seqlens_q,
                                             cu_seqlens_k=cu_seqlens_k)
        q_rot = L.kv_store_qk_norm_rope(q, k, v, positions, self.q_norm_weight, self.k_norm_weight, k_cache, v_cache,
                                        slot_mapping, eps=self.eps, rope_theta=self.theta)
        o = L.attn_prefill_varlen(q_rot, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                                  self.scale, causal=True, block_table=block_tables)
        return torch.nn.functional.linear(o.view(n, self.hq * self.hd), self.w_o)

    def decode(self, x, context_lens, block_tables, k_cache, v_cache, workspace=None):
        """``x [B, hidden]``: one new token per row, at position ``context_lens[b] - 1`` (rows with context 0 are
        padding: nothing is stored, their output is the projection of a zero attention row)."""
        b = x.shape[0]
        q, k, v = self._project(x)
        bs = k_cache.shape[1]
        positions = (context_lens - 1).clamp_min(0)
        slot_mapping = L.kv_slot_mapping(block_tables, bs, b, context_lens=context_lens)
        q_rot = L.kv_store_qk_norm_rope(q, k, v, positions, self.q_norm_weight, self.k_norm_weight, k_cache, v_cache,
                                        slot_mapping, eps=self.eps, rope_theta=self.theta)
        o = L.attn_decode_paged(q_rot, k_cache, v_cache, context_lens, block_tables, self.scale, workspace=workspace)
        return torch.nn.functional.linear(o.view(b, self.hq * self.hd), self.w_o)
