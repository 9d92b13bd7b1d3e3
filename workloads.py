"""Seeded synthetic inputs for the paged-KV attention hot path.

Shared by the tests, ``bench.py`` and the smoke check: it is the only module both the CPU oracle side and
the HIP side take data from.  It draws data and metadata and nothing else -- no slot arithmetic, no
scatter, no attention: every step of the method is computed separately by the oracle and by the kernels.

Recipe (all seeded; ``seed`` is the workload number unless a test says otherwise):

* draws happen in the order lengths -> block permutation -> new-token tensors (q, k, v) -> history;
* each sequence takes ``ceil(Lk / block_size)`` physical blocks, handed out consecutively from a seeded
  permutation of the cache's blocks; block-table rows are padded with -1;
* tensors are N(0, 1) drawn in float32; bf16 tensors are those values rounded to nearest-even;
* "history" holds the K/V of positions that were cached before this step, as logical rows per sequence
  (``[sum(Lk - Lq), Hkv, hd]``, sequences back to back); how it reaches the cache is up to each side;
* cache memory not covered by history or new tokens is filled with a quiet-NaN pattern, so a read of a
  stale slot shows up as NaN.

Host (``device="cpu"``) cases use NumPy's PCG64 and return NumPy arrays (bf16 as raw ``uint16`` bits);
large device cases use torch's generator on the device and return torch tensors.  Both are deterministic
for a given seed, but they are different streams.
"""

from dataclasses import dataclass, field
import math

import numpy as np

NAN_BITS = {"bf16": 0x7FC0, "f32": 0x7FC00000}

# The workloads, named by what they are (shapes of the Qwen3-0.6B attention layer: 16 q heads, 8 kv heads,
# head_dim 128, block_size 256, unless stated).
WORKLOADS = {
    "tiny_fp32": "tiny fp32 layer: 2 seqs of 6 and 3 tokens, block_size 4, 8 blocks, 4/2 heads, head_dim 16; "
                 "store + causal prefill, then one decode step per sequence",
    "decode_batch64": "decode: batch 64, context_lens U[512,4096], block_size 256, 4096-block cache, "
                      "bf16 16/8/128; store one token per sequence then paged decode",
    "varlen_prefill_8seq": "varlen causal prefill: 8 seqs, lengths U[128,2048], bf16 16/8/128, block_size 256; "
                           "store all tokens then contiguous attention",
    "prefix_prefill_16seq": "prefix-cache / chunked prefill: 16 seqs, cached prefix U[256,4096] + new chunk "
                            "U[64,512], K/V read through block_tables, bf16 16/8/128",
    "long_decode_batch256": "padded long decode: batch 256 (last 32 rows padding, slot -1), context_lens "
                            "U[1024,32768], bf16 16/8/128; plus a store sweep of 16384 tokens into distinct "
                            "random slots",
}


def f32_to_bf16_bits(x):
    """Round float32 values to bf16 (nearest, ties to even); returns the raw 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    # 32-bit sums: only patterns >= 0xFFFF8000 (negative NaNs) wrap, and they give 0 either way, as the
    # 17-bit quotient 0x10000 of an exact sum would after the cast to 16 bits
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


@dataclass
class Case:
    """One step's inputs.  Integer metadata is always NumPy int32; tensors are NumPy (host cases) or torch
    (device cases).  ``Lq[b]`` new tokens of sequence ``b`` are its last positions out of ``Lk[b]``."""

    dtype: str                    # "bf16" or "f32"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    Lq: np.ndarray                # [B] new tokens per sequence (decode: 1 per batch row)
    Lk: np.ndarray                # [B] positions after this step (decode: context_lens, 0 = padding)
    cu_seqlens_q: np.ndarray      # [B+1]
    cu_seqlens_k: np.ndarray      # [B+1]
    cu_hist: np.ndarray           # [B+1] offsets of each sequence's history rows
    block_tables: np.ndarray      # [B, max_blocks] padded with -1
    q: object = None              # [sum Lq, Hq, hd]
    k: object = None              # [sum Lq, Hkv, hd] new-token keys
    v: object = None
    hist_k: object = None         # [sum of cached lengths, Hkv, hd]
    hist_v: object = None
    decode: bool = False          # one query per sequence, context_lens = Lk
    extra: dict = field(default_factory=dict)

    @property
    def batch(self):
        return len(self.Lq)

    @property
    def max_blocks(self):
        return self.block_tables.shape[1]

    @property
    def context_lens(self):
        return self.Lk.astype(np.int32)


def _assign_blocks(rng, lk, block_size, num_blocks, max_blocks=None):
    need = [math.ceil(int(n) / block_size) for n in lk]
    assert sum(need) <= num_blocks, "cache too small for the workload"
    perm = rng.permutation(num_blocks)
    width = max_blocks if max_blocks is not None else max(max(need), 1)
    bt = np.full((len(lk), width), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    return bt


def _cumsum0(x):
    return np.concatenate([[0], np.cumsum(np.asarray(x, dtype=np.int64))]).astype(np.int32)


def _host_tensor(rng, shape, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


def _device_tensor(gen, shape, dtype, device):
    import torch
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def _build(Lq, Lk, hist, *, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, dtype, seed,
           device, decode, max_blocks, rng, scale):
    rng = rng if rng is not None else np.random.default_rng(seed)
    bt = _assign_blocks(rng, Lk, block_size, num_blocks, max_blocks)
    nq, nh = int(Lq.sum()), int(hist.sum())
    qs = (nq, num_q_heads, head_dim)
    ks = (nq, num_kv_heads, head_dim)
    hs = (nh, num_kv_heads, head_dim)
    if device == "cpu":
        q, k, v = (_host_tensor(rng, s, dtype) for s in (qs, ks, ks))
        hk, hv = (_host_tensor(rng, hs, dtype) for _ in range(2))
    else:
        import torch
        gen = torch.Generator(device=device)
        gen.manual_seed(int(rng.integers(0, 2**62)))
        q, k, v = (_device_tensor(gen, s, dtype, device) for s in (qs, ks, ks))
        hk, hv = (_device_tensor(gen, hs, dtype, device) for _ in range(2))
    return Case(dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                block_size=block_size, num_blocks=num_blocks,
                scale=scale if scale is not None else 1.0 / math.sqrt(head_dim),
                Lq=Lq.astype(np.int32), Lk=Lk.astype(np.int32), cu_seqlens_q=_cumsum0(Lq),
                cu_seqlens_k=_cumsum0(Lk), cu_hist=_cumsum0(hist), block_tables=bt, q=q, k=k, v=v,
                hist_k=hk, hist_v=hv, decode=decode)


def make_case(Lq, Lk, *, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, dtype, seed,
              device="cpu", max_blocks=None, rng=None, scale=None):
    """Prefill step from per-sequence lengths: ``Lq[b]`` new tokens after ``Lk[b] - Lq[b]`` cached ones."""
    Lq = np.asarray(Lq, dtype=np.int64)
    Lk = np.asarray(Lk, dtype=np.int64)
    assert np.all(Lk >= Lq) and np.all(Lq >= 0)
    return _build(Lq, Lk, Lk - Lq, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                  block_size=block_size, num_blocks=num_blocks, dtype=dtype, seed=seed, device=device,
                  decode=False, max_blocks=max_blocks, rng=rng, scale=scale)


def tiny_fp32_prefill(device="cpu", seed=1):
    """Tiny fp32 layer, prefill part: two prompts of 6 and 3 tokens, fp32, block_size 4, 8 blocks.

    The block tables come from ``permutation(8)``: sequence 0 takes two blocks, sequence 1 one block.
    """
    return make_case([6, 3], [6, 3], num_q_heads=4, num_kv_heads=2, head_dim=16, block_size=4,
                     num_blocks=8, dtype="f32", seed=seed, device=device, scale=0.25)


def tiny_fp32_decode(prefill, device="cpu", seed=101):
    """Tiny fp32 layer, decode part: one new token per sequence after ``prefill`` (context 7 and 4).

    The sequences keep the blocks of the prefill step (7 tokens still fit in 2 blocks of 4, 4 in 1).
    The history is exactly the prefill step's keys and values.
    """
    rng = np.random.default_rng(seed)
    ctx = prefill.Lk + 1
    assert np.all(np.ceil(ctx / prefill.block_size) <= (prefill.block_tables >= 0).sum(axis=1))
    shape_q = (prefill.batch, prefill.num_q_heads, prefill.head_dim)
    shape_k = (prefill.batch, prefill.num_kv_heads, prefill.head_dim)
    q = _host_tensor(rng, shape_q, prefill.dtype)
    k = _host_tensor(rng, shape_k, prefill.dtype)
    v = _host_tensor(rng, shape_k, prefill.dtype)
    return Case(dtype=prefill.dtype, num_q_heads=prefill.num_q_heads, num_kv_heads=prefill.num_kv_heads,
                head_dim=prefill.head_dim, block_size=prefill.block_size, num_blocks=prefill.num_blocks,
                scale=prefill.scale, Lq=np.ones(prefill.batch, np.int32), Lk=ctx.astype(np.int32),
                cu_seqlens_q=_cumsum0(np.ones(prefill.batch)), cu_seqlens_k=_cumsum0(ctx),
                cu_hist=prefill.cu_seqlens_k.copy(), block_tables=prefill.block_tables.copy(), q=q, k=k, v=v,
                hist_k=prefill.k, hist_v=prefill.v, decode=True)


def decode_case(context_lens, *, num_q_heads=16, num_kv_heads=8, head_dim=128, block_size=256,
                num_blocks=4096, dtype="bf16", seed=2, device="cpu", max_blocks=None, rng=None, scale=None):
    """Decode step: every batch row has one query and one new K/V row; sequence ``b`` holds
    ``context_lens[b] - 1`` cached tokens and writes its new one at position ``context_lens[b] - 1``.

    A context length of 0 marks a padding row: it owns no block (all -1), writes nothing (slot -1) and
    reads nothing.
    """
    ctx = np.asarray(context_lens, dtype=np.int64)
    assert np.all(ctx >= 0)
    ones = np.ones(len(ctx), dtype=np.int64)
    return _build(ones, ctx, np.maximum(ctx - 1, 0), num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                  head_dim=head_dim, block_size=block_size, num_blocks=num_blocks, dtype=dtype, seed=seed,
                  device=device, decode=True, max_blocks=max_blocks, rng=rng, scale=scale)


def decode_batch64(device="cpu", seed=2):
    rng = np.random.default_rng(seed)
    ctx = rng.integers(512, 4096, size=64, endpoint=True)
    return decode_case(ctx, num_blocks=4096, seed=seed, device=device, max_blocks=16, rng=rng)


def varlen_prefill_8seq(device="cpu", seed=3):
    rng = np.random.default_rng(seed)
    lens = rng.integers(128, 2048, size=8, endpoint=True)
    return make_case(lens, lens, num_q_heads=16, num_kv_heads=8, head_dim=128, block_size=256,
                     num_blocks=1024, dtype="bf16", seed=seed, device=device, rng=rng)


def prefix_prefill_16seq(device="cpu", seed=4):
    rng = np.random.default_rng(seed)
    prefix = rng.integers(256, 4096, size=16, endpoint=True)
    chunk = rng.integers(64, 512, size=16, endpoint=True)
    return make_case(chunk, prefix + chunk, num_q_heads=16, num_kv_heads=8, head_dim=128, block_size=256,
                     num_blocks=4096, dtype="bf16", seed=seed, device=device, max_blocks=18, rng=rng)


def chunked_prefill(chunks, prefixes, device="cpu", seed=6):
    """New-token chunks on long cached prefixes (chunked prefill: few query tiles over long key ranges), paged
    bf16 16/8/128 cache with block_size 256; the history is each sequence's cached prefix."""
    rng = np.random.default_rng(seed)
    chunks, prefixes = np.asarray(chunks, np.int64), np.asarray(prefixes, np.int64)
    lk = chunks + prefixes
    num_blocks = int(sum(-(-x // 256) for x in lk)) + 16
    return make_case(chunks, lk, num_q_heads=16, num_kv_heads=8, head_dim=128, block_size=256,
                     num_blocks=num_blocks, dtype="bf16", seed=seed, device=device, rng=rng)


def long_decode_batch256(device="cpu", seed=5):
    """224 real rows followed by 32 padding rows (context 0, slot -1, block row all -1)."""
    rng = np.random.default_rng(seed)
    ctx = np.concatenate([rng.integers(1024, 32768, size=224, endpoint=True), np.zeros(32, np.int64)])
    return decode_case(ctx, num_blocks=32768, seed=seed, device=device, max_blocks=128, rng=rng)


@dataclass
class StoreSweep:
    key: list          # per set: [N, Hkv, hd]
    value: list
    slots: list        # per set: int32 [N], distinct
    num_blocks: int
    block_size: int
    num_kv_heads: int
    head_dim: int
    dtype: str


def store_sweep(n_tokens=16384, *, n_sets=8, num_blocks=4096, block_size=256, num_kv_heads=8,
                head_dim=128, dtype="bf16", seed=5, device="cpu"):
    """Independent (key, value, slots) sets for the store bandwidth sweep; slots distinct per set.

    Eight sets of 64 MiB of K and V rows (512 MiB, twice the GPU's 256 MB last-level cache), used in turn, so no
    set's rows are still cached when it comes round again: the sweep reads them from HBM."""
    rng = np.random.default_rng(seed)
    num_slots = num_blocks * block_size
    slots = [rng.choice(num_slots, n_tokens, replace=False).astype(np.int32) for _ in range(n_sets)]
    shape = (n_tokens, num_kv_heads, head_dim)
    if device == "cpu":
        keys = [_host_tensor(rng, shape, dtype) for _ in range(n_sets)]
        vals = [_host_tensor(rng, shape, dtype) for _ in range(n_sets)]
    else:
        import torch
        gen = torch.Generator(device=device)
        gen.manual_seed(int(rng.integers(0, 2**62)))
        keys = [_device_tensor(gen, shape, dtype, device) for _ in range(n_sets)]
        vals = [_device_tensor(gen, shape, dtype, device) for _ in range(n_sets)]
    return StoreSweep(key=keys, value=vals, slots=slots, num_blocks=num_blocks, block_size=block_size,
                      num_kv_heads=num_kv_heads, head_dim=head_dim, dtype=dtype)


def nan_cache_host(num_blocks, block_size, num_kv_heads, head_dim, dtype):
    """A host cache image filled with the quiet-NaN pattern (bf16 as uint16 bits)."""
    shape = (num_blocks, block_size, num_kv_heads, head_dim)
    if dtype == "bf16":
        return np.full(shape, NAN_BITS["bf16"], dtype=np.uint16)
    return np.full(shape, NAN_BITS["f32"], dtype=np.uint32).view(np.float32)
