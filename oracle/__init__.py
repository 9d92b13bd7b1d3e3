"""CPU oracle for the paged-KV attention hot path (store scatter, varlen prefill, paged decode).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the package ``paged_kv_cache_300_amd``, its
HIP kernels or its C ABI) imports, links or runs this package; only ``tests/``, the ``smoke()`` of
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` do.  It shares no code, headers, tables
or helpers with the HIP path.

It is deliberately plain: NumPy, float64 arithmetic, one sequence and one head at a time, with no
blocking, fusion or reordering beyond what the definitions below state.  bf16 data arrives as its raw
16-bit patterns (``uint16``) and is widened exactly before any arithmetic.

Sources (three web pages on the attention layer of nano-vLLM; cited by tag, page title and section):

* [P1] "Nano-VLLM全代码解析笔记(5)-laynorm和attention", m.demingchina.com/news/18656
  -- the attention.py walkthrough and its questions Q1-Q6.
* [P2] nano-vllm lesson on the Qwen3 attention sub-layer, www.yeyulingfeng.com/a/738130.html
  -- §2 (the seven steps), §3 (GQA), §4 (QK-Norm and RoPE), §5.1 (store_kvcache), §5.2 (FlashAttention /
  online softmax), §5.3 (prefill / decode calls).
* [P3] "课程 04 · KV 到底写到了哪一格", diomchen.github.io/lessons/0004-attention-slot-mapping.html
  -- §1 (the five tensors), §2 (slot_mapping), §3 (the scatter kernel), §4 (the two attention calls),
  §7 (exercise A), §9 (exercise C).

Pins (see ``tests/test_oracle_*.py``): every function here is checked against values the pages print
(``tests/golden``), closed forms, invariants, a textbook routine and brute force.  No function is
"parity unpinned"; the one convention the pages leave open (which query heads share a kv head) is a
reading, stated in ``attention.kv_head_of``.
"""

from .bf16 import bf16_bits_to_f64, as_f64
from .slots import slot_mapping_block_walk, slot_mapping_ref, decode_slot_ref
from .store import store_ref, scatter_rows_ref
from .qknorm_rope import rms_norm_ref, rope_ref, qk_norm_rope_ref
from .sublayer import project_split_ref, sublayer_step_ref
from .attention import (
    kv_head_of,
    attention_ref,
    decode_ref,
    online_softmax_blocks,
    merge_partials,
    gather_logical_kv,
)

__all__ = [
    "bf16_bits_to_f64",
    "as_f64",
    "slot_mapping_block_walk",
    "slot_mapping_ref",
    "decode_slot_ref",
    "store_ref",
    "scatter_rows_ref",
    "rms_norm_ref",
    "rope_ref",
    "qk_norm_rope_ref",
    "project_split_ref",
    "sublayer_step_ref",
    "kv_head_of",
    "attention_ref",
    "decode_ref",
    "online_softmax_blocks",
    "merge_partials",
    "gather_logical_kv",
]
