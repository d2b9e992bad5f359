"""CPU oracle for paged KV-cache decode. TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct reference for what the HIP library computes:
block geometry and slot translation, the scatter of new tokens into their
slots, whole-block copies for copy-on-write, and decode attention read through
a block table. Floating point is fp64 throughout.

Who may use it: the tests under tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py. The HIP library never imports, links or calls
anything here, and nothing here imports the library: the two share no code.
Inputs come from the seeded generators in the `workloads` package, which hold
none of this arithmetic.

Sources (three web pages on PagedAttention):
  [L]  "Paged Attention: OS-Inspired Memory Management for KV Caches"
       (modernaiengineering.com, Lesson 13.6)
  [B]  "What is PagedAttention and how does it manage KV cache?" (n4n.ai blog)
  [W]  the worksonmygpu.com deep-dive post on PagedAttention in vLLM

Every function is pinned by tests that do not re-type its formula: values the
pages print, closed forms, an independent library routine (torch CPU
scaled_dot_product_attention in fp64) and brute force on tiny inputs.
"""
from .geometry import (blocks_for, logical_block, block_offset, slot_of, empty_slots,
                       kv_bytes_per_token, contiguous_waste, paged_waste, decode_slots,
                       token_slots)
from .cache import gather, write_kv, copy_blocks, swap_blocks
from .attention import (decode, prefill, attend, attend_partial, merge_partials,
                        causal_attention)
from .block_manager import BlockManager, PoolExhausted

__all__ = [
    "blocks_for", "logical_block", "block_offset", "slot_of", "empty_slots",
    "kv_bytes_per_token", "contiguous_waste", "paged_waste", "decode_slots", "token_slots",
    "gather", "write_kv", "copy_blocks", "swap_blocks",
    "decode", "prefill", "attend", "attend_partial", "merge_partials", "causal_attention",
    "BlockManager", "PoolExhausted",
]
