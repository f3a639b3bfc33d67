"""Where a key or value lands in the paged KV pool -- test infrastructure (oracle).

"Candle model runner" section 2.4: position j of a sequence lives in block
floor(j / B) of its block table, slot j mod B. Section 3 "Where a key lands":
with B = 16 and table [7, 2, 9], position 37 is pool block 9, slot 5, and the
K of KV head h starts at element (h*16 + 5)*D of layer l's K slab of block 9.

The pool holds, per layer, a K part and a V part, each an array of blocks, and
each block's slab is [H_kv][B][D] (the slab layout of that worked example):
pool[layer][0 = K, 1 = V][block][kv_head][slot][channel].
"""

from __future__ import annotations


def kv_location(pos: int, block_table, block_tokens: int) -> tuple:
    """(pool block, slot) of absolute position ``pos``."""
    return int(block_table[pos // block_tokens]), pos % block_tokens


def slab_offset(kv_head: int, slot: int, block_tokens: int, head_dim: int) -> int:
    """Element offset of (kv_head, slot) inside one block's [H_kv][B][D] slab."""
    return (kv_head * block_tokens + slot) * head_dim


def kv_element_offset(layer: int, is_v: bool, pos: int, kv_head: int, block_table,
                      n_blocks: int, n_kv_heads: int, block_tokens: int, head_dim: int) -> int:
    """Element offset of channel 0 of (layer, K or V, position, kv head) in the pool."""
    block, slot = kv_location(pos, block_table, block_tokens)
    slab = block_tokens * n_kv_heads * head_dim
    base = ((layer * 2 + (1 if is_v else 0)) * n_blocks + block) * slab
    return base + slab_offset(kv_head, slot, block_tokens, head_dim)
