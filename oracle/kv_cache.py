"""Physical KV pool, the KV write and the block copy (oracle side).

The pages fix that the cache is a pool of fixed-size physical blocks that may sit
anywhere (agentalpha.top Q32 answer part 2; data.6616ai.com "PagedAttention：把虚拟
内存搬进 KV Cache"), but not how a block is laid out in memory.  The library's
interface fixes that layout, and the oracle writes it out independently here:

* K pool: ``[num_blocks, num_kv_heads, head_dim / X, block_size, X]`` with
  ``X = 16 / element_bytes`` (8 for bf16/fp16, 4 for fp32): element (block, head,
  offset, d) sits at ``[block, head, d // X, offset, d % X]``;
* V pool: ``[num_blocks, num_kv_heads, head_dim, block_size]``: element
  (block, head, offset, d) sits at ``[block, head, d, offset]``.

Pools hold raw storage bits so that copies are compared byte for byte.
"""
from __future__ import annotations

import numpy as np

from .numerics import ELEM_BYTES, bits_dtype


class Pool:
    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int,
                 dtype: str, fill_bits: int = 0):
        self.num_blocks, self.num_kv_heads = int(num_blocks), int(num_kv_heads)
        self.head_dim, self.block_size, self.dtype = int(head_dim), int(block_size), dtype
        self.x = 16 // ELEM_BYTES[dtype]
        bd = bits_dtype(dtype)
        self.k = np.full((num_blocks, num_kv_heads, head_dim // self.x, block_size, self.x),
                         fill_bits, dtype=bd)
        self.v = np.full((num_blocks, num_kv_heads, head_dim, block_size), fill_bits, dtype=bd)

    # logical views --------------------------------------------------------------
    def k_at(self, blocks: np.ndarray, offsets: np.ndarray) -> np.ndarray:
        """K bits of the tokens at (blocks[i], offsets[i]) as ``[n, num_kv_heads, head_dim]``."""
        g = self.k[blocks, :, :, offsets, :]  # [n, H, D/X, X]
        return g.reshape(len(blocks), self.num_kv_heads, self.head_dim)

    def v_at(self, blocks: np.ndarray, offsets: np.ndarray) -> np.ndarray:
        """V bits of the tokens at (blocks[i], offsets[i]) as ``[n, num_kv_heads, head_dim]``."""
        return self.v[blocks, :, :, offsets]  # [n, H, D]


def paged_kv_write(pool: Pool, k_new: np.ndarray, v_new: np.ndarray, slot_mapping) -> None:
    """Store token t's K/V ``[num_kv_heads, head_dim]`` in slot ``slot_mapping[t]``.

    A slot names physical block ``slot // B`` and offset ``slot % B`` (the block
    table's logical->physical indirection has already been applied by the block
    manager).  Negative slots are padding and skipped.  Stored data elsewhere is
    untouched: appending a token moves nothing (agentalpha.top Q32 answer part 2;
    ohmygp.com "破局思路", 按需分配).
    """
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0
    if not keep.any():
        return
    slots = slots[keep]
    blk = slots // pool.block_size
    off = slots % pool.block_size
    n = len(slots)
    pool.k[blk, :, :, off, :] = np.asarray(k_new)[keep].reshape(n, pool.num_kv_heads, pool.head_dim // pool.x, pool.x)
    pool.v[blk, :, :, off] = np.asarray(v_new)[keep]


def copy_blocks(pool: Pool, pairs) -> None:
    """Copy-on-write: for each (src, dst), block dst of K and of V becomes a copy of block src.

    Pairs come from writes into shared blocks (agentalpha.top Q32 answer part 3;
    data.6616ai.com "PagedAttention：把虚拟内存搬进 KV Cache"; ohmygp.com "破局思路").
    Destinations are distinct and never a source, so the order does not matter.
    """
    for src, dst in pairs:
        pool.k[int(dst)] = pool.k[int(src)]
        pool.v[int(dst)] = pool.v[int(src)]


def swap_blocks(src: Pool, dst: Pool, pairs) -> None:
    """Swap-out / swap-in: for each (s, d), block d of ``dst`` (K and V, every head
    and slot) becomes a copy of block s of ``src``.  The two pools have the same
    tile layout and may differ in block count (a device pool and a host pool).

    Preemption under memory pressure moves a request's KV blocks to CPU memory and
    back (data.6616ai.com "PagedAttention 之外", scheduler and preemption;
    "可能的追问", KV swapped out to the CPU when the device is full).
    """
    if (src.num_kv_heads, src.head_dim, src.block_size, src.dtype) != \
            (dst.num_kv_heads, dst.head_dim, dst.block_size, dst.dtype):
        raise ValueError("pools must share the tile layout")
    for s, d in pairs:
        dst.k[int(d)] = src.k[int(s)]
        dst.v[int(d)] = src.v[int(s)]
