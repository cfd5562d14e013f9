"""Memory-waste accounting of contiguous reservation versus paged allocation.

ohmygp.com "用模拟把浪费率算出来": every request reserves the maximum length in
the contiguous scheme, while paged allocation hands out whole blocks so that only
the tail block of a request can hold unused slots.  Three figures follow:
the contiguous waste 1 - used / reserved, the paged waste 1 - used / paged, and
the concurrency gain reserved / paged (how many more requests fit in the same
memory).  ``paged`` counts ceil(len / B) blocks of B slots per request.

agentalpha.top Q32, follow-up 2 and the résumé note after it: the block size trades
internal fragmentation (larger blocks waste more of the tail) against table size
(smaller blocks need more entries), and short sequences can take 16-token blocks while
long ones take 32-token blocks.  ``class_block_size`` and ``paged_footprint`` account a
batch under such a per-length-class choice.
"""
from __future__ import annotations

import numpy as np


def blocks_needed(length: int, block_size: int) -> int:
    """Number of blocks a request of ``length`` tokens occupies: ceil(length / B)."""
    return -(-int(length) // int(block_size))


def tail_waste(length: int, block_size: int) -> int:
    """Unused slots of the request: those of its partially filled tail block."""
    return blocks_needed(length, block_size) * int(block_size) - int(length)


def waste_report(lengths, max_len: int, block_size: int):
    """(contiguous waste, paged waste, concurrency gain) for a set of request lengths."""
    lengths = np.asarray(lengths, dtype=np.int64)
    used = float(lengths.sum())
    reserved = float(len(lengths) * int(max_len))
    paged = float(sum(blocks_needed(L, block_size) * block_size for L in lengths))
    return 1.0 - used / reserved, 1.0 - used / paged, reserved / paged


def class_block_size(length: int, threshold: int, small: int = 16, large: int = 32) -> int:
    """Block size of a request's length class: ``small`` below ``threshold`` tokens, else ``large``."""
    return int(small) if int(length) < int(threshold) else int(large)


def paged_footprint(lengths, block_sizes):
    """(allocated slots, wasted slots, table entries) of requests of ``lengths`` held in
    blocks of ``block_sizes`` (one block size per request)."""
    allocated = wasted = entries = 0
    for L, B in zip(lengths, block_sizes):
        n = blocks_needed(L, B)
        allocated += n * int(B)
        wasted += tail_waste(L, B)
        entries += n
    return allocated, wasted, entries
