"""Block-table representations and the memory they take.

TEST INFRASTRUCTURE ONLY (see the package docstring).

agentalpha.top Q32, follow-up 1 (block-table overhead for a 128K-token context): with
16-token blocks such a request needs 8192 table entries; at about 8 bytes an entry (a
4-byte physical block id plus state such as "full") that is 64 KB per request and
64 MB for 1000 concurrent requests.  Two ways to shrink it are named there: 16-bit
block ids while the pool has fewer than 65536 blocks, and a hierarchical table in
the manner of multi-level page tables for sparse cases.

The representations (restated here from their definitions, independently of the
library):

* flat: row b of a [N][W] matrix holds entries 0 .. W-1 of sequence b, padded past
  its table; entries are 4-byte ints, or 2-byte unsigned ints below 65536 blocks.
* two-level: a sequence's entries are cut into leaves of E = 512 / B ids (the
  entries of 512 tokens); row b of a [N][dir_width]
  directory names the leaf that holds each run of E entries of sequence b.  Leaves
  are numbered by sequence (in the given order) and then by position; a sequence's
  last leaf is padded with ``pad``; one final leaf holds only ``pad`` and every
  directory entry past a sequence's leaves names it.

Reading taken for "sparse": a batch whose table width W is set by its longest
sequence while most sequences are short, so most of a flat [N][W] matrix is padding.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

LEAF_TOKENS = 512  # context tokens whose block ids one leaf holds


def table_entries(context_len: int, block_size: int) -> int:
    """Entries of a request's table: one per block, ceil(L / B)."""
    return -(-int(context_len) // int(block_size))


def table_bytes_per_request(context_len: int, block_size: int, entry_bytes: int) -> int:
    """Bytes of one request's flat table at ``entry_bytes`` per entry."""
    return table_entries(context_len, block_size) * int(entry_bytes)


def flat_table_bytes(num_seqs: int, width: int, entry_bytes: int) -> int:
    """Bytes of a flat [N][W] table matrix."""
    return int(num_seqs) * int(width) * int(entry_bytes)


def leaf_entries(block_size: int) -> int:
    """Entries per two-level leaf: the blocks of 512 tokens."""
    return LEAF_TOKENS // int(block_size)


def two_level(tables: Sequence[Sequence[int]], block_size: int, dir_width: int,
              pad: int) -> Tuple[np.ndarray, np.ndarray]:
    """(directory int32 [n][dir_width], leaves int32 [num_leaves][E]) of ``tables``."""
    E = leaf_entries(block_size)
    leaves: List[List[int]] = []
    directory = np.zeros((len(tables), dir_width), dtype=np.int32)
    pad_rows = []  # (row, column) of directory entries that name the padding leaf
    for b, t in enumerate(tables):
        runs = [list(t[i:i + E]) for i in range(0, len(t), E)]
        if len(runs) > dir_width:
            raise ValueError("table needs more leaves than the directory width")
        for j in range(dir_width):
            if j < len(runs):
                directory[b, j] = len(leaves)
                leaves.append(runs[j] + [pad] * (E - len(runs[j])))
            else:
                pad_rows.append((b, j))
    if len(tables):
        for b, j in pad_rows:
            directory[b, j] = len(leaves)
        leaves.append([pad] * E)
    return directory, np.asarray(leaves, dtype=np.int32).reshape(len(leaves), E)


def two_level_entry(directory: np.ndarray, leaves: np.ndarray, b: int, j: int) -> int:
    """Entry j of sequence b: the (j mod E)-th id of the leaf the directory names for run j div E."""
    E = leaves.shape[1]
    return int(leaves[directory[b, j // E], j % E])


def two_level_bytes(num_seqs: int, dir_width: int, num_leaves: int, block_size: int) -> int:
    """Bytes of a two-level table: 4 per directory entry and per leaf entry."""
    return 4 * (int(num_seqs) * int(dir_width) + int(num_leaves) * leaf_entries(block_size))
