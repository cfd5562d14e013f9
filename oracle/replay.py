"""Replay a workload's operations through the oracle block manager, write and copy.

A workload (duck-typed: ``num_blocks``, ``block_size``, ``free_order``,
``prefill``, ``forks``, ``steps``, ``batch``, value accessors) lists prefill,
fork and decode-step operations; this module performs them in order on an oracle
pool and returns the final pool, the batch's block tables and context lengths,
and the slot mapping and copy pairs of the last (measured) step.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import numpy as np

from .block_manager import BlockManager
from .kv_cache import Pool, copy_blocks, paged_kv_write


@dataclasses.dataclass
class ReplayResult:
    bm: BlockManager
    pool: Pool
    block_tables: np.ndarray      # int32 [N, W]
    context_lens: np.ndarray      # int32 [N]
    last_slots: np.ndarray        # int64 [T]
    last_pairs: np.ndarray        # int64 [P, 2]
    copies: int                   # total CoW pairs over all steps


def replay(w, fill_bits: int, pad: int = 0, context=None,
           stop_before_last_step: bool = False) -> ReplayResult:
    bm = BlockManager(w.num_blocks, w.block_size, w.free_order)
    pool = Pool(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size, w.dtype, fill_bits)
    if context is None:
        context = w.all_context_kv()
    for seq, n in w.prefill:
        bm.add_seq(seq, n)
        if n:
            k, v = context[seq]
            paged_kv_write(pool, k, v, bm.slots(seq, 0, n))
    for parent, child in w.forks:
        bm.fork(parent, child)
    slots: List[int] = []
    pairs: List[Tuple[int, int]] = []
    copies = 0
    nsteps = len(w.steps) - (1 if stop_before_last_step else 0)
    for i in range(nsteps):
        slots, pairs = bm.step(w.steps[i])
        copies += len(pairs)
        copy_blocks(pool, pairs)
        k, v = w.step_kv(i)
        paged_kv_write(pool, k, v, slots)
    tables = np.asarray(bm.block_tables(w.batch, w.max_blocks_per_seq, pad), dtype=np.int32)
    lens = np.asarray([bm.lens[int(s)] for s in w.batch], dtype=np.int32)
    return ReplayResult(bm, pool, tables.reshape(len(w.batch), w.max_blocks_per_seq), lens,
                        np.asarray(slots, dtype=np.int64),
                        np.asarray(pairs, dtype=np.int64).reshape(-1, 2), copies)


def replay_prefill(w, fill_bits: int, context=None, pad: int = 0):
    """Place a prefill workload: every sequence (ascending) is added with its whole
    context and its K/V written at positions 0..L-1.  Returns (pool, block tables
    int32 [N, W], context lengths int32 [N])."""
    bm = BlockManager(w.num_blocks, w.block_size, w.free_order)
    pool = Pool(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size, w.dtype, fill_bits)
    if context is None:
        context = w.all_context_kv()
    for b in range(w.num_seqs):
        L = int(w.context_lens[b])
        bm.add_seq(b, L)
        if L:
            k, v = context[b]
            paged_kv_write(pool, k, v, bm.slots(b, 0, L))
    tables = np.asarray(bm.block_tables(range(w.num_seqs), w.max_blocks_per_seq, pad), dtype=np.int32)
    return pool, tables.reshape(w.num_seqs, w.max_blocks_per_seq), np.asarray(w.context_lens, dtype=np.int32)


def replay_prefix(w, fill_bits: int, cache: bool = True):
    """Place a prefix-sharing workload request by request.  With ``cache`` each request
    reuses the cached blocks of its prompt prefix and only its remaining tokens' K/V are
    written; without it every token is written.  Returns (pool, block tables int32
    [N, W], context lengths int32 [N], cached token count per request)."""
    from .block_manager import PrefixCachingBlockManager
    bm = (PrefixCachingBlockManager if cache else BlockManager)(w.num_blocks, w.block_size, w.free_order)
    pool = Pool(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size, w.dtype, fill_bits)
    cached = []
    for b in range(w.num_seqs):
        toks = w.tokens(b)
        L = len(toks)
        if cache:
            c = bm.add_seq_tokens(b, toks)
        else:
            bm.add_seq(b, L)
            c = 0
        k, v = w.kv(b)
        if L > c:
            paged_kv_write(pool, k[c:], v[c:], bm.slots(b, c, L - c))
        cached.append(c)
    tables = np.asarray(bm.block_tables(range(w.num_seqs), w.max_blocks_per_seq, 0), dtype=np.int32)
    lens = np.asarray([w.length(b) for b in range(w.num_seqs)], dtype=np.int32)
    return pool, tables.reshape(w.num_seqs, w.max_blocks_per_seq), lens, np.asarray(cached, dtype=np.int32)
