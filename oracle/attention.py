"""Decode attention over a paged KV pool, in float64 (oracle side).

Paging changes where K/V live, not what attention computes: the kernel reads KV
by block index, so the cache is contiguous logically and scattered physically
(data.6616ai.com "PagedAttention：把虚拟内存搬进 KV Cache"; ohmygp.com "破局思路",
块表映射).  The result is therefore plain softmax attention over the sequence's
logical K/V, written out here by its definition:

    s_j   = scale * sum_d q[b, h, d] * K[b, j, g, d]           for 0 <= j < L_b
    out   = sum_j exp(s_j - max s) V[b, j, g, :] / sum_j exp(s_j - max s)

with g = h // (Hq / Hkv) for grouped-query heads (consecutive query heads share a
KV head) and K/V[b, j] read from physical block ``table[b][j // B]`` at offset
``j % B``.  An empty context (L_b = 0) gives a zero output.

``paged_attention_prefill`` is the multi-token form over the same pool: each
sequence appends a chunk of C_b new tokens (their K/V already written to the pool,
so the context length L_b includes them), and query token t of the chunk sits at
position L_b - C_b + t and attends causally to positions 0 .. L_b - C_b + t.  This
is the prefill / chunked-prefill step that FlashAttention-style blockwise loading
serves over paged KV (agentalpha.top Q32 follow-up 3; data.6616ai.com "可能的追问");
decode is its C_b = 1 case.

``partitioned_attention`` computes the same result in independent partitions of
the context merged by log-sum-exp weights, the split-context form the pages tie
to FlashAttention-style blockwise loading over paged KV (agentalpha.top Q32
follow-up 3; data.6616ai.com "可能的追问").  In exact arithmetic it equals the
direct form; tests check the two agree to 1e-12 in float64.
"""
from __future__ import annotations

from typing import Iterable, Optional

import numpy as np

from .kv_cache import Pool
from .numerics import widen


def gather_context(pool: Pool, table_row: np.ndarray, length: int):
    """Logical K and V ``[length, Hkv, D]`` (float64) of one sequence, read through its table."""
    j = np.arange(length, dtype=np.int64)
    row = np.asarray(table_row, dtype=np.int64)
    blocks = row[j // pool.block_size]
    offs = j % pool.block_size
    return widen(pool.k_at(blocks, offs), pool.dtype), widen(pool.v_at(blocks, offs), pool.dtype)


def softmax_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Attention of queries ``q [G, D]`` over ``K, V [L, D]`` (float64)."""
    s = scale * (q @ K.T)                      # [G, L]
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    return (p @ V) / p.sum(axis=1, keepdims=True)


def paged_attention_decode(q_bits: np.ndarray, q_dtype: str, pool: Pool, block_tables: np.ndarray,
                           context_lens: np.ndarray, scale: float,
                           seqs: Optional[Iterable[int]] = None) -> np.ndarray:
    """Decode attention for every (or each listed) batch row: float64 ``[N, Hq, D]``.

    Rows not listed in ``seqs`` stay zero.
    """
    q = widen(q_bits, q_dtype)
    N, Hq, D = q.shape
    Hkv = pool.num_kv_heads
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    out = np.zeros((N, Hq, D), dtype=np.float64)
    for b in (range(N) if seqs is None else seqs):
        L = int(context_lens[b])
        if L == 0:
            continue
        K, V = gather_context(pool, block_tables[b], L)
        for g in range(Hkv):
            heads = slice(g * G, (g + 1) * G)
            out[b, heads] = softmax_attention(q[b, heads], K[:, g, :], V[:, g, :], scale)
    return out


def paged_attention_prefill(q_bits: np.ndarray, q_dtype: str, pool: Pool, block_tables: np.ndarray,
                            context_lens: np.ndarray, query_start: np.ndarray, scale: float,
                            seqs: Optional[Iterable[int]] = None) -> np.ndarray:
    """Causal attention of each sequence's chunk of new tokens: float64 ``[T, Hq, D]``.

    Rows of sequences not listed in ``seqs`` (when given) stay zero.

    ``q`` holds the chunks back to back (``[T, Hq, D]``); sequence b owns rows
    ``query_start[b] .. query_start[b+1]-1`` and its chunk is the last
    C_b = query_start[b+1] - query_start[b] of its L_b context tokens (C_b <= L_b).
    Row t of the chunk (position p = L_b - C_b + t) is softmax attention over the
    context tokens j <= p.
    """
    q = widen(q_bits, q_dtype)
    T, Hq, D = q.shape
    Hkv = pool.num_kv_heads
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    qs = np.asarray(query_start, dtype=np.int64)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for b in (range(len(qs) - 1) if seqs is None else seqs):
        C = int(qs[b + 1] - qs[b])
        L = int(context_lens[b])
        if C == 0:
            continue
        if C > L:
            raise ValueError("a chunk cannot be longer than its context")
        K, V = gather_context(pool, block_tables[b], L)
        pos = L - C + np.arange(C)                         # position of each chunk token
        visible = np.arange(L)[None, :] <= pos[:, None]    # [C, L] causal mask
        for h in range(Hq):
            g = h // G
            s = scale * (q[qs[b]:qs[b + 1], h, :] @ K[:, g, :].T)   # [C, L]
            s = np.where(visible, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)                                # masked entries give exp(-inf) = 0
            out[qs[b]:qs[b + 1], h, :] = (p @ V[:, g, :]) / p.sum(axis=1, keepdims=True)
    return out


def partitioned_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                          part_tokens: int) -> np.ndarray:
    """Same attention as ``softmax_attention`` computed per partition and merged.

    Partition p covers tokens [p*T, (p+1)*T).  Each keeps its own max m_p, sum
    l_p = sum exp(s - m_p) and normalised output o_p; the merge weights partition p
    by exp(m_p - M) * l_p with M = max_p m_p.
    """
    L = K.shape[0]
    ms, ls, os_ = [], [], []
    for start in range(0, L, part_tokens):
        s = scale * (q @ K[start:start + part_tokens].T)
        m = s.max(axis=1)
        p = np.exp(s - m[:, None])
        l = p.sum(axis=1)
        ms.append(m)
        ls.append(l)
        os_.append((p @ V[start:start + part_tokens]) / l[:, None])
    m = np.stack(ms)            # [P, G]
    l = np.stack(ls)
    o = np.stack(os_)           # [P, G, D]
    M = m.max(axis=0)
    w = np.exp(m - M) * l
    return (w[:, :, None] * o).sum(axis=0) / w.sum(axis=0)[:, None]
