"""Pins for the oracle's prefix cache (CPU only).

* FNV-1a 64 matches the published test vectors of its authors' reference;
* two prompts with a common prefix share exactly the full blocks that lie inside
  the common prefix and before the second prompt's last token;
* released cached blocks stay addressable until allocation evicts them, least
  recently released first;
* a prompt equal to a cached one still computes its last block;
* attention over a chunk computed on top of cached blocks equals attention with the
  whole prompt written (the cached blocks hold the same K/V);
* a request that does not fit changes nothing.
"""
import numpy as np
import pytest

from oracle.attention import paged_attention_prefill
from oracle.block_manager import (BlockManager, OutOfBlocks, PrefixCachingBlockManager, block_key, fnv1a64)
from oracle.kv_cache import Pool, paged_kv_write

B = 4


def test_fnv1a64_published_vectors():
    assert fnv1a64(b"") == 0xCBF29CE484222325
    assert fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert fnv1a64(b"foobar") == 0x85944171F73967E8


def test_block_key_chains_parent_and_tokens():
    k1 = block_key(0, [1, 2, 3, 4])
    assert k1 == fnv1a64(bytes(8) + b"".join(int(t).to_bytes(4, "little") for t in [1, 2, 3, 4]))
    assert block_key(k1, [5, 6, 7, 8]) != block_key(0, [5, 6, 7, 8])
    assert block_key(0, [-1, 0, 0, 0]) == fnv1a64(bytes(8) + b"\xff\xff\xff\xff" + bytes(12))


def test_common_prefix_shares_full_blocks():
    bm = PrefixCachingBlockManager(40, B, np.arange(40))
    system = list(range(100, 111))          # 11 tokens: 2 full blocks + 3
    a = system + [1, 2, 3, 4, 5, 6]         # 17 tokens
    b = system + [7, 8]                     # 13 tokens
    assert bm.add_seq_tokens(0, a) == 0
    assert bm.add_seq_tokens(1, b) == 2 * B  # blocks 0, 1 lie inside the 11 common tokens
    assert bm.tables[1][:2] == bm.tables[0][:2] and bm.tables[1][2] != bm.tables[0][2]
    assert all(bm.refcount[x] == 2 for x in bm.tables[0][:2])
    c = [999] + system
    assert bm.add_seq_tokens(2, c) == 0      # different first block: nothing shared


def test_last_block_is_always_computed():
    bm = PrefixCachingBlockManager(20, B, np.arange(20))
    p = list(range(3 * B))
    assert bm.add_seq_tokens(0, p) == 0
    assert bm.add_seq_tokens(1, p) == 2 * B  # the block holding the last token is fresh
    assert bm.tables[1][2] != bm.tables[0][2]


def test_released_blocks_stay_cached_until_evicted_in_release_order():
    bm = PrefixCachingBlockManager(8, B, np.arange(8))
    p = list(range(10, 10 + 3 * B + 1))      # 13 tokens: 3 cached full blocks + a tail
    q = list(range(50, 50 + 3 * B + 1))
    bm.add_seq_tokens(0, p)
    bm.add_seq_tokens(1, q)
    bm.free_seq(0)                           # p's full blocks released first, then q's
    bm.free_seq(1)
    assert len(bm.free) == 2 and list(bm.evictable) == bm_order(bm, p) + bm_order(bm, q)
    assert bm.add_seq_tokens(2, p) == 3 * B  # still cached
    bm.free_seq(2)                           # p's blocks are now the most recently released
    # an uncached 5-block prompt takes the 2 free blocks, then evicts q's 3 blocks
    bm.add_seq_tokens(3, list(range(200, 200 + 5 * B)))
    assert bm_order(bm, q) == [] and len(bm_order(bm, p)) == 3
    bm.free_seq(3)
    assert bm.add_seq_tokens(4, p) == 3 * B  # p survived the eviction
    bm.free_seq(4)
    assert bm.add_seq_tokens(5, q) == 0      # q did not


def bm_order(bm, prompt):
    """Cached blocks of the prompt's full blocks, in block order (those still cached)."""
    out, parent = [], 0
    for i in range(len(prompt) // B):
        key = block_key(parent, prompt[i * B:(i + 1) * B])
        if key in bm.cached:
            out.append(bm.cached[key])
        parent = key
    return out


def test_request_that_does_not_fit_changes_nothing():
    bm = PrefixCachingBlockManager(5, B, np.arange(5))
    bm.add_seq_tokens(0, list(range(4 * B + 1)))
    snap = (dict(bm.tables), list(bm.free), list(bm.refcount), dict(bm.cached), list(bm.evictable))
    with pytest.raises(OutOfBlocks):
        bm.add_seq_tokens(1, list(range(100, 100 + 2 * B)))
    assert (dict(bm.tables), list(bm.free), list(bm.refcount), dict(bm.cached), list(bm.evictable)) == snap


def test_plain_manager_is_unchanged():
    bm = BlockManager(10, B, np.arange(10))
    bm.add_seq(0, 9)
    bm.free_seq(0)
    assert list(bm.free) == [3, 4, 5, 6, 7, 8, 9, 0, 1, 2]


def _f32_bits(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)


def test_attention_on_cached_blocks_equals_full_write():
    rng = np.random.default_rng(9)
    H, D, G = 2, 8, 2
    system_len, suffix = 14, [3, 9, 5]
    sysK, sysV = rng.standard_normal((system_len, H, D)), rng.standard_normal((system_len, H, D))
    prompts, kvs = [], []
    for i, s in enumerate(suffix):
        toks = list(range(1000, 1000 + system_len)) + [i * 100 + j for j in range(s)]
        K = np.concatenate([sysK, rng.standard_normal((s, H, D))])
        V = np.concatenate([sysV, rng.standard_normal((s, H, D))])
        prompts.append(toks)
        kvs.append((_f32_bits(K), _f32_bits(V)))
    lens = np.asarray([len(p) for p in prompts])
    # plain placement: every token written, every token a query
    plain = BlockManager(30, B, np.arange(30))
    pool_a = Pool(30, H, D, B, "f32", fill_bits=0x7FC00000)
    for i, p in enumerate(prompts):
        plain.add_seq(i, len(p))
        paged_kv_write(pool_a, kvs[i][0], kvs[i][1], plain.slots(i, 0, len(p)))
    q_full = _f32_bits(rng.standard_normal((int(lens.sum()), H * G, D)))
    qs_full = np.concatenate([[0], np.cumsum(lens)])
    ref = paged_attention_prefill(q_full, "f32", pool_a, np.asarray(plain.block_tables(range(3), 8, 0)), lens,
                                  qs_full, 0.35)
    # cached placement: only uncached tokens written; only they are queries
    pc = PrefixCachingBlockManager(30, B, np.arange(30)[::-1])
    pool_b = Pool(30, H, D, B, "f32", fill_bits=0x7FC00000)
    chunks, rows = [], []
    for i, p in enumerate(prompts):
        c = pc.add_seq_tokens(i, p)
        paged_kv_write(pool_b, kvs[i][0][c:], kvs[i][1][c:], pc.slots(i, c, len(p) - c))
        chunks.append(len(p) - c)
        rows.append(np.arange(qs_full[i] + c, qs_full[i + 1]))
    assert chunks[0] == lens[0] and chunks[1] < lens[1] and chunks[2] < lens[2]
    rows = np.concatenate(rows)
    qs = np.concatenate([[0], np.cumsum(chunks)])
    got = paged_attention_prefill(q_full[rows], "f32", pool_b, np.asarray(pc.block_tables(range(3), 8, 0)), lens, qs,
                                  0.35)
    np.testing.assert_array_equal(got, ref[rows])
