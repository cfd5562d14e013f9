"""Pins for the oracle block manager, KV write and block copy (CPU only)."""
import json
import os

import numpy as np
import pytest

from oracle.block_manager import BlockManager, OutOfBlocks
from oracle.kv_cache import Pool, copy_blocks, paged_kv_write
from oracle.accounting import blocks_needed

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _free_order_starting(first, num_blocks):
    rest = [b for b in range(num_blocks) if b not in first]
    return list(first) + rest


def test_page_block_table_example_resolves():
    """The page's table (logical 0 -> 5, logical 1 -> 12) places tokens in blocks 5 and 12."""
    g = json.load(open(os.path.join(GOLDEN, "block_table_example.json")))
    B = g["block_size"]
    phys = g["logical_to_physical"]
    bm = BlockManager(16, B, _free_order_starting(phys, 16))
    bm.add_seq(0, 2 * B)
    assert bm.block_table(0) == phys
    # write token j's id into a one-head, D=4 fp32 pool and find it back in the physical blocks
    pool = Pool(16, 1, 4, B, "f32", fill_bits=0)
    ids = np.arange(1, 2 * B + 1, dtype=np.float32)
    k = np.repeat(ids[:, None, None], 4, axis=2).view(np.uint32)
    paged_kv_write(pool, k, k, bm.slots(0, 0, 2 * B))
    for j in range(2 * B):
        blk, off = phys[j // B], j % B
        assert pool.k[blk, 0, 0, off, 0].view(np.float32) == ids[j]
        assert pool.v[blk, 0, 3, off].view(np.float32) == ids[j]
    # every other block is untouched
    others = [b for b in range(16) if b not in phys]
    assert not pool.k[others].any() and not pool.v[others].any()


@pytest.mark.parametrize("B", [16, 32])
def test_blocks_per_sequence_is_ceil_and_tail_waste_below_one_block(B):
    rng = np.random.default_rng(7)
    lengths = rng.integers(0, 300, size=40)
    bm = BlockManager(2000, B, rng.permutation(2000))
    for s, L in enumerate(lengths):
        if s % 2:
            bm.add_seq(s, int(L))
        else:  # grow token by token
            bm.add_seq(s, 0)
            for _ in range(int(L)):
                bm.append_slot(s)
        n = len(bm.block_table(s))
        assert n == -(-int(L) // B) == blocks_needed(L, B)
        assert 0 <= n * B - int(L) <= B - 1


def test_page_block_size_tradeoff_figures():
    g = json.load(open(os.path.join(GOLDEN, "block_size_tradeoff.json")))
    c33, c128k = g["cases"]
    bm = BlockManager(8192, c33["block_size"], range(8192))
    bm.add_seq(0, c33["request_tokens"])
    assert len(bm.block_table(0)) * c33["block_size"] - c33["request_tokens"] == c33["wasted_tokens"]
    bm2 = BlockManager(8192, c128k["block_size"], range(8192))
    bm2.add_seq(0, c128k["request_tokens"])
    assert len(bm2.block_table(0)) == c128k["blocks"]


def _check_refcounts(bm):
    counts = np.zeros(bm.num_blocks, dtype=np.int64)
    for t in bm.tables.values():
        for b in t:
            counts[b] += 1
    assert list(counts) == bm.refcount
    free = list(bm.free)
    assert len(set(free)) == len(free)
    assert all(counts[b] == 0 for b in free)
    assert len(free) + int((counts > 0).sum()) == bm.num_blocks


def test_fork_shares_blocks_and_cow_copies_only_shared_tails():
    B = 16
    bm = BlockManager(64, B, range(64))
    bm.add_seq(0, 20)                      # two blocks, the second holds 4 tokens
    for c in (1, 2, 3):
        bm.fork(0, c)
    shared = bm.block_table(0)
    assert all(bm.refcount[b] == 4 for b in shared)
    slots, pairs = bm.step([0, 1, 2, 3])
    # the first three writers copy the shared tail; the last sharer writes in place
    assert [p[0] for p in pairs] == [shared[1]] * 3
    dsts = [p[1] for p in pairs]
    assert len(set(dsts)) == 3 and not set(dsts) & set(shared)
    assert bm.block_table(3) == shared
    assert [bm.block_table(s)[1] for s in (0, 1, 2)] == dsts
    assert bm.refcount[shared[0]] == 4 and bm.refcount[shared[1]] == 1
    assert slots == [d * B + 4 for d in dsts] + [shared[1] * B + 4]
    # the full first block stays shared: nothing copies it
    _check_refcounts(bm)


def test_block_aligned_prompt_needs_no_copy():
    bm = BlockManager(64, 16, range(64))
    bm.add_seq(0, 32)
    for c in (1, 2, 3):
        bm.fork(0, c)
    _, pairs = bm.step([0, 1, 2, 3])
    assert pairs == []
    tails = {bm.block_table(s)[-1] for s in range(4)}
    assert len(tails) == 4


def test_free_returns_blocks_to_back_and_exhaustion_raises():
    bm = BlockManager(4, 16, [3, 1, 0, 2])
    bm.add_seq(0, 17)                     # takes 3, 1
    bm.add_seq(1, 16)                     # takes 0
    bm.free_seq(0)                        # 3, 1 go behind 2
    assert list(bm.free) == [2, 3, 1]
    bm.add_seq(2, 48)
    assert bm.block_table(2) == [2, 3, 1]
    with pytest.raises(OutOfBlocks):
        bm.append_slot(1)  # position 16 needs a new block: none left
    with pytest.raises(OutOfBlocks):
        bm.add_seq(3, 1)


def test_each_sequence_reads_back_its_own_history():
    """Random add/fork/append/free with writes and CoW copies: every live sequence,
    read through its table, holds exactly the tokens it wrote or inherited."""
    rng = np.random.default_rng(11)
    for B in (4, 16):
        NB = 400
        bm = BlockManager(NB, B, rng.permutation(NB))
        pool = Pool(NB, 1, 4, B, "f32", fill_bits=0)
        hist = {}
        next_id, next_seq = [1.0], [0]

        def tok():
            next_id[0] += 1.0
            return next_id[0]

        def write(slots, vals):
            k = np.repeat(np.asarray(vals, np.float32)[:, None, None], 4, axis=2).view(np.uint32)
            paged_kv_write(pool, k, k, slots)

        for it in range(300):
            op = rng.random()
            live = sorted(hist)
            if op < 0.15 or not live:
                n = int(rng.integers(0, 3 * B))
                if sum(len(t) for t in bm.tables.values()) + n // B + 2 > NB // 2:
                    continue
                s = next_seq[0]; next_seq[0] += 1
                bm.add_seq(s, n)
                vals = [tok() for _ in range(n)]
                if n:
                    write(bm.slots(s, 0, n), vals)
                hist[s] = vals
            elif op < 0.3:
                p = int(rng.choice(live))
                c = next_seq[0]; next_seq[0] += 1
                bm.fork(p, c)
                hist[c] = list(hist[p])
            elif op < 0.38 and len(live) > 1:
                s = int(rng.choice(live))
                bm.free_seq(s)
                del hist[s]
            else:
                k = int(rng.integers(1, len(live) + 1))
                seqs = sorted(int(x) for x in rng.choice(live, size=k, replace=False))
                if len(bm.free) < 2 * len(seqs):
                    continue
                slots, pairs = bm.step(seqs)
                copy_blocks(pool, pairs)
                vals = [tok() for _ in seqs]
                write(slots, vals)
                for s, v in zip(seqs, vals):
                    hist[s].append(v)
            _check_refcounts(bm)
        for s, vals in hist.items():
            got = [float(pool.k[bm.slot_of(s, j) // B, 0, 0, bm.slot_of(s, j) % B, 0].view(np.float32))
                   for j in range(len(vals))]
            assert got == vals, f"sequence {s}"


def test_copy_blocks_copies_whole_blocks_only():
    rng = np.random.default_rng(3)
    pool = Pool(8, 2, 8, 4, "bf16", fill_bits=0)
    pool.k[:] = rng.integers(0, 2 ** 16, size=pool.k.shape, dtype=np.uint16)
    pool.v[:] = rng.integers(0, 2 ** 16, size=pool.v.shape, dtype=np.uint16)
    k0, v0 = pool.k.copy(), pool.v.copy()
    copy_blocks(pool, [(1, 5), (1, 6), (2, 7)])
    for s, d in [(1, 5), (1, 6), (2, 7)]:
        assert (pool.k[d] == k0[s]).all() and (pool.v[d] == v0[s]).all()
    for b in (0, 1, 2, 3, 4):
        assert (pool.k[b] == k0[b]).all() and (pool.v[b] == v0[b]).all()


def test_write_skips_negative_slots_and_touches_only_its_slots():
    pool = Pool(4, 2, 16, 4, "f16", fill_bits=0x7E00)
    k = np.arange(3 * 2 * 16, dtype=np.uint16).reshape(3, 2, 16)
    v = k + 1000
    paged_kv_write(pool, k, v, [5, -1, 14])
    # slot 5 = block 1 offset 1; slot 14 = block 3 offset 2
    assert (pool.k[1, :, :, 1, :].reshape(2, 16) == k[0]).all()
    assert (pool.v[3, :, :, 2] == v[2]).all()
    touched = np.zeros(pool.k.shape, bool)
    touched[1, :, :, 1, :] = True
    touched[3, :, :, 2, :] = True
    assert (pool.k[~touched] == 0x7E00).all()
    # layout: K element (block, head, offset, d) at [block, head, d // 8, offset, d % 8]
    assert pool.k[1, 1, 0, 1, 3] == k[0, 1, 3]
    assert pool.k[1, 1, 1, 1, 0] == k[0, 1, 8]
    assert pool.k[3, 0, 1, 2, 2] == k[2, 0, 10]
    # V element (block, head, offset, d) at [block, head, d, offset]
    assert pool.v[3, 1, 7, 2] == v[2, 1, 7]
