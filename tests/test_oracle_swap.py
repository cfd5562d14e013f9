"""Pins for the oracle's swap path: moving sequences between a device and a host block
manager, and the block copy between two pools (CPU only).

* a swap-out / swap-in round trip restores every moved sequence's logical K/V bit
  for bit, although the device blocks were reused by other sequences meanwhile and
  the sequences come back in other physical blocks;
* attention over a swapped-back sequence equals attention before the swap (the
  decode oracle is pinned elsewhere);
* blocks shared by moved sequences are copied once and stay shared; blocks shared
  with a sequence that stays keep their other reference;
* a move that does not fit changes nothing;
* the copy touches exactly the destination blocks of its pairs.
"""
import numpy as np
import pytest

from oracle.attention import gather_context, paged_attention_decode
from oracle.block_manager import BlockManager, OutOfBlocks, move_seqs
from oracle.kv_cache import Pool, paged_kv_write, swap_blocks

B, H, D = 4, 2, 8


def _f32_bits(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)


def _setup(rng, nb=24, lengths=(9, 6, 13)):
    gpu = BlockManager(nb, B, rng.permutation(nb))
    pool = Pool(nb, H, D, B, "f32", fill_bits=0x7FC00000)
    for s, L in enumerate(lengths):
        gpu.add_seq(s, L)
        paged_kv_write(pool, _f32_bits(rng.standard_normal((L, H, D))), _f32_bits(rng.standard_normal((L, H, D))),
                       gpu.slots(s, 0, L))
    return gpu, pool


def _logical(pool, bm, s):
    K, V = gather_context(pool, np.asarray(bm.tables[s]), bm.lens[s])
    return K.copy(), V.copy()


def test_round_trip_restores_logical_kv():
    rng = np.random.default_rng(1)
    gpu, pool = _setup(rng)
    gpu.fork(1, 3)  # 3 shares all of 1's blocks
    before = {s: _logical(pool, gpu, s) for s in (0, 1, 2, 3)}
    cpu = BlockManager(30, B, rng.permutation(30))
    host = Pool(30, H, D, B, "f32", fill_bits=0)
    out_pairs = move_seqs(gpu, cpu, [1, 3, 0])
    swap_blocks(pool, host, out_pairs)
    assert len(out_pairs) == len({b for s in (1, 0) for b in cpu.tables[s]})
    # the device reuses the freed blocks for a new sequence
    gpu.add_seq(7, 4 * B)
    paged_kv_write(pool, _f32_bits(rng.standard_normal((4 * B, H, D))),
                   _f32_bits(rng.standard_normal((4 * B, H, D))), gpu.slots(7, 0, 4 * B))
    in_pairs = move_seqs(cpu, gpu, [0, 1, 3])
    swap_blocks(host, pool, in_pairs)
    for s in (0, 1, 2, 3):
        K, V = _logical(pool, gpu, s)
        np.testing.assert_array_equal(K, before[s][0])
        np.testing.assert_array_equal(V, before[s][1])
    assert gpu.tables[1] == gpu.tables[3]  # still shared after the round trip
    assert all(gpu.refcount[b] == 2 for b in gpu.tables[1])
    assert cpu.tables == {} and len(cpu.free) == 30


def test_attention_after_round_trip_is_unchanged():
    rng = np.random.default_rng(2)
    gpu, pool = _setup(rng)
    q = _f32_bits(rng.standard_normal((3, 2 * H, D)))
    tables = lambda: np.asarray(gpu.block_tables([0, 1, 2], 8, 0), dtype=np.int32)
    lens = np.asarray([gpu.lens[s] for s in (0, 1, 2)])
    ref = paged_attention_decode(q, "f32", pool, tables(), lens, 0.3)
    cpu = BlockManager(10, B, np.arange(10))
    host = Pool(10, H, D, B, "f32")
    swap_blocks(pool, host, move_seqs(gpu, cpu, [2]))
    gpu.add_seq(9, 3 * B)  # takes the freed blocks
    paged_kv_write(pool, _f32_bits(rng.standard_normal((3 * B, H, D))),
                   _f32_bits(rng.standard_normal((3 * B, H, D))), gpu.slots(9, 0, 3 * B))
    swap_blocks(host, pool, move_seqs(cpu, gpu, [2]))
    np.testing.assert_array_equal(paged_attention_decode(q, "f32", pool, tables(), lens, 0.3), ref)


def test_shared_block_with_a_staying_sequence_keeps_its_reference():
    rng = np.random.default_rng(3)
    gpu, _ = _setup(rng)
    gpu.fork(0, 5)
    shared = list(gpu.tables[0])
    cpu = BlockManager(12, B, np.arange(12))
    pairs = move_seqs(gpu, cpu, [0])
    assert [p[0] for p in pairs] == shared and [p[1] for p in pairs] == list(range(len(shared)))
    assert all(gpu.refcount[b] == 1 for b in shared)  # 5 still holds them
    assert all(cpu.refcount[c] == 1 for c in cpu.tables[0])


def test_move_that_does_not_fit_changes_nothing():
    rng = np.random.default_rng(4)
    gpu, _ = _setup(rng)
    cpu = BlockManager(3, B, np.arange(3))
    snap = (dict(gpu.tables), list(gpu.free), list(gpu.refcount), list(cpu.free))
    with pytest.raises(OutOfBlocks):
        move_seqs(gpu, cpu, [0, 2])  # 3 + 4 blocks > 3
    assert (dict(gpu.tables), list(gpu.free), list(gpu.refcount), list(cpu.free)) == snap
    with pytest.raises(KeyError):
        move_seqs(gpu, cpu, [42])
    with pytest.raises(ValueError):
        move_seqs(gpu, cpu, [1, 1])


def test_swap_blocks_copies_exactly_the_pairs():
    rng = np.random.default_rng(5)
    a = Pool(6, H, D, B, "f32")
    a.k[:] = rng.integers(0, 2**32, a.k.shape, dtype=np.uint32)
    a.v[:] = rng.integers(0, 2**32, a.v.shape, dtype=np.uint32)
    b = Pool(9, H, D, B, "f32", fill_bits=7)
    swap_blocks(a, b, [(4, 0), (1, 8), (4, 3)])
    for s, d in [(4, 0), (1, 8), (4, 3)]:
        np.testing.assert_array_equal(b.k[d], a.k[s])
        np.testing.assert_array_equal(b.v[d], a.v[s])
    untouched = [1, 2, 4, 5, 6, 7]
    assert (b.k[untouched] == 7).all() and (b.v[untouched] == 7).all()
    with pytest.raises(ValueError):
        swap_blocks(a, Pool(2, H, D, 2 * B, "f32"), [(0, 0)])
