"""The library's host block manager against the oracle's, bit for bit (CPU only)."""
import numpy as np
import pytest

import synth
from oracle.block_manager import BlockManager as OracleBM, OutOfBlocks


def _same_state(lib_bm, ora, seqs):
    for s in seqs:
        assert lib_bm.block_table(s) == ora.block_table(s)
        assert lib_bm.seq_len(s) == ora.lens[s]
    assert [lib_bm.refcount(b) for b in range(ora.num_blocks)] == ora.refcount
    assert lib_bm.num_free() == len(ora.free)


def test_page_example_table(pkv_lib):
    order = [5, 12] + [b for b in range(16) if b not in (5, 12)]
    bm = pkv_lib.BlockManager(16, 16, order)
    bm.add_seq(0, 32)
    assert bm.block_table(0) == [5, 12]
    assert bm.slots(0, 0, 32).tolist() == list(range(80, 96)) + list(range(192, 208))


@pytest.mark.parametrize("B", [4, 16, 32])
def test_random_operations_match_oracle(pkv_lib, B):
    rng = np.random.default_rng(B)
    NB = 300
    order = rng.permutation(NB)
    lib_bm = pkv_lib.BlockManager(NB, B, order)
    ora = OracleBM(NB, B, order)
    live, next_seq = [], 0
    for it in range(600):
        op = rng.random()
        if op < 0.15 or not live:
            n = int(rng.integers(0, 3 * B))
            try:
                ora.add_seq(next_seq, n)
                ok = True
            except OutOfBlocks:
                ok = False
            if ok:
                lib_bm.add_seq(next_seq, n)
                live.append(next_seq)
            else:
                with pytest.raises(pkv_lib.PkvError) as e:
                    lib_bm.add_seq(next_seq, n)
                assert e.value.status == 5
            next_seq += 1
        elif op < 0.3:
            p = int(rng.choice(live))
            ora.fork(p, next_seq)
            lib_bm.fork(p, next_seq)
            live.append(next_seq)
            next_seq += 1
        elif op < 0.4 and len(live) > 1:
            s = int(live.pop(int(rng.integers(len(live)))))
            ora.free_seq(s)
            lib_bm.free_seq(s)
        else:
            k = int(rng.integers(1, len(live) + 1))
            seqs = sorted(int(x) for x in rng.choice(live, size=k, replace=False))
            if len(ora.free) < 2 * len(seqs):
                continue
            s1, p1 = ora.step(seqs)
            s2, p2 = lib_bm.step(seqs)
            assert s2.tolist() == s1
            assert p2.tolist() == [list(p) for p in p1]
        _same_state(lib_bm, ora, live)
    for s in live:
        L = ora.lens[s]
        assert lib_bm.slots(s, 0, L).tolist() == ora.slots(s, 0, L)


@pytest.mark.parametrize("name,kw", [("tiny_fp32", {}), ("mha_bf16", {}), ("gqa_bf16", {}),
                                      ("cow_fp16_p1020", {}), ("cow_fp16_p1024", {}),
                                      ("long_bf16_b16", {}), ("long_bf16_b32", {})])
def test_workload_tables_match_oracle(pkv_lib, name, kw):
    """Replaying a workload's operations gives the same tables, slots and copy pairs."""
    w = synth.by_name(name, **kw)
    lib_bm = pkv_lib.BlockManager(w.num_blocks, w.block_size, w.free_order)
    ora = OracleBM(w.num_blocks, w.block_size, w.free_order)
    for seq, n in w.prefill:
        lib_bm.add_seq(seq, n)
        ora.add_seq(seq, n)
        if seq < 3:
            assert lib_bm.slots(seq, 0, n).tolist() == ora.slots(seq, 0, n)
    for p, c in w.forks:
        lib_bm.fork(p, c)
        ora.fork(p, c)
    for seqs in w.steps:
        s1, p1 = ora.step(seqs)
        s2, p2 = lib_bm.step(seqs)
        assert s2.tolist() == s1 and p2.tolist() == [list(p) for p in p1]
    t1 = np.asarray(ora.block_tables(w.batch, w.max_blocks_per_seq, 0), np.int32)
    t2 = lib_bm.block_tables(w.batch, w.max_blocks_per_seq, 0)
    assert (t1 == t2).all()
    assert [lib_bm.seq_len(int(s)) for s in w.batch] == w.context_lens.tolist()
