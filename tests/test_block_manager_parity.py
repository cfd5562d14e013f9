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


@pytest.mark.parametrize("B", [4, 16])
def test_moves_between_two_managers_match_oracle(pkv_lib, B):
    """Random histories over a device manager and a host manager, with sequences
    moved back and forth in groups (swap-out / swap-in), failing moves included."""
    from oracle.block_manager import move_seqs
    rng = np.random.default_rng(100 + B)
    NG, NC = 120, 90
    og, oc = rng.permutation(NG), rng.permutation(NC)
    lg, lc = pkv_lib.BlockManager(NG, B, og), pkv_lib.BlockManager(NC, B, oc)
    rg, rc = OracleBM(NG, B, og), OracleBM(NC, B, oc)
    on_gpu, on_cpu, nxt = [], [], 0
    for it in range(500):
        op = rng.random()
        if op < 0.2 or not on_gpu:
            n = int(rng.integers(1, 4 * B))
            if len(rg.free) >= -(-n // B):
                rg.add_seq(nxt, n)
                lg.add_seq(nxt, n)
                on_gpu.append(nxt)
            nxt += 1
        elif op < 0.3:
            p = int(rng.choice(on_gpu))
            rg.fork(p, nxt)
            lg.fork(p, nxt)
            on_gpu.append(nxt)
            nxt += 1
        elif op < 0.45:
            k = int(rng.integers(1, min(4, len(on_gpu)) + 1))
            seqs = [int(x) for x in rng.choice(on_gpu, size=k, replace=False)]
            try:
                p1 = move_seqs(rg, rc, seqs)
                ok = True
            except OutOfBlocks:
                ok = False
            if ok:
                p2 = lg.move_seqs(lc, seqs)
                assert p2.tolist() == [list(p) for p in p1]
                on_gpu = [s for s in on_gpu if s not in seqs]
                on_cpu += seqs
            else:
                with pytest.raises(pkv_lib.PkvError) as e:
                    lg.move_seqs(lc, seqs)
                assert e.value.status == 5
        elif op < 0.6 and on_cpu:
            k = int(rng.integers(1, min(4, len(on_cpu)) + 1))
            seqs = [int(x) for x in rng.choice(on_cpu, size=k, replace=False)]
            try:
                p1 = move_seqs(rc, rg, seqs)
                ok = True
            except OutOfBlocks:
                ok = False
            if ok:
                p2 = lc.move_seqs(lg, seqs)
                assert p2.tolist() == [list(p) for p in p1]
                on_cpu = [s for s in on_cpu if s not in seqs]
                on_gpu += seqs
            else:
                with pytest.raises(pkv_lib.PkvError) as e:
                    lc.move_seqs(lg, seqs)
                assert e.value.status == 5
        elif op < 0.7 and len(on_gpu) > 1:
            s = on_gpu.pop(int(rng.integers(len(on_gpu))))
            rg.free_seq(s)
            lg.free_seq(s)
        else:
            seqs = sorted(on_gpu)
            if len(rg.free) < 2 * len(seqs):
                continue
            s1, p1 = rg.step(seqs)
            s2, p2 = lg.step(seqs)
            assert s2.tolist() == s1 and p2.tolist() == [list(p) for p in p1]
        _same_state(lg, rg, on_gpu)
        _same_state(lc, rc, on_cpu)
    # invalid moves are rejected and change nothing
    if on_gpu:
        s = on_gpu[0]
        free_before = lg.num_free()
        with pytest.raises(pkv_lib.PkvError):
            lg.move_seqs(lc, [s, s])
        with pytest.raises(pkv_lib.PkvError):
            lg.move_seqs(lc, [10 ** 6])
        assert lg.num_free() == free_before
