"""The library's host block manager against the oracle's, bit for bit (CPU only)."""
import numpy as np
import pytest

import synth
from oracle import tables as oracle_tables
from oracle.accounting import class_block_size, paged_footprint
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
    # two-level tables of the final state, in a shuffled sequence order
    E = 512 // B
    seqs = [int(x) for x in rng.permutation(live)]
    width = max(-(-len(ora.block_table(x)) // E) for x in seqs) + 1
    d, lv = lib_bm.block_tables_2l(seqs, width, 7)
    od, olv = oracle_tables.two_level([ora.block_table(x) for x in seqs], B, width, 7)
    assert np.array_equal(d, od) and np.array_equal(lv, olv)


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


@pytest.mark.parametrize("B", [4, 16])
def test_prefix_cache_matches_oracle(pkv_lib, B):
    """Random request streams over a small pool: prompts share system prefixes, some
    repeat exactly, sequences decode, fork and leave; evictions happen under pressure.
    Tables, counts, cached-block counts and every cached-token answer must match."""
    from oracle.block_manager import PrefixCachingBlockManager
    rng = np.random.default_rng(7 + B)
    NB = 60
    order = rng.permutation(NB)
    lib_bm = pkv_lib.BlockManager(NB, B, order, prefix_cache=True)
    ora = PrefixCachingBlockManager(NB, B, order)
    systems = [rng.integers(0, 1000, size=int(rng.integers(B, 5 * B))).tolist() for _ in range(4)]
    seen = []
    live, nxt, hits = [], 0, 0
    for it in range(700):
        op = rng.random()
        if op < 0.35 or not live:
            if seen and rng.random() < 0.2:
                prompt = list(seen[int(rng.integers(len(seen)))])
            else:
                prompt = systems[int(rng.integers(4))] + rng.integers(0, 1000, size=int(rng.integers(0, 2 * B))).tolist()
            if not prompt:
                continue
            try:
                c1 = ora.add_seq_tokens(nxt, prompt)
                ok = True
            except OutOfBlocks:
                ok = False
            if ok:
                c2 = lib_bm.add_seq_tokens(nxt, prompt)
                assert c2 == c1
                hits += c1 > 0
                live.append(nxt)
                seen.append(prompt)
            else:
                with pytest.raises(pkv_lib.PkvError) as e:
                    lib_bm.add_seq_tokens(nxt, prompt)
                assert e.value.status == 5
            nxt += 1
        elif op < 0.45:
            p = int(rng.choice(live))
            ora.fork(p, nxt)
            lib_bm.fork(p, nxt)
            live.append(nxt)
            nxt += 1
        elif op < 0.75 and live:
            s = live.pop(int(rng.integers(len(live))))
            ora.free_seq(s)
            lib_bm.free_seq(s)
        else:
            seqs = sorted(live)
            if ora._available() < 2 * len(seqs):
                continue
            s1, p1 = ora.step(seqs)
            s2, p2 = lib_bm.step(seqs)
            assert s2.tolist() == s1 and p2.tolist() == [list(p) for p in p1]
        for s in live:
            assert lib_bm.block_table(s) == ora.block_table(s)
        assert [lib_bm.refcount(b) for b in range(NB)] == ora.refcount
        assert lib_bm.num_free() == ora._available()
        assert lib_bm.num_cached() == len(ora.cached)
    assert hits > 20  # the stream did exercise reuse


def test_block_tables16_match_int32_tables(pkv_lib):
    """16-bit tables hold the int32 tables' ids as unsigned 16-bit values, including ids
    above 32767, and the same padding; ids or padding that do not fit are rejected."""
    NB = 65536
    order = list(range(NB - 1, -1, -1))  # the first blocks handed out have ids >= 32768
    bm = pkv_lib.BlockManager(NB, 16, order)
    bm.add_seq(0, 40)
    bm.add_seq(1, 0)
    bm.add_seq(2, 17)
    t32 = bm.block_tables([2, 0, 1], 4, 9)
    t16 = bm.block_tables16([2, 0, 1], 4, 9)
    assert t16.dtype == np.int16 and t16.shape == (3, 4)
    assert np.array_equal(t16.view(np.uint16).astype(np.int32), t32)
    assert t32.max() == NB - 1 and t16.view(np.uint16).max() == NB - 1
    with pytest.raises(pkv_lib.PkvError):
        bm.block_tables16([0], 4, 65536)
    with pytest.raises(pkv_lib.PkvError):
        bm.block_tables16([0], 2, 0)  # three blocks do not fit a width of two
    big = pkv_lib.BlockManager(NB + 1, 16, list(range(NB, -1, -1)))
    big.add_seq(0, 16)
    assert big.block_table(0) == [NB]
    with pytest.raises(pkv_lib.PkvError):
        big.block_tables16([0], 1, 0)


def test_length_class_pools_match_the_accounting(pkv_lib):
    """The library's managers allocate, for each block-size choice of the length-class
    batch, exactly the slots and table entries the oracle's accounting counts."""
    lw = synth.lenclass_bf16()
    lens = [int(x) for x in lw.base.context_lens]
    choices = {"all_b16": ([lw.base], [16] * len(lens)), "all_b32": ([lw.all32], [32] * len(lens)),
               "by_class": ([lw.short, lw.long], [class_block_size(x, lw.threshold) for x in lens])}
    for name, (parts, Bs) in choices.items():
        alloc = entries = 0
        for w in parts:
            bm = pkv_lib.BlockManager(w.num_blocks, w.block_size, w.free_order)
            for s, n in w.prefill:
                bm.add_seq(s, n)
            bm.step(w.steps[-1])
            used = w.num_blocks - bm.num_free()
            alloc += used * w.block_size
            entries += used
        assert (alloc, entries) == paged_footprint(lens, Bs)[::2], name
