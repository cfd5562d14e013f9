"""The benchmark's algorithmic byte counts (CPU only): the figures the roofline divides."""
import numpy as np

import bench
import synth


def test_unique_tokens_counts_shared_blocks_once():
    # block 5 is shared by both sequences (a forked prefix); sequence 1 reads 3 of its
    # slots, sequence 0 all 4; blocks 7 and 9 are private
    tables = np.array([[5, 7, 0], [5, 9, 0]])
    assert bench.unique_tokens(tables, [6, 3], 4) == 4 + 2
    assert bench.unique_tokens(tables, [6, 7], 4) == 4 + 2 + 3
    assert bench.unique_tokens(tables, [0, 0], 4) == 0


def test_algorithmic_bytes_items():
    w = synth.gqa_bf16(num_seqs=4, max_len=3000)
    lens = np.array([1, 1024, 1025, 3000])
    ab = bench.algorithmic_bytes(w, lens)
    H, D, e, Hq = 8, 128, 2, 32
    assert ab["kv"] == ab["kv_unique"] == 2 * lens.sum() * H * D * e
    assert ab["q"] == 4 * Hq * D * e
    # rows of one partition write their output; the others write and re-read partials
    assert ab["out"] == 2 * Hq * D * e
    assert ab["partials"] == 2 * (2 + 3) * Hq * (D + 2) * 4
    # one table entry per block per KV head, and one context length per sequence
    blocks = sum(-(-int(L) // 16) for L in lens)
    assert ab["tables"] == H * blocks * 4 + 4 * 4
    assert bench.algorithmic_bytes(w, lens, "int16")["tables"] == H * blocks * 2 + 4 * 4
    leaves = sum(-(-(-(-int(L) // 16)) // 32) for L in lens)
    assert bench.algorithmic_bytes(w, lens, "two_level")["tables"] == H * blocks * 4 + 4 * 4 + H * leaves * 4
    # with 2048-token partitions only the 3000-token row is split (2 partitions)
    assert bench.algorithmic_bytes(w, lens, partition_tokens=2048)["partials"] == 2 * 2 * Hq * (D + 2) * 4
    assert bench.algorithmic_bytes(w, lens, partition_tokens=2048)["out"] == 3 * Hq * D * e
    u = bench.algorithmic_bytes(w, lens, unique=100)
    assert u["kv_unique"] == 2 * 100 * H * D * e and u["total"] == ab["total"] - ab["kv"] + u["kv_unique"]


def test_spread_and_host_cpus():
    s = bench.spread([1.0, 2.0, 3.0, 4.0, 5.0, 6.0, 7.0, 8.0, 9.0, 10.0, 11.0])
    assert s == {"median": 6.0, "p10": 2.0, "p90": 10.0, "n": 11}
    h = bench.host_cpus()
    assert h["cpu_count"] >= h["affinity"] >= 1
