"""Checks of the seeded input generators and of the oracle replay of small workloads (CPU only)."""
import numpy as np
import torch

import synth
from oracle.replay import replay


def test_values_are_deterministic_and_rne_rounded():
    a = synth.normal_bits((1, 2, 3), (5, 7), "bf16")
    b = synth.normal_bits((1, 2, 3), (5, 7), "bf16")
    assert a.dtype == np.uint16 and (a == b).all()
    f32 = np.random.default_rng([1, 2, 3]).standard_normal(35, dtype=np.float32)
    # round-to-nearest-even by hand: add 0x7FFF + lsb, keep the top 16 bits
    u = f32.view(np.uint32).astype(np.uint64)
    rne = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    assert (a.reshape(-1) == rne).all()
    h = synth.normal_bits((4,), (100,), "f16")
    assert (h == np.random.default_rng([4]).standard_normal(100, dtype=np.float32).astype(np.float16).view(np.uint16)).all()


def test_length_mix_ranges_and_proportions():
    rng = np.random.default_rng(0)
    L = synth.skewed_lengths(rng, 200000)
    assert L.min() >= 32 and L.max() <= 4095
    assert abs((L < 512).mean() - 0.70) < 0.01
    assert abs(((L >= 512) & (L < 2048)).mean() - 0.25) < 0.01
    L2 = synth.skewed_lengths(np.random.default_rng(1), 200000, 2)
    assert L2.min() >= 64 and L2.max() <= 8191
    assert abs(L2.mean() - 1327.5) < 10


def test_config_shapes():
    t = synth.tiny_fp32()
    assert t.num_blocks == 64 and t.max_blocks_per_seq == 4 and (t.context_lens >= 1).all()
    assert (t.context_lens <= 64).all() and sorted(t.free_order.tolist()) == list(range(64))
    m = synth.mha_bf16()
    assert m.num_seqs == 64 and m.max_blocks_per_seq == 256 and m.num_kv_heads == 32
    need = sum(-(-int(L) // 16) for L in m.context_lens)
    assert m.num_blocks == int(np.ceil(1.1 * need))
    g = synth.gqa_bf16()
    assert g.num_seqs == 256 and g.max_blocks_per_seq == 512 and g.num_q_heads // g.num_kv_heads == 4
    lg = synth.long_bf16(16)
    assert lg.num_blocks == 65536 and lg.max_blocks_per_seq == 8192
    assert lg.kv_bytes_logical() == 4 * 2 ** 30
    assert synth.long_bf16(32).num_blocks == 32768


def test_cow_workload_copies_three_tails_per_prompt():
    w = synth.cow_fp16(1020, num_prompts=3, max_suffix=9)
    r = replay(w, synth.NAN_BITS["f16"])
    assert r.copies == 3 * 3
    assert (r.context_lens == w.context_lens).all()
    w2 = synth.cow_fp16(1024, num_prompts=3, max_suffix=9)
    assert replay(w2, synth.NAN_BITS["f16"]).copies == 0


def test_replayed_pool_holds_each_sequence_context():
    w = synth.gqa_bf16(num_seqs=6, max_len=300)
    ctx = w.all_context_kv()
    r = replay(w, synth.NAN_BITS["bf16"], context=ctx)
    kstep, vstep = w.step_kv(0)
    for b in range(w.num_seqs):
        L = int(r.context_lens[b])
        j = np.arange(L)
        blocks = r.block_tables[b][j // 16]
        k = r.pool.k_at(blocks, j % 16)
        assert (k[:L - 1] == ctx[b][0]).all() and (k[L - 1] == kstep[b]).all()
        v = r.pool.v_at(blocks, j % 16)
        assert (v[:L - 1] == ctx[b][1]).all() and (v[L - 1] == vstep[b]).all()


def test_prefill_workloads_are_consistent():
    import synth
    for name in synth.PREFILL_WORKLOADS:
        w = synth.by_name(name)
        qs = w.query_start()
        assert qs[0] == 0 and qs[-1] == w.num_tokens and np.all(np.diff(qs) == w.chunk_lens)
        assert np.all(w.chunk_lens <= w.context_lens) and np.all(w.chunk_lens > 0)
        need = sum(-(-int(L) // w.block_size) for L in w.context_lens)
        assert w.num_blocks >= need and sorted(w.free_order.tolist()) == list(range(w.num_blocks))
        assert w.max_blocks_per_seq * w.block_size >= w.context_lens.max()
        # flops: 4 * Hq * D per visible (query row, key) pair, counted by brute force on a prefix of the batch
        L, C = w.context_lens.astype(int), w.chunk_lens.astype(int)
        pairs = sum(sum(L[b] - C[b] + t + 1 for t in range(C[b])) for b in range(w.num_seqs))
        assert w.flops() == 4 * w.num_q_heads * w.head_dim * pairs


def test_swap_workload_fits_its_host_pool():
    import synth
    sw = synth.by_name("swap_bf16")
    w = sw.base
    need = sum(-(-int(w.context_lens[i]) // w.block_size) for i in range(len(sw.moved)))
    assert sw.host_blocks >= need and sw.moved == list(range(len(sw.moved)))
