"""Pins for the oracle's causal chunk (prefill) attention over a paged pool (CPU only).

Each pin comes from outside the oracle's own formula:
* a whole-sequence chunk equals torch's scaled_dot_product_attention with its own
  causal mask (is_causal=True) in float64;
* a chunk at the end of a longer context equals the last rows of that whole-sequence
  result, which fixes the causal alignment (the chunk's last token sees everything);
* a one-token chunk equals the decode oracle (pinned in test_oracle_attention.py);
* identical keys give uniform weights, so row t is the mean of V over positions
  0..p (a closed form);
* Python loops with math.fsum on a tiny case;
* the result does not depend on where the blocks sit in the pool.
"""
import math

import numpy as np
import pytest
import torch

from oracle.attention import paged_attention_decode, paged_attention_prefill
from oracle.block_manager import BlockManager
from oracle.kv_cache import Pool, paged_kv_write


def _f32_bits(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)


def _f32(bits):
    return np.asarray(bits).view(np.float32).astype(np.float64)


def _place(K, V, lengths, B, num_blocks, order):
    """Store per-sequence K/V ``[L, H, D]`` (fp32 bits) into a pool in the given free order."""
    H, D = K[0].shape[1], K[0].shape[2]
    bm = BlockManager(num_blocks, B, order)
    pool = Pool(num_blocks, H, D, B, "f32", fill_bits=0x7FC00000)
    W = max(1, max(-(-L // B) for L in lengths))
    for s, L in enumerate(lengths):
        bm.add_seq(s, L)
        paged_kv_write(pool, K[s], V[s], bm.slots(s, 0, L))
    tables = np.asarray(bm.block_tables(range(len(lengths)), W, pad=0), dtype=np.int32)
    return pool, tables


def _case(seed, lengths, chunks, Hq, Hkv, D, B, extra_blocks=3):
    rng = np.random.default_rng(seed)
    K = [_f32_bits(rng.standard_normal((L, Hkv, D))) for L in lengths]
    V = [_f32_bits(rng.standard_normal((L, Hkv, D))) for L in lengths]
    nb = sum(-(-L // B) for L in lengths) + extra_blocks
    pool, tables = _place(K, V, lengths, B, nb, rng.permutation(nb))
    qs = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q = _f32_bits(rng.standard_normal((int(qs[-1]), Hq, D)))
    return K, V, pool, tables, qs, q


def _sdpa_causal(q, K, V, scale, G):
    """torch SDPA (float64, is_causal) of ``q [L, Hq, D]`` over ``K, V [L, Hkv, D]``."""
    qt = torch.from_numpy(q).permute(1, 0, 2).unsqueeze(0)                      # [1, Hq, L, D]
    kt = torch.from_numpy(np.repeat(K, G, axis=1)).permute(1, 0, 2).unsqueeze(0).contiguous()
    vt = torch.from_numpy(np.repeat(V, G, axis=1)).permute(1, 0, 2).unsqueeze(0).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    return o[0].permute(1, 0, 2).numpy()                                        # [L, Hq, D]


@pytest.mark.parametrize("G", [1, 4])
def test_whole_sequence_matches_torch_causal_sdpa(G):
    lengths = [37, 16, 1, 50]
    Hkv, D, B = 2, 8, 16
    Hq = Hkv * G
    K, V, pool, tables, qs, q = _case(11 + G, lengths, lengths, Hq, Hkv, D, B)
    scale = 1 / math.sqrt(D)
    got = paged_attention_prefill(q, "f32", pool, tables, np.asarray(lengths), qs, scale)
    for b, L in enumerate(lengths):
        ref = _sdpa_causal(_f32(q[qs[b]:qs[b + 1]]), _f32(K[b]), _f32(V[b]), scale, G)
        np.testing.assert_allclose(got[qs[b]:qs[b + 1]], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("G", [1, 2])
def test_chunk_equals_last_rows_of_whole_sequence(G):
    """A chunk of C tokens at the end of an L-token context is the last C rows of
    the whole-sequence causal result (torch SDPA) computed with the same queries."""
    lengths = [45, 33, 20]
    chunks = [7, 33, 1]
    Hkv, D, B = 2, 8, 16
    Hq = Hkv * G
    rng = np.random.default_rng(40 + G)
    K = [_f32_bits(rng.standard_normal((L, Hkv, D))) for L in lengths]
    V = [_f32_bits(rng.standard_normal((L, Hkv, D))) for L in lengths]
    nb = sum(-(-L // B) for L in lengths) + 2
    pool, tables = _place(K, V, lengths, B, nb, rng.permutation(nb))
    full_q = [_f32_bits(rng.standard_normal((L, Hq, D))) for L in lengths]
    q = np.concatenate([full_q[b][L - C:] for b, (L, C) in enumerate(zip(lengths, chunks))])
    qs = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    scale = 0.3
    got = paged_attention_prefill(q, "f32", pool, tables, np.asarray(lengths), qs, scale)
    for b, (L, C) in enumerate(zip(lengths, chunks)):
        ref = _sdpa_causal(_f32(full_q[b]), _f32(K[b]), _f32(V[b]), scale, G)[L - C:]
        np.testing.assert_allclose(got[qs[b]:qs[b + 1]], ref, rtol=1e-12, atol=1e-12)


def test_one_token_chunks_equal_decode():
    lengths = [1, 17, 64, 100]
    Hq, Hkv, D, B = 8, 2, 16, 16
    K, V, pool, tables, qs, q = _case(7, lengths, [1] * len(lengths), Hq, Hkv, D, B)
    got = paged_attention_prefill(q, "f32", pool, tables, np.asarray(lengths), qs, 0.25)
    ref = paged_attention_decode(q, "f32", pool, tables, np.asarray(lengths), 0.25)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-14)


def test_identical_keys_give_prefix_means():
    """Equal scores: p_j = 1/(p+1) for every visible j, so row t is the mean of
    V[0..p] with p = L - C + t."""
    L, C, Hkv, D, B, G = 40, 12, 2, 4, 16, 2
    rng = np.random.default_rng(3)
    k_row = rng.standard_normal((1, Hkv, D))
    K = [_f32_bits(np.repeat(k_row, L, axis=0))]
    Vf = rng.standard_normal((L, Hkv, D)).astype(np.float32)
    V = [_f32_bits(Vf)]
    pool, tables = _place(K, V, [L], B, 5, rng.permutation(5))
    q = _f32_bits(rng.standard_normal((C, Hkv * G, D)))
    got = paged_attention_prefill(q, "f32", pool, tables, np.asarray([L]), np.asarray([0, C]), 0.5)
    cum = np.cumsum(Vf.astype(np.float64), axis=0)
    for t in range(C):
        p = L - C + t
        for h in range(Hkv * G):
            np.testing.assert_allclose(got[t, h], cum[p, h // G] / (p + 1), rtol=1e-12, atol=1e-13)


def test_brute_force_tiny():
    L, C, Hkv, D, B, G = 6, 4, 1, 4, 2, 2
    K, V, pool, tables, qs, q = _case(19, [L], [C], Hkv * G, Hkv, D, B)
    scale = 0.7
    got = paged_attention_prefill(q, "f32", pool, tables, np.asarray([L]), qs, scale)
    Kf, Vf, qf = _f32(K[0]).tolist(), _f32(V[0]).tolist(), _f32(q).tolist()
    for t in range(C):
        p = L - C + t
        for h in range(Hkv * G):
            g = h // G
            s = [scale * math.fsum(qf[t][h][d] * Kf[j][g][d] for d in range(D)) for j in range(p + 1)]
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            tot = math.fsum(w)
            ref = [math.fsum(w[j] * Vf[j][g][d] for j in range(p + 1)) / tot for d in range(D)]
            np.testing.assert_allclose(got[t, h], ref, rtol=1e-12, atol=1e-13)


def test_placement_does_not_change_the_result():
    lengths = [30, 19]
    chunks = [9, 19]
    Hq, Hkv, D, B = 4, 2, 8, 8
    rng = np.random.default_rng(23)
    K = [_f32_bits(rng.standard_normal((L, Hkv, D))) for L in lengths]
    V = [_f32_bits(rng.standard_normal((L, Hkv, D))) for L in lengths]
    qs = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q = _f32_bits(rng.standard_normal((int(qs[-1]), Hq, D)))
    nb = 12
    outs = []
    for order in (np.arange(nb), rng.permutation(nb)):
        pool, tables = _place(K, V, lengths, B, nb, order)
        outs.append(paged_attention_prefill(q, "f32", pool, tables, np.asarray(lengths), qs, 0.4))
    np.testing.assert_array_equal(outs[0], outs[1])


def test_rejects_chunk_longer_than_context():
    K, V, pool, tables, qs, q = _case(2, [4], [4], 2, 1, 4, 4)
    with pytest.raises(ValueError):
        paged_attention_prefill(q, "f32", pool, tables, np.asarray([3]), qs, 1.0)


def test_sequence_subset_matches_full_result():
    lengths = [20, 33, 9]
    chunks = [5, 33, 2]
    K, V, pool, tables, qs, q = _case(31, lengths, chunks, 4, 2, 8, 8)
    full = paged_attention_prefill(q, "f32", pool, tables, np.asarray(lengths), qs, 0.5)
    part = paged_attention_prefill(q, "f32", pool, tables, np.asarray(lengths), qs, 0.5, seqs=[1])
    np.testing.assert_array_equal(part[qs[1]:qs[2]], full[qs[1]:qs[2]])
    assert not part[:qs[1]].any() and not part[qs[2]:].any()
