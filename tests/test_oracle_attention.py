"""Pins for the oracle's decode attention (CPU only).

Each pin comes from outside the oracle's own formula: brute force with Python
loops on a contiguous layout, torch's scaled_dot_product_attention in float64,
closed forms, invariance under physical placement, and the fp64 identity of the
partitioned form.
"""
import math

import numpy as np
import pytest
import torch

from oracle.attention import paged_attention_decode, partitioned_attention, softmax_attention, gather_context
from oracle.block_manager import BlockManager
from oracle.kv_cache import Pool, paged_kv_write, copy_blocks
from oracle.numerics import widen


def _f32_bits(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)


def _place(K, V, lengths, B, num_blocks, order, dtype="f32", fill=0x7FC00000):
    """Store logical per-sequence K/V [L, H, D] (bits) into a pool in the given free order."""
    H, D = K[0].shape[1], K[0].shape[2]
    bm = BlockManager(num_blocks, B, order)
    pool = Pool(num_blocks, H, D, B, dtype, fill_bits=fill)
    W = max(1, max(-(-L // B) for L in lengths))
    for s, L in enumerate(lengths):
        bm.add_seq(s, L)
        if L:
            paged_kv_write(pool, K[s], V[s], bm.slots(s, 0, L))
    tables = np.asarray(bm.block_tables(range(len(lengths)), W, pad=0), dtype=np.int32)
    return pool, tables


def _brute(q, K, V, scale, G):
    """Python loops with math.exp / math.fsum on contiguous lists."""
    Hq, D = len(q), len(q[0])
    L = len(K)
    out = []
    for h in range(Hq):
        g = h // G
        s = [scale * math.fsum(q[h][d] * K[j][g][d] for d in range(D)) for j in range(L)]
        m = max(s)
        p = [math.exp(x - m) for x in s]
        tot = math.fsum(p)
        out.append([math.fsum(p[j] * V[j][g][d] for j in range(L)) / tot for d in range(D)])
    return out


@pytest.mark.parametrize("G", [1, 2])
def test_brute_force_tiny(G):
    rng = np.random.default_rng(5 + G)
    lengths = [5, 3]
    Hkv, D, B = 2, 4, 2
    Hq = Hkv * G
    K = [_f32_bits(rng.standard_normal((L, Hkv, D))) for L in lengths]
    V = [_f32_bits(rng.standard_normal((L, Hkv, D))) for L in lengths]
    q = _f32_bits(rng.standard_normal((2, Hq, D)))
    pool, tables = _place(K, V, lengths, B, 10, rng.permutation(10))
    out = paged_attention_decode(q, "f32", pool, tables, np.asarray(lengths), 0.5)
    for b, L in enumerate(lengths):
        ref = _brute(widen(q[b], "f32").tolist(), widen(K[b], "f32").tolist(),
                     widen(V[b], "f32").tolist(), 0.5, G)
        np.testing.assert_allclose(out[b], np.asarray(ref), rtol=0, atol=1e-14)


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 2), (12, 3)])
def test_matches_torch_sdpa_float64(Hq, Hkv):
    rng = np.random.default_rng(Hq * 10 + Hkv)
    lengths = [1, 17, 40, 33]
    D, B = 16, 16
    K = [_f32_bits(rng.standard_normal((L, Hkv, D))) for L in lengths]
    V = [_f32_bits(rng.standard_normal((L, Hkv, D))) for L in lengths]
    q = _f32_bits(rng.standard_normal((len(lengths), Hq, D)))
    pool, tables = _place(K, V, lengths, B, 20, rng.permutation(20))
    scale = 1.0 / math.sqrt(D)
    out = paged_attention_decode(q, "f32", pool, tables, np.asarray(lengths), scale)
    for b, L in enumerate(lengths):
        qt = torch.from_numpy(widen(q[b], "f32"))[None, :, None, :]          # [1, Hq, 1, D]
        kt = torch.from_numpy(widen(K[b], "f32")).permute(1, 0, 2)[None]    # [1, Hkv, L, D]
        vt = torch.from_numpy(widen(V[b], "f32")).permute(1, 0, 2)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kt.contiguous(), vt.contiguous(), scale=scale, enable_gqa=(Hq != Hkv))
        np.testing.assert_allclose(out[b], ref[0, :, 0, :].numpy(), rtol=0, atol=1e-13)


def test_bf16_and_f16_widening_matches_torch():
    rng = np.random.default_rng(1)
    x = torch.from_numpy(rng.standard_normal(1000).astype(np.float32))
    for dt, name in ((torch.bfloat16, "bf16"), (torch.float16, "f16")):
        t = x.to(dt)
        bits = t.view(torch.int16).numpy().view(np.uint16)
        np.testing.assert_array_equal(widen(bits, name), t.to(torch.float64).numpy())


def test_paged_equals_contiguous_for_any_placement():
    rng = np.random.default_rng(9)
    lengths = [37, 16, 1, 64]
    Hkv, D, B, NB = 2, 8, 16, 12
    K = [_f32_bits(rng.standard_normal((L, Hkv, D))) for L in lengths]
    V = [_f32_bits(rng.standard_normal((L, Hkv, D))) for L in lengths]
    q = _f32_bits(rng.standard_normal((4, 4, D)))
    outs = []
    for trial in range(4):
        order = np.arange(NB) if trial == 0 else rng.permutation(NB)
        pool, tables = _place(K, V, lengths, B, NB, order)
        outs.append(paged_attention_decode(q, "f32", pool, tables, np.asarray(lengths), 0.3))
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])
    # and the identity placement equals attention over the plain contiguous arrays
    for b, L in enumerate(lengths):
        Kc, Vc = widen(K[b], "f32"), widen(V[b], "f32")
        for h in range(4):
            ref = softmax_attention(widen(q[b, h:h + 1], "f32"), Kc[:, h // 2], Vc[:, h // 2], 0.3)
            np.testing.assert_allclose(outs[0][b, h], ref[0], rtol=0, atol=1e-14)


def test_closed_forms():
    rng = np.random.default_rng(2)
    Hkv, D, B = 1, 8, 4
    lengths = [1, 9, 9, 9, 0]
    K = [_f32_bits(rng.standard_normal((L, Hkv, D))) for L in lengths]
    V = [_f32_bits(rng.standard_normal((L, Hkv, D))) for L in lengths]
    # row 2: all keys equal; row 3: key 4 = 40 * q, the rest random
    K[2] = np.repeat(K[2][:1], 9, axis=0)
    q = rng.standard_normal((5, 1, D)).astype(np.float32)
    q[1] = 0.0
    K3 = widen(K[3], "f32")
    K3[4, 0] = 40.0 * q[3, 0]
    K[3] = _f32_bits(K3)
    pool, tables = _place(K, V, lengths, B, 20, rng.permutation(20))
    out = paged_attention_decode(_f32_bits(q), "f32", pool, tables, np.asarray(lengths), 1.0)
    np.testing.assert_array_equal(out[0, 0], widen(V[0], "f32")[0, 0])          # L = 1
    np.testing.assert_allclose(out[1, 0], widen(V[1], "f32")[:, 0].mean(0), atol=1e-15)  # q = 0
    np.testing.assert_allclose(out[2, 0], widen(V[2], "f32")[:, 0].mean(0), atol=1e-15)  # equal keys
    np.testing.assert_allclose(out[3, 0], widen(V[3], "f32")[4, 0], atol=1e-12)  # peaked
    np.testing.assert_array_equal(out[4], 0.0)                                    # empty context


def test_large_logits_do_not_overflow():
    """q x 30: logits near 1e3 overflow exp without the max subtraction."""
    rng = np.random.default_rng(4)
    L, D = 50, 64
    K = [_f32_bits(rng.standard_normal((L, 1, D)))]
    V = [_f32_bits(rng.standard_normal((L, 1, D)))]
    q = _f32_bits(30.0 * rng.standard_normal((1, 1, D)))
    pool, tables = _place(K, V, [L], 16, 8, rng.permutation(8))
    out = paged_attention_decode(q, "f32", pool, tables, np.asarray([L]), 1.0)
    assert np.isfinite(out).all()
    s = widen(K[0], "f32")[:, 0] @ widen(q, "f32")[0, 0]
    np.testing.assert_allclose(out[0, 0], widen(V[0], "f32")[int(np.argmax(s)), 0], atol=1e-9)


@pytest.mark.parametrize("L,T", [(1000, 512), (513, 512), (512, 512), (37, 5), (9, 1), (4096, 512)])
def test_partitioned_lse_identity(L, T):
    rng = np.random.default_rng(L + T)
    q = rng.standard_normal((4, 32))
    K = rng.standard_normal((L, 32))
    V = rng.standard_normal((L, 32))
    direct = softmax_attention(q, K, V, 0.2)
    part = partitioned_attention(q, K, V, 0.2, T)
    np.testing.assert_allclose(part, direct, rtol=0, atol=1e-12)


def test_unused_slots_and_table_padding_are_never_read():
    """NaN in every slot beyond each length and in the blocks the padding points at."""
    rng = np.random.default_rng(6)
    lengths = [3, 17]
    K = [_f32_bits(rng.standard_normal((L, 1, 8))) for L in lengths]
    V = [_f32_bits(rng.standard_normal((L, 1, 8))) for L in lengths]
    pool, tables = _place(K, V, lengths, 16, 8, rng.permutation(8))
    tables = np.concatenate([tables, np.full((2, 3), 7, np.int32)], axis=1)  # block 7 never allocated
    q = _f32_bits(rng.standard_normal((2, 1, 8)))
    out = paged_attention_decode(q, "f32", pool, tables, np.asarray(lengths), 0.5)
    assert np.isfinite(out).all()


def test_cow_samples_agree_on_shared_prefix():
    """After copy-on-write, every sample still holds the prompt: same q over the prefix -> same output."""
    rng = np.random.default_rng(8)
    B, P, Hkv, D = 16, 20, 2, 8
    bm = BlockManager(32, B, rng.permutation(32))
    pool = Pool(32, Hkv, D, B, "f16", fill_bits=0x7E00)
    kp = np.asarray(torch.randn(P, Hkv, D, dtype=torch.float16).view(torch.int16).numpy().view(np.uint16))
    vp = np.asarray(torch.randn(P, Hkv, D, dtype=torch.float16).view(torch.int16).numpy().view(np.uint16))
    bm.add_seq(0, P)
    paged_kv_write(pool, kp, vp, bm.slots(0, 0, P))
    for c in (1, 2, 3):
        bm.fork(0, c)
    for _ in range(3):
        slots, pairs = bm.step([0, 1, 2, 3])
        copy_blocks(pool, pairs)
        kn = rng.integers(0, 0x3C00, size=(4, Hkv, D), dtype=np.uint16)
        paged_kv_write(pool, kn, kn, slots)
    tables = np.asarray(bm.block_tables(range(4), 3, 0), np.int32)
    assert len({tuple(t[:2]) for t in tables}) == 4  # the tail block diverged for everyone
    q1 = torch.randn(1, 4, D, dtype=torch.float16).view(torch.int16).numpy().view(np.uint16)
    q = np.repeat(q1, 4, axis=0)
    out = paged_attention_decode(q, "f16", pool, tables, np.full(4, P), 0.35)
    for s in (1, 2, 3):
        np.testing.assert_array_equal(out[s], out[0])
    full = paged_attention_decode(q, "f16", pool, tables, np.full(4, P + 3), 0.35)
    assert not np.array_equal(full[1], full[0])


def test_gather_reads_only_table_prefix():
    pool = Pool(4, 1, 4, 4, "f32", fill_bits=0)
    for b in range(4):
        pool.k[b] = _f32_bits(np.full((1, 1, 4, 4), b))
    Kg, _ = gather_context(pool, np.array([2, 0, 3, 1]), 9)
    assert Kg[:, 0, 0].tolist() == [2.0] * 4 + [0.0] * 4 + [3.0]
