"""The C-ABI library loads and exports every declared symbol; host-side paths (CPU only)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "pkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(pkv_lib):
    names = _declared_functions()
    assert len(names) >= 20
    lib = ctypes.CDLL(pkv_lib.library_path())
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings_and_version(pkv_lib):
    lib = pkv_lib.load()
    assert lib.pkv_version().decode().startswith("pkv")
    assert lib.pkv_status_string(0) == b"PKV_OK"
    assert lib.pkv_status_string(5) == b"PKV_ERR_OUT_OF_BLOCKS"


def test_workspace_and_pool_sizes(pkv_lib):
    lib = pkv_lib.load()
    # partial outputs (8 sequences x 32 heads x 257 slots x 128 floats: 512-token
    # partitions of 131072 tokens, plus one for a split at the end of a shared prefix),
    # (max, sum) pairs, the item list (4 ints an item), per-row counters, per-sequence
    # partial counts, group records (4 ints), members and their own tokens, and a
    # counter block, each 256-byte aligned
    n = lib.pkv_paged_attention_workspace_bytes(8, 32, 128, 8192, 16)
    parts = 8192 * 16 // 512 + 1
    al = lambda x: (x + 255) // 256 * 256
    assert n == (al(8 * 32 * parts * 128 * 4) + al(8 * 32 * parts * 2 * 4) + al(8 * parts * 16) + al(8 * 32 * 4)
                 + al(8 * 4) + al(8 * 16) + al(8 * 4) + al(8 * 4) + 256)
    assert lib.pkv_paged_attention_workspace_bytes(-1, 32, 128, 8, 16) == 0
    d = pkv_lib.PoolDesc(65536, 16, 8, 128, 2)
    assert lib.pkv_pool_bytes(ctypes.byref(d)) == 2 * 2 ** 30


def test_host_side_argument_errors(pkv_lib):
    """Invalid arguments are rejected on the host, before any device work."""
    lib = pkv_lib.load()
    P = pkv_lib.PoolDesc
    fake = ctypes.c_void_p(0x1000)
    st = lib.pkv_paged_kv_write(None, fake, fake, fake, fake, fake, 4, None)
    assert st == 1 and b"null pool" in lib.pkv_last_error()
    st = lib.pkv_paged_kv_write(ctypes.byref(P(64, 24, 8, 128, 2)), fake, fake, fake, fake, fake, 4, None)
    assert st == 2 and b"block_size" in lib.pkv_last_error()
    st = lib.pkv_paged_kv_write(ctypes.byref(P(64, 16, 8, 96, 2)), fake, fake, fake, fake, fake, 4, None)
    assert st == 2
    st = lib.pkv_paged_kv_write(ctypes.byref(P(64, 16, 8, 128, 7)), fake, fake, fake, fake, fake, 4, None)
    assert st == 1
    st = lib.pkv_paged_kv_write(ctypes.byref(P(64, 16, 8, 128, 2)), fake, fake, ctypes.c_void_p(0x1008), fake,
                                fake, 4, None)
    assert st == 1 and b"misaligned" in lib.pkv_last_error()
    assert lib.pkv_paged_kv_write(ctypes.byref(P(64, 16, 8, 128, 2)), None, None, None, None, None, 0, None) == 0
    assert lib.pkv_copy_blocks(ctypes.byref(P(64, 16, 8, 128, 2)), fake, fake, None, 3, None) == 1
    assert lib.pkv_copy_blocks(ctypes.byref(P(64, 16, 8, 128, 2)), None, None, None, 0, None) == 0
    d = ctypes.byref(P(64, 16, 8, 128, 2))
    # num_q_heads not a multiple of num_kv_heads
    st = lib.pkv_paged_attention_decode(d, fake, fake, fake, fake, 4, 12, fake, 4, fake, 1.0, fake, 1 << 20, None)
    assert st == 1 and b"multiple" in lib.pkv_last_error()
    # workspace too small
    st = lib.pkv_paged_attention_decode(d, fake, fake, fake, fake, 4, 32, fake, 4, fake, 1.0, fake, 16, None)
    assert st == 3
    # fp32 with 8 query heads per kv head has no kernel
    st = lib.pkv_paged_attention_decode(ctypes.byref(P(64, 16, 4, 128, 0)), fake, fake, fake, fake, 4, 32, fake, 4,
                                        fake, 1.0, fake, 1 << 24, None)
    assert st == 2
    assert lib.pkv_paged_attention_decode(d, None, None, None, None, 0, 32, None, 4, None, 1.0, None, 0, None) == 0
    # 16-bit tables address at most 65536 blocks
    big = ctypes.byref(P(65537, 16, 8, 128, 2))
    for fn in (lib.pkv_paged_attention_decode_t16, lib.pkv_paged_attention_partitions_t16):
        st = fn(big, fake, fake, fake, fake, 4, 32, fake, 4, fake, 1.0, fake, 1 << 24, None)
        assert st == 2 and b"65536" in lib.pkv_last_error()
    st = lib.pkv_paged_attention_prefill_t16(big, fake, fake, fake, fake, 2, 32, fake, 10, 8, fake, 4, fake, 0.1,
                                             fake, 1 << 20, None)
    assert st == 2 and b"65536" in lib.pkv_last_error()
    # at 65536 blocks the 16-bit calls check their arguments like the int32 ones
    full = ctypes.byref(P(65536, 16, 8, 128, 2))
    st = lib.pkv_paged_attention_decode_t16(full, fake, fake, fake, fake, 4, 12, fake, 4, fake, 1.0, fake, 1 << 24, None)
    assert st == 1 and b"multiple" in lib.pkv_last_error()
    st = lib.pkv_paged_attention_partitions_t16(full, fake, fake, fake, fake, 4, 32, ctypes.c_void_p(0x1001), 4, fake,
                                                1.0, fake, 1 << 24, None)
    assert st == 1 and b"misaligned" in lib.pkv_last_error()


def test_noalloc_and_stream_read_host_side_errors(pkv_lib):
    """Sizes beyond the static scratch are rejected before any device call; the
    streaming-read probe checks its arguments."""
    lib = pkv_lib.load()
    d = pkv_lib.PoolDesc(64, 16, 8, 128, 2)
    fake = ctypes.c_void_p(0x1000)
    need = lib.pkv_paged_attention_workspace_bytes(4096, 32, 128, 512, 16)
    assert need > pkv_lib.NOALLOC_SCRATCH_BYTES
    st = lib.pkv_paged_attention_decode_noalloc(ctypes.byref(d), fake, fake, fake, fake, 4096, 32, fake, 512, fake,
                                                0.1, None)
    assert st == 3 and b"static scratch" in lib.pkv_last_error()
    assert lib.pkv_stream_read(fake, 100, 4, 8, fake, None) == 1     # not a multiple of 16
    assert lib.pkv_stream_read(fake, 4096, 4, 3, fake, None) == 1    # unroll
    assert lib.pkv_stream_read(fake, 4096, 0, 8, fake, None) == 1    # workgroups
    assert lib.pkv_stream_read(None, 4096, 4, 8, fake, None) == 1


def test_two_level_host_side_errors(pkv_lib):
    lib = pkv_lib.load()
    P = pkv_lib.PoolDesc
    fake = ctypes.c_void_p(0x1000)
    d = ctypes.byref(P(64, 16, 8, 128, 2))

    def dec(dir_=fake, dw=4, leaves=fake, nl=8, n=4, ws=1 << 24):
        return lib.pkv_paged_attention_decode_2l(d, fake, fake, fake, fake, n, 32, dir_, dw, leaves, nl, fake, 1.0,
                                                 fake, ws, None)

    assert dec(dw=0) == 1 and b"dir_width" in lib.pkv_last_error()
    assert dec(nl=-1) == 1
    assert dec(dw=(1 << 31) // 32) == 1  # dir_width * 32 entries overflows int32
    assert dec(dir_=None) == 1 and b"null" in lib.pkv_last_error()
    assert dec(dir_=ctypes.c_void_p(0x1002)) == 1 and b"misaligned" in lib.pkv_last_error()
    assert dec(leaves=None) == 1 and b"null" in lib.pkv_last_error()
    assert dec(leaves=ctypes.c_void_p(0x1002)) == 1 and b"misaligned" in lib.pkv_last_error()
    # the flat width is dir_width * 32 entries: the workspace is sized for 4 * 32 blocks
    need = lib.pkv_paged_attention_workspace_bytes(4, 32, 128, 4 * 32, 16)
    assert dec(ws=need - 1) == 3
    assert dec(n=0, dir_=None, leaves=None) == 0
    st = lib.pkv_paged_attention_partitions_2l(d, fake, fake, fake, fake, 4, 32, fake, 0, fake, 8, fake, 1.0, fake,
                                               1 << 24, None)
    assert st == 1
    st = lib.pkv_paged_attention_prefill_2l(d, fake, fake, fake, fake, 2, 32, fake, 10, 8, None, 4, fake, 8, fake,
                                            0.1, fake, 1 << 20, None)
    assert st == 1 and b"null" in lib.pkv_last_error()
    st = lib.pkv_paged_attention_prefill_2l(None, fake, fake, fake, fake, 2, 32, fake, 10, 8, fake, 4, fake, 8, fake,
                                            0.1, fake, 1 << 20, None)
    assert st == 1 and b"null pool" in lib.pkv_last_error()
    # the block manager's two-level tables
    bm = pkv_lib.BlockManager(64, 16, list(range(64)))
    bm.add_seq(0, 33 * 16)  # 33 blocks: two 32-entry leaves
    with pytest.raises(pkv_lib.PkvError):
        bm.block_tables_2l([0], 1, 0)
    d2, lv = bm.block_tables_2l([0], 3, 63)
    assert d2.tolist() == [[0, 1, 2]] and lv.shape == (3, 32)
    assert lv[1].tolist() == [32] + [63] * 31 and lv[2].tolist() == [63] * 32
    n = ctypes.c_int32(0)
    assert lib.pkv_bm_block_tables_2l(bm._h, (ctypes.c_int32 * 1)(0), 1, 3, 0, (ctypes.c_int32 * 3)(), None, 0,
                                      ctypes.byref(n)) == 0 and n.value == 3
    out = (ctypes.c_int32 * 64)()
    assert lib.pkv_bm_block_tables_2l(bm._h, (ctypes.c_int32 * 1)(0), 1, 3, 0, (ctypes.c_int32 * 3)(), out, 2,
                                      ctypes.byref(n)) == 1 and b"leaf_cap" in lib.pkv_last_error()
    odd = pkv_lib.BlockManager(8, 24, list(range(8)))
    odd.add_seq(0, 5)
    with pytest.raises(pkv_lib.PkvError):
        odd.block_tables_2l([0], 1, 0)


def test_block_manager_errors(pkv_lib):
    bm = pkv_lib.BlockManager(4, 16, [3, 1, 0, 2])
    bm.add_seq(0, 17)
    with pytest.raises(pkv_lib.PkvError) as e:
        bm.add_seq(0, 1)
    assert e.value.status == 1
    with pytest.raises(pkv_lib.PkvError) as e:
        bm.add_seq(1, 64)
    assert e.value.status == 5
    assert bm.num_free() == 2  # the failed call changed nothing
    with pytest.raises(pkv_lib.PkvError):
        bm.fork(7, 8)
    with pytest.raises(pkv_lib.PkvError):
        pkv_lib.BlockManager(4, 16, [0, 1, 1, 2])
    assert bm.refcount(99) == -1


def test_prefill_host_side_errors(pkv_lib):
    lib = pkv_lib.load()
    P = pkv_lib.PoolDesc
    fake = ctypes.c_void_p(0x1000)
    d = ctypes.byref(P(64, 16, 8, 128, 2))
    args = lambda **kw: dict(dict(k=fake, v=fake, out=fake, q=fake, n=2, hq=32, qs=fake, t=10, mq=8, tab=fake, w=4,
                                  lens=fake, ws=fake, wsb=1 << 20), **kw)

    def call(desc, **kw):
        a = args(**kw)
        return lib.pkv_paged_attention_prefill(desc, a["k"], a["v"], a["out"], a["q"], a["n"], a["hq"], a["qs"],
                                               a["t"], a["mq"], a["tab"], a["w"], a["lens"], 0.1, a["ws"],
                                               a["wsb"], None)

    assert call(None) == 1 and b"null pool" in lib.pkv_last_error()
    assert call(d, hq=12) == 1 and b"multiple" in lib.pkv_last_error()
    # fp32 pools have no prefill kernel
    assert call(ctypes.byref(P(64, 16, 8, 128, 0))) == 2 and b"bf16/fp16" in lib.pkv_last_error()
    assert call(d, qs=None) == 1 and b"null pointer" in lib.pkv_last_error()
    assert call(d, q=ctypes.c_void_p(0x1008)) == 1 and b"misaligned" in lib.pkv_last_error()
    assert call(d, n=-1) == 1
    # workspace: a 256-byte counter block, then 8 bytes per task of the bound
    # ceil(T * G / 64) + N (T = 10 tokens, G = 4, N = 2 -> 3 tasks)
    assert lib.pkv_paged_attention_prefill_workspace_bytes(2, 10, 32, 8) == 256 + 8 * 3
    assert lib.pkv_paged_attention_prefill_workspace_bytes(2, 10, 12, 8) == 0
    assert call(d, wsb=256 + 8 * 3 - 1) == 3 and b"workspace" in lib.pkv_last_error()
    assert call(d, ws=ctypes.c_void_p(0x1010)) == 3
    # nothing to do: no launch, no pointer checks
    assert call(d, n=0, k=None, v=None, out=None, q=None, qs=None, tab=None, lens=None) == 0
    assert call(d, t=0, k=None, v=None, out=None, q=None, qs=None, tab=None, lens=None) == 0


def test_swap_host_side_errors(pkv_lib):
    lib = pkv_lib.load()
    d = ctypes.byref(pkv_lib.PoolDesc(64, 16, 8, 128, 2))
    fake = ctypes.c_void_p(0x1000)
    assert lib.pkv_swap_blocks(d, fake, fake, fake, fake, fake, 0, None) == 0
    assert lib.pkv_swap_blocks(d, fake, None, fake, fake, fake, 3, None) == 1
    assert lib.pkv_swap_blocks(d, fake, fake, ctypes.c_void_p(0x1008), fake, fake, 3, None) == 1
    assert b"misaligned" in lib.pkv_last_error()
    assert lib.pkv_swap_blocks(d, fake, fake, fake, fake, fake, -1, None) == 1
    assert lib.pkv_swap_blocks(None, fake, fake, fake, fake, fake, 1, None) == 1


def test_prefix_cache_switch_and_plain_fallback(pkv_lib):
    bm = pkv_lib.BlockManager(8, 4, list(range(8)))
    assert bm.add_seq_tokens(0, [1, 2, 3, 4, 5]) == 0  # cache off: plain add
    assert pkv_lib.load().pkv_bm_set_prefix_cache(bm._h, 1) == 1  # a manager with sequences cannot switch
    bm.free_seq(0)
    assert pkv_lib.load().pkv_bm_set_prefix_cache(bm._h, 1) == 0
    assert bm.add_seq_tokens(1, [1, 2, 3, 4, 5]) == 0
    assert bm.add_seq_tokens(2, [1, 2, 3, 4, 5]) == 4 and bm.num_cached() == 1


def test_decode_partition_size_rule(pkv_lib):
    """The plan's partition size: 2048 when some context exceeds 1024 tokens and the token
    work per workgroup slot reaches two thirds of the longest item at head size 128, the
    whole longest item at head size 64 (768 slots without a device: 256 compute units x 3)."""
    import synth
    pt = pkv_lib.decode_partition_tokens
    assert pt([], 32, 8) == 1024
    assert pt([1024] * 4096, 32, 8) == 1024            # no context needs a second 1024 partition
    assert pt(synth.gqa_bf16().context_lens, 32, 8) == 2048
    assert pt(synth.gqa_bf16(num_seqs=32).context_lens, 32, 8) == 1024
    assert pt(synth.mha_bf16().context_lens, 32, 32) == 2048
    assert pt(synth.long_bf16(16, num_seqs=1).context_lens, 32, 8) == 2048
    assert pt(synth.cow_fp16(1020).context_lens, 32, 8) == 2048
    assert pt(synth.gqa_bf16(num_seqs=96).context_lens, 32, 8) == 1024
    # the boundary: 3 * tokens * workgroups per item against 2 * longest * slots
    assert pt([2048] + [0] * 15, 32, 8) == 1024            # 3 * 2048 * 8 < 2 * 2048 * 768
    assert pt([2048] * 64, 32, 8) == 2048                  # 3 * 131072 * 8 == 2 * 2048 * 768
    assert pt([2048] * 63, 32, 8) == 1024
    assert pt([3000] * 64, 32, 8) == 2048                  # the longest item is capped at 2048 tokens
    assert pt([3000] + [500] * 256, 32, 8) == 1024         # 131000 tokens: 3 * 131000 * 8 < 2 * 2048 * 768
    assert pt([3000] + [500] * 257, 32, 8) == 2048         # 131500 tokens
    assert pt([2048] * 64, 64, 2) == 1024                  # 32 query heads per kv head: 4 workgroups per item
    assert pt([2048] * 128, 64, 2) == 2048
    # head size 64 with 16-token blocks: 3 * tokens * workgroups per item against
    # 3 * longest * slots; with 32-token blocks the head size-128 threshold
    assert pt([2048] * 64, 32, 8, 64) == 1024
    assert pt([2048] * 96, 32, 8, 64) == 2048              # 3 * 196608 * 8 == 3 * 2048 * 768
    assert pt([2048] * 95, 32, 8, 64) == 1024
    assert pt([2048] * 64, 32, 8, 64, 32) == 2048
    assert pt([2048] * 63, 32, 8, 128, 32) == 1024
    assert pt(synth.gqa_bf16(num_seqs=128).context_lens, 32, 8) == 2048
    assert pt(synth.gqa_bf16(num_seqs=128).context_lens, 32, 8, 64) == 1024
    assert pt(synth.gqa_bf16(num_seqs=128).context_lens, 32, 8, 64, 32) == 2048
    assert pt(synth.gqa_bf16(num_seqs=160).context_lens, 32, 8, 64) == 2048
    lib = pkv_lib.load()
    out = ctypes.c_int32()
    pool = pkv_lib.PoolDesc(1, 16, 8, 128, 2)
    assert lib.pkv_decode_partition_tokens(ctypes.byref(pool), None, 3, 32, ctypes.byref(out)) == 1
    assert lib.pkv_decode_partition_tokens(ctypes.byref(pool), None, 0, 30, ctypes.byref(out)) == 1
    assert lib.pkv_decode_partition_tokens(None, None, 0, 32, ctypes.byref(out)) == 1
    assert lib.pkv_decode_partition_tokens(ctypes.byref(pool), None, 0, 32, ctypes.byref(out)) == 0
    odd = pkv_lib.PoolDesc(1, 16, 8, 96, 2)
    assert lib.pkv_decode_partition_tokens(ctypes.byref(odd), None, 0, 32, ctypes.byref(out)) == 2
    try:
        pkv_lib.set_decode_partition_tokens(2048)
        assert pt([100], 32, 8) == 2048
        pkv_lib.set_decode_partition_tokens(1024)
        assert pt(synth.gqa_bf16().context_lens, 32, 8) == 1024
        assert lib.pkv_set_decode_partition_tokens(1000) == 1
        assert lib.pkv_set_decode_partition_tokens(256) == 1
        pkv_lib.set_decode_partition_tokens(512)
        assert pt(synth.gqa_bf16().context_lens, 32, 8) == 512
    finally:
        pkv_lib.set_decode_partition_tokens(0)
    assert pt([100], 32, 8) == 1024


def test_plan_table_reference_errors(pkv_lib):
    """A bad table reference is rejected on the host before the plan launches."""
    lib = pkv_lib.load()
    P, T = pkv_lib.PoolDesc, pkv_lib.TableRef
    d = P(64, 16, 8, 128, 2)
    ws_bytes = lib.pkv_paged_attention_workspace_bytes(4, 32, 128, 8, 16)
    fake = ctypes.c_void_p(0x1000)
    for ref in (T(None, None, 4, 0), T(0x1000, None, 3, 0), T(0x1000, 0x2000, 2, 0), T(0x1002, None, 4, 0),
                T(0x1000, None, 4, 1)):
        st = lib.pkv_paged_attention_plan(ctypes.byref(d), 4, 32, 8, fake, ctypes.byref(ref), fake, ws_bytes, None)
        assert st == 1, (ref.entries, ref.leaf_dir, ref.entry_bytes)
        assert b"table reference" in lib.pkv_last_error()
    # two-level: the row width must be whole leaves (32 entries at block 16)
    st = lib.pkv_paged_attention_plan(ctypes.byref(d), 4, 32, 8, fake, ctypes.byref(T(0x1000, 0x2000, 4, 0)), fake,
                                      ws_bytes, None)
    assert st == 1
    # 16-bit entries cannot address a pool of more than 65536 blocks
    big = P(70000, 16, 8, 128, 2)
    st = lib.pkv_decode_prepare(ctypes.byref(big), fake, fake, fake, fake, fake, 4, 4, 32, 8, fake,
                                ctypes.byref(T(0x1000, None, 2, 0)), fake, ws_bytes, None)
    assert st == 2
