"""Pins of the block-table oracle (flat, 16-bit and two-level tables, table memory)."""
import json
import pathlib

import numpy as np
import pytest

from oracle import tables as T

GOLDEN = pathlib.Path(__file__).parent / "golden"


def test_page_table_memory_example():
    """agentalpha.top Q32 follow-up 1: 128K tokens, 16-token blocks, ~8 B an entry."""
    g = json.loads((GOLDEN / "table_memory.json").read_text())
    assert T.table_entries(g["context_tokens"], g["block_size"]) == g["entries_per_request"]
    per = T.table_bytes_per_request(g["context_tokens"], g["block_size"], g["bytes_per_entry"])
    assert per == g["bytes_per_request"]
    assert per * g["concurrent_requests"] // 1024 == g["bytes_total_kb"]
    # the 4-byte ids of the library's flat tables, and 16-bit ids, at the same size
    assert T.table_bytes_per_request(g["context_tokens"], g["block_size"], 4) == per // 2
    assert T.table_bytes_per_request(g["context_tokens"], g["block_size"], 2) == per // 4
    assert T.table_entries(1, 16) == 1 and T.table_entries(0, 16) == 0 and T.table_entries(17, 16) == 2


def test_two_level_hand_example():
    """Block size 32 (16-entry leaves): a 20-block, an empty and a 1-block table."""
    t0 = list(range(100, 120))
    d, lv = T.two_level([t0, [], [7]], 32, 3, 9)
    assert d.tolist() == [[0, 1, 3], [3, 3, 3], [2, 3, 3]]
    assert lv.shape == (4, 16)
    assert lv[0].tolist() == list(range(100, 116))
    assert lv[1].tolist() == [116, 117, 118, 119] + [9] * 12
    assert lv[2].tolist() == [7] + [9] * 15
    assert lv[3].tolist() == [9] * 16
    assert T.two_level_entry(d, lv, 0, 17) == 117 and T.two_level_entry(d, lv, 2, 0) == 7
    d, lv = T.two_level([], 16, 4, 0)
    assert d.shape == (0, 4) and lv.shape == (0, 32)
    with pytest.raises(ValueError):
        T.two_level([list(range(40))], 16, 1, 0)  # 40 entries need two 32-entry leaves


@pytest.mark.parametrize("B", [16, 32])
def test_two_level_lookup_brute_force(B):
    rng = np.random.default_rng(B)
    E = 512 // B
    tables = [list(rng.integers(0, 1 << 20, size=int(n))) for n in rng.integers(0, 4 * E + 3, size=40)]
    width = max(-(-len(t) // E) for t in tables) + 1
    d, lv = T.two_level(tables, B, width, -5)
    assert lv.shape[0] == sum(-(-len(t) // E) for t in tables) + 1
    for b, t in enumerate(tables):
        for j in range(width * E):
            assert T.two_level_entry(d, lv, b, j) == (t[j] if j < len(t) else -5)


def test_sparse_batch_memory():
    """One 128K-token request and 999 of 512 tokens, block 16: the flat matrix is as wide
    as the longest table (8192 entries a row); the two-level table holds a 256-entry
    directory row per request and only the leaves in use."""
    n, W = 1000, 8192
    assert T.flat_table_bytes(n, W, 4) == 32_768_000
    assert T.flat_table_bytes(n, W, 2) == 16_384_000
    leaves = 256 + 999 + 1  # 8192 / 32, one per short request, the padding leaf
    assert T.two_level_bytes(n, 256, leaves, 16) == 4 * (256_000 + 1256 * 32) == 1_184_768
