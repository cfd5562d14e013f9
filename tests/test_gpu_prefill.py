"""GPU parity of the paged prefill (causal chunk) attention against the oracle.

Every case places the workload through the library (block manager + KV write, unowned
slots NaN-poisoned), runs ``pkv_paged_attention_prefill`` and compares with the
fp64 oracle: |gpu - oracle| <= 2e-2 + 1e-2 |oracle| elementwise and relative L2
error per (row, head) below 1e-2 for bf16/fp16.
"""
import zlib

import numpy as np
import pytest
import torch

import paged_kv_cache_281_amd as pkv
import synth
from oracle.attention import paged_attention_prefill as oracle_prefill
from oracle.replay import replay_prefill
from tests.gpu_harness import compare, log, replay_prefill_gpu, rising_keys, run_prefill, to_bits, value_bits

pytestmark = pytest.mark.gpu
DEV = "cuda"

# name, dtype, Hq, Hkv, D, B, cached prefix per sequence, chunk per sequence
CASES = [
    ("bf16_g4_d128_b16", "bf16", 32, 8, 128, 16, [0, 100, 3, 700], [77, 1, 130, 33]),
    ("f16_g1_d64_b32", "f16", 4, 4, 64, 32, [0, 31, 5], [200, 64, 1]),
    ("bf16_g8_d64_b16", "bf16", 16, 2, 64, 16, [16, 0], [48, 257]),
    ("bf16_g16_d128_b32", "bf16", 32, 2, 128, 32, [0, 500], [40, 9]),
    ("f16_g2_d128_b16", "f16", 8, 4, 128, 16, [1000, 0, 17], [129, 15, 16]),
    ("bf16_g32_d128_b16", "bf16", 32, 1, 128, 16, [3, 0], [20, 35]),
    ("bf16_g3_d128_b16", "bf16", 12, 4, 128, 16, [10, 0], [50, 90]),
    ("bf16_g4_empty_chunk", "bf16", 8, 2, 128, 16, [5, 10, 0], [0, 20, 7]),
]


def _workload(case):
    name, dtype, hq, hkv, d, b, prefix, chunk = case
    L = np.asarray(prefix) + np.asarray(chunk)
    return synth.prefill_workload(name, zlib.crc32(name.encode()) % 1000, dtype, L, chunk, hq, hkv, d, b)


def _run_case(w, q_scale=1.0, seqs=None):
    log(f"prefill case {w.name}: N={w.num_seqs} T={w.num_tokens} max_chunk={w.max_query_len}")
    ctx = w.all_context_kv()
    q_bits = w.queries()
    if q_scale != 1.0:
        q_bits = synth.normal_bits((w.seed, 99), (w.num_tokens, w.num_q_heads, w.head_dim), w.dtype)
        qf = torch.from_numpy(q_bits.view(np.int16)).view(torch.bfloat16 if w.dtype == "bf16" else torch.float16)
        q_bits = (qf.float() * q_scale).to(qf.dtype).view(torch.int16).numpy().view(np.uint16)
    st = replay_prefill_gpu(w, ctx, DEV)
    out = run_prefill(w, st, q_bits, DEV)
    pool, tables, lens = replay_prefill(w, synth.NAN_BITS[w.dtype], context=ctx)
    assert np.array_equal(tables, st.tables.cpu().numpy())
    ref = oracle_prefill(q_bits, w.dtype, pool, tables, lens, w.query_start(), w.scale, seqs=seqs)
    qs = w.query_start()
    rows = np.concatenate([np.arange(qs[b], qs[b + 1]) for b in (range(w.num_seqs) if seqs is None else seqs)])
    err, rel = compare(w, out, ref, rows=rows)
    log(f"  max abs err {err:.3g}, max rel L2 {rel:.3g}")
    return out


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prefill_cases(case):
    _run_case(_workload(case))


def test_prefill_peaked_queries():
    """q x 30: logits of order 1e2..1e3 need the running max."""
    _run_case(_workload(CASES[0]), q_scale=30.0)


@pytest.mark.parametrize("case", [CASES[0], CASES[3]], ids=[CASES[0][0], CASES[3][0]])
def test_prefill_scores_rising_on_every_unit(case):
    """Keys that grow with their position and all-ones queries: every row's maximum
    passes the lazy-rescale threshold on every 32-token unit it sees (the raw-score
    limit and its update run unit after unit)."""
    w = _workload(case)
    ctx = rising_keys(w.all_context_kv(), w.dtype, w.head_dim, 8.0)
    q_bits = value_bits(np.ones((w.num_tokens, w.num_q_heads, w.head_dim), np.float32), w.dtype)
    log(f"prefill case {w.name} (rising keys): N={w.num_seqs} T={w.num_tokens}")
    st = replay_prefill_gpu(w, ctx, DEV)
    out = run_prefill(w, st, q_bits, DEV)
    pool, tables, lens = replay_prefill(w, synth.NAN_BITS[w.dtype], context=ctx)
    assert np.array_equal(tables, st.tables.cpu().numpy())
    ref = oracle_prefill(q_bits, w.dtype, pool, tables, lens, w.query_start(), w.scale)
    err, rel = compare(w, out, ref)
    log(f"  max abs err {err:.3g}, max rel L2 {rel:.3g}")


def test_prefill_placement_and_repeat_are_bitwise_equal():
    w = _workload(CASES[0])
    ctx = w.all_context_kv()
    q_bits = w.queries()
    st1 = replay_prefill_gpu(w, ctx, DEV)
    a = run_prefill(w, st1, q_bits, DEV)
    b = run_prefill(w, st1, q_bits, DEV)
    order = np.random.default_rng(5).permutation(w.num_blocks).astype(np.int32)
    st2 = replay_prefill_gpu(w, ctx, DEV, free_order=order)
    c = run_prefill(w, st2, q_bits, DEV)
    assert not np.array_equal(st1.tables.cpu().numpy(), st2.tables.cpu().numpy())
    assert np.array_equal(to_bits(a, w.dtype), to_bits(b, w.dtype))
    assert np.array_equal(to_bits(a, w.dtype), to_bits(c, w.dtype))


@pytest.mark.parametrize("name", ["prefill_bf16", "chunked_bf16"])
def test_prefill_full_size_sampled_sequences(name):
    """The benchmark workloads at full size; the oracle checks the shortest, the
    longest and two seeded random sequences."""
    w = synth.by_name(name)
    L = np.asarray(w.context_lens)
    rng = np.random.default_rng(17)
    seqs = sorted({int(L.argmin()), int(L.argmax()), *rng.choice(w.num_seqs, 2, replace=False).tolist()})
    _run_case(w, seqs=seqs)


def test_prefill_rejects_fp32_and_bad_arguments():
    kp, vp = pkv.alloc_pools(4, 16, 2, 64, torch.float32, DEV)
    q = torch.zeros(3, 2, 64, dtype=torch.float32, device=DEV)
    qs = torch.tensor([0, 3], dtype=torch.int32, device=DEV)
    tables = torch.zeros(1, 4, dtype=torch.int32, device=DEV)
    lens = torch.tensor([3], dtype=torch.int32, device=DEV)
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_attention_prefill(q, kp, vp, tables, lens, qs, 3, 0.125)
    assert e.value.status == 2


def test_prefill_pools_match_oracle():
    """The placement writes (whole runs of blocks, one launch per sequence) leave the
    pools bit-identical to the oracle's."""
    w = _workload(CASES[4])
    ctx = w.all_context_kv()
    st = replay_prefill_gpu(w, ctx, DEV)
    pool, _, _ = replay_prefill(w, synth.NAN_BITS[w.dtype], context=ctx)
    assert (to_bits(st.k_pool, w.dtype) == pool.k).all()
    assert (to_bits(st.v_pool, w.dtype) == pool.v).all()
