"""The decode step (KV write + plan + partition pass, and copy-on-write copies when the
step has pairs) captured as a HIP graph and replayed: every replay, with eager library
work and synchronisations between replays, gives the bits of the eager step, and the
eager result matches the oracle (int32, 16-bit and two-level tables)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_281_amd as pkv
import synth
from oracle.attention import paged_attention_decode as oracle_attention
from oracle.replay import replay as oracle_replay
from tests.gpu_harness import compare, log, replay_gpu, to_bits, to_device

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("name,tables", [("gqa", "int32"), ("cow", "int32"), ("long", "int32"), ("gqa", "int16"),
                                         ("long", "two_level")])
def test_graph_replays_match_eager_step(name, tables):
    if name == "gqa":
        w = synth.gqa_bf16(num_seqs=8, max_len=1500)
    elif name == "cow":
        w = synth.cow_fp16(1020, num_prompts=3, max_suffix=20)
    else:
        w = synth.long_bf16(16, num_seqs=2, context=40 * 1024)  # 40 partitions: the separate merge kernel
    log(f"graph replay {name}, {tables} tables: {w.num_seqs} sequences")
    ctx = w.all_context_kv()
    st = replay_gpu(w, ctx, DEV)
    width = w.max_blocks_per_seq
    if tables == "int16":
        st.tables = torch.from_numpy(st.bm.block_tables16(w.batch, width, 0)).to(DEV)
    elif tables == "two_level":
        E = pkv.LEAF_TOKENS // w.block_size
        ld, lv = st.bm.block_tables_2l(w.batch, -(-width // E), 0)
        st.tables = pkv.TwoLevelTables(torch.from_numpy(ld).to(DEV), torch.from_numpy(lv).to(DEV))
        width = ld.shape[1] * E
    # rebuild the last step's inputs: undo nothing, just re-run it (writes are idempotent)
    slots = torch.from_numpy(st.last_slots).to(DEV)
    pairs = torch.from_numpy(st.last_pairs).to(DEV)
    k, v = (to_device(x, w.dtype, DEV) for x in w.step_kv(len(w.steps) - 1))
    q = to_device(w.queries(), w.dtype, DEV)
    out = torch.empty_like(q)
    ws = pkv.alloc_workspace(w.num_seqs, w.num_q_heads, w.head_dim, width, w.block_size, DEV)

    def step():
        if len(st.last_pairs):
            pkv.copy_blocks(st.k_pool, st.v_pool, pairs)
        pkv.decode_prepare(st.k_pool, st.v_pool, k, v, slots, q, st.tables, st.context_lens, ws)
        pkv.paged_attention_partitions(q, st.k_pool, st.v_pool, st.tables, st.context_lens, w.scale, out, ws)

    step()
    torch.cuda.synchronize()
    eager = to_bits(out, w.dtype).copy()
    ora = oracle_replay(w, synth.NAN_BITS[w.dtype], context=ctx)
    ref = oracle_attention(w.queries(), w.dtype, ora.pool, ora.block_tables, ora.context_lens, w.scale)
    compare(w, out, ref)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for i in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(out, w.dtype), eager), f"replay {i} differs"
        # eager library work between replays
        pkv.paged_attention_decode(q, st.k_pool, st.v_pool, st.tables, st.context_lens, w.scale)
        torch.cuda.synchronize()
