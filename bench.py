"""Benchmark of one paged decode step on one MI355X.

A step is one pass of the whole hot path over one batch: the copy-on-write block
copies of the step (if any), then one launch that writes the step's new tokens
into their slots (from the host block manager) and plans the attention, then the
attention partition pass, whose last finisher per row does the log-sum-exp merge
(a separate merge kernel for rows of more than 32 partitions).  Inputs are seeded
synthetic data already resident in HBM.  The timed steps are stream launches; the
same step captured as a HIP graph is replayed afterwards and reported beside them
(``--eager`` skips the replays).

Prints one JSON line.  ``value`` is KV GB/s over the whole step (attention's
algorithmic K+V bytes / step time); ``roofline`` describes the dominant kernel
(the attention partition pass) against MI355X's 8 TB/s HBM peak; ``cpu_baseline``
times the fp64 oracle on a bounded sample of the same workload.

Without ``--workload`` the line is the long-context decode step (8 sequences of 131,072
tokens, block 16: the largest single-GPU configuration), and it carries, as
sub-records, the GQA batch (256 sequences), long context at block 32, long context at
512-token partitions, and the device's streaming-read ceiling (``pkv_stream_read`` over
4 GiB).  ``--workload stream_ceiling`` prints that ceiling as its own line.

With a prefill workload (``--workload prefill_bf16`` or ``chunked_bf16``) a step is
the KV write of every sequence's chunk followed by the causal chunk attention (its
plan pass and its attention pass);
``value`` is attention TFLOP/s over the step and the roofline is the prefill kernel
against the dense bf16 MFMA peak (2.5 PFLOP/s).

With ``--workload swap_bf16`` a step moves 64 sequences of the GQA batch to a host
block manager, copies their blocks to pinned host memory, and brings them back; the
roofline is the swap-out copy against PCIe 5.0 x16 (63 GB/s per direction).
With ``--workload prefix_bf16`` the same prefill batch (64 requests over 4 system
prompts) is timed with the prefix cache (only uncached tokens written and attended
from) and without it.
With ``--workload lenclass_bf16`` the GQA batch is held three ways: all in one block-16
pool, all in one block-32 pool, and by length class (sequences under 1024 tokens in a
block-16 pool, the others in a block-32 pool, one decode step over both).  ``value`` is
the per-class step's K+V GB/s; every configuration's step time and memory are reported.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention KV GB/s (% of HBM peak) + decode tokens/sec, 1 GPU"
PREFILL_METRIC = "paged prefill attention TFLOP/s (% of dense bf16 MFMA peak), 1 GPU"
SWAP_METRIC = "KV block swap GB/s between the device pool and pinned host memory, 1 GPU"
PCIE_PEAK_GBS = 63.0  # PCIe 5.0 x16, one direction
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
PARTITION_TOKENS = 1024  # the library's shorter decode partition (the plan may pick 2048)
FUSE_MAX_PARTS = 32  # rows split into more partitions are merged by the separate merge kernel
LEAF_TOKENS = 512  # the library's two-level leaf
KERNEL_SRC = os.path.join(ROOT, "paged_kv_cache_281_amd", "csrc", "paged_attention.hip")
PREFILL_SRC = os.path.join(ROOT, "paged_kv_cache_281_amd", "csrc", "paged_prefill.hip")


def spread(ms):
    """median, p10 and p90 of a list of kernel times (ms)."""
    a = np.asarray(ms, dtype=np.float64)
    return {"median": round(float(np.median(a)), 5), "p10": round(float(np.percentile(a, 10)), 5),
            "p90": round(float(np.percentile(a, 90)), 5), "n": int(a.size)}


def host_cpus():
    """Host CPUs as the oracle saw them: the machine's count and this process's affinity."""
    return {"cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0))}


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def unique_tokens(tables, lens, block_size):
    """Distinct (block, offset) slots the batch reads: a block shared by several
    sequences counts once, with the most slots any of them reads."""
    used = {}
    for row, L in zip(tables, lens):
        L = int(L)
        for j in range(-(-L // block_size)):
            n = min(block_size, L - j * block_size)
            b = int(row[j])
            used[b] = max(used.get(b, 0), n)
    return sum(used.values())


def algorithmic_bytes(w, lens, table_format="int32", unique=None, partition_tokens=PARTITION_TOKENS):
    """Bytes the attention partition pass must move, by item (see the design notes).
    Table entries are 4 bytes (2 for 16-bit tables); two-level tables add one 4-byte
    directory entry per leaf read.  K+V count every context token of every sequence
    (``kv``); with ``unique`` (distinct slots read) the total counts shared blocks
    once, the bytes that must come from HBM."""
    e = w.elem_bytes
    H, D, B, Hq = w.num_kv_heads, w.head_dim, w.block_size, w.num_q_heads
    G = Hq // H
    groups = H * max(1, -(-G // 16)) if G > 1 and w.dtype != "f32" else H
    lens = np.asarray(lens, dtype=np.int64)
    kv = int(2 * lens.sum() * H * D * e)
    q = int(len(lens) * Hq * D * e)
    parts = -(-lens // partition_tokens)
    single = parts <= 1
    out = int(single.sum() * Hq * D * e)
    partials = int(2 * parts[~single].sum() * Hq * (D + 2) * 4)  # written, then read by the merge
    eb = 2 if table_format == "int16" else 4
    tables = int(groups * (-(-lens // B)).sum() * eb + len(lens) * 4)
    if table_format == "two_level":
        leaf = LEAF_TOKENS // B
        tables += int(groups * (-(-(-(-lens // B)) // leaf)).sum() * 4)
    kv_hbm = kv if unique is None else int(2 * unique * H * D * e)
    return {"kv": kv, "kv_unique": kv_hbm, "q": q, "out": out, "partials": partials, "tables": tables,
            "total": kv_hbm + q + out + partials + tables, "merge_long": bool((parts > FUSE_MAX_PARTS).any())}


def partition_tokens_of(w, lens):
    """The decode partition size the library's plan pass picks for this batch."""
    import paged_kv_cache_281_amd as pkv
    return pkv.decode_partition_tokens(lens, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size)


def stored_traffic(workload, kernel="attn_partition", src=KERNEL_SRC):
    """HBM bytes per launch of a kernel from a committed rocprofv3 PMC summary, if its
    kernel source hash matches the current source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    cur = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if not h or not t or h.group(1) != cur:
        return None
    return float(t.group(1))


def cpu_baseline(w, ctx, target_s):
    """The fp64 oracle (as it stands) on a bounded sample: the measured step's KV write
    and attention for the first sequences of the batch, until ``target_s`` elapses."""
    import synth
    from oracle.attention import paged_attention_decode as oracle_attention
    from oracle.kv_cache import paged_kv_write as oracle_write
    from oracle.replay import replay as oracle_replay
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    ora = oracle_replay(w, synth.NAN_BITS[w.dtype], context=ctx)
    q = w.queries()
    k_new, v_new = w.step_kv(len(w.steps) - 1)
    done, kv_bytes = 0, 0
    t0 = time.perf_counter()
    for b in range(w.num_seqs):
        oracle_write(ora.pool, k_new[b:b + 1], v_new[b:b + 1], ora.last_slots[b:b + 1])
        oracle_attention(q, w.dtype, ora.pool, ora.block_tables, ora.context_lens, w.scale, seqs=[b])
        done += 1
        kv_bytes += 2 * int(ora.context_lens[b]) * w.num_kv_heads * w.head_dim * w.elem_bytes
        if time.perf_counter() - t0 > target_s:
            break
    el = time.perf_counter() - t0
    return {"value": kv_bytes / el / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle", **host_cpus(),
            "tokens_per_s": done / el,
            "sample": f"KV write + attention of the first {done} of {w.num_seqs} sequences of the batch "
                      f"({kv_bytes / 1e9:.3f} GB of KV) in {el:.1f} s; fp64 NumPy, BLAS threads {threads}"}


def cpu_baseline_prefill(w, ctx, target_s):
    """The fp64 oracle (as it stands) on a bounded sample of a prefill batch: chunk
    attention of one sequence at a time, shortest first, until ``target_s`` elapses."""
    import synth
    from oracle.attention import paged_attention_prefill as oracle_prefill
    from oracle.replay import replay_prefill
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    pool, tables, lens = replay_prefill(w, synth.NAN_BITS[w.dtype], context=ctx)
    q = w.queries()
    qs = w.query_start()
    L = np.asarray(w.context_lens, dtype=np.int64)
    C = np.asarray(w.chunk_lens, dtype=np.int64)
    done, flops = 0, 0
    t0 = time.perf_counter()
    for b in np.argsort(L, kind="stable"):
        oracle_prefill(q, w.dtype, pool, tables, lens, qs, w.scale, seqs=[int(b)])
        done += 1
        flops += 4 * w.num_q_heads * w.head_dim * int(C[b] * (L[b] - C[b]) + C[b] * (C[b] + 1) // 2)
        if time.perf_counter() - t0 > target_s:
            break
    el = time.perf_counter() - t0
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle", **host_cpus(),
            "sample": f"chunk attention of the {done} shortest of {w.num_seqs} sequences "
                      f"({flops / 1e9:.2f} GFLOP) in {el:.1f} s; fp64 NumPy, BLAS threads {threads}"}


def prefill_main(args, w, dev):
    """One prefill step per iteration: the chunks' KV write, then the causal chunk attention."""
    import torch
    import paged_kv_cache_281_amd as pkv
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}
    npi = np.int16
    log(f"prefill workload {w.name}: N={w.num_seqs} tokens={w.num_tokens} max_chunk={w.max_query_len} "
        f"context={int(w.context_lens.sum())} Hq={w.num_q_heads} Hkv={w.num_kv_heads} D={w.head_dim} "
        f"B={w.block_size} {w.dtype}")
    ctx = w.all_context_kv()

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(npi)).to(dev).view(tdt[w.dtype])

    bm = pkv.BlockManager(w.num_blocks, w.block_size, w.free_order)
    kp, vp = pkv.alloc_pools(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, tdt[w.dtype], dev)
    kp.view(torch.int16).fill_(0)
    vp.view(torch.int16).fill_(0)
    k_chunk, v_chunk, s_chunk = [], [], []
    for b in range(w.num_seqs):
        L, C = int(w.context_lens[b]), int(w.chunk_lens[b])
        bm.add_seq(b, L)
        k, v = ctx.pop(b)
        slots = bm.slots(b, 0, L)
        if L - C:  # the cached prefix is written once, before the timed steps
            pkv.paged_kv_write(kp, vp, up(k[:L - C]), up(v[:L - C]), torch.from_numpy(slots[:L - C]).to(dev))
        k_chunk.append(k[L - C:])
        v_chunk.append(v[L - C:])
        s_chunk.append(slots[L - C:])
    k_new = up(np.concatenate(k_chunk))
    v_new = up(np.concatenate(v_chunk))
    slots_d = torch.from_numpy(np.concatenate(s_chunk)).to(dev)
    tables = torch.from_numpy(bm.block_tables(list(range(w.num_seqs)), w.max_blocks_per_seq, 0)).to(dev)
    lens = torch.from_numpy(np.asarray(w.context_lens, dtype=np.int32)).to(dev)
    qs = torch.from_numpy(w.query_start()).to(dev)
    q = up(w.queries())
    out = torch.empty_like(q)
    ws = pkv.alloc_prefill_workspace(w.num_seqs, w.num_tokens, w.num_q_heads, w.num_kv_heads, dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    def step(e=None):
        pkv.paged_kv_write(kp, vp, k_new, v_new, slots_d)
        if e is not None:
            e[0].record(stream)
        pkv.paged_attention_prefill(q, kp, vp, tables, lens, qs, w.max_query_len, w.scale, out, ws)
        if e is not None:
            e[1].record(stream)

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    attn_all = [e[0].elapsed_time(e[1]) for e in ev]
    attn_ms = float(np.mean(attn_all))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        pkv.paged_kv_write(kp, vp, k_new, v_new, slots_d)
    e1.record(stream)
    torch.cuda.synchronize()
    write_ms = e0.elapsed_time(e1) / 10
    log(f"step {ms_step:.4f} ms (prefill attention {attn_ms:.4f}, chunk KV write alone {write_ms:.4f})")
    flops = w.flops()
    achieved = flops / (attn_ms * 1e-3) / 1e12
    res = {
        "metric": PREFILL_METRIC,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
                   "query_tokens": w.num_tokens, "max_chunk": w.max_query_len,
                   "context_tokens": int(w.context_lens.sum()), "flops": flops, "kv_bytes": w.kv_bytes()},
        "tokens_per_s": round(w.num_tokens / (ms_step * 1e-3), 1),
        "kernel_ms": {"attn_prefill": round(attn_ms, 5), "kv_write_alone": round(write_ms, 5)},
        "attn_prefill_ms_spread": spread(attn_all),
        "roofline": {"kernel": "attn_prefill_mfma", "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": stored_traffic(w.name, "attn_prefill", PREFILL_SRC), "algorithmic_flops": flops},
    }
    if not args.no_cpu_baseline:
        del kp, vp
        torch.cuda.empty_cache()
        log("timing the oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline_prefill(w, w.all_context_kv(), args.cpu_seconds)
    print(json.dumps(res), flush=True)


def swap_main(args, sw, dev):
    """One step: move the chosen sequences to the host manager and copy their blocks out,
    then move them back and copy in.  Pools hold arbitrary bytes (the copy moves bits)."""
    import torch
    import paged_kv_cache_281_amd as pkv
    w = sw.base
    tdt = torch.bfloat16
    bm = pkv.BlockManager(w.num_blocks, w.block_size, w.free_order)
    for seq, n in w.prefill:
        bm.add_seq(seq, n)
    kp, vp = pkv.alloc_pools(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, tdt, dev)
    kp.view(torch.int16).random_()
    vp.view(torch.int16).random_()
    hk, hv = pkv.alloc_host_pools(sw.host_blocks, w.block_size, w.num_kv_heads, w.head_dim, tdt)
    hbm = pkv.BlockManager(sw.host_blocks, w.block_size, np.arange(sw.host_blocks, dtype=np.int32))
    block_bytes = 2 * w.num_kv_heads * w.block_size * w.head_dim * 2
    stream = torch.cuda.current_stream(dev)
    log(f"swap workload: {len(sw.moved)} of {w.num_seqs} sequences, host pool {sw.host_blocks} blocks")

    host_us = []

    def step(e=None):
        t = time.perf_counter()
        p_out = bm.move_seqs(hbm, sw.moved)
        host_us.append((time.perf_counter() - t) * 1e6)
        d_out = torch.from_numpy(p_out).to(dev, non_blocking=False)
        if e is not None:
            e[0].record(stream)
        pkv.swap_blocks(kp, vp, hk, hv, d_out)
        if e is not None:
            e[1].record(stream)
        p_in = hbm.move_seqs(bm, sw.moved)
        d_in = torch.from_numpy(p_in).to(dev, non_blocking=False)
        if e is not None:
            e[2].record(stream)
        pkv.swap_blocks(hk, hv, kp, vp, d_in)
        if e is not None:
            e[3].record(stream)
        return len(p_out), len(p_in)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        n_out, n_in = step(ev[i])
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    out_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    in_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))
    moved_bytes = n_out * block_bytes
    gbs_out = moved_bytes / (out_ms * 1e-3) / 1e9
    gbs_in = moved_bytes / (in_ms * 1e-3) / 1e9
    # on-box ceiling: one contiguous DMA copy of the same bytes each way
    flat = torch.empty(moved_bytes, dtype=torch.uint8, device=dev)
    hflat = torch.empty(moved_bytes, dtype=torch.uint8, pin_memory=True)
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    hflat.copy_(flat, non_blocking=True)
    torch.cuda.synchronize()
    e0.record(stream)
    hflat.copy_(flat, non_blocking=True)
    e1.record(stream)
    flat.copy_(hflat, non_blocking=True)
    e2.record(stream)
    torch.cuda.synchronize()
    dma_out = moved_bytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
    dma_in = moved_bytes / (e1.elapsed_time(e2) * 1e-3) / 1e9
    log(f"step {ms_step:.3f} ms: out {out_ms:.3f} ms ({gbs_out:.1f} GB/s), in {in_ms:.3f} ms ({gbs_in:.1f} GB/s); "
        f"contiguous DMA {dma_out:.1f} / {dma_in:.1f} GB/s")
    res = {
        "metric": SWAP_METRIC,
        "value": round(2 * moved_bytes / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": sw.name, "moved_sequences": len(sw.moved), "blocks_each_way": n_out,
                   "bytes_each_way": moved_bytes, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size},
        "kernel_ms": {"swap_out": round(out_ms, 5), "swap_in": round(in_ms, 5)},
        "swap_out_gbs": round(gbs_out, 2),
        "swap_in_gbs": round(gbs_in, 2),
        "contiguous_dma_gbs": {"device_to_host": round(dma_out, 2), "host_to_device": round(dma_in, 2)},
        "host_block_manager_move_us": round(float(np.median(host_us)), 1),
        "roofline": {"kernel": "copy_blocks_kernel (swap out)", "bound": "pcie", "achieved": round(gbs_out, 2),
                     "peak": PCIE_PEAK_GBS, "unit": "GB/s", "frac": round(gbs_out / PCIE_PEAK_GBS, 4),
                     "traffic": None, "algorithmic_bytes": moved_bytes},
    }
    if not args.no_cpu_baseline:
        from oracle.kv_cache import Pool, swap_blocks as oracle_swap
        src = Pool(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size, "bf16")
        dst = Pool(sw.host_blocks, w.num_kv_heads, w.head_dim, w.block_size, "bf16")
        pairs = bm.move_seqs(hbm, sw.moved)
        t = time.perf_counter()
        reps = 0
        while time.perf_counter() - t < min(args.cpu_seconds, 5.0):
            oracle_swap(src, dst, pairs)
            reps += 1
        el = time.perf_counter() - t
        res["cpu_baseline"] = {"value": round(reps * moved_bytes / el / 1e9, 3), "unit": "GB/s", "cores": 1,
                               "kind": "oracle", **host_cpus(),
                               "sample": f"{reps} oracle block copies of {len(pairs)} blocks in host memory "
                                         f"(NumPy, one thread) in {el:.1f} s"}
    print(json.dumps(res), flush=True)


def prefix_main(args, w, dev):
    """Prefill of requests sharing system prompts, with the prefix cache (only uncached
    tokens are written and attended from) and without it (whole prompts); same requests,
    same queries per position."""
    import torch
    import paged_kv_cache_281_amd as pkv
    tdt = torch.bfloat16

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(tdt)

    flops_row = 4 * w.num_q_heads * w.head_dim
    lens = np.asarray([w.length(b) for b in range(w.num_seqs)], dtype=np.int64)
    stream = torch.cuda.current_stream(dev)
    res_runs = {}
    for cache in (True, False):
        t = time.perf_counter()
        bm = pkv.BlockManager(w.num_blocks, w.block_size, w.free_order, prefix_cache=cache)
        cached = np.asarray([bm.add_seq_tokens(b, w.tokens(b)) for b in range(w.num_seqs)], dtype=np.int64)
        host_ms = (time.perf_counter() - t) * 1e3
        kp, vp = pkv.alloc_pools(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, tdt, dev)
        kp.view(torch.int16).fill_(0)
        vp.view(torch.int16).fill_(0)
        ks, vs, ss, qs_rows = [], [], [], []
        for b in range(w.num_seqs):
            k, v = w.kv(b)
            c, L = int(cached[b]), int(lens[b])
            ks.append(k[c:])
            vs.append(v[c:])
            ss.append(bm.slots(b, c, L - c))
            qs_rows.append(w.queries(b)[c:])
        k_new, v_new = up(np.concatenate(ks)), up(np.concatenate(vs))
        slots = torch.from_numpy(np.concatenate(ss)).to(dev)
        q = up(np.concatenate(qs_rows))
        chunks = lens - cached
        qstart = torch.from_numpy(np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)).to(dev)
        tables = torch.from_numpy(bm.block_tables(list(range(w.num_seqs)), w.max_blocks_per_seq, 0)).to(dev)
        lens_d = torch.from_numpy(lens.astype(np.int32)).to(dev)
        out = torch.empty_like(q)
        ws = pkv.alloc_prefill_workspace(w.num_seqs, q.shape[0], w.num_q_heads, w.num_kv_heads, dev)
        mq = int(chunks.max())
        torch.cuda.synchronize()

        def step(e=None):
            pkv.paged_kv_write(kp, vp, k_new, v_new, slots)
            if e is not None:
                e[0].record(stream)
            pkv.paged_attention_prefill(q, kp, vp, tables, lens_d, qstart, mq, w.scale, out, ws)
            if e is not None:
                e[1].record(stream)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(ev[i])
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        attn = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
        flops = flops_row * int(np.sum(chunks * (lens - chunks) + chunks * (chunks + 1) // 2))
        res_runs["cached" if cache else "uncached"] = {
            "ms_per_step": round(ms, 5), "attn_ms": round(attn, 5), "computed_tokens": int(chunks.sum()),
            "cached_tokens": int(cached.sum()), "flops": flops, "attn_tflops": round(flops / (attn * 1e-3) / 1e12, 2),
            "host_block_manager_ms": round(host_ms, 2)}
        log(f"{'with' if cache else 'without'} prefix cache: step {ms:.4f} ms, attention {attn:.4f} ms, "
            f"{int(chunks.sum())} of {int(lens.sum())} prompt tokens computed")
        del kp, vp
        torch.cuda.empty_cache()
    c, u = res_runs["cached"], res_runs["uncached"]
    total = int(lens.sum())
    res = {
        "metric": "prompt tokens/s of a prefill batch sharing system prompts, with prefix caching, 1 GPU",
        "value": round(total / (c["ms_per_step"] * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": c["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "requests": w.num_seqs, "system_prompts": len(w.system_lens),
                   "prompt_tokens": total, "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "block_size": w.block_size},
        "with_cache": c, "without_cache": u,
        "speedup": round(u["ms_per_step"] / c["ms_per_step"], 3),
        "roofline": {"kernel": "attn_prefill_lds (cached run)", "bound": "mfma", "achieved": c["attn_tflops"],
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(c["attn_tflops"] / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "algorithmic_flops": c["flops"]},
    }
    print(json.dumps(res), flush=True)


def lenclass_main(args, lw, dev):
    """Decode step of one batch under three block-size choices (see the module docstring)."""
    import torch
    import paged_kv_cache_281_amd as pkv
    base = lw.base
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[base.dtype]
    log(f"length-class workload: {base.num_seqs} sequences, threshold {lw.threshold}: "
        f"{lw.short.num_seqs} in block 16, {lw.long.num_seqs} in block 32")
    t = time.perf_counter()
    ctx = base.all_context_kv()
    log(f"generated context values in {time.perf_counter() - t:.1f} s")

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(tdt)

    def setup(w):
        p = {"w": w}
        bm = pkv.BlockManager(w.num_blocks, w.block_size, w.free_order)
        kp, vp = pkv.alloc_pools(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, tdt, dev)
        kp.view(torch.int16).fill_(0)
        vp.view(torch.int16).fill_(0)
        for seq, n in w.prefill:
            bm.add_seq(seq, n)
            if n:
                k, v = ctx[seq]
                pkv.paged_kv_write(kp, vp, up(k[:n]), up(v[:n]), torch.from_numpy(bm.slots(seq, 0, n)).to(dev))
        slots, pairs = bm.step(w.steps[-1])
        assert len(pairs) == 0
        k_new, v_new = (up(x) for x in w.step_kv(0))
        lens_np = np.asarray([bm.seq_len(int(s)) for s in w.batch], dtype=np.int32)
        used_blocks = w.num_blocks - bm.num_free()
        p.update(bm=bm, kp=kp, vp=vp, k_new=k_new, v_new=v_new, slots=torch.from_numpy(slots).to(dev),
                 tables=torch.from_numpy(bm.block_tables(w.batch, w.max_blocks_per_seq, 0)).to(dev),
                 lens_np=lens_np, lens=torch.from_numpy(lens_np).to(dev), q=up(w.queries()),
                 ws=pkv.alloc_workspace(w.num_seqs, w.num_q_heads, w.head_dim, w.max_blocks_per_seq,
                                        w.block_size, dev),
                 blocks=used_blocks, slots_alloc=used_blocks * w.block_size)
        p["out"] = torch.empty_like(p["q"])
        return p

    stream = torch.cuda.current_stream(dev)
    results = {}
    for name, parts_w in (("all_b16", [base]), ("all_b32", [lw.all32]), ("by_class", [lw.short, lw.long])):
        parts = [setup(w) for w in parts_w]
        torch.cuda.synchronize()

        def step(ev=None):
            for i, p in enumerate(parts):
                w = p["w"]
                pkv.decode_prepare(p["kp"], p["vp"], p["k_new"], p["v_new"], p["slots"], p["q"], p["tables"],
                                   p["lens"], p["ws"])
                if ev is not None:
                    ev[i][0].record(stream)
                pkv.paged_attention_partitions(p["q"], p["kp"], p["vp"], p["tables"], p["lens"], w.scale, p["out"],
                                               p["ws"])
                if ev is not None:
                    ev[i][1].record(stream)

        evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in parts] for _ in range(args.steps)]
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step()
        torch.cuda.synchronize()
        step_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        for i in range(args.steps):
            step(evs[i])
        torch.cuda.synchronize()
        part_ms = [float(np.mean([e[i][0].elapsed_time(e[i][1]) for e in evs])) for i in range(len(parts))]
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            step()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        conc_ms = None
        if len(parts) > 1:
            # the pools are independent: one graph branch per pool (fork / join on
            # streams of default priority), so the two partition passes can overlap;
            # reported beside the one-branch step, which is the step timed
            branches = [torch.cuda.Stream(device=dev) for _ in parts]

            def step_branches():
                cur = torch.cuda.current_stream(dev)
                for b in branches:
                    b.wait_stream(cur)
                for p, b in zip(parts, branches):
                    with torch.cuda.stream(b):
                        pkv.decode_prepare(p["kp"], p["vp"], p["k_new"], p["v_new"], p["slots"], p["q"],
                                           p["tables"], p["lens"], p["ws"])
                        pkv.paged_attention_partitions(p["q"], p["kp"], p["vp"], p["tables"], p["lens"],
                                                       p["w"].scale, p["out"], p["ws"])
                for b in branches:
                    cur.wait_stream(b)

            g2 = torch.cuda.CUDAGraph()
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                step_branches()
            stream.wait_stream(side)
            torch.cuda.synchronize()
            with torch.cuda.graph(g2):
                step_branches()
            for _ in range(args.warmup):
                g2.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                g2.replay()
            torch.cuda.synchronize()
            conc_ms = (time.perf_counter() - t0) * 1e3 / args.steps
            log(f"{name}: pools as parallel graph branches {conc_ms:.4f} ms (one branch {graph_ms:.4f}, "
                f"stream launches {step_ms:.4f})")
        abs_ = [algorithmic_bytes(p["w"], p["lens_np"], partition_tokens=partition_tokens_of(p["w"], p["lens_np"]))
                for p in parts]
        kv = sum(a["kv"] for a in abs_)
        used = sum(int(p["lens_np"].sum()) for p in parts)
        alloc = sum(p["slots_alloc"] for p in parts)
        per_slot = 2 * base.num_kv_heads * base.head_dim * base.elem_bytes
        results[name] = {
            "block_sizes": [p["w"].block_size for p in parts], "sequences": [p["w"].num_seqs for p in parts],
            "ms_per_step": round(step_ms, 5), "graph_ms_per_step": round(graph_ms, 5),
            "parallel_branches_ms_per_step": None if conc_ms is None else round(conc_ms, 5),
            "partition_kernel_ms": [round(x, 5) for x in part_ms],
            "kv_gbs": round(kv / (step_ms * 1e-3) / 1e9, 2),
            "partition_kernel_gbs": round(sum(a["total"] for a in abs_) / (sum(part_ms) * 1e-3) / 1e9, 2),
            "tokens": used, "allocated_slots": alloc, "wasted_slots": alloc - used,
            "kv_bytes_allocated": alloc * per_slot, "table_entries": sum(p["blocks"] for p in parts),
            "kv_bytes": kv, "algorithmic_bytes": sum(a["total"] for a in abs_),
        }
        log(f"{name}: step {step_ms:.4f} ms (graph replays {graph_ms:.4f}), partition kernels {part_ms}, "
            f"waste {alloc - used} slots, {results[name]['table_entries']} table entries")
        del parts, g
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    r = results["by_class"]
    achieved = r["algorithmic_bytes"] / (sum(r["partition_kernel_ms"]) * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": r["kv_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": base.dtype,
        "data": "synthetic",
        "config": {"workload": lw.name, "threshold": lw.threshold, "num_seqs": base.num_seqs,
                   "num_q_heads": base.num_q_heads, "num_kv_heads": base.num_kv_heads, "head_dim": base.head_dim,
                   "block_sizes": "16 below the threshold, 32 from it", "context_tokens": r["tokens"],
                   "kv_bytes": r["kv_bytes"]},
        "pct_hbm_peak": round(100.0 * r["kv_gbs"] / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(base.num_seqs / (r["ms_per_step"] * 1e-3), 1),
        "step_launch": "stream",
        "configurations": results,
        "roofline": {"kernel": "attn_partition (block-16 and block-32 launches)", "bound": "hbm",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "algorithmic_bytes": r["algorithmic_bytes"]},
    }
    if not args.no_cpu_baseline:
        log("timing the oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(base, ctx, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def stream_ceiling(dev, gib=4, reps=10, configs=None):
    """The device's streaming-read rate: one read of a ``gib`` GiB buffer by the library's
    probe kernel (``pkv_stream_read``: 16-byte non-temporal loads, grid-stride), over a
    sweep of workgroup counts and loads in flight; HIP events around ``reps`` launches."""
    import torch
    import paged_kv_cache_281_amd as pkv
    n = gib << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    src.fill_(1)
    stream = torch.cuda.current_stream(dev)
    configs = configs or [(wg, u) for u in (4, 8) for wg in (2048, 4096, 8192, 16384, 32768, 65536)]
    sink = torch.empty(4 * max(wg for wg, _ in configs), dtype=torch.int32, device=dev)
    rows = []
    for wg, u in configs:
        pkv.stream_read(src, sink, wg, u)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            pkv.stream_read(src, sink, wg, u)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        rows.append({"workgroups": wg, "loads_in_flight": u, "ms": round(ms, 4), "gbs": round(n / (ms * 1e-3) / 1e9, 1)})
    del src, sink
    torch.cuda.empty_cache()
    best = max(rows, key=lambda r: r["gbs"])
    return {"bytes": n, "best_gbs": best["gbs"], "best": best, "frac_of_peak": round(best["gbs"] / HBM_PEAK_GBS, 4),
            "sweep": rows, "kernel": "stream_read_kernel (pkv_stream_read)"}


def stream_main(args, dev):
    """``--workload stream_ceiling``: the streaming-read ceiling as its own JSON line."""
    log("streaming-read ceiling: 4 GiB, sweep of launch shapes")
    t0 = time.perf_counter()
    c = stream_ceiling(dev, reps=max(1, args.steps))
    log(f"best {c['best_gbs']} GB/s ({c['best']}) in {time.perf_counter() - t0:.1f} s")
    res = {"metric": "HBM streaming-read GB/s (% of HBM peak), 1 GPU", "value": c["best_gbs"], "unit": "GB/s",
           "n_gpus": 1, "steps": args.steps, "warmup": 1, "ms_per_step": c["best"]["ms"], "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
           "config": {"workload": "stream_ceiling", "bytes": c["bytes"]},
           "roofline": {"kernel": c["kernel"], "bound": "hbm", "achieved": c["best_gbs"], "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": c["frac_of_peak"], "traffic": None, "algorithmic_bytes": c["bytes"]},
           "sweep": c["sweep"]}
    print(json.dumps(res), flush=True)


def decode_run(args, name, dev, table_format="int32", partition_tokens=0, with_cpu=False, num_seqs=None, shape=None):
    """One decode workload: set-up, ``args.steps`` timed steps (graph replays unless
    ``--eager``), the passes alone, and flushed partition timings.  Returns the bench
    record (the JSON line's fields) for that workload."""
    import torch
    import paged_kv_cache_281_amd as pkv
    import synth
    pkv.set_decode_partition_tokens(partition_tokens)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
    ti = {"f32": (np.int32, torch.int32), "f16": (np.int16, torch.int16), "bf16": (np.int16, torch.int16)}
    w = synth.by_name(name, **({"num_seqs": num_seqs} if num_seqs else {}), **(shape or {}))
    log(f"workload {w.name}: N={w.num_seqs} Hq={w.num_q_heads} Hkv={w.num_kv_heads} D={w.head_dim} "
        f"B={w.block_size} {w.dtype} tokens={int(w.context_lens.sum())} partition={partition_tokens or 'plan'}")
    t = time.perf_counter()
    ctx = w.all_context_kv()
    log(f"generated context values in {time.perf_counter() - t:.1f} s")
    npi, tint = ti[w.dtype]

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(npi)).to(dev).view(tdt[w.dtype])

    # ---- set-up: every operation before the measured step ----------------------------
    bm = pkv.BlockManager(w.num_blocks, w.block_size, w.free_order)
    kp, vp = pkv.alloc_pools(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, tdt[w.dtype], dev)
    kp.view(tint).fill_(0)
    vp.view(tint).fill_(0)
    for seq, n in w.prefill:
        bm.add_seq(seq, n)
        if n:
            k, v = ctx.pop(seq)
            pkv.paged_kv_write(kp, vp, up(k), up(v), torch.from_numpy(bm.slots(seq, 0, n)).to(dev))
    for p, c in w.forks:
        bm.fork(p, c)
    for i, seqs in enumerate(w.steps[:-1]):
        slots, pairs = bm.step(seqs)
        if len(pairs):
            pkv.copy_blocks(kp, vp, torch.from_numpy(pairs).to(dev))
        k, v = w.step_kv(i)
        pkv.paged_kv_write(kp, vp, up(k), up(v), torch.from_numpy(slots).to(dev))
    # the measured step: host block manager once (its cost is reported separately)
    th = time.perf_counter()
    slots, pairs = bm.step(w.steps[-1])
    host_bm_us = (time.perf_counter() - th) * 1e6
    k_new, v_new = (up(x) for x in w.step_kv(len(w.steps) - 1))
    slots_d = torch.from_numpy(slots).to(dev)
    pairs_d = torch.from_numpy(pairs).to(dev)
    width = w.max_blocks_per_seq
    if table_format == "two_level":
        E = LEAF_TOKENS // w.block_size
        ld, lv = bm.block_tables_2l(w.batch, -(-width // E), 0)
        tables = pkv.TwoLevelTables(torch.from_numpy(ld).to(dev), torch.from_numpy(lv).to(dev))
        table_bytes = int(ld.nbytes + lv.nbytes)
        width = ld.shape[1] * E
    else:
        tab = bm.block_tables16 if table_format == "int16" else bm.block_tables
        tables = torch.from_numpy(tab(w.batch, width, 0)).to(dev)
        table_bytes = int(tables.numel() * tables.element_size())
    lens_np = np.asarray([bm.seq_len(int(s)) for s in w.batch], dtype=np.int32)
    lens = torch.from_numpy(lens_np).to(dev)
    q = up(w.queries())
    out = torch.empty_like(q)
    ws = pkv.alloc_workspace(w.num_seqs, w.num_q_heads, w.head_dim, width, w.block_size, dev)
    torch.cuda.synchronize()
    log(f"set-up done; step has {len(pairs)} copy pairs, {len(slots)} new tokens")

    stream = torch.cuda.current_stream(dev)

    def step(e=None):
        if len(pairs):
            pkv.copy_blocks(kp, vp, pairs_d)
        pkv.decode_prepare(kp, vp, k_new, v_new, slots_d, q, tables, lens, ws)
        if e is not None:
            e[0].record(stream)
        pkv.paged_attention_partitions(q, kp, vp, tables, lens, w.scale, out, ws)
        if e is not None:
            e[1].record(stream)

    # timed region: exactly `steps` steps launched on the stream, nothing else in it
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    # the same steps again with HIP events around each partition pass (on the stream it
    # is launched on): the kernel's duration for the roofline (the events add a little
    # time to each step, so these steps are not the ones timed above)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    events_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    graph_ms = None
    if not args.eager:
        # the same step captured once as a HIP graph and replayed (data.6616ai.com
        # "PagedAttention 之外": graph capture removes the per-launch CPU cost of decode);
        # on this device a replay costs a few microseconds more than the stream launches
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            step()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    log(f"step {ms_step:.4f} ms as stream launches (with events {events_ms:.4f}, graph replays "
        f"{graph_ms if graph_ms is None else round(graph_ms, 4)})")
    part_all = [e[0].elapsed_time(e[1]) for e in ev]
    part_ms = float(np.mean(part_all))

    # outside the timed region: the other passes on their own, then the partition
    # pass after flushing L2 / MALL with a 512 MiB write
    def timed(fn, reps=10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    copy_ms = timed(lambda: pkv.copy_blocks(kp, vp, pairs_d)) if len(pairs) else 0.0
    prep_ms = timed(lambda: pkv.decode_prepare(kp, vp, k_new, v_new, slots_d, q, tables, lens, ws))
    write_ms = timed(lambda: pkv.paged_kv_write(kp, vp, k_new, v_new, slots_d))
    plan_ms = timed(lambda: pkv.paged_attention_plan(q, kp, vp, tables, lens, ws))
    log(f"step {ms_step:.4f} ms (partitions {part_ms:.4f}; alone: copy {copy_ms:.4f}, write+plan {prep_ms:.4f}, "
        f"write {write_ms:.4f}, plan {plan_ms:.4f})")
    flushed = []
    if args.flush_reps > 0:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(args.flush_reps):
            pkv.paged_attention_plan(q, kp, vp, tables, lens, ws)
            scratch.fill_(1)
            e0.record(stream)
            pkv.paged_attention_partitions(q, kp, vp, tables, lens, w.scale, out, ws)
            e1.record(stream)
            torch.cuda.synchronize()
            flushed.append(e0.elapsed_time(e1))
        del scratch

    uniq = unique_tokens(bm.block_tables(w.batch, w.max_blocks_per_seq, 0), lens_np, w.block_size)
    pt = partition_tokens_of(w, lens_np)
    ab = algorithmic_bytes(w, lens_np, table_format, uniq, pt)
    kv_gbs = ab["kv"] / (ms_step * 1e-3) / 1e9
    hbm_gbs = ab["kv_unique"] / (ms_step * 1e-3) / 1e9
    achieved = ab["total"] / (part_ms * 1e-3) / 1e9
    tag = w.name if not partition_tokens else f"{w.name}_p{partition_tokens}"
    traffic = stored_traffic(tag) if table_format == "int32" else None
    res = {
        "metric": METRIC,
        "value": round(kv_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
                   "context_tokens": int(lens_np.sum()), "max_context": int(lens_np.max()),
                   "partition_tokens": pt, "partition_rule": "fixed" if partition_tokens else "plan",
                   "copy_pairs": int(len(pairs)), "kv_bytes": ab["kv"], "kv_bytes_unique": ab["kv_unique"],
                   "tables": table_format, "table_bytes": table_bytes},
        # % of HBM peak counts each distinct block once (the bytes HBM must deliver); the
        # logical rate counts a block shared by several sequences once per sequence
        "pct_hbm_peak": round(100.0 * hbm_gbs / HBM_PEAK_GBS, 2),
        "hbm_kv_gbs": round(hbm_gbs, 2),
        "logical_kv_gbs": round(kv_gbs, 2),
        "tokens_per_s": round(w.num_seqs / (ms_step * 1e-3), 1),
        "attention_kv_gbs": round(ab["kv"] / ((plan_ms + part_ms) * 1e-3) / 1e9, 2),
        "kernel_ms": {"attn_partitions": round(part_ms, 5), "copy_blocks_alone": round(copy_ms, 5),
                      "write_and_plan_alone": round(prep_ms, 5), "kv_write_alone": round(write_ms, 5),
                      "attn_plan_alone": round(plan_ms, 5)},
        "attn_partitions_ms_after_cache_flush": round(float(np.median(flushed)), 5) if flushed else None,
        "attn_partitions_ms_spread": spread(part_all),
        "attn_partitions_ms_after_cache_flush_spread": spread(flushed) if flushed else None,
        "host_block_manager_step_us": round(host_bm_us, 1),
        "step_launch": "stream",
        "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 5),
        "events_ms_per_step": round(events_ms, 5),
        "roofline": {"kernel": "attn_partition" + (" + attn_merge_long" if ab["merge_long"] else ""),
                     "bound": "hbm", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": ab},
    }
    pkv.set_decode_partition_tokens(0)
    if with_cpu:
        del kp, vp
        torch.cuda.empty_cache()
        log("timing the oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(w, w.all_context_kv(), args.cpu_seconds)
    return res


def sub_record(r, partition_tokens=0):
    """The fields of a decode record carried inside the headline line."""
    return {"workload": r["config"]["workload"], "partition_tokens": r["config"]["partition_tokens"],
            "partition_rule": r["config"]["partition_rule"], "ms_per_step": r["ms_per_step"],
            "value": r["value"], "unit": r["unit"], "pct_hbm_peak": r["pct_hbm_peak"],
            "tokens_per_s": r["tokens_per_s"], "kernel_ms": r["kernel_ms"],
            "attn_partitions_ms_spread": r["attn_partitions_ms_spread"],
            "roofline": {k: r["roofline"][k] for k in ("kernel", "bound", "achieved", "peak", "unit", "frac", "traffic")},
            "algorithmic_bytes": r["roofline"]["algorithmic_bytes"]["total"],
            "context_tokens": r["config"]["context_tokens"], "block_size": r["config"]["block_size"]}


HEADLINE = "long_bf16_b16"
# other decode configurations the headline line carries: (key, workload, fixed partition size)
SUB_RECORDS = [("gqa_bf16", "gqa_bf16", 0), ("long_bf16_b32", "long_bf16_b32", 0),
               ("long_bf16_b16_p512", "long_bf16_b16", 512), ("cow_fp16_p1020", "cow_fp16_p1020", 0),
               ("cow_fp16_p1020_shuffled", "cow_fp16_p1020_shuffled", 0)]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None,
                    help=f"one workload's line; default: {HEADLINE} with the other decode configurations "
                         f"({', '.join(k for k, _, _ in SUB_RECORDS)}) and the streaming-read ceiling as sub-records")
    ap.add_argument("--num-seqs", type=int, default=None,
                    help="override the workload's number of sequences (decode workloads)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flush-reps", type=int, default=10,
                    help="extra partition-pass timings, each after a 512 MiB cache flush")
    ap.add_argument("--eager", action="store_true",
                    help="skip the HIP-graph replays of the decode step (the timed steps are stream launches)")
    ap.add_argument("--tables", choices=["int32", "int16", "two_level"], default="int32",
                    help="block-table format of the decode step (flat int32, flat 16-bit, or two-level)")
    ap.add_argument("--head-dim", type=int, choices=[64, 128], default=None,
                    help="gqa_bf16 / mha_bf16 / prefill_bf16 / chunked_bf16 at another head size (same lengths)")
    ap.add_argument("--block-size", type=int, choices=[16, 32], default=None,
                    help="gqa_bf16 / mha_bf16 / prefill_bf16 / chunked_bf16 at another block size (same lengths)")
    ap.add_argument("--partition-tokens", type=int, choices=[0, 512, 1024, 2048], default=0,
                    help="fix the decode partition size (0: the plan pass chooses per batch)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the path runs on one GPU, see the design notes for how it would shard)", file=sys.stderr)
        sys.exit(2)

    import torch
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "reps": 5}))
        return

    import paged_kv_cache_281_amd as pkv
    import synth
    pkv.load()
    if args.workload == "stream_ceiling":
        stream_main(args, dev)
        return
    name = args.workload or HEADLINE
    if name in synth.LENCLASS_WORKLOADS:
        lenclass_main(args, synth.by_name(name), dev)
        return
    if name in synth.PREFIX_WORKLOADS:
        prefix_main(args, synth.by_name(name), dev)
        return
    if name in synth.SWAP_WORKLOADS:
        swap_main(args, synth.by_name(name), dev)
        return
    if name in synth.PREFILL_WORKLOADS:
        shape = {k: v for k, v in (("head_dim", args.head_dim), ("block", args.block_size)) if v}
        kw = dict(shape, **({"num_seqs": args.num_seqs} if args.num_seqs else {}))
        prefill_main(args, synth.by_name(name, **kw), dev)
        return
    if args.workload is not None:
        shape = {k: v for k, v in (("head_dim", args.head_dim), ("block", args.block_size)) if v}
        res = decode_run(args, name, dev, args.tables, args.partition_tokens, not args.no_cpu_baseline,
                         args.num_seqs, shape)
        print(json.dumps(res), flush=True)
        return
    # the headline line: the largest single-GPU configuration, with the other decode
    # configurations and the streaming-read ceiling carried as sub-records
    subs = {}
    for key, wname, pt in SUB_RECORDS:
        subs[key] = sub_record(decode_run(args, wname, dev, "int32", pt, False))
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    ceiling = stream_ceiling(dev, reps=5)
    log(f"streaming-read ceiling {ceiling['best_gbs']} GB/s ({ceiling['best']})")
    res = decode_run(args, HEADLINE, dev, "int32", 0, not args.no_cpu_baseline)
    res["sub_records"] = subs
    # the forked batch with its samples scattered through the batch, against the same
    # batch in prompt order (shared prefixes are found wherever their sequences sit)
    res["cow_shuffled_over_ordered"] = round(subs["cow_fp16_p1020_shuffled"]["ms_per_step"] /
                                             subs["cow_fp16_p1020"]["ms_per_step"], 4)
    res["hbm_read_ceiling"] = {k: ceiling[k] for k in ("bytes", "best_gbs", "best", "frac_of_peak", "kernel")}
    res["roofline"]["frac_of_read_ceiling"] = round(res["roofline"]["achieved"] / ceiling["best_gbs"], 4)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
