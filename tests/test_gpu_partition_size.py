"""Decode partition size (1024 or 2048 tokens, chosen per launch by the plan pass, or 512
when fixed by the caller) and the plan's task list.

- Parity against the oracle with the size fixed at 512, 1024 and 2048 (both launch
  paths: decode_prepare + partitions, and the one-call decode), on shapes that reach
  every partition kernel, rows of several partitions with a ragged tail, and a row
  that needs the separate merge kernel at 1024 but not at 2048.
- The size the device picks equals the host rule (pkv_decode_partition_tokens).
- The task list is a permutation of the expected (sequence, partition) items, full
  partitions first, tail items in non-increasing length class, and the tail items of
  sequences that share their first block (copy-on-write samples) listed together and
  flagged for cached K/V loads.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_281_amd as pkv
import synth
from gpu_harness import log, replay_gpu
from test_gpu_parity import _custom, _run_case

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture
def partition_tokens():
    """Sets the process-wide partition size for one test and restores the plan's choice."""
    def set_(tokens):
        pkv.set_decode_partition_tokens(tokens)
    yield set_
    pkv.set_decode_partition_tokens(0)


CASES = [
    ("tiny_fp32", lambda: synth.tiny_fp32(seed=7, num_seqs=16)),
    ("f32_g4_d64_b32", lambda: _custom("f32_g4", "f32", 8, 2, 64, 32, [1, 1023, 2048, 2049, 4500], seed=5)),
    ("mha_bf16", lambda: synth.mha_bf16(num_seqs=6, max_len=4500)),
    ("gqa_bf16", lambda: synth.gqa_bf16(num_seqs=12, max_len=6000)),
    ("f16_g8_d64_b16", lambda: _custom("f16_g8", "f16", 16, 2, 64, 16, [2, 2047, 2048, 2049, 3000, 6143], seed=9)),
    ("cow_fp16_p1020", lambda: synth.cow_fp16(1020, num_prompts=3, max_suffix=200)),
    # shared-prefix groups (cached K/V loads) in the 32-token-block kernel, and flagged
    # tasks in the vector-ALU kernel (one query head per kv head), which streams them
    ("cow_fp16_b32", lambda: synth.cow_fp16(1020, num_prompts=3, max_suffix=200, block=32)),
    ("cow_fp16_mha", lambda: synth.cow_fp16(1020, num_prompts=3, max_suffix=200, hq=8, hkv=8)),
    ("long_bf16_b16", lambda: synth.long_bf16(16, num_seqs=2, context=5000)),
    ("long_bf16_b32", lambda: synth.long_bf16(32, num_seqs=2, context=5000)),
    # 40 partitions at 1024 (separate merge kernel), 20 at 2048 (merged by the last finisher)
    ("long_merge", lambda: synth.long_bf16(16, num_seqs=1, context=40000)),
]


@pytest.mark.parametrize("tokens", [512, 1024, 2048])
@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
def test_parity_at_each_partition_size(name, make, tokens, partition_tokens):
    partition_tokens(tokens)
    w = make()
    log(f"partition size {tokens}: {name}")
    _run_case(w, fused=True)
    _run_case(w, check_pools=False)


def _counters(ws: torch.Tensor) -> np.ndarray:
    # the workspace ends with a 256-byte counter block: [number of items, log2 partition size, ...]
    return ws[-256:].view(torch.int32)[:2].cpu().numpy()


SHARED = 1 << 30  # task flag: the sequence shares its first block with a neighbour


def _tasks(ws: torch.Tensor, n: int, hq: int, d: int, parts: int, count: int) -> np.ndarray:
    # workspace regions (each 256-byte aligned): partial outputs, (max, sum) pairs, tasks
    al = lambda x: (x + 255) // 256 * 256
    off = al(n * hq * parts * d * 4) + al(n * hq * parts * 2 * 4)
    return ws[off:off + count * 8].view(torch.int32).view(-1, 2).cpu().numpy()


def _items(tasks: np.ndarray) -> np.ndarray:
    """The (item, length) pairs with the shared-group flag cleared."""
    t = tasks.copy()
    t[:, 0] &= ~SHARED
    return t


def _plan(lens, hq, hkv, tables, d=128, block=16):
    """Runs the plan pass alone on a batch; returns the counters and the task list."""
    n = len(lens)
    W = tables.shape[1]
    q = torch.zeros(n, hq, d, dtype=torch.bfloat16, device=DEV)
    kp, vp = pkv.alloc_pools(1, block, hkv, d, torch.bfloat16, DEV)  # the plan reads no K/V
    ws = pkv.alloc_workspace(n, hq, d, W, block, DEV)
    lens_d = torch.from_numpy(np.asarray(lens, dtype=np.int32)).to(DEV)
    pkv.paged_attention_plan(q, kp, vp, tables, lens_d, ws)
    torch.cuda.synchronize()
    cnt = _counters(ws)
    parts = -(-W * block // pkv.PARTITION_TOKENS_MIN)
    return cnt, _tasks(ws, n, hq, d, parts, int(cnt[0])), parts


BATCHES = [
    ("gqa_256", lambda: synth.gqa_bf16().context_lens, 32, 8),
    ("gqa_32", lambda: synth.gqa_bf16(num_seqs=32).context_lens, 32, 8),
    ("mha_64", lambda: synth.mha_bf16().context_lens, 32, 32),
    ("long_1", lambda: synth.long_bf16(16, num_seqs=1).context_lens, 32, 8),
    ("gqa_96", lambda: synth.gqa_bf16(num_seqs=96).context_lens, 32, 8),
    ("boundary_63", lambda: np.full(63, 2048), 32, 8),
    ("boundary_64", lambda: np.full(64, 2048), 32, 8),
    ("short", lambda: np.array([0, 1, 1024, 17]), 32, 8),
    ("many", lambda: np.random.default_rng(4).integers(0, 3000, size=3000), 8, 8),
]


@pytest.mark.parametrize("name,lens_fn,hq,hkv", BATCHES, ids=[b[0] for b in BATCHES])
def test_device_choice_matches_host_rule(name, lens_fn, hq, hkv):
    lens = np.asarray(lens_fn(), dtype=np.int64)
    W = max(1, int(-(-lens.max() // 16)))
    tables = torch.arange(len(lens), dtype=torch.int32, device=DEV).repeat_interleave(W).view(len(lens), W)
    cnt, tasks, parts = _plan(lens, hq, hkv, tables.contiguous())
    pt = pkv.decode_partition_tokens(lens, hq, hkv)
    log(f"{name}: host rule {pt}, device log2 {cnt[1]}, {cnt[0]} items")
    assert 1 << int(cnt[1]) == pt
    expect = sorted((b * parts + p, int(L)) for b, L in enumerate(lens) for p in range(max(1, -(-int(L) // pt))))
    assert sorted(map(tuple, _items(tasks).tolist())) == expect
    assert not (tasks[:, 0] & SHARED).any()  # distinct first blocks: no groups


def _group_classes(lens, first, pt):
    """Tail class of each sequence's group (0: no tail item), the plan's grouping restated:
    a sequence follows the previous one when both are non-empty, share the first block and
    lie in the same aligned run of 16."""
    n = len(lens)
    cls = np.zeros(n, dtype=np.int64)
    for b, L in enumerate(lens):
        rem = int(L) % pt
        cls[b] = -(-rem // (pt // 64)) if rem else (1 if L == 0 else 0)
    head = np.ones(n, dtype=bool)
    for b in range(1, n):
        head[b] = not (b % 16 and lens[b] > 0 and lens[b - 1] > 0 and first[b] == first[b - 1])
    groups, g = [], []
    for b in range(n):
        if head[b] and g:
            groups.append(g)
            g = []
        g.append(b)
    groups.append(g)
    out = np.zeros(n, dtype=np.int64)
    for g in groups:
        out[g] = max(cls[g])
    return out, groups


def _check_order(tasks, parts, lens, first, pt):
    """The task list holds every expected item once, full partitions first (in the top
    class, with the tails that fill more than 63/64 of a partition), tail items in
    non-increasing group class, each group's tail items together in sequence order.
    Items of a group of two or more sequences carry the shared flag, the others not.
    Returns the groups."""
    flags = (tasks[:, 0] & SHARED) != 0
    tasks = _items(tasks)
    expect = sorted((b * parts + p, int(L)) for b, L in enumerate(lens) for p in range(max(1, -(-int(L) // pt))))
    assert sorted(map(tuple, tasks.tolist())) == expect
    gcls, groups = _group_classes(lens, first, pt)
    size = np.zeros(len(lens), dtype=np.int64)
    for g in groups:
        size[g] = len(g)
    assert np.array_equal(flags, size[tasks[:, 0] // parts] > 1)
    b_of, p_of = tasks[:, 0] // parts, tasks[:, 0] % parts
    tail = (p_of == lens[b_of] // pt) & ((lens[b_of] % pt != 0) | (lens[b_of] == 0))
    key = np.where(tail, gcls[b_of], 64)  # full partitions share the top class with tails of > 63/64 of one
    assert (np.diff(key) <= 0).all(), "classes must not increase along the list"
    pos = {int(t): i for i, t in enumerate(tasks[:, 0])}
    for g in groups:
        tail_pos = [pos[b * parts + int(lens[b]) // pt] for b in g if lens[b] % pt or lens[b] == 0]
        if tail_pos:
            assert tail_pos == list(range(tail_pos[0], tail_pos[0] + len(tail_pos))), (g, tail_pos)
    return groups


@pytest.mark.parametrize("tokens", [512, 1024, 2048])
def test_task_list_order_and_shared_prefix_groups(tokens, partition_tokens):
    partition_tokens(tokens)
    w = synth.cow_fp16(1020, num_prompts=8, max_suffix=256)
    st = replay_gpu(w, w.all_context_kv(), DEV)
    tables = st.tables.contiguous()
    lens = st.context_lens.cpu().numpy().astype(np.int64)
    cnt, tasks, parts = _plan(lens, w.num_q_heads, w.num_kv_heads, tables)
    assert 1 << int(cnt[1]) == tokens
    groups = _check_order(tasks, parts, lens, tables[:, 0].cpu().numpy(), tokens)
    assert len(groups) == 8  # one group per prompt: its 4 samples share the prompt's first block


def test_plan_groups_only_equal_first_blocks():
    """Equal first blocks group sequences in aligned runs of 16 (here 3 groups); distinct
    first blocks leave every sequence on its own (40 groups)."""
    lens = np.array([100 + 37 * i for i in range(40)], dtype=np.int64)
    pt = pkv.decode_partition_tokens(lens, 32, 8)
    assert pt == 1024
    W = int(-(-lens.max() // 16))  # rows wide enough for every context (longer ones are clamped)
    same = torch.zeros(40, W, dtype=torch.int32, device=DEV)
    diff = torch.arange(40, dtype=torch.int32, device=DEV).repeat_interleave(W).view(40, W).contiguous()
    for tables, n_groups in ((same, 3), (diff, 40)):
        cnt, tasks, parts = _plan(lens, 32, 8, tables)
        groups = _check_order(tasks, parts, lens, tables[:, 0].cpu().numpy(), pt)
        assert len(groups) == n_groups
    # with one first block: runs 16..31 (largest tail class 62), 0..15 (41), 32..39 (33)
    cnt, tasks, parts = _plan(lens, 32, 8, same)
    tasks = _items(tasks)
    b_of, p_of = tasks[:, 0] // parts, tasks[:, 0] % parts
    tails = [int(b) for b, p in zip(b_of, p_of) if p == lens[b] // 1024]
    assert tails == list(range(16, 32)) + list(range(0, 16)) + list(range(32, 40))


def _plan_prepare(lens, hq, hkv, tables, d=128, block=16):
    """The plan as the fused write + plan launch runs it (256 threads; no tokens written)."""
    n = len(lens)
    W = tables.shape[1]
    q = torch.zeros(n, hq, d, dtype=torch.bfloat16, device=DEV)
    kp, vp = pkv.alloc_pools(1, block, hkv, d, torch.bfloat16, DEV)
    kv_new = torch.zeros(0, hkv, d, dtype=torch.bfloat16, device=DEV)
    slots = torch.zeros(0, dtype=torch.int64, device=DEV)
    ws = pkv.alloc_workspace(n, hq, d, W, block, DEV)
    lens_d = torch.from_numpy(np.asarray(lens, dtype=np.int32)).to(DEV)
    pkv.decode_prepare(kp, vp, kv_new, kv_new, slots, q, tables, lens_d, ws)
    torch.cuda.synchronize()
    cnt = _counters(ws)
    parts = -(-W * block // pkv.PARTITION_TOKENS_MIN)
    return cnt, _tasks(ws, n, hq, d, parts, int(cnt[0])), parts


@pytest.mark.parametrize("seed", range(6))
def test_task_list_on_random_batches(seed):
    """Random batches (more sequences than either plan launch has threads, empty
    contexts, contexts that are whole partitions, runs of shared first blocks that cross
    the aligned runs of 16) through both plan launches: a valid task list in the order
    the plan promises, and the partition size of the host rule."""
    rng = np.random.default_rng(seed)
    n = int(rng.choice([1, 17, 300, 1500]))
    lens = rng.integers(0, 9000, size=n)
    lens[rng.random(n) < 0.05] = 0
    whole = rng.random(n) < 0.05
    lens[whole] = 2048 * rng.integers(1, 4, size=int(whole.sum()))
    # first blocks: runs of equal ids of random length (1..40), distinct between runs
    first = np.zeros(n, dtype=np.int64)
    b, run_id = 0, 0
    while b < n:
        k = int(rng.integers(1, 41))
        first[b:b + k] = run_id
        b += k
        run_id += 1
    W = max(1, int(-(-lens.max() // 16)))
    rows = np.repeat(first[:, None], W, axis=1).astype(np.int32)
    tables = torch.from_numpy(rows).to(DEV)
    pt = pkv.decode_partition_tokens(lens, 32, 8)
    for run in (_plan, _plan_prepare):
        cnt, tasks, parts = run(lens, 32, 8, tables)
        log(f"seed {seed} {run.__name__}: N={n} partition {1 << int(cnt[1])} (rule {pt}), {cnt[0]} items")
        assert 1 << int(cnt[1]) == pt
        _check_order(tasks, parts, lens.astype(np.int64), first, pt)
