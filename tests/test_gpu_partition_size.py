"""Decode partition size (1024 or 2048 tokens, chosen per launch by the plan pass, or 512
when fixed by the caller) and the plan's task list.

- Parity against the oracle with the size fixed at 512, 1024 and 2048 (both launch
  paths: decode_prepare + partitions, and the one-call decode), on shapes that reach
  every partition kernel, rows of several partitions with a ragged tail, and a row
  that needs the separate merge kernel at 1024 but not at 2048.
- The size the device picks equals the host rule (pkv_decode_partition_tokens).
- The item list holds exactly the expected items, in non-increasing length class:
  every sequence's own partitions, and for each group of sequences that share their
  leading blocks (copy-on-write samples, wherever they sit in the batch) the
  shared-prefix items that read those blocks once for several sequences.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_281_amd as pkv
import synth
from gpu_harness import log, replay_gpu, to_device
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


FUSED = 1 << 28  # item flag: a shared-prefix item that also computes its members' own tokens
FUSED_MAX_UNITS = 192  # 16-token units of a fused item at most
FUSED_MAX_PARTS = 4  # parts a fused group's work is cut into at most
PREFIX = 1 << 29  # item flag: a shared-prefix item (x holds the offset of its sequences)
SHARED = 1 << 30  # item flag: cached K/V loads (a group that needs several items)
MIN_SHARED = 256  # shortest shared prefix given shared-prefix items
WIN = 512  # sequences are grouped within aligned windows of this many


def _regions(n, hq, d, parts):
    """Byte offsets of the workspace regions (each 256-byte aligned)."""
    al = lambda x: (x + 255) // 256 * 256
    r = {"o": 0}
    r["ml"] = al(n * hq * parts * d * 4)
    r["tasks"] = r["ml"] + al(n * hq * parts * 2 * 4)
    r["done"] = r["tasks"] + al(n * parts * 16)
    r["seq_np"] = r["done"] + al(n * hq * 4)
    r["seq_grp"] = r["seq_np"] + al(n * 4)
    r["members"] = r["seq_grp"] + al(n * 16)
    r["member_own"] = r["members"] + al(n * 4)
    return r


def _read_plan(ws, n, hq, d, parts):
    """(counters, items [count, 4], partial count per sequence, members list, their own tokens)."""
    cnt = _counters(ws)
    r = _regions(n, hq, d, parts)
    i32 = lambda off, k: ws[off:off + 4 * k].view(torch.int32).cpu().numpy()
    tasks = i32(r["tasks"], 4 * int(cnt[0])).reshape(-1, 4)
    return cnt, tasks, i32(r["seq_np"], n), i32(r["members"], n), i32(r["member_own"], n)


def _plan(lens, hq, hkv, tables, d=128, block=16, prepare=False):
    """Runs the plan pass alone (or as the fused write + plan launch runs it, 1024
    threads, no tokens written) on a batch; returns what it wrote."""
    n = len(lens)
    W = tables.shape[1]
    q = torch.zeros(n, hq, d, dtype=torch.bfloat16, device=DEV)
    kp, vp = pkv.alloc_pools(1, block, hkv, d, torch.bfloat16, DEV)  # the plan reads no K/V
    ws = pkv.alloc_workspace(n, hq, d, W, block, DEV)
    lens_d = torch.from_numpy(np.asarray(lens, dtype=np.int32)).to(DEV)
    if prepare:
        kv_new = torch.zeros(0, hkv, d, dtype=torch.bfloat16, device=DEV)
        slots = torch.zeros(0, dtype=torch.int64, device=DEV)
        pkv.decode_prepare(kp, vp, kv_new, kv_new, slots, q, tables, lens_d, ws)
    else:
        pkv.paged_attention_plan(q, kp, vp, tables, lens_d, ws)
    torch.cuda.synchronize()
    parts = -(-W * block // pkv.PARTITION_TOKENS_MIN) + 1
    return _read_plan(ws, n, hq, d, parts)


def _groups(lens, rows, block, cm):
    """The shared-prefix groups the plan must find, restated: within aligned windows of
    WIN sequences, sequences of at least MIN_SHARED tokens with the same first block;
    the prefix is the shortest run of leading entries equal to the first member's, cut
    to blocks both fill; groups of two or more with a prefix of MIN_SHARED tokens or
    more.  Returns [(members, prefix tokens)]."""
    out = []
    if cm < 2:
        return out
    n = len(lens)
    for w0 in range(0, n, WIN):
        by_first = {}
        for b in range(w0, min(n, w0 + WIN)):
            if lens[b] >= MIN_SHARED and rows[b][0] >= 0:
                by_first.setdefault(int(rows[b][0]), []).append(b)
        for mem in by_first.values():
            if len(mem) < 2:
                continue
            a = mem[0]
            S = int(lens[a]) // block
            for b in mem[1:]:
                cap = min(int(lens[a]), int(lens[b])) // block
                j = 0
                while j < cap and rows[a][j] == rows[b][j]:
                    j += 1
                S = min(S, j)
            if S * block >= MIN_SHARED:
                out.append((mem, S * block))
    return out


def _fused(mem, S, lens, pt, cm, block):
    """A group whose items also compute its members' own tokens: block 16, the prefix in
    one partition, and the prefix plus min(cm, members) members of the group's longest
    context in at most FUSED_MAX_UNITS units."""
    per = min(cm, len(mem))
    maxl = max(int(lens[b]) for b in mem)
    return block == 16 and S <= pt and S // 16 + per * (-(-(maxl - S) // 16)) <= FUSED_MAX_UNITS


def _fused_parts(tasks, members, groups):
    """The parts of each fused group's work, read from its items (every item of a group
    carries the same count); checks that the batch has one count, cut to what each
    group's prefix allows (four prefix units per wave and part at least)."""
    x, wv = tasks[:, 0], tasks[:, 3]
    gid = {b: i for i, (mem, _) in enumerate(groups) for b in mem}
    parts = {}
    for a, v in zip(x, wv):
        if a & FUSED:
            g = gid[int(members[int(a) & (FUSED - 1)])]
            parts.setdefault(g, set()).add(int(v) >> 24)
    assert all(len(v) == 1 for v in parts.values()), "one part count per group"
    parts = {g: v.pop() for g, v in parts.items()}
    if parts:
        top = max(parts.values())
        assert 1 <= top <= FUSED_MAX_PARTS
        for g, n in parts.items():
            cap = groups[g][1] // 16 // 4  # four prefix units per wave
            assert n == min(top, cap), (n, top, cap)
    return {groups[g][0][0]: n for g, n in parts.items()}


def _check_plan(plan, lens, rows, pt, cm, block=16):
    """The item list holds exactly the expected items: every sequence's own partitions
    (after its shared prefix), and for every group ceil(members / cm) shared-prefix items
    per prefix partition whose sequences are the group's members, each once (a fused
    group: per column set, one item per part of its work, which also holds its members'
    own tokens, and no own items); partial counts per sequence; items in non-increasing
    length class.  Returns the groups."""
    cnt, tasks, seq_np, members, member_own = plan
    lens = np.asarray(lens, dtype=np.int64)
    if pt >= 1024:  # the partition kernels' grid then holds ceil(W * B / 1024) + 1 items per sequence
        assert int(cnt[0]) <= len(lens) * (-(-np.asarray(rows).shape[1] * block // 1024) + 1)
    groups = _groups(lens, rows, block, cm)
    sp = {b: S for mem, S in groups for b in mem}
    fused = {b for mem, S in groups if _fused(mem, S, lens, pt, cm, block) for b in mem}
    parts_by_first = _fused_parts(tasks, members, [(m, S) for m, S in groups if _fused(m, S, lens, pt, cm, block)])
    parts_of = {b: parts_by_first[mem[0]] for mem, S in groups if mem[0] in parts_by_first for b in mem}
    own, want_np = [], []
    for b, L in enumerate(lens):
        L = int(L)
        S = sp.get(b, 0)
        if b in fused:
            want_np.append(parts_of[b])
            continue
        npp = -(-S // pt)
        full, rem = (L - S) // pt, (L - S) % pt
        npb = 1 if L == 0 else npp + full + (rem > 0)
        want_np.append(npb)
        own += [(b, S + q * pt, pt, npp + q, npb) for q in range(full)]
        if rem or L == 0:
            own.append((b, S + full * pt, rem, npp + full, npb))
    assert np.array_equal(seq_np, want_np)
    x, tok0, ntok, wv = (tasks[:, i] for i in range(4))
    is_prefix = (x & PREFIX) != 0
    got_own = [(int(a), int(t), int(k), int(v & 0xffff), int(v >> 16))
               for a, t, k, v in zip(x[~is_prefix], tok0[~is_prefix], ntok[~is_prefix], wv[~is_prefix])]
    assert sorted(got_own) == sorted(own)
    assert not (x[~is_prefix] & SHARED).any()
    # shared-prefix items: (group, partition) -> the members its items cover
    group_of = {b: min(mem) for mem, _ in groups for b in mem}
    seen = {}
    for a, t, k, v in zip(x[is_prefix], tok0[is_prefix], ntok[is_prefix], wv[is_prefix]):
        off, p, nm = int(a) & (FUSED - 1), int(v) & 0xffff, (int(v) >> 16) & 0xff
        mem = [int(m) for m in members[off:off + nm]]
        assert 1 <= nm <= cm
        assert len({group_of.get(m, -1) for m in mem}) == 1 and mem[0] in group_of, "an item mixes groups"
        if a & FUSED:  # the members' own tokens, beside their ids
            assert [int(o) for o in member_own[off:off + nm]] == [int(lens[m]) - sp[m] for m in mem]
        seen.setdefault((group_of[mem[0]], p, int(t), int(k), bool(a & SHARED), bool(a & FUSED)), []).extend(mem)
    want = {}
    for mem, S in groups:
        ncs = -(-len(mem) // cm)
        if _fused(mem, S, lens, pt, cm, block):
            for p in range(parts_of[mem[0]]):
                want[(min(mem), p, 0, S, ncs > 1, True)] = sorted(mem)
            continue
        for p in range(-(-S // pt)):
            want[(min(mem), p, p * pt, min(pt, S - p * pt), ncs > 1, False)] = sorted(mem)
    assert {k: sorted(v) for k, v in seen.items()} == want
    # longest first: classes of pt/64 tokens never increase along the list (a fused item
    # is classed by its share of the prefix plus its members' longest own tokens, at most
    # a partition)
    size = ntok.astype(np.int64).copy()
    for i, (a, v) in enumerate(zip(x, wv)):
        if a & FUSED:
            mem = [int(m) for m in members[int(a) & (FUSED - 1):][:(int(v) >> 16) & 0xff]]
            S = sp[mem[0]]
            g = next(g for g, _ in groups if mem[0] in g)
            whole = S + min(cm, len(g)) * (max(int(lens[b]) for b in g) - S)
            size[i] = min(pt, -(-whole // parts_of[mem[0]]))
    cls = np.where(size > 0, -(-size // (pt // 64)), 1)
    assert (np.diff(cls) <= 0).all(), "classes must not increase along the list"
    return groups


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
    rows = np.repeat(np.arange(len(lens), dtype=np.int32)[:, None], W, axis=1)
    plan = _plan(lens, hq, hkv, torch.from_numpy(rows).to(DEV))
    pt = pkv.decode_partition_tokens(lens, hq, hkv)
    log(f"{name}: host rule {pt}, device log2 {plan[0][1]}, {plan[0][0]} items")
    assert 1 << int(plan[0][1]) == pt
    assert _check_plan(plan, lens, rows, pt, 16 // (hq // hkv) if 1 <= hq // hkv <= 8 else 0) == []


@pytest.mark.parametrize("tokens", [512, 1024, 2048])
def test_shared_prefix_groups_of_forked_samples(tokens, partition_tokens):
    """Copy-on-write samples: each prompt's 4 samples share its first 63 blocks (the
    tail block was copied for three of them), so every prompt becomes one group with a
    1008-token prefix and one shared-prefix item per prefix partition."""
    partition_tokens(tokens)
    w = synth.cow_fp16(1020, num_prompts=8, max_suffix=256)
    st = replay_gpu(w, w.all_context_kv(), DEV)
    lens = st.context_lens.cpu().numpy().astype(np.int64)
    rows = st.tables.cpu().numpy()
    plan = _plan(lens, w.num_q_heads, w.num_kv_heads, st.tables.contiguous())
    assert 1 << int(plan[0][1]) == tokens
    groups = _check_plan(plan, lens, rows, tokens, 4)
    assert sorted(sorted(m) for m, _ in groups) == [[4 * k + i for i in range(4)] for k in range(8)]
    assert all(S == 1008 for _, S in groups)


def test_groups_form_wherever_members_sit():
    """The same forked batch with its samples shuffled through the batch gives the same
    groups (as sets of sequences) and the same prefixes."""
    w = synth.cow_fp16(1020, num_prompts=8, max_suffix=256)
    st = replay_gpu(w, w.all_context_kv(), DEV)
    lens = st.context_lens.cpu().numpy().astype(np.int64)
    rows = st.tables.cpu().numpy()
    perm = np.random.default_rng(3).permutation(len(lens))
    pt = pkv.decode_partition_tokens(lens, 32, 8)
    ordered = _check_plan(_plan(lens, 32, 8, st.tables.contiguous()), lens, rows, pt, 4)
    shuffled = _check_plan(_plan(lens[perm], 32, 8, torch.from_numpy(rows[perm]).to(DEV)), lens[perm], rows[perm],
                           pt, 4)
    back = sorted((sorted(int(perm[b]) for b in m), S) for m, S in shuffled)
    assert back == sorted((sorted(m), S) for m, S in ordered)


def test_plan_groups_only_equal_leading_blocks():
    """One first block for all rows: sequences of 256 tokens or more form one group whose
    prefix is the shortest member's whole blocks (35 members in 9 items of 4); distinct
    first blocks give no groups, nor do rows that agree on only 160 leading tokens."""
    lens = np.array([100 + 37 * i for i in range(40)], dtype=np.int64)
    W = int(-(-lens.max() // 16))
    pt = pkv.decode_partition_tokens(lens, 32, 8)
    same = np.zeros((40, W), dtype=np.int32)
    diff = np.repeat(np.arange(40, dtype=np.int32)[:, None], W, axis=1)
    early = same.copy()
    early[:, 10:] = np.arange(40, dtype=np.int32)[:, None]  # rows agree on 10 blocks (160 tokens) only
    for rows, n_groups in ((same, 1), (diff, 0), (early, 0)):
        plan = _plan(lens, 32, 8, torch.from_numpy(rows).to(DEV))
        groups = _check_plan(plan, lens, rows, pt, 4)
        assert len(groups) == n_groups
    g = _groups(lens, same, 16, 4)
    assert len(g[0][0]) == 35 and g[0][1] == (285 // 16) * 16


@pytest.mark.parametrize("seed", range(6))
def test_task_list_on_random_batches(seed):
    """Random batches (more sequences than either plan launch has threads, several
    grouping windows, empty contexts, contexts that are whole partitions, groups of
    sequences with equal leading blocks scattered through the batch, rows that diverge
    at random places) through both plan launches: the expected items, in the order the
    plan promises, and the partition size of the host rule."""
    rng = np.random.default_rng(seed)
    n = int(rng.choice([1, 17, 300, 1500]))
    lens = rng.integers(0, 9000, size=n)
    lens[rng.random(n) < 0.05] = 0
    whole = rng.random(n) < 0.05
    lens[whole] = 2048 * rng.integers(1, 4, size=int(whole.sum()))
    W = max(1, int(-(-lens.max() // 16)))
    # rows: a group id per sequence (few groups, scattered), the group's shared entries up
    # to a random divergence point, then entries of the sequence's own
    gid = rng.integers(0, max(1, n // 5), size=n)
    base = rng.integers(0, 1 << 20, size=(int(gid.max()) + 1, W)).astype(np.int32)
    rows = base[gid].copy()
    cut = rng.integers(0, W + 1, size=n)
    own_ids = (np.arange(n, dtype=np.int64)[:, None] * W + np.arange(W)[None, :] + (1 << 21)).astype(np.int32)
    mask = np.arange(W)[None, :] >= cut[:, None]
    rows[mask] = own_ids[mask]
    tables = torch.from_numpy(rows).to(DEV)
    pt = pkv.decode_partition_tokens(lens, 32, 8)
    for prepare in (False, True):
        plan = _plan(lens, 32, 8, tables, prepare=prepare)
        log(f"seed {seed} prepare={prepare}: N={n} partition {1 << int(plan[0][1])} (rule {pt}), {plan[0][0]} items")
        assert 1 << int(plan[0][1]) == pt
        _check_plan(plan, lens, rows, pt, 4)


def test_grid_holds_the_longest_item_list():
    """With partitions of 1024 tokens or more the partition grid holds ceil(W * B / 1024)
    + 1 items per sequence.  Three samples of one 512-token prompt at 8 query heads per KV
    head (two members per column set) form one fused group of two column sets, each cut
    into three parts: six items, exactly the grid of three sequences with 45-block rows.
    Both launch paths match the oracle."""
    w = synth.cow_fp16(512, num_prompts=1, samples=3, max_suffix=200, hq=16, hkv=2)
    st = replay_gpu(w, w.all_context_kv(), DEV)
    lens = st.context_lens.cpu().numpy().astype(np.int64)
    rows = st.tables.cpu().numpy()
    plan = _plan(lens, w.num_q_heads, w.num_kv_heads, st.tables.contiguous())
    assert 1 << int(plan[0][1]) == 1024
    groups = _check_plan(plan, lens, rows, 1024, 2)
    assert len(groups) == 1
    assert int(plan[0][0]) == len(lens) * (-(-rows.shape[1] * 16 // 1024) + 1) == 6
    _run_case(w, fused=True)
    _run_case(w, check_pools=False)


def test_partition_size_changed_between_plan_and_partitions(partition_tokens):
    """A plan made with 512-token partitions lists more items (20) than the grid of
    1024-token partitions holds (12); the partition pass sizes its grid from its
    workspace's plan, not from the size set when it is launched, so the output equals
    the one-call decode at 512 bit for bit."""
    w = synth.long_bf16(16, num_seqs=2, context=5000)
    st = replay_gpu(w, w.all_context_kv(), DEV)
    q = to_device(w.queries(), w.dtype, DEV)
    partition_tokens(512)
    ref = pkv.paged_attention_decode(q, st.k_pool, st.v_pool, st.tables, st.context_lens, w.scale)
    ws = pkv.alloc_workspace(w.num_seqs, w.num_q_heads, w.head_dim, w.max_blocks_per_seq, w.block_size, DEV)
    pkv.paged_attention_plan(q, st.k_pool, st.v_pool, st.tables, st.context_lens, ws)
    partition_tokens(0)
    out = torch.full_like(q, float("nan"))
    pkv.paged_attention_partitions(q, st.k_pool, st.v_pool, st.tables, st.context_lens, w.scale, out, ws)
    torch.cuda.synchronize()
    cnt = _counters(ws)
    log(f"plan at 512: {cnt[0]} items, partitions launched with the plan's choice in force")
    assert int(cnt[1]) == 9 and int(cnt[0]) == 20
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("n,block,want", [(128, 16, 1024), (160, 16, 2048), (128, 32, 2048)])
def test_device_choice_at_head_size_64(n, block, want):
    """At head size 64 with 16-token blocks the plan needs the token work per slot to
    reach the whole longest item (not two thirds of it) before it takes 2048-token
    partitions: GQA batches of 128 and 160 sequences fall on either side; with 32-token
    blocks 128 sequences already take 2048.  The device agrees with the host rule."""
    lens = np.asarray(synth.gqa_bf16(num_seqs=n).context_lens, dtype=np.int64)
    W = int(-(-lens.max() // block))
    rows = np.repeat(np.arange(len(lens), dtype=np.int32)[:, None], W, axis=1)
    plan = _plan(lens, 32, 8, torch.from_numpy(rows).to(DEV), d=64, block=block)
    pt = pkv.decode_partition_tokens(lens, 32, 8, 64, block)
    log(f"D=64 B={block}, {n} sequences: host rule {pt}, device log2 {plan[0][1]}")
    assert pt == want and 1 << int(plan[0][1]) == want
    _check_plan(plan, lens, rows, pt, 4, block)
