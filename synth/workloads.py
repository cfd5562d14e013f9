"""Workload definitions and seeded generators.

Every random draw comes from ``numpy.random.Generator(PCG64)`` seeded by a tuple
of integers, so a tensor can be regenerated on its own (one sequence's context,
one decode step's new tokens) without drawing the rest.  Values are drawn in
fp32 and rounded to the storage type with a round-to-nearest-even cast; the
arrays handed out are the raw storage bits (uint16 for bf16/fp16, uint32 for
fp32), so both sides see identical bytes.

Length mix: the interview post (ohmygp.com, "用模拟把浪费率算出来") simulates
request lengths drawn 70% from [32, 512), 25% from [512, 2048) and 5% from
[2048, 4096).  ``skewed_lengths`` draws from that mix, optionally with every
range scaled by an integer factor (factor 2 gives lengths up to 8191).
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import math
import os
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

# storage dtype name -> (numpy bits dtype, torch dtype, element bytes)
DTYPES: Dict[str, Tuple[type, torch.dtype, int]] = {
    "f32": (np.uint32, torch.float32, 4),
    "f16": (np.uint16, torch.float16, 2),
    "bf16": (np.uint16, torch.bfloat16, 2),
}

# quiet-NaN bit patterns used to poison pool memory that no sequence owns
NAN_BITS = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0}

# seed-tuple tags for the different value streams of one workload
_TAG_CTX_K, _TAG_CTX_V, _TAG_STEP_K, _TAG_STEP_V, _TAG_Q, _TAG_PF_Q = 1, 2, 3, 4, 5, 6
_TAG_SYS_TOK, _TAG_SFX_TOK, _TAG_SYS_K, _TAG_SYS_V, _TAG_SFX_K, _TAG_SFX_V, _TAG_REQ_Q = 7, 8, 9, 10, 11, 12, 13


def _gen_threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def normal_bits(key: Sequence[int], shape: Sequence[int], dtype: str) -> np.ndarray:
    """N(0,1) values of ``shape`` as raw ``dtype`` storage bits, from seed tuple ``key``."""
    n = int(np.prod(shape)) if len(shape) else 1
    rng = np.random.default_rng(list(key))
    x = rng.standard_normal(size=n, dtype=np.float32)
    bits_np, tdt, _ = DTYPES[dtype]
    if dtype == "f32":
        return x.view(np.uint32).reshape(shape)
    t = torch.from_numpy(x).to(tdt)  # round-to-nearest-even
    return t.view(torch.int16).numpy().view(np.uint16).reshape(shape)


def skewed_lengths(rng: np.random.Generator, n: int, factor: int = 1) -> np.ndarray:
    """Lengths from the interview post's skewed mix, every range scaled by ``factor``."""
    r = rng.random(n)
    u = rng.random(n)
    short = factor * 32 + np.floor(u * (480 * factor))
    mid = factor * 512 + np.floor(u * (1536 * factor))
    long_ = factor * 2048 + np.floor(u * (2048 * factor))
    return np.where(r < 0.7, short, np.where(r < 0.95, mid, long_)).astype(np.int64)


@dataclasses.dataclass
class Workload:
    """One decode workload: shapes, pool, block-manager operations and value seeds.

    Operations, replayed in this order by both sides:
      1. ``prefill``: for each (seq, n): add the sequence with n tokens and write
         their K/V (positions 0..n-1) from ``context_kv(seq, n)``.
      2. ``forks``: for each (parent, child): the child shares the parent's blocks.
      3. ``steps``: each entry is a list of sequence ids, ascending; every listed
         sequence appends one token; the step's copy-on-write pairs are copied
         before the step's tokens are written.  The last step is the measured one.
      4. attention over ``batch`` (output row i is sequence ``batch[i]``) with
         queries ``queries()``.
    """

    name: str
    seed: int
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    scale: float
    free_order: np.ndarray
    prefill: List[Tuple[int, int]]
    forks: List[Tuple[int, int]]
    steps: List[List[int]]
    batch: np.ndarray
    context_lens: np.ndarray  # length of each batch sequence after the last step
    notes: str = ""

    # ---- shapes -------------------------------------------------------------
    @property
    def num_seqs(self) -> int:
        return int(len(self.batch))

    @property
    def elem_bytes(self) -> int:
        return DTYPES[self.dtype][2]

    def kv_bytes_logical(self) -> int:
        """K+V bytes that attention reads: each context token once per KV head."""
        return int(2 * int(self.context_lens.sum()) * self.num_kv_heads * self.head_dim * self.elem_bytes)

    # ---- values -------------------------------------------------------------
    def context_kv(self, seq: int, n: int) -> Tuple[np.ndarray, np.ndarray]:
        shape = (n, self.num_kv_heads, self.head_dim)
        return (normal_bits((self.seed, _TAG_CTX_K, seq), shape, self.dtype),
                normal_bits((self.seed, _TAG_CTX_V, seq), shape, self.dtype))

    def all_context_kv(self, threads: Optional[int] = None) -> Dict[int, Tuple[np.ndarray, np.ndarray]]:
        """Context K/V of every prefilled sequence, drawn on a thread pool."""
        threads = threads or _gen_threads()
        jobs = [(s, n) for s, n in self.prefill]
        out: Dict[int, Tuple[np.ndarray, np.ndarray]] = {}
        with _cf.ThreadPoolExecutor(threads) as ex:
            futs = {}
            for s, n in jobs:
                shape = (n, self.num_kv_heads, self.head_dim)
                futs[ex.submit(normal_bits, (self.seed, _TAG_CTX_K, s), shape, self.dtype)] = (s, 0)
                futs[ex.submit(normal_bits, (self.seed, _TAG_CTX_V, s), shape, self.dtype)] = (s, 1)
            parts: Dict[Tuple[int, int], np.ndarray] = {}
            for f in _cf.as_completed(futs):
                parts[futs[f]] = f.result()
        for s, _ in jobs:
            out[s] = (parts[(s, 0)], parts[(s, 1)])
        return out

    def step_kv(self, step: int) -> Tuple[np.ndarray, np.ndarray]:
        shape = (len(self.steps[step]), self.num_kv_heads, self.head_dim)
        return (normal_bits((self.seed, _TAG_STEP_K, step), shape, self.dtype),
                normal_bits((self.seed, _TAG_STEP_V, step), shape, self.dtype))

    def queries(self) -> np.ndarray:
        return normal_bits((self.seed, _TAG_Q), (self.num_seqs, self.num_q_heads, self.head_dim), self.dtype)


@dataclasses.dataclass
class PrefillWorkload:
    """One prefill / chunked-prefill batch over a paged pool.

    Replayed by both sides in this order: for each sequence b (ascending) add it with
    ``context_lens[b]`` tokens and write their K/V (positions 0..L-1) from
    ``context_kv(b)``; the last ``chunk_lens[b]`` of them are the chunk.  Attention
    then takes ``queries()`` (the chunks' tokens back to back, ``[T, Hq, D]``).
    """

    name: str
    seed: int
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    scale: float
    free_order: np.ndarray
    context_lens: np.ndarray
    chunk_lens: np.ndarray
    notes: str = ""

    @property
    def num_seqs(self) -> int:
        return int(len(self.context_lens))

    @property
    def elem_bytes(self) -> int:
        return DTYPES[self.dtype][2]

    def query_start(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.chunk_lens)]).astype(np.int32)

    @property
    def num_tokens(self) -> int:
        return int(np.sum(self.chunk_lens))

    @property
    def max_query_len(self) -> int:
        return int(np.max(self.chunk_lens)) if len(self.chunk_lens) else 0

    def flops(self) -> int:
        """2 flops per multiply-add in q.K and in p.V: 4 * Hq * D per visible (row, key) pair."""
        L = self.context_lens.astype(np.int64)
        C = self.chunk_lens.astype(np.int64)
        pairs = int(np.sum(C * (L - C) + C * (C + 1) // 2))
        return 4 * self.num_q_heads * self.head_dim * pairs

    def kv_bytes(self) -> int:
        """K+V bytes of every context token once per KV head (each is read at least once)."""
        return int(2 * int(self.context_lens.sum()) * self.num_kv_heads * self.head_dim * self.elem_bytes)

    def context_kv(self, seq: int) -> Tuple[np.ndarray, np.ndarray]:
        shape = (int(self.context_lens[seq]), self.num_kv_heads, self.head_dim)
        return (normal_bits((self.seed, _TAG_CTX_K, seq), shape, self.dtype),
                normal_bits((self.seed, _TAG_CTX_V, seq), shape, self.dtype))

    def all_context_kv(self, threads: Optional[int] = None) -> Dict[int, Tuple[np.ndarray, np.ndarray]]:
        threads = threads or _gen_threads()
        with _cf.ThreadPoolExecutor(threads) as ex:
            futs = [ex.submit(self.context_kv, b) for b in range(self.num_seqs)]
            return {b: f.result() for b, f in enumerate(futs)}

    def queries(self) -> np.ndarray:
        return normal_bits((self.seed, _TAG_PF_Q), (self.num_tokens, self.num_q_heads, self.head_dim), self.dtype)


def prefill_workload(name: str, seed: int, dtype: str, context_lens, chunk_lens, hq: int, hkv: int, d: int,
                     block: int, slack: float = 1.1, notes: str = "") -> PrefillWorkload:
    """A prefill batch with the given context and chunk lengths; the pool holds
    ``slack`` times the blocks the batch needs, handed out in a seeded random order."""
    L = np.asarray(context_lens, dtype=np.int64)
    C = np.asarray(chunk_lens, dtype=np.int64)
    if np.any(C > L) or np.any(C < 0):
        raise ValueError("chunks must lie inside their contexts")
    rng = np.random.default_rng([seed, 7])
    need = int(sum(-(-int(x) // block) for x in L))
    num_blocks = max(1, int(math.ceil(slack * need)))
    width = int(max(1, max(-(-int(x) // block) for x in L)))
    return PrefillWorkload(name=name, seed=seed, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                           block_size=block, num_blocks=num_blocks, max_blocks_per_seq=width,
                           scale=1.0 / math.sqrt(d), free_order=rng.permutation(num_blocks).astype(np.int32),
                           context_lens=L.astype(np.int32), chunk_lens=C.astype(np.int32), notes=notes)


def prefill_bf16(seed: int = 1005, num_seqs: int = 64, head_dim: int = 128, block: int = 16) -> PrefillWorkload:
    """Whole-prompt prefill: 64 prompts with lengths from the interview post's request
    mix (each prompt is its own chunk), 32 q / 8 kv heads, D=128, B=16, bf16 (head and
    block size can be changed; the lengths stay the same)."""
    rng = np.random.default_rng(seed)
    L = skewed_lengths(rng, num_seqs, 1)
    return prefill_workload("prefill_bf16" + _shape_tag(head_dim, block), seed, "bf16", L, L, 32, 8, head_dim, block,
                            notes="prompt lengths from the skewed request mix; chunk = whole prompt")


def chunked_bf16(seed: int = 1006, num_seqs: int = 16, chunk: int = 512, head_dim: int = 128,
                 block: int = 16) -> PrefillWorkload:
    """Chunked prefill: 16 sequences whose earlier tokens (the skewed mix scaled x2, up
    to 8191) are already cached, each appending a chunk of 512 tokens; 32 q / 8 kv
    heads, D=128, B=16, bf16 (head and block size can be changed)."""
    rng = np.random.default_rng(seed)
    prefix = skewed_lengths(rng, num_seqs, 2)
    C = np.full(num_seqs, chunk, dtype=np.int64)
    return prefill_workload("chunked_bf16" + _shape_tag(head_dim, block), seed, "bf16", prefix + C, C, 32, 8,
                            head_dim, block, notes="cached prefix from the x2 skewed mix, then a 512-token chunk")


def _decode_workload(name: str, seed: int, dtype: str, lengths: np.ndarray, hq: int, hkv: int,
                     d: int, block: int, rng: np.random.Generator, num_blocks: Optional[int] = None,
                     width: Optional[int] = None, slack: float = 1.1, notes: str = "") -> Workload:
    """Batch decode: each sequence holds len-1 context tokens, the step writes token len-1."""
    lengths = np.asarray(lengths, dtype=np.int64)
    n = len(lengths)
    need = int(sum(-(-int(L) // block) for L in lengths))
    if num_blocks is None:
        num_blocks = int(math.ceil(slack * need))
    if width is None:
        width = int(max(1, max(-(-int(L) // block) for L in lengths)))
    free_order = rng.permutation(num_blocks).astype(np.int32)
    return Workload(
        name=name, seed=seed, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
        block_size=block, num_blocks=num_blocks, max_blocks_per_seq=width,
        scale=1.0 / math.sqrt(d), free_order=free_order,
        prefill=[(b, int(lengths[b]) - 1) for b in range(n)], forks=[],
        steps=[list(range(n))], batch=np.arange(n, dtype=np.int32),
        context_lens=lengths.astype(np.int32), notes=notes)


def tiny_fp32(seed: int = 1000, num_seqs: int = 4) -> Workload:
    """4 sequences, lengths U{1..64}, 8 q = 8 kv heads, D=64, B=16, pool of 64 blocks, fp32."""
    rng = np.random.default_rng(seed)
    lengths = rng.integers(1, 65, size=num_seqs)
    return _decode_workload("tiny_fp32", seed, "f32", lengths, 8, 8, 64, 16, rng,
                            num_blocks=64, width=4)


def _shape_tag(head_dim: int, block: int) -> str:
    """Name suffix of a batch built at another head size or block size than its default."""
    return (f"_d{head_dim}" if head_dim != 128 else "") + (f"_b{block}" if block != 16 else "")


def mha_bf16(seed: int = 1001, num_seqs: int = 64, max_len: Optional[int] = None, head_dim: int = 128,
             block: int = 16) -> Workload:
    """MHA 32 q = 32 kv heads, D=128, B=16, skewed mix, pool = need + 10%, bf16 (head and
    block size can be changed; the lengths stay the same)."""
    rng = np.random.default_rng(seed)
    lengths = skewed_lengths(rng, num_seqs, 1)
    if max_len is not None:
        lengths = np.minimum(lengths, max_len)
    return _decode_workload("mha_bf16" + _shape_tag(head_dim, block), seed, "bf16", lengths, 32, 32, head_dim,
                            block, rng, width=4096 // block if max_len is None else None)


def gqa_bf16(seed: int = 1002, num_seqs: int = 256, max_len: Optional[int] = None, head_dim: int = 128,
             block: int = 16) -> Workload:
    """GQA 32 q over 8 kv heads (4 per group), D=128, B=16, skewed mix x2 (up to 8191), bf16
    (head and block size can be changed; the lengths stay the same)."""
    rng = np.random.default_rng(seed)
    lengths = skewed_lengths(rng, num_seqs, 2)
    if max_len is not None:
        lengths = np.minimum(lengths, max_len)
    return _decode_workload("gqa_bf16" + _shape_tag(head_dim, block), seed, "bf16", lengths, 32, 8, head_dim,
                            block, rng, width=8192 // block if max_len is None else None)


def long_bf16(block_size: int = 16, seed: int = 1004, num_seqs: int = 8, context: int = 131072) -> Workload:
    """Long context: every sequence holds ``context`` tokens, 32 q / 8 kv heads, D=128, bf16.

    The pool holds exactly the blocks the batch needs (65536 at B=16, 32768 at B=32
    for 8 x 131072 tokens), placed by a random permutation.
    """
    rng = np.random.default_rng(seed)
    lengths = np.full(num_seqs, context, dtype=np.int64)
    need = num_seqs * (-(-context // block_size))
    return _decode_workload(f"long_bf16_b{block_size}", seed, "bf16", lengths, 32, 8, 128, block_size,
                            rng, num_blocks=need, width=-(-context // block_size))


def cow_fp16(prompt_len: int = 1020, seed: int = 1003, num_prompts: int = 64, samples: int = 4,
             max_suffix: int = 256, block: int = 16, hq: int = 32, hkv: int = 8, shuffle: bool = False) -> Workload:
    """Parallel sampling: prompts of ``prompt_len`` tokens, each forked into ``samples`` samples.

    Sample i of prompt k is sequence ``samples*k + i``; sample 0 is the prompt's own
    sequence.  Each sample has generated s ~ U{0..max_suffix} tokens before the
    measured step (one decode step per token, all samples stepping together), then
    the measured step appends one more token to every sample.  32 q / 8 kv heads,
    D=128, B=16, fp16 (block size and head counts can be changed for test cases).
    With ``shuffle`` the attention batch lists the same sequences in a seeded random
    order (a prompt's samples scattered through the batch); everything else is equal.
    """
    rng = np.random.default_rng(seed)
    n = num_prompts * samples
    suffix = rng.integers(0, max_suffix + 1, size=n)
    lengths = prompt_len + suffix + 1
    full_shared = prompt_len // block
    need = num_prompts * (-(-prompt_len // block))
    need += int(sum(-(-int(L) // block) - full_shared for L in lengths))
    num_blocks = int(math.ceil(1.1 * need))
    free_order = rng.permutation(num_blocks).astype(np.int32)
    steps: List[List[int]] = []
    for tau in range(int(suffix.max()) if n else 0):
        steps.append([i for i in range(n) if suffix[i] > tau])
    steps.append(list(range(n)))
    width = -(-(prompt_len + max_suffix + 1) // block)
    batch = np.arange(n, dtype=np.int32)
    if shuffle:
        batch = np.random.default_rng((seed, 1)).permutation(n).astype(np.int32)
    return Workload(
        name=f"cow_fp16_p{prompt_len}" + ("_shuffled" if shuffle else ""), seed=seed, dtype="f16", num_q_heads=hq, num_kv_heads=hkv,
        head_dim=128, block_size=block, num_blocks=num_blocks, max_blocks_per_seq=width,
        scale=1.0 / math.sqrt(128), free_order=free_order,
        prefill=[(samples * k, prompt_len) for k in range(num_prompts)],
        forks=[(samples * k, samples * k + i) for k in range(num_prompts) for i in range(1, samples)],
        steps=steps, batch=batch, context_lens=lengths[batch].astype(np.int32),
        notes=f"suffix lengths {suffix.tolist()}")


WORKLOADS = {
    "tiny_fp32": tiny_fp32,
    "mha_bf16": mha_bf16,
    "gqa_bf16": gqa_bf16,
    "cow_fp16_p1020": lambda **kw: cow_fp16(1020, **kw),
    "cow_fp16_p1024": lambda **kw: cow_fp16(1024, **kw),
    "cow_fp16_p1020_shuffled": lambda **kw: cow_fp16(1020, shuffle=True, **kw),
    "long_bf16_b16": lambda **kw: long_bf16(16, **kw),
    "long_bf16_b32": lambda **kw: long_bf16(32, **kw),
}


def restrict(base: Workload, name: str, seqs: Sequence[int], block: int, slack: float = 1.1) -> Workload:
    """``base`` (a one-step decode batch) restricted to ``seqs`` and held in blocks of
    ``block`` tokens, in a pool of ``slack`` times the blocks it needs placed by a seeded
    permutation.  Sequence ids and context values are those of ``base``; the step's new
    tokens and the queries are drawn for the restricted batch."""
    seqs = sorted(int(x) for x in seqs)
    pos = {int(s): i for i, s in enumerate(base.batch)}
    lengths = np.asarray([int(base.context_lens[pos[s]]) for s in seqs], dtype=np.int64)
    need = int(sum(-(-int(L) // block) for L in lengths))
    num_blocks = max(1, int(math.ceil(slack * need)))
    width = int(max([1] + [-(-int(L) // block) for L in lengths]))
    rng = np.random.default_rng([base.seed, block, len(seqs)])
    return Workload(
        name=name, seed=base.seed, dtype=base.dtype, num_q_heads=base.num_q_heads,
        num_kv_heads=base.num_kv_heads, head_dim=base.head_dim, block_size=block, num_blocks=num_blocks,
        max_blocks_per_seq=width, scale=base.scale, free_order=rng.permutation(num_blocks).astype(np.int32),
        prefill=[(s, int(L) - 1) for s, L in zip(seqs, lengths)], forks=[], steps=[seqs],
        batch=np.asarray(seqs, dtype=np.int32), context_lens=lengths.astype(np.int32),
        notes=f"{base.name} restricted to {len(seqs)} sequences, block {block}")


@dataclasses.dataclass
class LengthClassWorkload:
    """One decode batch under a per-length-class block size (agentalpha.top Q32, the
    résumé note after follow-up 2: short sequences in 16-token blocks, long ones in
    32-token blocks).  ``short`` and ``long`` split ``base`` at ``threshold`` tokens
    into a block-16 and a block-32 workload with pools of their own; ``all16`` (=
    ``base``) and ``all32`` hold the whole batch in one pool of either block size."""

    name: str
    threshold: int
    base: Workload
    short: Workload
    long: Workload
    all32: Workload


def lenclass_bf16(threshold: int = 1024, num_seqs: int = 256, max_len: Optional[int] = None) -> LengthClassWorkload:
    """The GQA batch (256 sequences, mix x2, 32/8 heads, D=128, bf16) split at 1024
    tokens: the mix's short range (70%) in block 16, the rest in block 32."""
    base = gqa_bf16(num_seqs=num_seqs, max_len=max_len)
    L = base.context_lens
    short = [int(s) for s, x in zip(base.batch, L) if int(x) < threshold]
    long_ = [int(s) for s, x in zip(base.batch, L) if int(x) >= threshold]
    return LengthClassWorkload(
        "lenclass_bf16", threshold, base,
        restrict(base, "lenclass_bf16_short_b16", short, 16),
        restrict(base, "lenclass_bf16_long_b32", long_, 32),
        restrict(base, "lenclass_bf16_all_b32", list(base.batch), 32))


LENCLASS_WORKLOADS = {"lenclass_bf16": lenclass_bf16}


@dataclasses.dataclass
class SwapWorkload:
    """Preemption by swapping: the ``base`` decode workload's sequences are placed
    (prefill operations only), then ``moved`` sequences go out to a host pool of
    ``host_blocks`` blocks and come back (data.6616ai.com "PagedAttention 之外")."""

    name: str
    base: Workload
    moved: List[int]
    host_blocks: int


def swap_bf16(num_moved: int = 64) -> SwapWorkload:
    """The GQA batch (256 sequences, mix x2, 32/8 heads, D=128, B=16, bf16); its first
    64 sequences are swapped out and back in."""
    base = gqa_bf16()
    moved = [int(s) for s in base.batch[:num_moved]]
    need = sum(-(-int(base.context_lens[i]) // base.block_size) for i in range(num_moved))
    return SwapWorkload("swap_bf16", base, moved, int(math.ceil(1.1 * need)))


SWAP_WORKLOADS = {"swap_bf16": swap_bf16}


@dataclasses.dataclass
class PrefixWorkload:
    """Requests that share system prompts (data.6616ai.com "PagedAttention 之外",
    prefix caching).  Request b is system prompt ``system_of[b]`` followed by its own
    suffix.  Token ids and K/V of a system prompt are drawn once per prompt, so equal
    prefixes hold equal K/V (as K/V at a position depend only on the tokens up to it);
    suffix values and every query row are drawn per request."""

    name: str
    seed: int
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    scale: float
    free_order: np.ndarray
    system_lens: List[int]
    system_of: List[int]
    suffix_lens: List[int]

    @property
    def num_seqs(self) -> int:
        return len(self.system_of)

    @property
    def elem_bytes(self) -> int:
        return DTYPES[self.dtype][2]

    def length(self, b: int) -> int:
        return self.system_lens[self.system_of[b]] + self.suffix_lens[b]

    def tokens(self, b: int) -> np.ndarray:
        s = self.system_of[b]
        sys_tok = np.random.default_rng([self.seed, _TAG_SYS_TOK, s]).integers(0, 32000, self.system_lens[s])
        sfx_tok = np.random.default_rng([self.seed, _TAG_SFX_TOK, b]).integers(0, 32000, self.suffix_lens[b])
        return np.concatenate([sys_tok, sfx_tok]).astype(np.int32)

    def kv(self, b: int) -> Tuple[np.ndarray, np.ndarray]:
        s = self.system_of[b]
        hs = (self.system_lens[s], self.num_kv_heads, self.head_dim)
        hx = (self.suffix_lens[b], self.num_kv_heads, self.head_dim)
        k = np.concatenate([normal_bits((self.seed, _TAG_SYS_K, s), hs, self.dtype),
                            normal_bits((self.seed, _TAG_SFX_K, b), hx, self.dtype)])
        v = np.concatenate([normal_bits((self.seed, _TAG_SYS_V, s), hs, self.dtype),
                            normal_bits((self.seed, _TAG_SFX_V, b), hx, self.dtype)])
        return k, v

    def queries(self, b: int) -> np.ndarray:
        """Query rows of every position of request b ``[L_b, Hq, D]``."""
        return normal_bits((self.seed, _TAG_REQ_Q, b), (self.length(b), self.num_q_heads, self.head_dim), self.dtype)


def prefix_bf16(seed: int = 1007, num_requests: int = 64, num_systems: int = 4) -> PrefixWorkload:
    """64 requests over 4 system prompts of U{512..2047} tokens; user suffixes from the
    interview post's request mix; 32 q / 8 kv heads, D=128, B=16, bf16."""
    rng = np.random.default_rng(seed)
    system_lens = rng.integers(512, 2048, size=num_systems).tolist()
    system_of = rng.integers(0, num_systems, size=num_requests).tolist()
    suffix_lens = skewed_lengths(rng, num_requests, 1).tolist()
    B = 16
    L = [system_lens[s] + x for s, x in zip(system_of, suffix_lens)]
    need = sum(-(-x // B) for x in L)
    nb = int(math.ceil(1.1 * need))
    return PrefixWorkload("prefix_bf16", seed, "bf16", 32, 8, 128, B, nb, max(-(-x // B) for x in L),
                          1.0 / math.sqrt(128), rng.permutation(nb).astype(np.int32), system_lens, system_of,
                          suffix_lens)


PREFIX_WORKLOADS = {"prefix_bf16": prefix_bf16}

PREFILL_WORKLOADS = {
    "prefill_bf16": prefill_bf16,
    "chunked_bf16": chunked_bf16,
}


def by_name(name: str, **kw):
    if name in LENCLASS_WORKLOADS:
        return LENCLASS_WORKLOADS[name](**kw)
    if name in PREFIX_WORKLOADS:
        return PREFIX_WORKLOADS[name](**kw)
    if name in SWAP_WORKLOADS:
        return SWAP_WORKLOADS[name](**kw)
    if name in PREFILL_WORKLOADS:
        return PREFILL_WORKLOADS[name](**kw)
    return WORKLOADS[name](**kw)
