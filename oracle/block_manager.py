"""Block manager: per-sequence block tables, on-demand allocation, fork and copy-on-write.

Follows:
* agentalpha.top Q32, answer part 2 (PagedAttention的解决方案): the KV cache is cut
  into fixed-size blocks (16 tokens by default) allocated on demand; each request
  keeps a block table from logical block to physical block (its example: logical
  0 -> physical 5, logical 1 -> physical 12); a new token either lands in the
  current block or opens a new one, and stored data never moves.
* agentalpha.top Q32, answer part 3 (Copy-on-Write) and ohmygp.com "破局思路"
  (写时共享): sequences that share a prefix map their logical blocks to the same
  physical blocks, a reference count tracks the sharers, and a block is copied
  only when one sharer writes into it.
* data.6616ai.com "PagedAttention：把虚拟内存搬进 KV Cache": blocks are requested one
  at a time as a request grows; shared prefix blocks are refcounted and copied
  only at divergence.

Readings where the pages leave the policy open (all stated in the design notes):
* the free list starts in a caller-given order and hands out blocks from its
  front; a block whose count drops to zero goes to its back;
* a sequence added with n tokens receives ceil(n / B) blocks at once;
* appending at position ``pos``: when ``pos % B == 0`` a fresh block is opened;
  otherwise, when the tail block is shared (count > 1), the writer takes a fresh
  block, the pair (old tail -> fresh) is emitted for copying, and the old tail
  loses one reference; the last remaining sharer writes in place;
* a batch step visits sequences in the order given (ascending ids).

Moving sequences between two managers (a device pool and a host pool) models the
swap-out / swap-in of preemption (data.6616ai.com "PagedAttention 之外", scheduler
and preemption; "可能的追问"): the moved sequences get fresh blocks in the
destination, taken from its free list in the order their blocks are first met;
a block shared by several moved sequences is copied once and stays shared; the
source blocks are then released as by ``free_seq``.  The (source, destination)
block pairs to copy are returned in that order.
"""
from __future__ import annotations

import collections
from typing import Dict, List, Optional, Sequence, Tuple


class OutOfBlocks(RuntimeError):
    pass


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, free_order: Sequence[int]):
        order = [int(x) for x in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of range(num_blocks)")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.free = collections.deque(order)
        self.refcount = [0] * self.num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}

    # -- allocation -----------------------------------------------------------
    def _available(self) -> int:
        """Blocks an allocation may take."""
        return len(self.free)

    def _take(self) -> int:
        if not self.free:
            raise OutOfBlocks("no free block")
        blk = self.free.popleft()
        self.refcount[blk] = 1
        return blk

    def add_seq(self, seq: int, num_tokens: int) -> None:
        """Register ``seq`` holding ``num_tokens`` tokens: ceil(n/B) fresh blocks."""
        if seq in self.tables:
            raise ValueError(f"sequence {seq} exists")
        nblk = -(-int(num_tokens) // self.block_size)
        if nblk > self._available():
            raise OutOfBlocks("not enough free blocks")
        self.tables[seq] = [self._take() for _ in range(nblk)]
        self.lens[seq] = int(num_tokens)

    def fork(self, parent: int, child: int) -> None:
        """``child`` shares every block of ``parent``; each shared block gains a reference."""
        if child in self.tables:
            raise ValueError(f"sequence {child} exists")
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for blk in self.tables[child]:
            self.refcount[blk] += 1

    def append_slot(self, seq: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Reserve the slot of the next token of ``seq``.

        Returns (slot, cow) where slot = physical_block * B + offset and cow is
        (src_block, dst_block) when the write lands in a shared block, else None.
        """
        B = self.block_size
        table = self.tables[seq]
        pos = self.lens[seq]
        cow = None
        if pos % B == 0:
            table.append(self._take())
        else:
            tail = table[-1]
            if self.refcount[tail] > 1:
                fresh = self._take()
                self.refcount[tail] -= 1
                table[-1] = fresh
                cow = (tail, fresh)
        slot = table[pos // B] * B + pos % B
        self.lens[seq] = pos + 1
        return slot, cow

    def step(self, seqs: Sequence[int]) -> Tuple[List[int], List[Tuple[int, int]]]:
        """One decode step: append a slot for each sequence in order; collect CoW pairs."""
        slots, pairs = [], []
        for s in seqs:
            slot, cow = self.append_slot(int(s))
            slots.append(slot)
            if cow is not None:
                pairs.append(cow)
        return slots, pairs

    def free_seq(self, seq: int) -> None:
        """Drop ``seq``; blocks whose count reaches zero return to the back of the free list."""
        for blk in self.tables.pop(seq):
            self.refcount[blk] -= 1
            if self.refcount[blk] == 0:
                self._release(blk)
        del self.lens[seq]

    def _release(self, blk: int) -> None:
        self.free.append(blk)

    # -- lookups --------------------------------------------------------------
    def slot_of(self, seq: int, pos: int) -> int:
        """Slot of logical position ``pos``: block table[pos // B], offset pos % B."""
        B = self.block_size
        return self.tables[seq][pos // B] * B + pos % B

    def slots(self, seq: int, pos0: int, count: int) -> List[int]:
        return [self.slot_of(seq, p) for p in range(pos0, pos0 + count)]

    def block_table(self, seq: int) -> List[int]:
        return list(self.tables[seq])

    def block_tables(self, seqs: Sequence[int], width: int, pad: int) -> List[List[int]]:
        rows = []
        for s in seqs:
            t = self.tables[int(s)]
            if len(t) > width:
                raise ValueError("table wider than width")
            rows.append(t + [pad] * (width - len(t)))
        return rows


def move_seqs(src: BlockManager, dst: BlockManager, seqs: Sequence[int]) -> List[Tuple[int, int]]:
    """Move ``seqs`` (in order) from ``src`` to ``dst``; returns the block pairs to copy.

    All or nothing: unknown or duplicate sequences, a sequence already in ``dst``,
    or too few free blocks in ``dst`` raise before anything changes.
    """
    seqs = [int(s) for s in seqs]
    if len(set(seqs)) != len(seqs):
        raise ValueError("duplicate sequence")
    for s in seqs:
        if s not in src.tables:
            raise KeyError(f"unknown sequence {s}")
        if s in dst.tables:
            raise ValueError(f"sequence {s} exists in the destination")
    if src.block_size != dst.block_size:
        raise ValueError("block sizes differ")
    distinct = {b for s in seqs for b in src.tables[s]}
    if len(distinct) > dst._available():
        raise OutOfBlocks("destination has too few free blocks")
    mapping: Dict[int, int] = {}
    pairs: List[Tuple[int, int]] = []
    for s in seqs:
        table = []
        for b in src.tables[s]:
            if b in mapping:
                c = mapping[b]
                dst.refcount[c] += 1
            else:
                c = dst._take()
                mapping[b] = c
                pairs.append((b, c))
            table.append(c)
        dst.tables[s] = table
        dst.lens[s] = src.lens[s]
    for s in seqs:
        src.free_seq(s)
    return pairs


# ---------------------------------------------------------------------------------
# Prefix caching: data.6616ai.com "PagedAttention 之外" (the KV blocks of a prefix
# shared across requests, such as a system prompt, are cached and reused, saving
# prefill compute; vLLM's automatic prefix caching).  Readings (stated in the design
# notes): each full block of a prompt is keyed by FNV-1a 64 over the key of the block
# before it (0 for the first) followed by its token ids; a lookup also checks the
# stored parent key and tokens.  A new prompt reuses the cached blocks of its longest
# cached prefix of full blocks, never the block holding its last token (that token is
# always computed).  Its other full blocks are registered when allocated (unless the
# key is taken); its partial tail and blocks filled later by decoding are not cached.
# A cached block whose count drops to zero stays addressable in an evictable list in
# release order; allocation takes the free list first, then evicts the least
# recently released cached block.
# ---------------------------------------------------------------------------------
FNV64_OFFSET = 0xCBF29CE484222325
FNV64_PRIME = 0x100000001B3
_MASK64 = (1 << 64) - 1


def fnv1a64(data: bytes, h: int = FNV64_OFFSET) -> int:
    """FNV-1a, 64-bit: for each byte, h ^= byte, then h *= prime (mod 2^64)."""
    for byte in data:
        h ^= byte
        h = (h * FNV64_PRIME) & _MASK64
    return h


def block_key(parent_key: int, tokens: Sequence[int]) -> int:
    data = int(parent_key).to_bytes(8, "little") + b"".join(
        int(t).to_bytes(4, "little", signed=True) for t in tokens)
    return fnv1a64(data)


class PrefixCachingBlockManager(BlockManager):
    def __init__(self, num_blocks: int, block_size: int, free_order: Sequence[int]):
        super().__init__(num_blocks, block_size, free_order)
        self.cached: Dict[int, int] = {}                      # key -> block
        self.info: Dict[int, Tuple[int, int, Tuple[int, ...]]] = {}  # block -> (key, parent key, tokens)
        self.evictable: "collections.OrderedDict[int, None]" = collections.OrderedDict()

    def _available(self) -> int:
        return len(self.free) + len(self.evictable)

    def _take(self) -> int:
        if self.free:
            blk = self.free.popleft()
        elif self.evictable:
            blk, _ = self.evictable.popitem(last=False)
            key = self.info.pop(blk)[0]
            del self.cached[key]
        else:
            raise OutOfBlocks("no free block")
        self.refcount[blk] = 1
        return blk

    def _release(self, blk: int) -> None:
        if blk in self.info:
            self.evictable[blk] = None
        else:
            self.free.append(blk)

    def add_seq_tokens(self, seq: int, tokens: Sequence[int]) -> int:
        """Register ``seq`` with prompt ``tokens``; returns the number of leading tokens
        whose KV is already in the pool (a multiple of B)."""
        if seq in self.tables:
            raise ValueError(f"sequence {seq} exists")
        B = self.block_size
        tokens = [int(t) for t in tokens]
        n = len(tokens)
        nblk = -(-n // B)
        lookup = max(n - 1, 0) // B      # full blocks entirely before the last token
        keys, hits, parent = [], [], 0
        for i in range(n // B):
            toks = tuple(tokens[i * B:(i + 1) * B])
            key = block_key(parent, toks)
            keys.append((key, parent, toks))
            blk = self.cached.get(key)
            if i < lookup and len(hits) == i and blk is not None and self.info[blk][1:] == (parent, toks):
                hits.append(blk)
            parent = key
        pinned_evictable = sum(1 for b in hits if self.refcount[b] == 0)
        if nblk - len(hits) > self._available() - pinned_evictable:
            raise OutOfBlocks("not enough free blocks")
        for b in hits:
            if self.refcount[b] == 0:
                del self.evictable[b]
            self.refcount[b] += 1
        table = list(hits)
        for i in range(len(hits), nblk):
            blk = self._take()
            if i < len(keys) and keys[i][0] not in self.cached:
                self.cached[keys[i][0]] = blk
                self.info[blk] = keys[i]
            table.append(blk)
        self.tables[seq] = table
        self.lens[seq] = n
        return len(hits) * B
