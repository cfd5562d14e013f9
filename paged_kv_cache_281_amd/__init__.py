"""Paged KV-cache decode for AMD Instinct MI355X (gfx950).

A thin Python binding of ``libpkv.so`` (C ABI declared in ``include/pkv.h``).
This module only marshals arguments -- torch tensors become device pointers and
the current HIP stream -- and raises on a non-zero status.  Every step of the
path runs in the library's HIP kernels; there is no fallback: if the library is
missing, every call raises.

Pool tensors use the library's physical layout, with X = 16 / element_bytes:
  K pool ``[num_blocks, num_kv_heads, head_dim // X, block_size, X]``
  V pool ``[num_blocks, num_kv_heads, head_dim, block_size]``
"""
from __future__ import annotations

import ctypes
import os
from typing import List, NamedTuple, Optional, Sequence, Tuple

import numpy as np
import torch

__all__ = [
    "load", "load_debug", "library_path", "PoolDesc", "pool_shapes", "alloc_pools", "alloc_host_pools", "pool_desc",
    "paged_kv_write", "copy_blocks", "swap_blocks", "workspace_bytes", "alloc_workspace", "TwoLevelTables",
    "paged_attention_decode", "paged_attention_partitions", "paged_attention_plan", "decode_prepare",
    "prefill_workspace_bytes", "alloc_prefill_workspace", "paged_attention_prefill", "BlockManager", "PkvError",
    "PARTITION_TOKENS_MIN", "PARTITION_TOKENS", "PARTITION_TOKENS_MAX", "LEAF_TOKENS", "DTYPE_CODES", "decode_partition_tokens", "TableRef",
    "set_decode_partition_tokens", "stream_read", "paged_attention_decode_noalloc", "NOALLOC_SCRATCH_BYTES",
]

PARTITION_TOKENS_MIN = 512  # smallest decode partition, only when fixed (PKV_PARTITION_TOKENS_MIN; the workspace unit)
PARTITION_TOKENS = 1024  # decode split-context partition (PKV_PARTITION_TOKENS)
PARTITION_TOKENS_MAX = 2048  # the longer partition the plan may choose (PKV_PARTITION_TOKENS_MAX)
LEAF_TOKENS = 512  # tokens whose block ids one two-level leaf holds (PKV_LEAF_TOKENS)
DTYPE_CODES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
_c_i32, _c_i64, _c_vp, _c_sz, _c_f = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float

_LIB = None


class PkvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class PoolDesc(ctypes.Structure):
    _fields_ = [("num_blocks", _c_i32), ("block_size", _c_i32), ("num_kv_heads", _c_i32),
                ("head_dim", _c_i32), ("dtype", _c_i32)]


class TableRef(ctypes.Structure):
    """pkv_table_ref: where the plan pass reads each sequence's first block id."""
    _fields_ = [("entries", _c_vp), ("leaf_dir", _c_vp), ("entry_bytes", _c_i32), ("reserved", _c_i32)]


def library_path() -> str:
    """The in-tree libpkv.so, or the file named by the PKV_LIBRARY environment variable."""
    return os.environ.get("PKV_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")


def load():
    """Load libpkv.so (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m paged_kv_cache_281_amd.build`")
    _LIB = _bind(ctypes.CDLL(path))
    return _LIB


def load_debug():
    """The debug build (libpkv_debug.so, PKV_DEBUG=1): same C ABI, with every device
    precondition checked on the host before launch.  Raises if it has not been built."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv_debug.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m paged_kv_cache_281_amd.build --debug`")
    return _bind(ctypes.CDLL(path))


def _bind(lib):
    P = ctypes.POINTER
    sig = {
        "pkv_version": ([], ctypes.c_char_p),
        "pkv_status_string": ([_c_i32], ctypes.c_char_p),
        "pkv_last_error": ([], ctypes.c_char_p),
        "pkv_pool_bytes": ([P(PoolDesc)], _c_sz),
        "pkv_paged_kv_write": ([P(PoolDesc), _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_vp], _c_i32),
        "pkv_copy_blocks": ([P(PoolDesc), _c_vp, _c_vp, _c_vp, _c_i32, _c_vp], _c_i32),
        "pkv_paged_attention_workspace_bytes": ([_c_i32, _c_i32, _c_i32, _c_i32, _c_i32], _c_sz),
        "pkv_paged_attention_decode": ([P(PoolDesc), _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_vp, _c_i32,
                                        _c_vp, _c_f, _c_vp, _c_sz, _c_vp], _c_i32),
        "pkv_paged_attention_partitions": ([P(PoolDesc), _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_vp,
                                            _c_i32, _c_vp, _c_f, _c_vp, _c_sz, _c_vp], _c_i32),
        "pkv_paged_attention_plan": ([P(PoolDesc), _c_i32, _c_i32, _c_i32, _c_vp, P(TableRef), _c_vp, _c_sz, _c_vp],
                                     _c_i32),
        "pkv_decode_prepare": ([P(PoolDesc), _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_vp,
                                P(TableRef), _c_vp, _c_sz, _c_vp], _c_i32),
        "pkv_decode_partition_tokens": ([P(PoolDesc), _c_vp, _c_i32, _c_i32, P(_c_i32)], _c_i32),
        "pkv_set_decode_partition_tokens": ([_c_i32], _c_i32),
        "pkv_paged_attention_prefill": ([P(PoolDesc), _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_vp, _c_i32,
                                         _c_i32, _c_vp, _c_i32, _c_vp, _c_f, _c_vp, _c_sz, _c_vp], _c_i32),
        "pkv_paged_attention_prefill_workspace_bytes": ([_c_i32, _c_i32, _c_i32, _c_i32], _c_sz),
        "pkv_swap_blocks": ([P(PoolDesc), _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_vp], _c_i32),
        "pkv_bm_move_seqs": ([_c_vp, _c_vp, _c_vp, _c_i32, _c_vp, _c_i32, P(_c_i32)], _c_i32),
        "pkv_paged_attention_decode_t16": ([P(PoolDesc), _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_vp, _c_i32,
                                            _c_vp, _c_f, _c_vp, _c_sz, _c_vp], _c_i32),
        "pkv_paged_attention_partitions_t16": ([P(PoolDesc), _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_vp,
                                                _c_i32, _c_vp, _c_f, _c_vp, _c_sz, _c_vp], _c_i32),
        "pkv_paged_attention_prefill_t16": ([P(PoolDesc), _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_vp, _c_i32,
                                             _c_i32, _c_vp, _c_i32, _c_vp, _c_f, _c_vp, _c_sz, _c_vp], _c_i32),
        "pkv_bm_block_tables16": ([_c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_vp], _c_i32),
        "pkv_paged_attention_decode_2l": ([P(PoolDesc), _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_vp, _c_i32,
                                           _c_vp, _c_i32, _c_vp, _c_f, _c_vp, _c_sz, _c_vp], _c_i32),
        "pkv_paged_attention_partitions_2l": ([P(PoolDesc), _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_vp,
                                               _c_i32, _c_vp, _c_i32, _c_vp, _c_f, _c_vp, _c_sz, _c_vp], _c_i32),
        "pkv_paged_attention_prefill_2l": ([P(PoolDesc), _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_vp, _c_i32,
                                            _c_i32, _c_vp, _c_i32, _c_vp, _c_i32, _c_vp, _c_f, _c_vp, _c_sz, _c_vp],
                                           _c_i32),
        "pkv_bm_block_tables_2l": ([_c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_vp, _c_vp, _c_i32, P(_c_i32)], _c_i32),
        "pkv_stream_read": ([_c_vp, _c_sz, _c_i32, _c_i32, _c_vp, _c_vp], _c_i32),
        "pkv_paged_attention_decode_noalloc": ([P(PoolDesc), _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_vp,
                                                _c_i32, _c_vp, _c_f, _c_vp], _c_i32),
        "pkv_bm_create": ([_c_i32, _c_i32, _c_vp, P(_c_vp)], _c_i32),
        "pkv_bm_set_prefix_cache": ([_c_vp, _c_i32], _c_i32),
        "pkv_bm_add_seq_tokens": ([_c_vp, _c_i32, _c_vp, _c_i32, P(_c_i32)], _c_i32),
        "pkv_bm_num_cached": ([_c_vp], _c_i32),
        "pkv_bm_destroy": ([_c_vp], None),
        "pkv_bm_add_seq": ([_c_vp, _c_i32, _c_i32], _c_i32),
        "pkv_bm_fork": ([_c_vp, _c_i32, _c_i32], _c_i32),
        "pkv_bm_append_slot": ([_c_vp, _c_i32, P(_c_i64), P(_c_i32), P(_c_i32)], _c_i32),
        "pkv_bm_step": ([_c_vp, _c_vp, _c_i32, _c_vp, _c_vp, P(_c_i32)], _c_i32),
        "pkv_bm_free_seq": ([_c_vp, _c_i32], _c_i32),
        "pkv_bm_seq_len": ([_c_vp, _c_i32, P(_c_i32)], _c_i32),
        "pkv_bm_slots": ([_c_vp, _c_i32, _c_i32, _c_i32, _c_vp], _c_i32),
        "pkv_bm_block_table": ([_c_vp, _c_i32, _c_vp, _c_i32, P(_c_i32)], _c_i32),
        "pkv_bm_block_tables": ([_c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_vp], _c_i32),
        "pkv_bm_refcount": ([_c_vp, _c_i32], _c_i32),
        "pkv_bm_num_free": ([_c_vp], _c_i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


def _check(status: int) -> None:
    if status != 0:
        lib = load()
        raise PkvError(status, f"{lib.pkv_status_string(status).decode()}: {lib.pkv_last_error().decode()}")


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _require(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


# ---- pools ------------------------------------------------------------------------
def pool_shapes(num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int, dtype: torch.dtype):
    x = 16 // torch.empty((), dtype=dtype).element_size()
    return ((num_blocks, num_kv_heads, head_dim // x, block_size, x),
            (num_blocks, num_kv_heads, head_dim, block_size))


def alloc_pools(num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int, dtype: torch.dtype,
                device="cuda") -> Tuple[torch.Tensor, torch.Tensor]:
    """Uninitialised K and V pools in the library's layout."""
    ks, vs = pool_shapes(num_blocks, block_size, num_kv_heads, head_dim, dtype)
    return torch.empty(ks, dtype=dtype, device=device), torch.empty(vs, dtype=dtype, device=device)


def pool_desc(k_pool: torch.Tensor, v_pool: torch.Tensor) -> PoolDesc:
    _require(k_pool.dim() == 5 and v_pool.dim() == 4, "K pool must be 5-D and V pool 4-D")
    nb, h, dx, B, x = k_pool.shape
    _require(k_pool.dtype in DTYPE_CODES and v_pool.dtype == k_pool.dtype, "unsupported or mismatched pool dtype")
    _require(x * k_pool.element_size() == 16, "K pool last dimension must span 16 bytes")
    _require(tuple(v_pool.shape) == (nb, h, dx * x, B), "V pool shape does not match the K pool")
    _require(k_pool.is_contiguous() and v_pool.is_contiguous(), "pools must be contiguous")
    _require(k_pool.is_cuda and v_pool.is_cuda, "pools must be device tensors")
    return PoolDesc(nb, B, h, dx * x, DTYPE_CODES[k_pool.dtype])


# ---- kernels ------------------------------------------------------------------------
def paged_kv_write(k_pool: torch.Tensor, v_pool: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                   slot_mapping: torch.Tensor) -> None:
    """Store token t's K/V ``[num_kv_heads, head_dim]`` in slot ``slot_mapping[t]`` (negative: skip)."""
    d = pool_desc(k_pool, v_pool)
    T = k_new.shape[0]
    for t in (k_new, v_new):
        _require(tuple(t.shape) == (T, d.num_kv_heads, d.head_dim), "k_new/v_new must be [T, Hkv, D]")
        _require(t.dtype == k_pool.dtype and t.is_contiguous() and t.device == k_pool.device, "k_new/v_new dtype/layout/device")
    _require(slot_mapping.dtype == torch.int64 and tuple(slot_mapping.shape) == (T,) and slot_mapping.is_contiguous()
             and slot_mapping.device == k_pool.device, "slot_mapping must be a contiguous int64 [T] device tensor")
    _check(load().pkv_paged_kv_write(ctypes.byref(d), _ptr(k_pool), _ptr(v_pool), _ptr(k_new), _ptr(v_new),
                                     _ptr(slot_mapping), T, _stream(k_pool.device)))


def copy_blocks(k_pool: torch.Tensor, v_pool: torch.Tensor, pairs: torch.Tensor) -> None:
    """For each row (src, dst) of the int64 ``[P, 2]`` device tensor, block dst becomes a copy of src."""
    d = pool_desc(k_pool, v_pool)
    _require(pairs.dtype == torch.int64 and pairs.dim() == 2 and pairs.shape[1] == 2 and pairs.is_contiguous()
             and pairs.device == k_pool.device, "pairs must be a contiguous int64 [P, 2] device tensor")
    _check(load().pkv_copy_blocks(ctypes.byref(d), _ptr(k_pool), _ptr(v_pool), _ptr(pairs), pairs.shape[0],
                                  _stream(k_pool.device)))


def alloc_host_pools(num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int, dtype: torch.dtype):
    """K and V pools of the device layout in pinned host memory (the swap target)."""
    ks, vs = pool_shapes(num_blocks, block_size, num_kv_heads, head_dim, dtype)
    return (torch.empty(ks, dtype=dtype, pin_memory=True), torch.empty(vs, dtype=dtype, pin_memory=True))


def swap_blocks(src_k: torch.Tensor, src_v: torch.Tensor, dst_k: torch.Tensor, dst_v: torch.Tensor,
                pairs: torch.Tensor) -> None:
    """For each row (s, d) of the int64 ``[P, 2]`` tensor, block d of the destination
    pools becomes a copy of block s of the source pools.  Pools are device tensors or
    pinned host tensors of the same tile layout (block counts may differ); ``pairs``
    is a device or pinned host tensor.  Runs on the current stream of the device
    involved."""
    for t in (src_k, src_v, dst_k, dst_v, pairs):
        _require(t.is_cuda or t.is_pinned(), "swap operands must be device tensors or pinned host tensors")
    _require(src_k.shape[1:] == dst_k.shape[1:] and src_v.shape[1:] == dst_v.shape[1:]
             and src_k.dtype == dst_k.dtype, "source and destination pools must share the tile layout")
    _require(src_k.dim() == 5 and src_v.dim() == 4 and src_k.shape[0] == src_v.shape[0]
             and dst_k.shape[0] == dst_v.shape[0], "K pools must be 5-D and V pools 4-D")
    _require(all(t.is_contiguous() for t in (src_k, src_v, dst_k, dst_v)), "pools must be contiguous")
    _require(pairs.dtype == torch.int64 and pairs.dim() == 2 and pairs.shape[1] == 2 and pairs.is_contiguous(),
             "pairs must be a contiguous int64 [P, 2] tensor")
    dev = next((t.device for t in (src_k, dst_k, pairs) if t.is_cuda), None)
    _require(dev is not None, "one operand must live on the device")
    nb, h, dx, B, x = src_k.shape
    _require(src_k.dtype in DTYPE_CODES and x * src_k.element_size() == 16, "unsupported pool layout")
    d = PoolDesc(nb, B, h, dx * x, DTYPE_CODES[src_k.dtype])
    _check(load().pkv_swap_blocks(ctypes.byref(d), _ptr(src_k), _ptr(src_v), _ptr(dst_k), _ptr(dst_v), _ptr(pairs),
                                  pairs.shape[0], _stream(dev)))


def workspace_bytes(num_seqs: int, num_q_heads: int, head_dim: int, max_blocks_per_seq: int, block_size: int) -> int:
    return int(load().pkv_paged_attention_workspace_bytes(num_seqs, num_q_heads, head_dim, max_blocks_per_seq,
                                                          block_size))


def alloc_workspace(num_seqs: int, num_q_heads: int, head_dim: int, max_blocks_per_seq: int, block_size: int,
                    device="cuda") -> torch.Tensor:
    n = workspace_bytes(num_seqs, num_q_heads, head_dim, max_blocks_per_seq, block_size)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


class TwoLevelTables(NamedTuple):
    """Two-level block tables: row b of ``leaf_dir`` (int32 ``[N, dir_width]``) names,
    for every run of ``LEAF_TOKENS // block_size`` entries of sequence b's table,
    the row of ``leaves`` (int32 ``[num_leaves, LEAF_TOKENS // block_size]``) that
    holds them.  Accepted wherever the attention calls take ``block_tables``."""
    leaf_dir: torch.Tensor
    leaves: torch.Tensor


def _tables(block_tables, N: int, d: PoolDesc, device):
    """(entry point suffix, the table arguments of the C call, flat width W)."""
    if isinstance(block_tables, TwoLevelTables):
        ld, lv = block_tables
        E = LEAF_TOKENS // d.block_size
        _require(ld.dtype == torch.int32 and ld.dim() == 2 and ld.shape[0] == N and ld.is_contiguous()
                 and ld.device == device, "leaf_dir must be a contiguous int32 [N, dir_width] device tensor")
        _require(lv.dtype == torch.int32 and lv.dim() == 2 and lv.shape[1] == E and lv.is_contiguous()
                 and lv.device == device, f"leaves must be a contiguous int32 [num_leaves, {E}] device tensor")
        return "_2l", (_ptr(ld), ld.shape[1], _ptr(lv), lv.shape[0]), ld.shape[1] * E
    _require(block_tables.dtype in (torch.int32, torch.int16) and block_tables.dim() == 2
             and block_tables.shape[0] == N and block_tables.is_contiguous() and block_tables.device == device,
             "block_tables must be a contiguous int32 (or 16-bit) [N, W] device tensor, or TwoLevelTables")
    suffix = "_t16" if block_tables.dtype == torch.int16 else ""
    return suffix, (_ptr(block_tables), block_tables.shape[1]), block_tables.shape[1]


def _attn_args(q, k_pool, v_pool, block_tables, context_lens, out, workspace):
    d = pool_desc(k_pool, v_pool)
    _require(q.dim() == 3 and q.shape[2] == d.head_dim and q.dtype == k_pool.dtype and q.is_contiguous()
             and q.device == k_pool.device, "q must be a contiguous [N, Hq, D] device tensor of the pool dtype")
    N, Hq, _ = q.shape
    _, _, W = _tables(block_tables, N, d, k_pool.device)
    _require(context_lens.dtype == torch.int32 and tuple(context_lens.shape) == (N,) and context_lens.is_contiguous()
             and context_lens.device == k_pool.device, "context_lens must be a contiguous int32 [N] device tensor")
    if out is None:
        out = torch.empty_like(q)
    _require(out.shape == q.shape and out.dtype == q.dtype and out.is_contiguous() and out.device == q.device,
             "out must match q")
    if workspace is None:
        workspace = alloc_workspace(N, Hq, d.head_dim, W, d.block_size, device=q.device)
    return d, N, Hq, W, out, workspace


def paged_attention_decode(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, block_tables: torch.Tensor,
                           context_lens: torch.Tensor, scale: float, out: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """softmax(scale * q K^T) V per sequence and query head, K/V read through the block tables."""
    d, N, Hq, W, out, ws = _attn_args(q, k_pool, v_pool, block_tables, context_lens, out, workspace)
    suffix, targs, _ = _tables(block_tables, N, d, k_pool.device)
    fn = getattr(load(), "pkv_paged_attention_decode" + suffix)
    _check(fn(ctypes.byref(d), _ptr(k_pool), _ptr(v_pool), _ptr(out), _ptr(q), N, Hq, *targs, _ptr(context_lens),
              float(scale), _ptr(ws), ws.numel(), _stream(q.device)))
    return out


NOALLOC_SCRATCH_BYTES = 128 << 20  # PKV_NOALLOC_SCRATCH_BYTES


def paged_attention_decode_noalloc(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                                   block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                                   out: torch.Tensor) -> torch.Tensor:
    """``paged_attention_decode`` without a workspace and without allocating: the library's
    fixed per-GPU scratch array holds the partials (``pkv_paged_attention_decode_noalloc``).
    ``out`` is caller-provided; int32 flat tables only.  Calls that overlap on one GPU race."""
    d = pool_desc(k_pool, v_pool)
    _require(q.dim() == 3 and q.shape[2] == d.head_dim and q.dtype == k_pool.dtype and q.is_contiguous()
             and q.device == k_pool.device, "q must be a contiguous [N, Hq, D] device tensor of the pool dtype")
    N, Hq, _ = q.shape
    _require(block_tables.dtype == torch.int32 and block_tables.dim() == 2 and block_tables.shape[0] == N
             and block_tables.is_contiguous() and block_tables.device == q.device,
             "block_tables must be a contiguous int32 [N, W] device tensor")
    _require(context_lens.dtype == torch.int32 and tuple(context_lens.shape) == (N,) and context_lens.is_contiguous()
             and context_lens.device == q.device, "context_lens must be a contiguous int32 [N] device tensor")
    _require(out is not None and out.shape == q.shape and out.dtype == q.dtype and out.is_contiguous()
             and out.device == q.device, "out must match q")
    _check(load().pkv_paged_attention_decode_noalloc(ctypes.byref(d), _ptr(k_pool), _ptr(v_pool), _ptr(out), _ptr(q),
                                                     N, Hq, _ptr(block_tables), block_tables.shape[1],
                                                     _ptr(context_lens), float(scale), _stream(q.device)))
    return out


def prefill_workspace_bytes(num_seqs: int, num_tokens: int, num_q_heads: int, num_kv_heads: int) -> int:
    return int(load().pkv_paged_attention_prefill_workspace_bytes(num_seqs, num_tokens, num_q_heads, num_kv_heads))


def alloc_prefill_workspace(num_seqs: int, num_tokens: int, num_q_heads: int, num_kv_heads: int,
                            device="cuda") -> torch.Tensor:
    n = prefill_workspace_bytes(num_seqs, num_tokens, num_q_heads, num_kv_heads)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def paged_attention_prefill(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                            block_tables: torch.Tensor, context_lens: torch.Tensor, query_start: torch.Tensor,
                            max_query_len: int, scale: float, out: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Causal attention of each sequence's chunk of new tokens over its paged context.

    ``q`` is ``[T, Hq, D]`` with sequence b's chunk in rows ``query_start[b] ..
    query_start[b+1]-1``; their K/V must already be in the pool (``context_lens``
    counts them).  ``max_query_len`` (host int) bounds every chunk length.
    """
    d = pool_desc(k_pool, v_pool)
    _require(q.dim() == 3 and q.shape[2] == d.head_dim and q.dtype == k_pool.dtype and q.is_contiguous()
             and q.device == k_pool.device, "q must be a contiguous [T, Hq, D] device tensor of the pool dtype")
    T, Hq, _ = q.shape
    _require(query_start.dtype == torch.int32 and query_start.dim() == 1 and query_start.is_contiguous()
             and query_start.device == k_pool.device, "query_start must be a contiguous int32 [N+1] device tensor")
    N = query_start.shape[0] - 1
    _require(N >= 0, "query_start needs N+1 entries")
    suffix, targs, _ = _tables(block_tables, N, d, k_pool.device)
    _require(context_lens.dtype == torch.int32 and tuple(context_lens.shape) == (N,) and context_lens.is_contiguous()
             and context_lens.device == k_pool.device, "context_lens must be a contiguous int32 [N] device tensor")
    if out is None:
        out = torch.empty_like(q)
    _require(out.shape == q.shape and out.dtype == q.dtype and out.is_contiguous() and out.device == q.device,
             "out must match q")
    if workspace is None:
        workspace = alloc_prefill_workspace(N, T, Hq, d.num_kv_heads, q.device)
    fn = getattr(load(), "pkv_paged_attention_prefill" + suffix)
    _check(fn(ctypes.byref(d), _ptr(k_pool), _ptr(v_pool), _ptr(out), _ptr(q), N, Hq, _ptr(query_start), T,
              int(max_query_len), *targs, _ptr(context_lens), float(scale), _ptr(workspace), workspace.numel(),
              _stream(q.device)))
    return out


def _table_ref(block_tables) -> TableRef:
    """The plan's view of the tables (first block id of each sequence)."""
    if isinstance(block_tables, TwoLevelTables):
        ld, lv = block_tables
        return TableRef(_ptr(lv), _ptr(ld), 4, 0)
    return TableRef(_ptr(block_tables), None, block_tables.element_size(), 0)


def paged_attention_plan(q, k_pool, v_pool, block_tables, context_lens, workspace) -> None:
    """First pass of ``paged_attention_decode``: the partition size and the (sequence,
    partition) task list."""
    d, N, Hq, W, _, ws = _attn_args(q, k_pool, v_pool, block_tables, context_lens, q, workspace)
    tr = _table_ref(block_tables)
    _check(load().pkv_paged_attention_plan(ctypes.byref(d), N, Hq, W, _ptr(context_lens), ctypes.byref(tr), _ptr(ws),
                                           ws.numel(), _stream(q.device)))


def decode_partition_tokens(context_lens, num_q_heads: int, num_kv_heads: int, head_dim: int = 128,
                            block_size: int = 16) -> int:
    """The partition size the plan pass picks for these context lengths (host values) on
    a 16-bit pool of this head and block size."""
    lens = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    out = _c_i32()
    pool = PoolDesc(1, int(block_size), int(num_kv_heads), int(head_dim), DTYPE_CODES[torch.bfloat16])
    _check(load().pkv_decode_partition_tokens(ctypes.byref(pool), lens.ctypes.data if lens.size else None, lens.size,
                                              int(num_q_heads), ctypes.byref(out)))
    return out.value


def set_decode_partition_tokens(tokens: int) -> None:
    """Fix the decode partition size of later calls (512, 1024 or 2048), or 0 for the plan's choice."""
    _check(load().pkv_set_decode_partition_tokens(int(tokens)))


def decode_prepare(k_pool, v_pool, k_new, v_new, slot_mapping, q, block_tables, context_lens, workspace) -> None:
    """The step's KV write and the attention plan pass in one launch (see ``paged_kv_write``
    and ``paged_attention_plan``); follow with ``paged_attention_partitions``."""
    d = pool_desc(k_pool, v_pool)
    T = k_new.shape[0]
    for t in (k_new, v_new):
        _require(tuple(t.shape) == (T, d.num_kv_heads, d.head_dim), "k_new/v_new must be [T, Hkv, D]")
        _require(t.dtype == k_pool.dtype and t.is_contiguous() and t.device == k_pool.device, "k_new/v_new dtype/layout/device")
    _require(slot_mapping.dtype == torch.int64 and tuple(slot_mapping.shape) == (T,) and slot_mapping.is_contiguous()
             and slot_mapping.device == k_pool.device, "slot_mapping must be a contiguous int64 [T] device tensor")
    _, N, Hq, W, _, ws = _attn_args(q, k_pool, v_pool, block_tables, context_lens, q, workspace)
    tr = _table_ref(block_tables)
    _check(load().pkv_decode_prepare(ctypes.byref(d), _ptr(k_pool), _ptr(v_pool), _ptr(k_new), _ptr(v_new),
                                     _ptr(slot_mapping), T, N, Hq, W, _ptr(context_lens), ctypes.byref(tr), _ptr(ws),
                                     ws.numel(), _stream(q.device)))


def paged_attention_partitions(q, k_pool, v_pool, block_tables, context_lens, scale, out, workspace) -> None:
    """Second pass of ``paged_attention_decode`` (partitions, with the merge of split rows)."""
    d, N, Hq, W, out, ws = _attn_args(q, k_pool, v_pool, block_tables, context_lens, out, workspace)
    suffix, targs, _ = _tables(block_tables, N, d, k_pool.device)
    fn = getattr(load(), "pkv_paged_attention_partitions" + suffix)
    _check(fn(ctypes.byref(d), _ptr(k_pool), _ptr(v_pool), _ptr(out), _ptr(q), N, Hq, *targs, _ptr(context_lens),
              float(scale), _ptr(ws), ws.numel(), _stream(q.device)))


def stream_read(src: torch.Tensor, sink: torch.Tensor, workgroups: int, unroll: int = 8) -> None:
    """Diagnostic: read every byte of the contiguous device tensor ``src`` once
    (``pkv_stream_read``); ``sink`` is an int32 device tensor of ``4 * workgroups`` entries."""
    _require(src.is_cuda and src.is_contiguous() and sink.is_cuda and sink.dtype == torch.int32
             and sink.numel() >= 4 * workgroups, "src must be a contiguous device tensor, sink int32 [4 * workgroups]")
    _check(load().pkv_stream_read(_ptr(src), src.numel() * src.element_size(), int(workgroups), int(unroll),
                                  _ptr(sink), _stream(src.device)))


# ---- host block manager ----------------------------------------------------------------
class BlockManager:
    """Host-side block manager of libpkv (tables, on-demand allocation, fork, copy-on-write)."""

    def __init__(self, num_blocks: int, block_size: int, free_order: Sequence[int], prefix_cache: bool = False):
        self._lib = load()
        order = np.ascontiguousarray(np.asarray(free_order, dtype=np.int32))
        _require(order.shape == (num_blocks,), "free_order must hold num_blocks entries")
        h = _c_vp()
        _check(self._lib.pkv_bm_create(num_blocks, block_size, order.ctypes.data, ctypes.byref(h)))
        self._h = h
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)
        if prefix_cache:
            _check(self._lib.pkv_bm_set_prefix_cache(self._h, 1))

    def add_seq_tokens(self, seq: int, tokens: Sequence[int]) -> int:
        """Add ``seq`` with prompt ``tokens``; returns how many leading tokens already
        have their K/V in the pool (prefix cache hits)."""
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        c = _c_i32()
        _check(self._lib.pkv_bm_add_seq_tokens(self._h, seq, t.ctypes.data, len(t), ctypes.byref(c)))
        return c.value

    def num_cached(self) -> int:
        return int(self._lib.pkv_bm_num_cached(self._h))

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.pkv_bm_destroy(h)
            self._h = None

    def add_seq(self, seq: int, num_tokens: int) -> None:
        _check(self._lib.pkv_bm_add_seq(self._h, seq, num_tokens))

    def fork(self, parent: int, child: int) -> None:
        _check(self._lib.pkv_bm_fork(self._h, parent, child))

    def append_slot(self, seq: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        slot, src, dst = _c_i64(), _c_i32(), _c_i32()
        _check(self._lib.pkv_bm_append_slot(self._h, seq, ctypes.byref(slot), ctypes.byref(src), ctypes.byref(dst)))
        return slot.value, (None if src.value < 0 else (src.value, dst.value))

    def step(self, seqs: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
        s = np.ascontiguousarray(np.asarray(seqs, dtype=np.int32))
        n = len(s)
        slots = np.empty(n, dtype=np.int64)
        pairs = np.empty((max(n, 1), 2), dtype=np.int64)
        npairs = _c_i32()
        _check(self._lib.pkv_bm_step(self._h, s.ctypes.data, n, slots.ctypes.data, pairs.ctypes.data,
                                     ctypes.byref(npairs)))
        return slots, pairs[:npairs.value].copy()

    def free_seq(self, seq: int) -> None:
        _check(self._lib.pkv_bm_free_seq(self._h, seq))

    def move_seqs(self, dst: "BlockManager", seqs: Sequence[int]) -> np.ndarray:
        """Move ``seqs`` to manager ``dst``; returns the int64 ``[P, 2]`` (source block,
        destination block) pairs to copy with ``swap_blocks``."""
        s = np.ascontiguousarray(np.asarray(seqs, dtype=np.int32))
        cap = max(1, self.num_blocks)
        pairs = np.empty((cap, 2), dtype=np.int64)
        n = _c_i32()
        _check(self._lib.pkv_bm_move_seqs(self._h, dst._h, s.ctypes.data, len(s), pairs.ctypes.data, cap,
                                          ctypes.byref(n)))
        return pairs[:n.value].copy()

    def seq_len(self, seq: int) -> int:
        n = _c_i32()
        _check(self._lib.pkv_bm_seq_len(self._h, seq, ctypes.byref(n)))
        return n.value

    def slots(self, seq: int, pos0: int, count: int) -> np.ndarray:
        out = np.empty(count, dtype=np.int64)
        _check(self._lib.pkv_bm_slots(self._h, seq, pos0, count, out.ctypes.data))
        return out

    def block_table(self, seq: int) -> List[int]:
        n = _c_i32()
        cap = self.num_blocks
        out = np.empty(cap, dtype=np.int32)
        _check(self._lib.pkv_bm_block_table(self._h, seq, out.ctypes.data, cap, ctypes.byref(n)))
        return out[:n.value].tolist()

    def block_tables16(self, seqs: Sequence[int], width: int, pad: int) -> np.ndarray:
        """Tables as 16-bit entries (``int16`` storage of the unsigned ids), for the
        ``_t16`` attention calls on pools of at most 65536 blocks."""
        s = np.ascontiguousarray(np.asarray(seqs, dtype=np.int32))
        out = np.empty((len(s), width), dtype=np.uint16)
        _check(self._lib.pkv_bm_block_tables16(self._h, s.ctypes.data, len(s), width, pad, out.ctypes.data))
        return out.view(np.int16)

    def block_tables_2l(self, seqs: Sequence[int], dir_width: int, pad: int) -> Tuple[np.ndarray, np.ndarray]:
        """Two-level tables (host arrays ``leaf_dir`` [n, dir_width], ``leaves``
        [num_leaves, LEAF_TOKENS // block_size]) for ``TwoLevelTables``."""
        s = np.ascontiguousarray(np.asarray(seqs, dtype=np.int32))
        ld = np.empty((len(s), dir_width), dtype=np.int32)
        n = ctypes.c_int32(0)
        _check(self._lib.pkv_bm_block_tables_2l(self._h, s.ctypes.data, len(s), dir_width, pad, ld.ctypes.data,
                                                None, 0, ctypes.byref(n)))
        lv = np.empty((n.value, LEAF_TOKENS // self.block_size), dtype=np.int32)
        _check(self._lib.pkv_bm_block_tables_2l(self._h, s.ctypes.data, len(s), dir_width, pad, ld.ctypes.data,
                                                lv.ctypes.data, n.value, ctypes.byref(n)))
        return ld, lv

    def block_tables(self, seqs: Sequence[int], width: int, pad: int) -> np.ndarray:
        s = np.ascontiguousarray(np.asarray(seqs, dtype=np.int32))
        out = np.empty((len(s), width), dtype=np.int32)
        _check(self._lib.pkv_bm_block_tables(self._h, s.ctypes.data, len(s), width, pad, out.ctypes.data))
        return out

    def refcount(self, block: int) -> int:
        return int(self._lib.pkv_bm_refcount(self._h, block))

    def num_free(self) -> int:
        return int(self._lib.pkv_bm_num_free(self._h))
