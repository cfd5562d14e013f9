"""Seeded synthetic inputs for the paged KV-cache decode path.

This package draws context lengths, free-list orders and N(0,1) values, and lists
the block-manager operations (prefill, fork, decode steps) that a workload
performs; prefill workloads list each sequence's context and new-chunk lengths.  It holds none of the method's arithmetic: no slot resolution, no
attention, no copy-on-write decision.  The oracle side and the HIP side of every
test and of the benchmark consume the same arrays from here.
"""
from .workloads import (  # noqa: F401
    DTYPES, NAN_BITS, Workload, normal_bits, skewed_lengths,
    tiny_fp32, mha_bf16, gqa_bf16, cow_fp16, long_bf16, by_name, WORKLOADS,
    PrefillWorkload, prefill_workload, prefill_bf16, chunked_bf16, PREFILL_WORKLOADS,
    SwapWorkload, swap_bf16, SWAP_WORKLOADS, PrefixWorkload, prefix_bf16, PREFIX_WORKLOADS,
    restrict, LengthClassWorkload, lenclass_bf16, LENCLASS_WORKLOADS,
)
