/*
 * pkv.h -- paged KV cache on AMD Instinct MI355X (gfx950): C ABI (decode attention,
 * KV write, copy-on-write, prefill / chunked prefill, swap, prefix caching).
 *
 * The method (pages: agentalpha.top "Q32：vLLM PagedAttention 原理", data.6616ai.com
 * "vLLM" article, ohmygp.com "batch-008-day-02-interview-1"): the KV cache is cut
 * into fixed-size physical blocks (16 tokens by default) that may sit anywhere in a
 * pool; each sequence's block table maps its logical blocks to physical ones; a new
 * token takes one slot and opens a new block only when the current one is full;
 * sequences sharing a prefix share refcounted blocks, and a shared block is copied
 * only when a sharer writes into it; attention reads K/V by block index.
 *
 * Conventions for every call below.
 *  - Device pointers are caller-owned device memory (e.g. torch tensors); the
 *    library never allocates or frees on these paths and keeps no pointer after the
 *    call returns.  Host pointers are marked "host".
 *  - Kernels are enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and run asynchronously; a PKV_OK return means the launch was accepted.
 *  - A call returns a pkv_status.  On failure nothing is enqueued and
 *    pkv_last_error() returns a message for the calling thread.
 *  - Preconditions marked "device" are not checked on the host (that would need a
 *    device->host sync); violating them is undefined behaviour.  A debug build of
 *    the library (PKV_DEBUG=1, libpkv_debug.so) checks them: each call waits for
 *    `stream`, copies the slots, block tables, context lengths, copy pairs or chunk
 *    offsets it is about to use to the host, and returns INVALID_ARG on a violation
 *    before enqueuing anything (so every debug call is synchronous).
 *
 * KV pool layout (the pages do not fix one).  Let X = 16 / element_bytes (8 for
 * bf16/fp16, 4 for fp32), H = num_kv_heads, D = head_dim, B = block_size.
 *  - K pool: [num_blocks][H][D / X][B][X]: element (block, head, offset, d) at
 *    ((((block * H + head) * (D / X) + d / X) * B + offset) * X + d % X).
 *  - V pool: [num_blocks][H][D][B]: element (block, head, offset, d) at
 *    (((block * H + head) * D + d) * B + offset).
 *  One (block, head) tile of K or V is B * D * element_bytes contiguous bytes.
 *  A slot is physical_block * B + offset.
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1,   /* null pointer, bad size, misalignment, unknown sequence */
  PKV_ERR_UNSUPPORTED = 2,   /* a valid shape or dtype this build has no kernel for */
  PKV_ERR_WORKSPACE = 3,     /* workspace smaller than the required size */
  PKV_ERR_LAUNCH = 4,        /* the HIP runtime rejected a launch */
  PKV_ERR_OUT_OF_BLOCKS = 5  /* block manager: no free block left */
} pkv_status;

typedef enum { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2 } pkv_dtype;

/* Shape and element type of a K/V pool pair.  Supported: head_dim in {64, 128},
 * block_size in {16, 32}, any num_kv_heads >= 1, num_blocks >= 1. */
typedef struct {
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype; /* pkv_dtype */
} pkv_pool_desc;

/* Library version string and status names.  Never NULL. */
const char* pkv_version(void);
const char* pkv_status_string(int32_t status);
/* Message of the calling thread's most recent failure ("" if none). */
const char* pkv_last_error(void);

/* Bytes of one pool (K or V) for `pool`; 0 if the descriptor is invalid. */
size_t pkv_pool_bytes(const pkv_pool_desc* pool);

/*
 * KV write: store each new token's K and V in its slot.
 * Pages: agentalpha.top Q32 answer part 2 (a new token lands in the current block
 * or opens a new one; nothing stored moves); ohmygp.com "破局思路" (one slot per
 * decoded token; a new block only when the current one is full).
 *   k_new, v_new  device, [num_tokens][H][D] contiguous, pool dtype, 16-byte aligned.
 *   slot_mapping  device int64 [num_tokens]; token t goes to block slot/B, offset
 *                 slot%B; slot < 0 skips the token (padding).
 *   k_pool, v_pool device, layout above, 16-byte aligned; only the written slots change.
 * Device preconditions: every slot < num_blocks * B; non-negative slots distinct.
 * num_tokens == 0 enqueues nothing.  Errors: INVALID_ARG, UNSUPPORTED, LAUNCH.
 */
int32_t pkv_paged_kv_write(const pkv_pool_desc* pool, void* k_pool, void* v_pool,
                           const void* k_new, const void* v_new,
                           const int64_t* slot_mapping, int32_t num_tokens, void* stream);

/*
 * Copy-on-write block copy: for each pair (src, dst), block dst of the K pool and of
 * the V pool (all heads, all slots) becomes a copy of block src.
 * Pages: agentalpha.top Q32 answer part 3 (copy a shared block only when a sharer
 * writes into it); data.6616ai.com "PagedAttention：把虚拟内存搬进 KV Cache" (refcounted
 * shared prefix, copied only at divergence); ohmygp.com "破局思路" (写时共享).
 *   src_dst_pairs device int64 [num_pairs][2].
 * Device preconditions: ids < num_blocks; destinations distinct; no destination is
 * also a source (a source may repeat).  num_pairs == 0 enqueues nothing.
 * Errors: INVALID_ARG, UNSUPPORTED, LAUNCH.
 */
int32_t pkv_copy_blocks(const pkv_pool_desc* pool, void* k_pool, void* v_pool,
                        const int64_t* src_dst_pairs, int32_t num_pairs, void* stream);

/*
 * Swap copy: for each pair (s, d), block d of the destination pools (K and V, every
 * head and slot) becomes a copy of block s of the source pools.  Pages:
 * data.6616ai.com "PagedAttention 之外" (preemption swaps a request's KV to CPU memory)
 * and "可能的追问" (swapped out when the device is full, resumed later).  The two
 * pools share the tile layout `pool` describes (its num_blocks is not used); one of
 * them is typically pinned host memory (hipHostMalloc / torch pin_memory), which
 * the copy kernel reads or writes directly over the host link.
 *   src_k, src_v, dst_k, dst_v  device or pinned host, 16-byte aligned.
 *   src_dst_pairs  device or pinned host int64 [num_pairs][2].
 * Device preconditions: block ids inside their pools; destinations distinct and the
 * source and destination ranges do not overlap.  num_pairs == 0 enqueues nothing.
 * Errors: INVALID_ARG, UNSUPPORTED, LAUNCH.
 */
int32_t pkv_swap_blocks(const pkv_pool_desc* pool, const void* src_k, const void* src_v, void* dst_k,
                        void* dst_v, const int64_t* src_dst_pairs, int32_t num_pairs, void* stream);

/* Context tokens per split-context partition of the attention pass: the plan pass picks
 * PKV_PARTITION_TOKENS or PKV_PARTITION_TOKENS_MAX for each launch (see
 * pkv_decode_partition_tokens); PKV_PARTITION_TOKENS_MIN is used only when fixed with
 * pkv_set_decode_partition_tokens.  Workspaces are sized for the smallest. */
#define PKV_PARTITION_TOKENS_MIN 512
#define PKV_PARTITION_TOKENS 1024
#define PKV_PARTITION_TOKENS_MAX 2048
/* Context tokens whose block ids one leaf of a two-level block table holds. */
#define PKV_LEAF_TOKENS 512

/* Workspace bytes pkv_paged_attention_decode needs for these sizes (0 on bad input):
 * fp32 partial results of every (sequence, query head, partition), the task list and
 * per-row counters. */
size_t pkv_paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                           int32_t max_blocks_per_seq, int32_t block_size);

/*
 * Decode attention over the paged pool, one query token per sequence.
 * Pages: data.6616ai.com "PagedAttention：把虚拟内存搬进 KV Cache" (the attention
 * kernel reads K/V by block index: logically contiguous, physically scattered);
 * agentalpha.top Q32 follow-up 3 (blockwise, FlashAttention-style loading adapted to
 * non-contiguous blocks by pointer indexing).  For each sequence b and query head h,
 * with G = num_q_heads / H and kv head g = h / G:
 *     s_j = scale * dot(q[b][h], K[b, j, g])   for 0 <= j < context_lens[b]
 *     out[b][h] = sum_j softmax(s)_j * V[b, j, g]
 * where token j of sequence b sits in block block_tables[b][j / B] at offset j % B.
 * Long contexts are split into partitions of PKV_PARTITION_TOKENS or
 * PKV_PARTITION_TOKENS_MAX tokens (chosen per call from the context lengths, as
 * pkv_decode_partition_tokens states) whose partial results are merged with
 * log-sum-exp weights (in `workspace`).  Context lengths above
 * max_blocks_per_seq * B break the contract; they are clamped to it (no access goes
 * past the table row).
 *   q, out        device [num_seqs][num_q_heads][D], pool dtype, contiguous, 16-byte aligned.
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq]; entries at index
 *                 >= ceil(context_lens[b] / B) are never followed (the plan pass
 *                 reads entry 0 of every row, an empty context's included, and compares
 *                 the leading entries of rows whose first entries are equal, up to the
 *                 shorter context's full blocks, without following them).
 *   context_lens  device int32 [num_seqs]; 0 gives a zero output row.
 *   workspace     device, >= pkv_paged_attention_workspace_bytes(...), 256-byte aligned;
 *                 contents on entry do not matter.
 * num_q_heads must be a multiple of H.  Accumulation is fp32; the output is rounded
 * to the pool dtype.  The reduction order depends only on logical token positions,
 * so results do not depend on the physical placement of blocks.
 * Device preconditions: context_lens[b] <= max_blocks_per_seq * B; table entries that
 * are read are < num_blocks.  num_seqs == 0 enqueues nothing.
 * Errors: INVALID_ARG, UNSUPPORTED (dtype/head_dim/block_size/group size), WORKSPACE, LAUNCH.
 */
int32_t pkv_paged_attention_decode(const pkv_pool_desc* pool, const void* k_pool, const void* v_pool,
                                   void* out, const void* q, int32_t num_seqs, int32_t num_q_heads,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens, float scale,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode attention that allocates nothing and takes no workspace: for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops or
 * harnesses that forbid allocation).  Same arguments (minus the workspace), kernels and
 * results as pkv_paged_attention_decode; its workspace is a fixed device array of
 * PKV_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU, held from the first
 * call on that GPU until the process ends.  Nothing in it needs clearing between calls
 * (the plan pass rewrites what the attention pass reads).  Every call on a GPU uses that
 * GPU's one array, so calls that overlap in time on one GPU (on different streams, or
 * from different threads) race and give undefined results; calls ordered on one stream
 * are safe.  Sizes whose workspace (pkv_paged_attention_workspace_bytes) exceeds
 * PKV_NOALLOC_SCRATCH_BYTES are rejected with WORKSPACE before anything is enqueued.
 * Errors: those of pkv_paged_attention_decode; LAUNCH also when the array's device
 * address cannot be looked up.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (128u << 20)
int32_t pkv_paged_attention_decode_noalloc(const pkv_pool_desc* pool, const void* k_pool, const void* v_pool,
                                           void* out, const void* q, int32_t num_seqs, int32_t num_q_heads,
                                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                                           const int32_t* context_lens, float scale, void* stream);

/*
 * Causal attention of chunks of new tokens over the paged pool (prefill and chunked
 * prefill).  Pages: agentalpha.top Q32 follow-up 3 (FlashAttention loads K/V block by
 * block; over paged storage that loading goes through the block table);
 * data.6616ai.com "可能的追问" (FlashAttention fused with paged reads).  Sequence b
 * appends a chunk of C_b = query_start[b+1] - query_start[b] tokens whose K/V are
 * already written to the pool, so its context_lens[b] = L_b counts them.  Query row
 * query_start[b] + t (t < C_b) sits at position p = L_b - C_b + t; for each query head
 * h, with kv head g = h / (num_q_heads / H):
 *     s_j = scale * dot(q[row][h], K[b, j, g])   for 0 <= j <= p
 *     out[row][h] = sum_j softmax(s)_j * V[b, j, g]
 * Decode is the C_b = 1 case.  bf16 and fp16 pools only (fp32: UNSUPPORTED).
 *   q, out        device [num_tokens][num_q_heads][D], pool dtype, contiguous,
 *                 16-byte aligned; sequence b's chunk is rows query_start[b] ..
 *                 query_start[b+1]-1.
 *   query_start   device int32 [num_seqs + 1], non-decreasing, query_start[0] = 0,
 *                 query_start[num_seqs] = num_tokens.
 *   num_tokens, max_query_len  host: the total rows and an upper bound on every C_b
 *                 (it sizes the grid).
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq]; context_lens device
 *                 int32 [num_seqs].
 *   workspace     device, >= pkv_paged_attention_prefill_workspace_bytes(...),
 *                 256-byte aligned; contents on entry do not matter.  It holds the
 *                 (sequence, tile) task list a plan pass builds before the attention
 *                 pass (longest first; no task for rows a chunk does not have).
 * Accumulation is fp32, the output is rounded to the pool dtype, and the reduction
 * order depends only on logical positions.  Nothing is allocated.
 * Device preconditions: C_b <= max_query_len; C_b <= context_lens[b] <=
 * max_blocks_per_seq * B; chunks do not overlap; table entries that are read are
 * < num_blocks.  A sequence whose chunk breaks them (longer than its context, or
 * outside q) gets no output rows written.  num_seqs == 0 or num_tokens == 0 enqueues
 * nothing.  Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, LAUNCH.
 */
int32_t pkv_paged_attention_prefill(const pkv_pool_desc* pool, const void* k_pool, const void* v_pool,
                                    void* out, const void* q, int32_t num_seqs, int32_t num_q_heads,
                                    const int32_t* query_start, int32_t num_tokens, int32_t max_query_len,
                                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                                    const int32_t* context_lens, float scale, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * 16-bit block tables: the same calls with uint16 table entries, for pools of at most
 * 65536 blocks (agentalpha.top Q32 follow-up 1: a block table can use 16-bit indices
 * while there are fewer than 65536 blocks, halving its memory).  Tables are otherwise
 * identical; a pool with more blocks is UNSUPPORTED.  Results are bit-identical to the
 * int32-table calls on the same data.
 */
int32_t pkv_paged_attention_decode_t16(const pkv_pool_desc* pool, const void* k_pool, const void* v_pool, void* out,
                                       const void* q, int32_t num_seqs, int32_t num_q_heads,
                                       const uint16_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, float scale, void* workspace,
                                       size_t workspace_bytes, void* stream);
int32_t pkv_paged_attention_partitions_t16(const pkv_pool_desc* pool, const void* k_pool, const void* v_pool,
                                           void* out, const void* q, int32_t num_seqs, int32_t num_q_heads,
                                           const uint16_t* block_tables, int32_t max_blocks_per_seq,
                                           const int32_t* context_lens, float scale, void* workspace,
                                           size_t workspace_bytes, void* stream);
int32_t pkv_paged_attention_prefill_t16(const pkv_pool_desc* pool, const void* k_pool, const void* v_pool,
                                        void* out, const void* q, int32_t num_seqs, int32_t num_q_heads,
                                        const int32_t* query_start, int32_t num_tokens, int32_t max_query_len,
                                        const uint16_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, float scale, void* workspace,
                                        size_t workspace_bytes, void* stream);

/*
 * Two-level block tables (agentalpha.top Q32 follow-up 1: a hierarchical table, in the
 * manner of multi-level page tables, keeps mostly empty tables small).  A sequence's
 * entries are cut into leaves of E = PKV_LEAF_TOKENS / block_size int32 block ids
 * (512 tokens' entries: 32 at block size 16, 16 at 32):
 *   leaves    device int32 [num_leaves][E];
 *   leaf_dir  device int32 [num_seqs][dir_width]: the leaf that holds entries
 *             j*E .. j*E+E-1 of sequence b is leaf_dir[b][j].
 * Entry j of sequence b is leaves[leaf_dir[b][j / E]][j % E].  Each call equals the
 * flat-table call with max_blocks_per_seq = dir_width * E on the table those lookups
 * give, bit for bit.  Only the directory entries and leaf entries of a sequence's
 * first ceil(L / B) blocks are followed; directory entries followed must lie in
 * 0 .. num_leaves - 1 (a device precondition, checked by the debug library).  A batch
 * whose longest table sets the width of every row stores dir_width int32 per
 * sequence plus the leaves it uses, instead of dir_width * E per sequence.
 * Errors: as the flat calls; INVALID_ARG also when dir_width <= 0, num_leaves < 0,
 * dir_width * E exceeds INT32_MAX, or leaf_dir is null or misaligned.
 */
int32_t pkv_paged_attention_decode_2l(const pkv_pool_desc* pool, const void* k_pool, const void* v_pool, void* out,
                                      const void* q, int32_t num_seqs, int32_t num_q_heads, const int32_t* leaf_dir,
                                      int32_t dir_width, const int32_t* leaves, int32_t num_leaves,
                                      const int32_t* context_lens, float scale, void* workspace,
                                      size_t workspace_bytes, void* stream);
int32_t pkv_paged_attention_partitions_2l(const pkv_pool_desc* pool, const void* k_pool, const void* v_pool,
                                          void* out, const void* q, int32_t num_seqs, int32_t num_q_heads,
                                          const int32_t* leaf_dir, int32_t dir_width, const int32_t* leaves,
                                          int32_t num_leaves, const int32_t* context_lens, float scale,
                                          void* workspace, size_t workspace_bytes, void* stream);
int32_t pkv_paged_attention_prefill_2l(const pkv_pool_desc* pool, const void* k_pool, const void* v_pool,
                                       void* out, const void* q, int32_t num_seqs, int32_t num_q_heads,
                                       const int32_t* query_start, int32_t num_tokens, int32_t max_query_len,
                                       const int32_t* leaf_dir, int32_t dir_width, const int32_t* leaves,
                                       int32_t num_leaves, const int32_t* context_lens, float scale,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes pkv_paged_attention_prefill needs for these sizes (0 on bad input). */
size_t pkv_paged_attention_prefill_workspace_bytes(int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                                   int32_t num_kv_heads);

/*
 * The two passes of pkv_paged_attention_decode, exposed separately (same arguments,
 * same results when called in this order on one stream with the same workspace and
 * context_lens) so that each pass can be timed on its own:
 *  - plan: picks the partition size, lists the work items in the workspace, longest
 *    first, and clears the per-row completion counters.  `tables` (a host struct; NULL
 *    allowed, which skips this) lets it find shared prefixes (agentalpha.top "Q32：
 *    vLLM PagedAttention 原理", standard answer part 3; data.6616ai.com
 *    "PagedAttention：把虚拟内存搬进 KV Cache", copy-on-write sharing): sequences of
 *    256 tokens or more whose rows start with the same blocks, anywhere within windows
 *    of 512 sequences, form a group whose common leading blocks (compared entry by
 *    entry, cut to blocks every member fills) are attended once for the whole group on
 *    16-bit pools with 1 to 8 query heads per kv head, the members' query heads side by
 *    side in one item.  Each column of a result depends only on its own sequence's
 *    tokens and on how its work is split, never on its position in the batch or on the
 *    other members of its group; a grouped call and an ungrouped one (NULL `tables`)
 *    split the work differently and may differ in the last bits;
 *  - partitions: one workgroup per item and kv-head group; writes the final output of
 *    sequences that fit one item and partial results of the others; the workgroup
 *    that completes the last partial of a row merges that row's partials with
 *    log-sum-exp weights.  Its grid holds as many items as the last plan pass this
 *    process launched on the workspace could list (half as many when that plan could
 *    not use 512-token partitions), so the partition size may change between the calls.
 * A partitions pass without a preceding plan pass on that workspace gives undefined
 * output values (but stays within the buffers).  Errors as pkv_paged_attention_decode.
 */
typedef struct {
  const void* entries;      /* flat tables: device rows [num_seqs][max_blocks_per_seq] of
                               entry_bytes each; two-level tables: the device int32 leaves */
  const int32_t* leaf_dir;  /* two-level tables: the device leaf directory
                               [num_seqs][max_blocks_per_seq / (PKV_LEAF_TOKENS / B)]; NULL if flat */
  int32_t entry_bytes;      /* 4 (int32) or 2 (16-bit) for flat tables, 4 for two-level */
  int32_t reserved;         /* 0 */
} pkv_table_ref;
int32_t pkv_paged_attention_plan(const pkv_pool_desc* pool, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 const pkv_table_ref* tables, void* workspace, size_t workspace_bytes,
                                 void* stream);
int32_t pkv_paged_attention_partitions(const pkv_pool_desc* pool, const void* k_pool, const void* v_pool,
                                       void* out, const void* q, int32_t num_seqs, int32_t num_q_heads,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, float scale,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode-step preparation: the KV write of the step's new tokens (as pkv_paged_kv_write)
 * and the plan pass of the step's attention (as pkv_paged_attention_plan) in a single
 * launch.  A decode step is then [pkv_copy_blocks if the step has copy pairs],
 * pkv_decode_prepare, pkv_paged_attention_partitions, with the same results as
 * pkv_copy_blocks + pkv_paged_kv_write + pkv_paged_attention_decode.
 * Arguments and errors are those of the two calls it replaces; num_tokens == 0 only
 * plans, num_seqs == 0 only writes.  `tables` is as for pkv_paged_attention_plan.
 */
int32_t pkv_decode_prepare(const pkv_pool_desc* pool, void* k_pool, void* v_pool,
                           const void* k_new, const void* v_new, const int64_t* slot_mapping,
                           int32_t num_tokens, int32_t num_seqs, int32_t num_q_heads,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           const pkv_table_ref* tables, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * The partition size (in tokens) the plan pass picks for a decode call with these
 * context lengths (host copy) on the current device.  Fewer, longer partitions save
 * each workgroup's fixed start and end (table entries, queries and first K/V unit;
 * combine, partial stores, merge), but a batch too small to keep the chip busy ends
 * when its longest items do.  The plan takes PKV_PARTITION_TOKENS_MAX when some
 * context exceeds PKV_PARTITION_TOKENS and
 *     3 * sum_b(context_lens[b]) * workgroups_per_item >= k * min(max_b context_lens[b], PKV_PARTITION_TOKENS_MAX) * slots
 * with k = 3 for pools of head_dim 64 and block_size 16 (the token work per resident
 * workgroup slot reaches the longest item) and k = 2 otherwise (two thirds of it),
 * workgroups_per_item = H * ceil(G / 16) and slots = 3 resident workgroups per compute
 * unit (768 on MI355X); else PKV_PARTITION_TOKENS.  A value set with
 * pkv_set_decode_partition_tokens takes precedence.  The pool descriptor gives H,
 * head_dim and block_size (num_blocks and dtype are checked, not used).  Host-only and
 * synchronous; no device is needed (without one, 256 compute units are assumed).
 * Errors: INVALID_ARG (bad pool descriptor, null pointers, num_seqs < 0, num_q_heads
 * not a positive multiple of H), UNSUPPORTED (head_dim or block_size).
 */
int32_t pkv_decode_partition_tokens(const pkv_pool_desc* pool, const int32_t* context_lens_host, int32_t num_seqs,
                                    int32_t num_q_heads, int32_t* tokens);
/*
 * Fixes the decode partition size of every later plan pass in the process:
 * PKV_PARTITION_TOKENS_MIN, PKV_PARTITION_TOKENS or PKV_PARTITION_TOKENS_MAX, or 0 for
 * the per-call choice above (the default).  For tuning and tests; results are the same
 * either way up to fp32 rounding of the merge.  Errors: INVALID_ARG (any other value).
 */
int32_t pkv_set_decode_partition_tokens(int32_t tokens);

/*
 * Host-side block manager: block tables, on-demand allocation, fork and
 * copy-on-write decisions.  Pages: agentalpha.top Q32 answer parts 2-3;
 * data.6616ai.com "PagedAttention：把虚拟内存搬进 KV Cache"; ohmygp.com "破局思路".
 * Policy:
 *  - the free list starts as `free_order` (host, a permutation of 0..num_blocks-1)
 *    and hands out blocks from its front; freed blocks go to its back;
 *  - add_seq(seq, n) gives a new sequence ceil(n / B) blocks;
 *  - append_slot at position pos: pos % B == 0 opens a fresh block; otherwise, if the
 *    tail block is shared (refcount > 1), the writer takes a fresh block, reports
 *    (old tail, fresh) as a copy pair and drops one reference to the old tail;
 *    the slot is table[pos / B] * B + pos % B;
 *  - fork(parent, child): the child shares all of the parent's blocks (+1 reference each);
 *  - free_seq drops one reference per block; blocks reaching zero become free.
 * Sequence ids are any non-negative int32.  A pkv_bm is not thread-safe.
 * Every call is host-only and synchronous.  Errors: INVALID_ARG (unknown or duplicate
 * sequence, bad sizes), OUT_OF_BLOCKS (the state is unchanged when it is returned).
 */
typedef struct pkv_bm pkv_bm;

int32_t pkv_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order, pkv_bm** out);
void pkv_bm_destroy(pkv_bm* bm);
int32_t pkv_bm_add_seq(pkv_bm* bm, int32_t seq, int32_t num_tokens);
int32_t pkv_bm_fork(pkv_bm* bm, int32_t parent, int32_t child);
/* Reserve the next token's slot; cow_src and cow_dst receive -1 when no copy is needed. */
int32_t pkv_bm_append_slot(pkv_bm* bm, int32_t seq, int64_t* slot, int32_t* cow_src, int32_t* cow_dst);
/* One decode step over `seqs` (host, n entries, visited in order): slots_out (host, n)
 * receives each slot, pairs_out (host, [n][2] capacity) the copy pairs in order,
 * *num_pairs their count.  On OUT_OF_BLOCKS the sequences before the failing one
 * have been appended. */
int32_t pkv_bm_step(pkv_bm* bm, const int32_t* seqs, int32_t n, int64_t* slots_out,
                    int64_t* pairs_out, int32_t* num_pairs);
int32_t pkv_bm_free_seq(pkv_bm* bm, int32_t seq);
int32_t pkv_bm_seq_len(const pkv_bm* bm, int32_t seq, int32_t* len);
/* Slots of positions pos0 .. pos0+count-1 of `seq` (host out, count entries). */
int32_t pkv_bm_slots(const pkv_bm* bm, int32_t seq, int32_t pos0, int32_t count, int64_t* out);
/* The block table of `seq` into out (host, cap entries); *n = its length. */
int32_t pkv_bm_block_table(const pkv_bm* bm, int32_t seq, int32_t* out, int32_t cap, int32_t* n);
/* Tables of `seqs` (host, n) as a host int32 [n][width] matrix padded with `pad`. */
int32_t pkv_bm_block_tables(const pkv_bm* bm, const int32_t* seqs, int32_t n, int32_t width,
                            int32_t pad, int32_t* out);
/* The same as a host uint16 matrix (INVALID_ARG if a block id or `pad` exceeds 65535). */
int32_t pkv_bm_block_tables16(const pkv_bm* bm, const int32_t* seqs, int32_t n, int32_t width,
                              int32_t pad, uint16_t* out);
/* Two-level tables of `seqs` (host, n) for the _2l calls: each table cut into leaves of
 * PKV_LEAF_TOKENS / block_size entries, numbered by sequence (in `seqs` order) and
 * then position; dir_out (host int32 [n][dir_width]) receives the leaf of every run,
 * leaves_out (host int32 [leaf_cap][entries]) the leaves, the last leaf of a sequence
 * padded with `pad`.  One more leaf, last, holds only `pad` and is named by the
 * directory entries past a sequence's leaves.  *num_leaves = the leaves written
 * (sum over seqs of ceil(blocks / entries), plus 1 when n > 0); with leaves_out null
 * only *num_leaves is set.  INVALID_ARG when a table needs more than dir_width leaves
 * or the leaves exceed leaf_cap. */
int32_t pkv_bm_block_tables_2l(const pkv_bm* bm, const int32_t* seqs, int32_t n, int32_t dir_width, int32_t pad,
                               int32_t* dir_out, int32_t* leaves_out, int32_t leaf_cap, int32_t* num_leaves);
/* Swap-out / swap-in bookkeeping (data.6616ai.com "PagedAttention 之外", scheduler and
 * preemption; "可能的追问": under memory pressure a request's KV goes to CPU memory and
 * comes back later).  Moves `seqs` (host, n, in order) from manager `src` to `dst`
 * (for example a device pool's manager and a pinned host pool's): each moved
 * sequence gets fresh blocks of `dst`, taken from its free list in the order the
 * source blocks are first met; a block shared by several moved sequences is copied
 * once and stays shared; the source blocks are then released as by free_seq.
 * pairs_out (host, [cap][2]) receives the (source block, destination block) pairs to
 * copy with pkv_swap_blocks, *num_pairs their count.  All or nothing: unknown,
 * duplicate or already-present sequences and a too-small cap are INVALID_ARG, too few
 * free destination blocks OUT_OF_BLOCKS, and neither changes any state. */
int32_t pkv_bm_move_seqs(pkv_bm* src, pkv_bm* dst, const int32_t* seqs, int32_t n, int64_t* pairs_out,
                         int32_t cap, int32_t* num_pairs);
/* Reference count of `block` (-1 if out of range); blocks an allocation may take
 * (free, plus released cached blocks when prefix caching is on). */
int32_t pkv_bm_refcount(const pkv_bm* bm, int32_t block);
int32_t pkv_bm_num_free(const pkv_bm* bm);

/*
 * Prefix caching.  Pages: data.6616ai.com "PagedAttention 之外" (the KV blocks of a
 * prefix shared across requests, such as a system prompt, can be cached and reused,
 * saving prefill compute in multi-turn and few-shot use).  Policy:
 *  - every full block of a prompt is keyed by FNV-1a 64 over the key of the block
 *    before it (0 for the first; 8 bytes little-endian) followed by its token ids
 *    (4 bytes each, little-endian); a lookup also compares the stored parent key and
 *    tokens;
 *  - add_seq_tokens reuses the cached blocks of the prompt's longest cached prefix of
 *    full blocks, never the block holding its last token, and returns in
 *    *cached_tokens how many leading tokens already have their K/V in the pool (the
 *    caller writes and computes only the rest); its other full blocks are registered
 *    as they are allocated (unless the key is taken); partial tails and blocks filled
 *    by decoding are not cached;
 *  - a cached block whose count drops to zero stays addressable in an evictable list
 *    in release order; allocation takes the free list first, then evicts the least
 *    recently released cached block.
 * set_prefix_cache switches it on or off for a manager without sequences or cached
 * blocks (INVALID_ARG otherwise).  Without it, add_seq_tokens is add_seq with
 * *cached_tokens = 0.  OUT_OF_BLOCKS leaves the state unchanged.
 */
int32_t pkv_bm_set_prefix_cache(pkv_bm* bm, int32_t enable);
int32_t pkv_bm_add_seq_tokens(pkv_bm* bm, int32_t seq, const int32_t* tokens, int32_t n, int32_t* cached_tokens);
/* Number of blocks registered in the prefix cache (in use or evictable). */
int32_t pkv_bm_num_cached(const pkv_bm* bm);

/*
 * Diagnostics: the device's streaming-read rate, the ceiling the bandwidth-bound
 * attention kernels are measured against (data.6616ai.com "PagedAttention 之外" and
 * ohmygp.com "先搞清敌人": decode is limited by memory bandwidth, not compute).  Reads
 * `bytes` bytes from `src` once, with 16-byte non-temporal loads in a grid-stride loop
 * over `workgroups` workgroups of 256 threads, `unroll` loads in flight per thread, and
 * stores one xor of what each wave read into `sink`.
 *   src   device, 16-byte aligned, `bytes` a positive multiple of 16.
 *   sink  device uint32 [workgroups * 4].
 * Errors: INVALID_ARG (null or misaligned pointers, bad sizes, unroll not 1, 2, 4 or 8),
 * LAUNCH.
 */
int32_t pkv_stream_read(const void* src, size_t bytes, int32_t workgroups, int32_t unroll, void* sink,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
