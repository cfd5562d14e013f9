// Internal declarations shared by the host-side translation units of libpkv.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "pkv.h"

namespace pkv {

// Records `msg` as the calling thread's last error and returns `status`.
int32_t set_error(int32_t status, const char* msg);

// Element bytes of a pkv_dtype, 0 if unknown.
inline int elem_bytes(int32_t dtype) {
  switch (dtype) {
    case PKV_F32: return 4;
    case PKV_F16: return 2;
    case PKV_BF16: return 2;
    default: return 0;
  }
}

// Partial-result slots per sequence: partitions of PKV_PARTITION_TOKENS_MIN tokens (the
// smallest size a launch can use) for max_blocks_per_seq blocks, plus one: a sequence
// whose leading blocks are read with other sequences' (a shared prefix) is split at the
// end of that prefix, which can cost one more partition.
inline int64_t max_partitions(int64_t max_blocks_per_seq, int64_t block_size) {
  return (max_blocks_per_seq * block_size + PKV_PARTITION_TOKENS_MIN - 1) / PKV_PARTITION_TOKENS_MIN + 1;
}

// Items per sequence the plan can list when its partitions hold at least
// PKV_PARTITION_TOKENS tokens: a sequence's own partitions plus one for a split at the
// end of a shared prefix; a fused group of c members lists ceil(c / cm) column sets
// (cm >= 2) of at most min(4, max_partitions) parts, which stays within c times this
// count.  The partition kernels' grid holds this many items per sequence then, half of
// what 512-token partitions need.
inline int64_t grid_partitions(int64_t max_blocks_per_seq, int64_t block_size) {
  return (max_blocks_per_seq * block_size + PKV_PARTITION_TOKENS - 1) / PKV_PARTITION_TOKENS + 1;
}

// Kernel launchers (defined in the .hip files).  They assume validated arguments
// and return a hipError_t value as int.
int launch_kv_write(const pkv_pool_desc& pool, void* k_pool, void* v_pool, const void* k_new,
                    const void* v_new, const int64_t* slots, int32_t num_tokens, void* stream);
int launch_copy_blocks(const pkv_pool_desc& pool, void* k_pool, void* v_pool, const int64_t* pairs,
                       int32_t num_pairs, void* stream);
// Whole-block copy from one pool pair to another of the same tile layout.
int launch_pool_copy(const pkv_pool_desc& pool, const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                     const int64_t* pairs, int32_t num_pairs, void* stream);

// Streaming-read probe (stream_read.hip).
int launch_stream_read(const void* src, size_t bytes, int32_t workgroups, int32_t unroll, void* sink, void* stream);

struct AttnArgs {
  const void* k_pool;
  const void* v_pool;
  void* out;
  const void* q;
  const void* block_tables;  // int32, or uint16 when table_bytes == 2; two-level: the leaves
  const int32_t* table_dir = nullptr;  // two-level tables: leaf directory [N][W / leaf entries], else null
  const int32_t* context_lens;
  float* ws_o;   // [num_seqs][num_q_heads][max_partitions][head_dim]
  float* ws_ml;  // [num_seqs][num_q_heads][max_partitions][2]: running max (log2 units), sum
  int* tasks;    // [num_seqs * max_partitions] x 4 ints: the plan's work items, longest first
  int* counters; // [64]: counters[0] = number of items
  int* done;     // [num_seqs * num_q_heads]: finished partitions per (sequence, head group)
  int* seq_np;   // [num_seqs]: partial results of each sequence's rows
  int* seq_grp;  // [num_seqs] x 4 ints: the plan's shared-prefix group of each sequence
  int* members;  // [num_seqs]: sequences of each shared-prefix group, group by group
  int* member_own;  // [num_seqs]: beside members, each member's own tokens
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, dtype;
  int32_t max_blocks_per_seq, max_parts;
  int32_t grid_parts = 0;  // items per sequence in the partition grid (0: max_parts)
  int32_t table_bytes;  // 4 (int32 entries) or 2 (uint16 entries)
  float scale;
  int32_t slots = 768;     // resident partition workgroups on the device (plan's size choice)
  int32_t force_log2 = 0;  // 0, or the log2 of a partition size fixed by the caller
};

// Decode partition sizes (log2 of tokens): the plan pass chooses between kLgPartMin and
// kLgPartMax; kLgPartFloor is only used when fixed by the caller, and sizes the workspace.
constexpr int kLgPartFloor = 9;  // PKV_PARTITION_TOKENS_MIN
constexpr int kLgPartMin = 10;   // PKV_PARTITION_TOKENS
constexpr int kLgPartMax = 11;   // PKV_PARTITION_TOKENS_MAX
static_assert((1 << kLgPartFloor) == PKV_PARTITION_TOKENS_MIN && (1 << kLgPartMin) == PKV_PARTITION_TOKENS &&
                  (1 << kLgPartMax) == PKV_PARTITION_TOKENS_MAX,
              "partition sizes");
constexpr int kSlotsPerCU = 3;  // partition workgroups resident per compute unit

// The plan's partition size for a batch of `tokens` context tokens in total, the longest
// `lmax`, with `hy` workgroups per (sequence, partition) item: the larger size once the
// batch's token work per resident workgroup slot reaches two thirds of its longest item
// (capped at the larger size), or the whole longest item at head size 64 with 16-token
// blocks, else the smaller one.  Measured on MI355X: at head size 128, batches below
// that ratio (GQA batches of 32 to 96 sequences) ran 1-19% faster with the smaller
// size, batches at or above it (GQA batches of 112 to 256 sequences, a 64-sequence MHA
// batch, 256 forked samples, one or eight 128K-token sequences) up to 5% faster with
// the larger one; block 32 at head size 64 or 128 changed over at the same ratio.  At
// head size 64 with 16-token blocks the GQA batches changed over later: 112 and 128
// sequences (ratios 1.05 and 1.2) 2-5% faster with the smaller size, 160 and 192 (1.6
// and 2.0) 0.5-1.2% faster with the larger one; MHA batches there ran alike with either.
__host__ __device__ inline int choose_partition_log2(unsigned long long tokens, int lmax, int hy, int head_dim,
                                                     int block_size, int slots, int force_log2) {
  if (force_log2) return force_log2;
  if (lmax <= (1 << kLgPartMin)) return kLgPartMin;
  const unsigned long long longest = lmax < (1 << kLgPartMax) ? lmax : (1 << kLgPartMax);
  const unsigned long long need = head_dim <= 64 && block_size == 16 ? 3ull : 2ull;
  return 3ull * tokens * static_cast<unsigned long long>(hy) >= need * longest * static_cast<unsigned long long>(slots)
             ? kLgPartMax
             : kLgPartMin;
}

// Resident partition workgroups on the current device (cached per device).
int32_t resident_slots();
// The partition size fixed by pkv_set_decode_partition_tokens (log2), or 0.
int32_t forced_partition_log2();
int32_t set_forced_partition_log2(int32_t log2_tokens);

// Byte offsets of the workspace regions (each 256-byte aligned) and the total size.
struct WorkspaceLayout {
  size_t o, ml, tasks, done, seq_np, seq_grp, members, member_own, counters, total;
};
inline WorkspaceLayout workspace_layout(int64_t n, int64_t hq, int64_t d, int64_t parts) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  WorkspaceLayout w;
  w.o = 0;
  w.ml = al(static_cast<size_t>(n * hq * parts * d) * sizeof(float));
  w.tasks = w.ml + al(static_cast<size_t>(n * hq * parts * 2) * sizeof(float));
  w.done = w.tasks + al(static_cast<size_t>(n * parts) * 4 * sizeof(int32_t));
  w.seq_np = w.done + al(static_cast<size_t>(n * hq) * sizeof(int32_t));
  w.seq_grp = w.seq_np + al(static_cast<size_t>(n) * sizeof(int32_t));
  w.members = w.seq_grp + al(static_cast<size_t>(n) * 4 * sizeof(int32_t));
  w.member_own = w.members + al(static_cast<size_t>(n) * sizeof(int32_t));
  w.counters = w.member_own + al(static_cast<size_t>(n) * sizeof(int32_t));
  w.total = w.counters + 256;
  return w;
}

// Returns -1 when no kernel exists for the shape/dtype/group size, else a hipError_t.
int launch_attn_plan(const AttnArgs& a, void* stream);
// The KV write of num_tokens tokens and the plan pass in one launch.
int launch_decode_prepare(const AttnArgs& a, const pkv_pool_desc& pool, void* k_pool, void* v_pool,
                          const void* k_new, const void* v_new, const int64_t* slots, int32_t num_tokens,
                          void* stream);
int launch_attn_partitions(const AttnArgs& a, void* stream);
// Whether a partition kernel exists for this configuration.
bool attn_supported(int32_t dtype, int32_t head_dim, int32_t block_size, int32_t group);

struct PrefillArgs {
  const void* k_pool;
  const void* v_pool;
  void* out;
  const void* q;
  const void* block_tables;  // int32, or uint16 when table_bytes == 2; two-level: the leaves
  const int32_t* table_dir = nullptr;  // two-level tables: leaf directory [N][W / leaf entries], else null
  const int32_t* context_lens;
  const int32_t* query_start;  // [num_seqs + 1]
  void* workspace;             // prefill_workspace_bytes(...) bytes, 256-byte aligned
  int32_t num_seqs, num_tokens, max_query_len, num_q_heads, num_kv_heads, head_dim, block_size, dtype;
  int32_t max_blocks_per_seq;
  int32_t table_bytes;
  float scale;
};
// Prefill workspace: a 256-byte counter block, then the (sequence, tile) task list.
constexpr size_t kPrefillCounterBytes = 256;
// Upper bound on the (sequence, tile) tasks of a batch with tiles of tile_rows rows.
int64_t prefill_task_bound(int64_t num_tokens, int64_t num_seqs, int64_t group, int64_t tile_rows);
// Workspace bytes a prefill launch needs (for the smallest tile).
size_t prefill_workspace_bytes(int64_t num_tokens, int64_t num_seqs, int64_t group);
// Whether a prefill kernel exists for this configuration.
bool prefill_supported(int32_t dtype, int32_t head_dim, int32_t block_size);
int launch_prefill(const PrefillArgs& a, void* stream);

}  // namespace pkv
