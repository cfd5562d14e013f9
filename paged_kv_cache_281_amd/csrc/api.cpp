// C ABI of libpkv: argument validation, workspace sizing and dispatch to the
// gfx950 kernels.  No entry point allocates device memory or synchronises, except in
// a debug build (PKV_DEBUG=1), whose entry points wait for the stream to check the
// device arrays they are given.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "pkv.h"
#include "pkv_internal.h"

namespace pkv {
namespace {
thread_local std::string g_last_error;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int32_t launch_status(int rc, const char* what) {
  if (rc == 0) return PKV_OK;
  if (rc < 0) return set_error(PKV_ERR_UNSUPPORTED, what);
  char buf[256];
  std::snprintf(buf, sizeof(buf), "%s: launch failed: %s", what, hipGetErrorString(static_cast<hipError_t>(rc)));
  return set_error(PKV_ERR_LAUNCH, buf);
}

int32_t check_pool(const pkv_pool_desc* pool, const char* who) {
  char buf[256];
  if (!pool) {
    std::snprintf(buf, sizeof(buf), "%s: null pool descriptor", who);
    return set_error(PKV_ERR_INVALID_ARG, buf);
  }
  if (pool->num_blocks <= 0 || pool->block_size <= 0 || pool->num_kv_heads <= 0 || pool->head_dim <= 0) {
    std::snprintf(buf, sizeof(buf), "%s: pool sizes must be positive", who);
    return set_error(PKV_ERR_INVALID_ARG, buf);
  }
  if (elem_bytes(pool->dtype) == 0) {
    std::snprintf(buf, sizeof(buf), "%s: unknown dtype %d", who, pool->dtype);
    return set_error(PKV_ERR_INVALID_ARG, buf);
  }
  if (pool->head_dim != 64 && pool->head_dim != 128) {
    std::snprintf(buf, sizeof(buf), "%s: head_dim %d unsupported (64 or 128)", who, pool->head_dim);
    return set_error(PKV_ERR_UNSUPPORTED, buf);
  }
  if (pool->block_size != 16 && pool->block_size != 32) {
    std::snprintf(buf, sizeof(buf), "%s: block_size %d unsupported (16 or 32)", who, pool->block_size);
    return set_error(PKV_ERR_UNSUPPORTED, buf);
  }
  return PKV_OK;
}

struct AttnCheck {
  int32_t status;
  AttnArgs args;
};

size_t workspace_bytes_for(int64_t n, int64_t hq, int64_t d, int64_t parts) {
  // partial outputs, (max, sum) pairs, the task list and counters
  return workspace_layout(n, hq, d, parts).total;
}

AttnCheck check_attention(const char* who, const pkv_pool_desc* pool, const void* k_pool, const void* v_pool,
                          void* out, const void* q, int32_t num_seqs, int32_t num_q_heads,
                          const void* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                          float scale, const void* workspace, size_t workspace_bytes, bool need_pools,
                          bool need_out = true, int table_bytes = 4) {
  AttnCheck c{PKV_OK, {}};
  char buf[256];
  if ((c.status = check_pool(pool, who)) != PKV_OK) return c;
  if (num_seqs < 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0) {
    std::snprintf(buf, sizeof(buf), "%s: num_seqs >= 0, num_q_heads > 0, max_blocks_per_seq > 0 required", who);
    c.status = set_error(PKV_ERR_INVALID_ARG, buf);
    return c;
  }
  if (num_q_heads % pool->num_kv_heads != 0) {
    std::snprintf(buf, sizeof(buf), "%s: num_q_heads %d is not a multiple of num_kv_heads %d", who, num_q_heads,
                  pool->num_kv_heads);
    c.status = set_error(PKV_ERR_INVALID_ARG, buf);
    return c;
  }
  const int group = num_q_heads / pool->num_kv_heads;
  if (!attn_supported(pool->dtype, pool->head_dim, pool->block_size, group)) {
    std::snprintf(buf, sizeof(buf), "%s: no kernel for dtype %d, head_dim %d, block_size %d, group %d", who,
                  pool->dtype, pool->head_dim, pool->block_size, group);
    c.status = set_error(PKV_ERR_UNSUPPORTED, buf);
    return c;
  }
  const int64_t parts = max_partitions(max_blocks_per_seq, pool->block_size);
  if (num_seqs > 65535 || parts > 65535 || static_cast<int64_t>(num_seqs) * parts * num_q_heads > (int64_t{1} << 23)) {
    std::snprintf(buf, sizeof(buf), "%s: num_seqs and partitions per sequence must be <= 65535 and "
                  "num_seqs * partitions * num_q_heads <= 2^23", who);
    c.status = set_error(PKV_ERR_UNSUPPORTED, buf);
    return c;
  }
  if (num_seqs > 0) {
    if ((need_pools && (!k_pool || !v_pool || !q || !block_tables)) || (need_out && !out) || !context_lens) {
      std::snprintf(buf, sizeof(buf), "%s: null pointer argument", who);
      c.status = set_error(PKV_ERR_INVALID_ARG, buf);
      return c;
    }
    if ((need_out && !aligned(out, 16)) ||
        (need_pools && (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(q, 16))) ||
        !aligned(block_tables, table_bytes) || !aligned(context_lens, 4)) {
      std::snprintf(buf, sizeof(buf), "%s: misaligned pointer (pools, q, out need 16 bytes)", who);
      c.status = set_error(PKV_ERR_INVALID_ARG, buf);
      return c;
    }
  }
  const size_t need = workspace_bytes_for(num_seqs, num_q_heads, pool->head_dim, parts);
  if (num_seqs > 0 && (workspace_bytes < need || !workspace || !aligned(workspace, 256))) {
    std::snprintf(buf, sizeof(buf), "%s: workspace of %zu bytes (256-byte aligned) needed, got %zu", who, need,
                  workspace_bytes);
    c.status = set_error(PKV_ERR_WORKSPACE, buf);
    return c;
  }
  AttnArgs& a = c.args;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.out = out;
  a.q = q;
  a.block_tables = block_tables;
  a.table_bytes = table_bytes;
  a.context_lens = context_lens;
  const WorkspaceLayout L = workspace_layout(num_seqs, num_q_heads, pool->head_dim, parts);
  char* ws = static_cast<char*>(const_cast<void*>(workspace));
  a.ws_o = reinterpret_cast<float*>(ws + L.o);
  a.ws_ml = reinterpret_cast<float*>(ws + L.ml);
  a.tasks = reinterpret_cast<int*>(ws + L.tasks);
  a.counters = reinterpret_cast<int*>(ws + L.counters);
  a.done = reinterpret_cast<int*>(ws + L.done);
  a.seq_np = reinterpret_cast<int*>(ws + L.seq_np);
  a.seq_grp = reinterpret_cast<int*>(ws + L.seq_grp);
  a.members = reinterpret_cast<int*>(ws + L.members);
  a.member_own = reinterpret_cast<int*>(ws + L.member_own);
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.head_dim = pool->head_dim;
  a.block_size = pool->block_size;
  a.dtype = pool->dtype;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_parts = static_cast<int32_t>(parts);
  a.scale = scale;
  a.slots = resident_slots();
  a.force_log2 = forced_partition_log2();
  return c;
}

// The block tables a plan pass is given (optional): which sequences share a first block.
int32_t apply_table_ref(const char* who, const pkv_pool_desc& pool, const pkv_table_ref* t, int32_t num_seqs,
                        int32_t max_blocks_per_seq, AttnArgs& a) {
  if (!t || num_seqs == 0) return PKV_OK;
  char buf[256];
  const int32_t E = PKV_LEAF_TOKENS / pool.block_size;
  const bool two = t->leaf_dir != nullptr;
  if (!t->entries || (t->entry_bytes != 4 && t->entry_bytes != 2) || (two && t->entry_bytes != 4) ||
      (two && max_blocks_per_seq % E != 0) || t->reserved != 0) {
    std::snprintf(buf, sizeof(buf), "%s: bad table reference (entries, entry_bytes 2 or 4, two-level: 4 and "
                  "max_blocks_per_seq a multiple of %d, reserved 0)", who, E);
    return set_error(PKV_ERR_INVALID_ARG, buf);
  }
  if (!aligned(t->entries, t->entry_bytes) || !aligned(t->leaf_dir, 4)) {
    std::snprintf(buf, sizeof(buf), "%s: misaligned table reference", who);
    return set_error(PKV_ERR_INVALID_ARG, buf);
  }
  if (t->entry_bytes == 2 && pool.num_blocks > 65536) {
    std::snprintf(buf, sizeof(buf), "%s: 16-bit block tables address at most 65536 blocks", who);
    return set_error(PKV_ERR_UNSUPPORTED, buf);
  }
  a.block_tables = t->entries;
  a.table_bytes = t->entry_bytes;
  a.table_dir = t->leaf_dir;
  return PKV_OK;
}

}  // namespace

int32_t set_error(int32_t status, const char* msg) {
  g_last_error = msg ? msg : "";
  return status;
}

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int32_t> g_slots[kMaxDevices];
std::atomic<int32_t> g_force_log2{0};

// The smallest partition (log2 of tokens) that each workspace's last plan pass could
// use, so that a partition pass launched on its own sizes its grid for that plan's item
// list even if the partition size was changed in between.  A workspace that is not on
// record gets the grid of 512-token partitions, which holds any list.
struct PlanFloor {
  const void* ws = nullptr;
  int32_t lg = 0;
};
constexpr int kPlanFloors = 64;
std::mutex g_plan_mu;
PlanFloor g_plan_floor[kPlanFloors];
int g_plan_next = 0;

int32_t plan_floor_log2(int32_t force_log2) { return force_log2 ? force_log2 : kLgPartMin; }

void record_plan(const void* ws, int32_t force_log2) {
  const int32_t lg = plan_floor_log2(force_log2);
  std::lock_guard<std::mutex> lock(g_plan_mu);
  for (PlanFloor& r : g_plan_floor) {
    if (r.ws == ws) {
      r.lg = lg;
      return;
    }
  }
  g_plan_floor[g_plan_next] = {ws, lg};
  g_plan_next = (g_plan_next + 1) % kPlanFloors;
}

int32_t recorded_plan_floor(const void* ws) {
  std::lock_guard<std::mutex> lock(g_plan_mu);
  for (const PlanFloor& r : g_plan_floor)
    if (r.ws == ws) return r.lg;
  return kLgPartFloor;
}

// Items per sequence in the partition grid after a plan whose partitions hold at least
// 2^floor_lg tokens.
int32_t grid_parts_for(const AttnArgs& a, int32_t floor_lg) {
  return floor_lg >= kLgPartMin ? static_cast<int32_t>(grid_partitions(a.max_blocks_per_seq, a.block_size))
                                : a.max_parts;
}
}  // namespace

int32_t resident_slots() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return 256 * kSlotsPerCU;
  }
  int32_t v = g_slots[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
      (void)hipGetLastError();
      cus = 256;
    }
    v = cus * kSlotsPerCU;
    g_slots[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

int32_t forced_partition_log2() { return g_force_log2.load(std::memory_order_relaxed); }

int32_t set_forced_partition_log2(int32_t lg) {
  g_force_log2.store(lg, std::memory_order_relaxed);
  return PKV_OK;
}

// ---------------------------------------------------------------------------------
// Precondition checks of a debug build (PKV_DEBUG=1).  A release build trusts the
// device arrays it is given (block ids, slots, lengths, copy pairs, chunk offsets);
// a debug build waits for the caller's stream, copies the arrays the call is about
// to use to the host and rejects violations with INVALID_ARG before any launch, so
// every debug call is synchronous.
// ---------------------------------------------------------------------------------
#ifndef PKV_DEBUG
#define PKV_DEBUG 0
#endif
constexpr bool kDebugChecks = PKV_DEBUG != 0;

template <class T>
bool fetch_host(const T* p, int64_t n, void* stream, std::vector<T>& out) {
  out.assign(static_cast<size_t>(n), T{});
  if (n == 0) return true;
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return false;
  return hipMemcpy(out.data(), p, static_cast<size_t>(n) * sizeof(T), hipMemcpyDefault) == hipSuccess;
}

int32_t debug_fail(const char* who, const char* what) {
  char buf[256];
  std::snprintf(buf, sizeof(buf), "%s: debug check failed: %s", who, what);
  return set_error(PKV_ERR_INVALID_ARG, buf);
}

// slots < num_blocks * B; non-negative slots distinct
int32_t debug_check_slots(const char* who, const pkv_pool_desc& pool, const int64_t* slots, int32_t n,
                          void* stream) {
  std::vector<int64_t> h;
  if (!fetch_host(slots, n, stream, h)) return debug_fail(who, "cannot read slot_mapping");
  const int64_t limit = static_cast<int64_t>(pool.num_blocks) * pool.block_size;
  std::vector<int64_t> seen;
  for (int64_t x : h) {
    if (x >= limit) return debug_fail(who, "slot past the pool");
    if (x >= 0) seen.push_back(x);
  }
  std::sort(seen.begin(), seen.end());
  if (std::adjacent_find(seen.begin(), seen.end()) != seen.end()) return debug_fail(who, "duplicate slot");
  return PKV_OK;
}

// 0 <= context_lens[b] <= W * B; table entries that are read lie in the pool
template <class Tab = int32_t>
int32_t debug_check_tables(const char* who, const pkv_pool_desc& pool, const Tab* tables, int32_t W,
                           const int32_t* lens, int32_t n, void* stream) {
  std::vector<int32_t> hl;
  std::vector<Tab> ht;
  if (!fetch_host(lens, n, stream, hl)) return debug_fail(who, "cannot read context_lens");
  if (tables && !fetch_host(tables, static_cast<int64_t>(n) * W, stream, ht))
    return debug_fail(who, "cannot read block_tables");
  for (int32_t b = 0; b < n; ++b) {
    if (hl[b] < 0 || static_cast<int64_t>(hl[b]) > static_cast<int64_t>(W) * pool.block_size)
      return debug_fail(who, "context length outside 0 .. max_blocks_per_seq * block_size");
    if (!tables) continue;
    const int32_t used = (hl[b] + pool.block_size - 1) / pool.block_size;
    for (int32_t j = 0; j < used; ++j) {
      const int64_t blk = static_cast<int64_t>(ht[static_cast<size_t>(b) * W + j]);
      if (blk < 0 || blk >= pool.num_blocks) return debug_fail(who, "block table entry outside the pool");
    }
  }
  return PKV_OK;
}

// two-level tables: the directory entries that are read name leaves 0 .. num_leaves - 1,
// and the leaf entries that are read lie in the pool
int32_t debug_check_tables_2l(const char* who, const pkv_pool_desc& pool, const int32_t* dir,
                              const int32_t* leaves, int32_t num_leaves, int32_t W, const int32_t* lens,
                              int32_t n, void* stream) {
  const int32_t E = PKV_LEAF_TOKENS / pool.block_size;
  const int32_t Wd = W / E;
  std::vector<int32_t> hl, hd, hv;
  if (!fetch_host(lens, n, stream, hl)) return debug_fail(who, "cannot read context_lens");
  if (!fetch_host(dir, static_cast<int64_t>(n) * Wd, stream, hd)) return debug_fail(who, "cannot read leaf_dir");
  if (!fetch_host(leaves, static_cast<int64_t>(num_leaves) * E, stream, hv)) return debug_fail(who, "cannot read leaves");
  for (int32_t b = 0; b < n; ++b) {
    if (hl[b] < 0 || static_cast<int64_t>(hl[b]) > static_cast<int64_t>(W) * pool.block_size)
      return debug_fail(who, "context length outside 0 .. dir_width * leaf entries * block_size");
    const int32_t used = (hl[b] + pool.block_size - 1) / pool.block_size;
    for (int32_t j = 0; j < used; ++j) {
      const int32_t leaf = hd[static_cast<size_t>(b) * Wd + j / E];
      if (leaf < 0 || leaf >= num_leaves) return debug_fail(who, "leaf directory entry outside the leaves");
      const int32_t blk = hv[static_cast<size_t>(leaf) * E + j % E];
      if (blk < 0 || blk >= pool.num_blocks) return debug_fail(who, "block table entry outside the pool");
    }
  }
  return PKV_OK;
}

// copy pairs: ids in the pool, destinations distinct and never a source
int32_t debug_check_pairs(const char* who, const pkv_pool_desc& pool, const int64_t* pairs, int32_t n,
                          void* stream) {
  std::vector<int64_t> h;
  if (!fetch_host(pairs, 2 * static_cast<int64_t>(n), stream, h)) return debug_fail(who, "cannot read pairs");
  std::vector<int64_t> src, dst;
  for (int32_t i = 0; i < n; ++i) {
    if (h[2 * i] < 0 || h[2 * i] >= pool.num_blocks || h[2 * i + 1] < 0 || h[2 * i + 1] >= pool.num_blocks)
      return debug_fail(who, "block id outside the pool");
    src.push_back(h[2 * i]);
    dst.push_back(h[2 * i + 1]);
  }
  std::sort(src.begin(), src.end());
  std::sort(dst.begin(), dst.end());
  if (std::adjacent_find(dst.begin(), dst.end()) != dst.end()) return debug_fail(who, "duplicate destination");
  for (int64_t d : dst)
    if (std::binary_search(src.begin(), src.end(), d)) return debug_fail(who, "a destination is also a source");
  return PKV_OK;
}

// chunk offsets: query_start[0] = 0, non-decreasing, query_start[N] = T, every chunk
// at most max_query_len and at most its context
int32_t debug_check_chunks(const char* who, const int32_t* qstart, const int32_t* lens, int32_t n, int32_t T,
                           int32_t max_query_len, void* stream) {
  std::vector<int32_t> hq, hl;
  if (!fetch_host(qstart, static_cast<int64_t>(n) + 1, stream, hq) || !fetch_host(lens, n, stream, hl))
    return debug_fail(who, "cannot read query_start / context_lens");
  if (hq[0] != 0 || hq[n] != T) return debug_fail(who, "query_start must run from 0 to num_tokens");
  for (int32_t b = 0; b < n; ++b) {
    const int32_t C = hq[b + 1] - hq[b];
    if (C < 0) return debug_fail(who, "query_start decreases");
    if (C > max_query_len) return debug_fail(who, "a chunk is longer than max_query_len");
    if (C > hl[b]) return debug_fail(who, "a chunk is longer than its context");
  }
  return PKV_OK;
}

}  // namespace pkv

using pkv::set_error;

extern "C" {

const char* pkv_version(void) { return "pkv 0.1 (gfx950)"; }

const char* pkv_status_string(int32_t status) {
  switch (status) {
    case PKV_OK: return "PKV_OK";
    case PKV_ERR_INVALID_ARG: return "PKV_ERR_INVALID_ARG";
    case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED";
    case PKV_ERR_WORKSPACE: return "PKV_ERR_WORKSPACE";
    case PKV_ERR_LAUNCH: return "PKV_ERR_LAUNCH";
    case PKV_ERR_OUT_OF_BLOCKS: return "PKV_ERR_OUT_OF_BLOCKS";
    default: return "PKV_ERR_UNKNOWN";
  }
}

const char* pkv_last_error(void) { return pkv::g_last_error.c_str(); }

size_t pkv_pool_bytes(const pkv_pool_desc* pool) {
  if (!pool || pool->num_blocks <= 0 || pool->block_size <= 0 || pool->num_kv_heads <= 0 || pool->head_dim <= 0)
    return 0;
  const int eb = pkv::elem_bytes(pool->dtype);
  return static_cast<size_t>(pool->num_blocks) * pool->num_kv_heads * pool->block_size * pool->head_dim * eb;
}

namespace {
int32_t check_write(const char* who, const pkv_pool_desc* pool, const void* k_pool, const void* v_pool,
                    const void* k_new, const void* v_new, const int64_t* slot_mapping, int32_t num_tokens) {
  char buf[256];
  int32_t st = pkv::check_pool(pool, who);
  if (st != PKV_OK) return st;
  if (num_tokens < 0) {
    std::snprintf(buf, sizeof(buf), "%s: negative num_tokens", who);
    return set_error(PKV_ERR_INVALID_ARG, buf);
  }
  if (num_tokens == 0) return PKV_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !slot_mapping) {
    std::snprintf(buf, sizeof(buf), "%s: null pointer argument", who);
    return set_error(PKV_ERR_INVALID_ARG, buf);
  }
  if (!pkv::aligned(k_pool, 16) || !pkv::aligned(v_pool, 16) || !pkv::aligned(k_new, 16) ||
      !pkv::aligned(v_new, 16) || !pkv::aligned(slot_mapping, 8)) {
    std::snprintf(buf, sizeof(buf), "%s: misaligned pointer", who);
    return set_error(PKV_ERR_INVALID_ARG, buf);
  }
  return PKV_OK;
}
}  // namespace

int32_t pkv_paged_kv_write(const pkv_pool_desc* pool, void* k_pool, void* v_pool, const void* k_new,
                           const void* v_new, const int64_t* slot_mapping, int32_t num_tokens, void* stream) {
  int32_t st = check_write("pkv_paged_kv_write", pool, k_pool, v_pool, k_new, v_new, slot_mapping, num_tokens);
  if (st != PKV_OK || num_tokens == 0) return st;
  if (pkv::kDebugChecks && (st = pkv::debug_check_slots("pkv_paged_kv_write", *pool, slot_mapping, num_tokens,
                                                        stream)) != PKV_OK)
    return st;
  return pkv::launch_status(pkv::launch_kv_write(*pool, k_pool, v_pool, k_new, v_new, slot_mapping, num_tokens, stream),
                            "pkv_paged_kv_write");
}

int32_t pkv_decode_prepare(const pkv_pool_desc* pool, void* k_pool, void* v_pool, const void* k_new,
                           const void* v_new, const int64_t* slot_mapping, int32_t num_tokens, int32_t num_seqs,
                           int32_t num_q_heads, int32_t max_blocks_per_seq, const int32_t* context_lens,
                           const pkv_table_ref* tables, void* workspace, size_t workspace_bytes, void* stream) {
  int32_t st = check_write("pkv_decode_prepare", pool, k_pool, v_pool, k_new, v_new, slot_mapping, num_tokens);
  if (st != PKV_OK) return st;
  pkv::AttnCheck c = pkv::check_attention("pkv_decode_prepare", pool, nullptr, nullptr, nullptr, nullptr,
                                          num_seqs, num_q_heads, nullptr, max_blocks_per_seq, context_lens, 1.0f,
                                          workspace, workspace_bytes, false, false);
  if (c.status != PKV_OK) return c.status;
  if ((st = pkv::apply_table_ref("pkv_decode_prepare", *pool, tables, num_seqs, max_blocks_per_seq, c.args)) != PKV_OK)
    return st;
  if (num_seqs == 0) return pkv_paged_kv_write(pool, k_pool, v_pool, k_new, v_new, slot_mapping, num_tokens, stream);
  if (pkv::kDebugChecks) {
    if ((st = pkv::debug_check_slots("pkv_decode_prepare", *pool, slot_mapping, num_tokens, stream)) != PKV_OK ||
        (st = pkv::debug_check_tables<int32_t>("pkv_decode_prepare", *pool, nullptr, max_blocks_per_seq, context_lens,
                                      num_seqs, stream)) != PKV_OK)
      return st;
  }
  pkv::record_plan(workspace, c.args.force_log2);
  return pkv::launch_status(pkv::launch_decode_prepare(c.args, *pool, k_pool, v_pool, k_new, v_new, slot_mapping,
                                                       num_tokens, stream),
                            "pkv_decode_prepare");
}

int32_t pkv_copy_blocks(const pkv_pool_desc* pool, void* k_pool, void* v_pool, const int64_t* src_dst_pairs,
                        int32_t num_pairs, void* stream) {
  int32_t st = pkv::check_pool(pool, "pkv_copy_blocks");
  if (st != PKV_OK) return st;
  if (num_pairs < 0) return set_error(PKV_ERR_INVALID_ARG, "pkv_copy_blocks: negative num_pairs");
  if (num_pairs == 0) return PKV_OK;
  if (!k_pool || !v_pool || !src_dst_pairs) return set_error(PKV_ERR_INVALID_ARG, "pkv_copy_blocks: null pointer argument");
  if (!pkv::aligned(k_pool, 16) || !pkv::aligned(v_pool, 16) || !pkv::aligned(src_dst_pairs, 8))
    return set_error(PKV_ERR_INVALID_ARG, "pkv_copy_blocks: misaligned pointer");
  if (pkv::kDebugChecks) {
    const int32_t dst = pkv::debug_check_pairs("pkv_copy_blocks", *pool, src_dst_pairs, num_pairs, stream);
    if (dst != PKV_OK) return dst;
  }
  return pkv::launch_status(pkv::launch_copy_blocks(*pool, k_pool, v_pool, src_dst_pairs, num_pairs, stream),
                            "pkv_copy_blocks");
}

int32_t pkv_swap_blocks(const pkv_pool_desc* pool, const void* src_k, const void* src_v, void* dst_k,
                        void* dst_v, const int64_t* src_dst_pairs, int32_t num_pairs, void* stream) {
  int32_t st = pkv::check_pool(pool, "pkv_swap_blocks");
  if (st != PKV_OK) return st;
  if (num_pairs < 0) return set_error(PKV_ERR_INVALID_ARG, "pkv_swap_blocks: negative num_pairs");
  if (num_pairs == 0) return PKV_OK;
  if (!src_k || !src_v || !dst_k || !dst_v || !src_dst_pairs)
    return set_error(PKV_ERR_INVALID_ARG, "pkv_swap_blocks: null pointer argument");
  if (!pkv::aligned(src_k, 16) || !pkv::aligned(src_v, 16) || !pkv::aligned(dst_k, 16) || !pkv::aligned(dst_v, 16) ||
      !pkv::aligned(src_dst_pairs, 8))
    return set_error(PKV_ERR_INVALID_ARG, "pkv_swap_blocks: misaligned pointer");
  return pkv::launch_status(
      pkv::launch_pool_copy(*pool, src_k, src_v, dst_k, dst_v, src_dst_pairs, num_pairs, stream), "pkv_swap_blocks");
}

int32_t pkv_decode_partition_tokens(const pkv_pool_desc* pool, const int32_t* context_lens_host, int32_t num_seqs,
                                    int32_t num_q_heads, int32_t* tokens) {
  const int32_t st = pkv::check_pool(pool, "pkv_decode_partition_tokens");
  if (st != PKV_OK) return st;
  if (!tokens || num_seqs < 0 || (num_seqs > 0 && !context_lens_host) || num_q_heads <= 0 ||
      num_q_heads % pool->num_kv_heads != 0)
    return pkv::set_error(PKV_ERR_INVALID_ARG, "pkv_decode_partition_tokens: bad arguments");
  const int32_t num_kv_heads = pool->num_kv_heads;
  unsigned long long total = 0;
  int lmax = 0;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int L = std::max(context_lens_host[b], 0);
    total += static_cast<unsigned long long>(L);
    lmax = std::max(lmax, L);
  }
  const int G = num_q_heads / num_kv_heads;
  const int hy = num_kv_heads * ((G + 15) / 16);
  *tokens = 1 << pkv::choose_partition_log2(total, lmax, hy, pool->head_dim, pool->block_size, pkv::resident_slots(),
                                            pkv::forced_partition_log2());
  return PKV_OK;
}

int32_t pkv_set_decode_partition_tokens(int32_t tokens) {
  if (tokens == 0) return pkv::set_forced_partition_log2(0);
  if (tokens == PKV_PARTITION_TOKENS_MIN) return pkv::set_forced_partition_log2(pkv::kLgPartFloor);
  if (tokens == PKV_PARTITION_TOKENS) return pkv::set_forced_partition_log2(pkv::kLgPartMin);
  if (tokens == PKV_PARTITION_TOKENS_MAX) return pkv::set_forced_partition_log2(pkv::kLgPartMax);
  return pkv::set_error(PKV_ERR_INVALID_ARG, "pkv_set_decode_partition_tokens: 0, 512, 1024 or 2048 expected");
}

int32_t pkv_stream_read(const void* src, size_t bytes, int32_t workgroups, int32_t unroll, void* sink,
                        void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || !pkv::aligned(src, 16) || !pkv::aligned(sink, 4) ||
      workgroups <= 0 || workgroups > (1 << 24) || (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8))
    return set_error(PKV_ERR_INVALID_ARG, "pkv_stream_read: src and sink non-null and aligned, bytes a positive "
                                          "multiple of 16, workgroups in 1 .. 2^24, unroll 1, 2, 4 or 8 required");
  return pkv::launch_status(pkv::launch_stream_read(src, bytes, workgroups, unroll, sink, stream), "pkv_stream_read");
}

size_t pkv_paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                           int32_t max_blocks_per_seq, int32_t block_size) {
  if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0 || max_blocks_per_seq <= 0 || block_size <= 0) return 0;
  return pkv::workspace_bytes_for(num_seqs, num_q_heads, head_dim, pkv::max_partitions(max_blocks_per_seq, block_size));
}

}  // extern "C"

namespace pkv {
namespace {

// 16-bit tables address at most 65536 blocks.
int32_t check_t16(const pkv_pool_desc* pool, const char* who) {
  if (pool && pool->num_blocks > 65536) {
    char buf[256];
    std::snprintf(buf, sizeof(buf), "%s: 16-bit block tables address at most 65536 blocks, the pool has %d", who,
                  pool->num_blocks);
    return set_error(PKV_ERR_UNSUPPORTED, buf);
  }
  return PKV_OK;
}

// A two-level table as the calls take it (null dir: a flat table).
struct LeafRef {
  const int32_t* dir = nullptr;
  int32_t num_leaves = 0;
};

// Entries per leaf of a two-level table, and the flat width it stands for.
int32_t two_level_width(const char* who, const pkv_pool_desc* pool, int32_t num_seqs, const int32_t* dir,
                        int32_t dir_width, int32_t num_leaves, int32_t* W) {
  int32_t st = check_pool(pool, who);
  if (st != PKV_OK) return st;
  const int32_t E = PKV_LEAF_TOKENS / pool->block_size;
  char buf[256];
  if (dir_width <= 0 || num_leaves < 0 || dir_width > 0x7fffffff / E) {
    std::snprintf(buf, sizeof(buf), "%s: dir_width in 1 .. %d and num_leaves >= 0 required", who, 0x7fffffff / E);
    return set_error(PKV_ERR_INVALID_ARG, buf);
  }
  if (num_seqs > 0 && !dir) {
    std::snprintf(buf, sizeof(buf), "%s: null pointer argument", who);
    return set_error(PKV_ERR_INVALID_ARG, buf);
  }
  if (!aligned(dir, 4)) {
    std::snprintf(buf, sizeof(buf), "%s: misaligned leaf_dir", who);
    return set_error(PKV_ERR_INVALID_ARG, buf);
  }
  *W = dir_width * E;
  return PKV_OK;
}

template <class Tab>
int32_t partitions_impl(const char* who, const pkv_pool_desc* pool, const void* k_pool, const void* v_pool, void* out,
                        const void* q, int32_t num_seqs, int32_t num_q_heads, const Tab* block_tables,
                        int32_t max_blocks_per_seq, const int32_t* context_lens, float scale, void* workspace,
                        size_t workspace_bytes, void* stream, LeafRef two = {}, bool with_plan = false) {
  // every argument is checked before the first launch (the plan pass included)
  AttnCheck c = check_attention(who, pool, k_pool, v_pool, out, q, num_seqs, num_q_heads, block_tables,
                                max_blocks_per_seq, context_lens, scale, workspace, workspace_bytes, true, true,
                                static_cast<int>(sizeof(Tab)));
  if (c.status != PKV_OK) return c.status;
  if (num_seqs == 0) return PKV_OK;
  if (kDebugChecks) {
    const int32_t st =
        two.dir ? debug_check_tables_2l(who, *pool, two.dir, reinterpret_cast<const int32_t*>(block_tables),
                                        two.num_leaves, max_blocks_per_seq, context_lens, num_seqs, stream)
                : debug_check_tables(who, *pool, block_tables, max_blocks_per_seq, context_lens, num_seqs, stream);
    if (st != PKV_OK) return st;
  }
  c.args.table_dir = two.dir;
  c.args.grid_parts =
      grid_parts_for(c.args, with_plan ? plan_floor_log2(c.args.force_log2) : recorded_plan_floor(workspace));
  if (kDebugChecks && !with_plan) {
    std::vector<int32_t> cnt;
    if (!fetch_host(c.args.counters, 1, stream, cnt)) return debug_fail(who, "cannot read the plan's item count");
    if (cnt[0] < 0 || static_cast<int64_t>(cnt[0]) > static_cast<int64_t>(num_seqs) * c.args.grid_parts)
      return debug_fail(who, "the plan's item list does not fit the partition grid");
  }
  if (with_plan) {
    record_plan(workspace, c.args.force_log2);
    const int rc = launch_attn_plan(c.args, stream);
    if (rc != 0) return launch_status(rc, who);
  }
  return launch_status(launch_attn_partitions(c.args, stream), who);
}

}  // namespace
}  // namespace pkv

extern "C" {

int32_t pkv_paged_attention_partitions(const pkv_pool_desc* pool, const void* k_pool, const void* v_pool, void* out,
                                       const void* q, int32_t num_seqs, int32_t num_q_heads,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, float scale, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  return pkv::partitions_impl("pkv_paged_attention_partitions", pool, k_pool, v_pool, out, q, num_seqs, num_q_heads,
                              block_tables, max_blocks_per_seq, context_lens, scale, workspace, workspace_bytes,
                              stream);
}

int32_t pkv_paged_attention_partitions_t16(const pkv_pool_desc* pool, const void* k_pool, const void* v_pool,
                                           void* out, const void* q, int32_t num_seqs, int32_t num_q_heads,
                                           const uint16_t* block_tables, int32_t max_blocks_per_seq,
                                           const int32_t* context_lens, float scale, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  const int32_t st = pkv::check_t16(pool, "pkv_paged_attention_partitions_t16");
  if (st != PKV_OK) return st;
  return pkv::partitions_impl("pkv_paged_attention_partitions_t16", pool, k_pool, v_pool, out, q, num_seqs,
                              num_q_heads, block_tables, max_blocks_per_seq, context_lens, scale, workspace,
                              workspace_bytes, stream);
}

int32_t pkv_paged_attention_partitions_2l(const pkv_pool_desc* pool, const void* k_pool, const void* v_pool,
                                          void* out, const void* q, int32_t num_seqs, int32_t num_q_heads,
                                          const int32_t* leaf_dir, int32_t dir_width, const int32_t* leaves,
                                          int32_t num_leaves, const int32_t* context_lens, float scale,
                                          void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "pkv_paged_attention_partitions_2l";
  int32_t W = 0;
  const int32_t st = pkv::two_level_width(who, pool, num_seqs, leaf_dir, dir_width, num_leaves, &W);
  if (st != PKV_OK) return st;
  return pkv::partitions_impl(who, pool, k_pool, v_pool, out, q, num_seqs, num_q_heads, leaves, W, context_lens,
                              scale, workspace, workspace_bytes, stream, pkv::LeafRef{leaf_dir, num_leaves});
}

int32_t pkv_paged_attention_plan(const pkv_pool_desc* pool, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 const pkv_table_ref* tables, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  pkv::AttnCheck c = pkv::check_attention("pkv_paged_attention_plan", pool, nullptr, nullptr, nullptr, nullptr,
                                          num_seqs, num_q_heads, nullptr, max_blocks_per_seq, context_lens, 1.0f,
                                          workspace, workspace_bytes, false, false);
  if (c.status != PKV_OK) return c.status;
  const int32_t tst =
      pkv::apply_table_ref("pkv_paged_attention_plan", *pool, tables, num_seqs, max_blocks_per_seq, c.args);
  if (tst != PKV_OK) return tst;
  if (num_seqs == 0) return PKV_OK;
  if (pkv::kDebugChecks) {
    const int32_t st = pkv::debug_check_tables<int32_t>("pkv_paged_attention_plan", *pool, nullptr, max_blocks_per_seq,
                                               context_lens, num_seqs, stream);
    if (st != PKV_OK) return st;
  }
  pkv::record_plan(workspace, c.args.force_log2);
  return pkv::launch_status(pkv::launch_attn_plan(c.args, stream), "pkv_paged_attention_plan");
}

int32_t pkv_paged_attention_decode(const pkv_pool_desc* pool, const void* k_pool, const void* v_pool, void* out,
                                   const void* q, int32_t num_seqs, int32_t num_q_heads, const int32_t* block_tables,
                                   int32_t max_blocks_per_seq, const int32_t* context_lens, float scale,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return pkv::partitions_impl("pkv_paged_attention_decode", pool, k_pool, v_pool, out, q, num_seqs, num_q_heads,
                              block_tables, max_blocks_per_seq, context_lens, scale, workspace, workspace_bytes,
                              stream, {}, true);
}

int32_t pkv_paged_attention_decode_t16(const pkv_pool_desc* pool, const void* k_pool, const void* v_pool, void* out,
                                       const void* q, int32_t num_seqs, int32_t num_q_heads,
                                       const uint16_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, float scale, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  const int32_t st = pkv::check_t16(pool, "pkv_paged_attention_decode_t16");
  if (st != PKV_OK) return st;
  return pkv::partitions_impl("pkv_paged_attention_decode_t16", pool, k_pool, v_pool, out, q, num_seqs, num_q_heads,
                              block_tables, max_blocks_per_seq, context_lens, scale, workspace, workspace_bytes,
                              stream, {}, true);
}

int32_t pkv_paged_attention_decode_2l(const pkv_pool_desc* pool, const void* k_pool, const void* v_pool, void* out,
                                      const void* q, int32_t num_seqs, int32_t num_q_heads, const int32_t* leaf_dir,
                                      int32_t dir_width, const int32_t* leaves, int32_t num_leaves,
                                      const int32_t* context_lens, float scale, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  const char* who = "pkv_paged_attention_decode_2l";
  int32_t W = 0;
  const int32_t st = pkv::two_level_width(who, pool, num_seqs, leaf_dir, dir_width, num_leaves, &W);
  if (st != PKV_OK) return st;
  return pkv::partitions_impl(who, pool, k_pool, v_pool, out, q, num_seqs, num_q_heads, leaves, W, context_lens,
                              scale, workspace, workspace_bytes, stream, pkv::LeafRef{leaf_dir, num_leaves}, true);
}

size_t pkv_paged_attention_prefill_workspace_bytes(int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                                   int32_t num_kv_heads) {
  if (num_seqs < 0 || num_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads) return 0;
  return pkv::prefill_workspace_bytes(num_tokens, num_seqs, num_q_heads / num_kv_heads);
}

}  // extern "C"

namespace pkv {
namespace {

template <class Tab>
int32_t prefill_impl(const char* who, const pkv_pool_desc* pool, const void* k_pool, const void* v_pool, void* out,
                     const void* q, int32_t num_seqs, int32_t num_q_heads, const int32_t* query_start,
                     int32_t num_tokens, int32_t max_query_len, const Tab* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, float scale, void* workspace, size_t workspace_bytes,
                     void* stream, LeafRef two = {}) {
  char buf[256];
  int32_t st = check_pool(pool, who);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || num_tokens < 0 || max_query_len < 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0) {
    std::snprintf(buf, sizeof(buf), "%s: num_seqs, num_tokens, max_query_len >= 0 and num_q_heads, "
                  "max_blocks_per_seq > 0 required", who);
    return set_error(PKV_ERR_INVALID_ARG, buf);
  }
  if (num_q_heads % pool->num_kv_heads != 0) {
    std::snprintf(buf, sizeof(buf), "%s: num_q_heads %d is not a multiple of num_kv_heads %d", who, num_q_heads,
                  pool->num_kv_heads);
    return set_error(PKV_ERR_INVALID_ARG, buf);
  }
  if (!prefill_supported(pool->dtype, pool->head_dim, pool->block_size)) {
    std::snprintf(buf, sizeof(buf), "%s: no kernel for dtype %d, head_dim %d, block_size %d (bf16/fp16 only)", who,
                  pool->dtype, pool->head_dim, pool->block_size);
    return set_error(PKV_ERR_UNSUPPORTED, buf);
  }
  if (num_seqs == 0 || num_tokens == 0 || max_query_len == 0) return PKV_OK;
  const int group = num_q_heads / pool->num_kv_heads;
  const int64_t grid = prefill_task_bound(num_tokens, num_seqs, group, 64) * pool->num_kv_heads;
  if (grid > 0x7fffffff || static_cast<int64_t>(num_tokens) * num_q_heads > 0x7fffffff) {
    std::snprintf(buf, sizeof(buf), "%s: problem too large for one launch", who);
    return set_error(PKV_ERR_UNSUPPORTED, buf);
  }
  if (!k_pool || !v_pool || !out || !q || !query_start || !block_tables || !context_lens) {
    std::snprintf(buf, sizeof(buf), "%s: null pointer argument", who);
    return set_error(PKV_ERR_INVALID_ARG, buf);
  }
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(q, 16) || !aligned(out, 16) ||
      !aligned(query_start, 4) || !aligned(block_tables, sizeof(Tab)) || !aligned(context_lens, 4)) {
    std::snprintf(buf, sizeof(buf), "%s: misaligned pointer (pools, q, out need 16 bytes)", who);
    return set_error(PKV_ERR_INVALID_ARG, buf);
  }
  const size_t need = prefill_workspace_bytes(num_tokens, num_seqs, group);
  if (workspace_bytes < need || !workspace || !aligned(workspace, 256)) {
    std::snprintf(buf, sizeof(buf), "%s: workspace of %zu bytes (256-byte aligned) needed, got %zu", who, need,
                  workspace_bytes);
    return set_error(PKV_ERR_WORKSPACE, buf);
  }
  if (kDebugChecks) {
    int32_t dst = debug_check_chunks(who, query_start, context_lens, num_seqs, num_tokens, max_query_len, stream);
    if (dst == PKV_OK)
      dst = two.dir ? debug_check_tables_2l(who, *pool, two.dir, reinterpret_cast<const int32_t*>(block_tables),
                                            two.num_leaves, max_blocks_per_seq, context_lens, num_seqs, stream)
                    : debug_check_tables(who, *pool, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                                         stream);
    if (dst != PKV_OK) return dst;
  }
  PrefillArgs a;
  a.workspace = workspace;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.out = out;
  a.q = q;
  a.block_tables = block_tables;
  a.table_bytes = static_cast<int32_t>(sizeof(Tab));
  a.table_dir = two.dir;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.max_query_len = max_query_len;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.head_dim = pool->head_dim;
  a.block_size = pool->block_size;
  a.dtype = pool->dtype;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.scale = scale;
  return launch_status(launch_prefill(a, stream), who);
}

}  // namespace
}  // namespace pkv

extern "C" {

int32_t pkv_paged_attention_prefill(const pkv_pool_desc* pool, const void* k_pool, const void* v_pool,
                                    void* out, const void* q, int32_t num_seqs, int32_t num_q_heads,
                                    const int32_t* query_start, int32_t num_tokens, int32_t max_query_len,
                                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                                    const int32_t* context_lens, float scale, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return pkv::prefill_impl("pkv_paged_attention_prefill", pool, k_pool, v_pool, out, q, num_seqs, num_q_heads,
                           query_start, num_tokens, max_query_len, block_tables, max_blocks_per_seq, context_lens,
                           scale, workspace, workspace_bytes, stream);
}

int32_t pkv_paged_attention_prefill_t16(const pkv_pool_desc* pool, const void* k_pool, const void* v_pool,
                                        void* out, const void* q, int32_t num_seqs, int32_t num_q_heads,
                                        const int32_t* query_start, int32_t num_tokens, int32_t max_query_len,
                                        const uint16_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, float scale, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  const int32_t st = pkv::check_t16(pool, "pkv_paged_attention_prefill_t16");
  if (st != PKV_OK) return st;
  return pkv::prefill_impl("pkv_paged_attention_prefill_t16", pool, k_pool, v_pool, out, q, num_seqs, num_q_heads,
                           query_start, num_tokens, max_query_len, block_tables, max_blocks_per_seq, context_lens,
                           scale, workspace, workspace_bytes, stream);
}

int32_t pkv_paged_attention_prefill_2l(const pkv_pool_desc* pool, const void* k_pool, const void* v_pool,
                                       void* out, const void* q, int32_t num_seqs, int32_t num_q_heads,
                                       const int32_t* query_start, int32_t num_tokens, int32_t max_query_len,
                                       const int32_t* leaf_dir, int32_t dir_width, const int32_t* leaves,
                                       int32_t num_leaves, const int32_t* context_lens, float scale,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "pkv_paged_attention_prefill_2l";
  int32_t W = 0;
  const int32_t st = pkv::two_level_width(who, pool, num_seqs, leaf_dir, dir_width, num_leaves, &W);
  if (st != PKV_OK) return st;
  return pkv::prefill_impl(who, pool, k_pool, v_pool, out, q, num_seqs, num_q_heads, query_start, num_tokens,
                           max_query_len, leaves, W, context_lens, scale, workspace, workspace_bytes, stream,
                           pkv::LeafRef{leaf_dir, num_leaves});
}

}  // extern "C"
