// Copy-on-write block copy: block dst of the K and V pools becomes a copy of block src.
//
// Pages: agentalpha.top "Q32：vLLM PagedAttention 原理", answer part 3 (a shared block
// is copied only when a sharer writes into it); data.6616ai.com vLLM article,
// "PagedAttention：把虚拟内存搬进 KV Cache" (refcounted prefix, copied at divergence);
// ohmygp.com interview post, "破局思路" (写时共享).
//
// The same kernel serves the swap copy between a device pool and a pinned host pool
// (data.6616ai.com "PagedAttention 之外": preemption swaps KV out to CPU memory).
//
// A block of one pool is num_kv_heads * block_size * head_dim * element_bytes
// contiguous bytes (all heads' tiles).  The grid is (chunks, pool, pair) folded into
// one dimension; each workgroup copies one 16 KiB chunk of one block with 16-byte
// vector loads and stores, four per thread.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 4;
constexpr int64_t kChunkVecs = kThreads * kPerThread;  // 16-byte vectors per workgroup

// Source and destination pools may be the same (copy-on-write) or different (swap
// between a device pool and a pinned host pool).
__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(const u32x4* src_k, const u32x4* src_v, u32x4* dst_k,
                                                               u32x4* dst_v, const int64_t* __restrict__ pairs,
                                                               int64_t block_vecs, int chunks) {
  const int chunk = blockIdx.x % chunks;
  const int which = (blockIdx.x / chunks) & 1;
  const int pair = blockIdx.x / (2 * chunks);
  const int64_t src = pairs[2 * pair];
  const int64_t dst = pairs[2 * pair + 1];
  const u32x4* s = (which ? src_v : src_k) + src * block_vecs;
  u32x4* d = (which ? dst_v : dst_k) + dst * block_vecs;
  u32x4 tmp[kPerThread];
  const int64_t base = chunk * kChunkVecs + threadIdx.x;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int64_t j = base + i * kThreads;
    if (j < block_vecs) tmp[i] = s[j];
  }
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int64_t j = base + i * kThreads;
    if (j < block_vecs) d[j] = tmp[i];
  }
}

}  // namespace

int launch_pool_copy(const pkv_pool_desc& pool, const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                     const int64_t* pairs, int32_t num_pairs, void* stream) {
  const int64_t block_bytes = static_cast<int64_t>(pool.num_kv_heads) * pool.block_size * pool.head_dim *
                              elem_bytes(pool.dtype);
  const int64_t block_vecs = block_bytes / 16;
  const int chunks = static_cast<int>((block_vecs + kChunkVecs - 1) / kChunkVecs);
  // keep every launch under 2^31 work-items
  const int64_t max_pairs = std::max<int64_t>(1, (int64_t{1} << 31) / (int64_t{2} * chunks * kThreads));
  for (int64_t p0 = 0; p0 < num_pairs; p0 += max_pairs) {
    const int64_t np = std::min<int64_t>(max_pairs, num_pairs - p0);
    const unsigned grid = static_cast<unsigned>(np * 2 * chunks);
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(src_k), static_cast<const u32x4*>(src_v), static_cast<u32x4*>(dst_k),
                       static_cast<u32x4*>(dst_v), pairs + 2 * p0, block_vecs, chunks);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return static_cast<int>(e);
  }
  return 0;
}

int launch_copy_blocks(const pkv_pool_desc& pool, void* k_pool, void* v_pool, const int64_t* pairs,
                       int32_t num_pairs, void* stream) {
  return launch_pool_copy(pool, k_pool, v_pool, k_pool, v_pool, pairs, num_pairs, stream);
}

}  // namespace pkv
