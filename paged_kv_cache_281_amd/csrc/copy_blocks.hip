// Copy-on-write block copy: block dst of the K and V pools becomes a copy of block src.
//
// Pages: agentalpha.top "Q32：vLLM PagedAttention 原理", answer part 3 (a shared block
// is copied only when a sharer writes into it); data.6616ai.com vLLM article,
// "PagedAttention：把虚拟内存搬进 KV Cache" (refcounted prefix, copied at divergence);
// ohmygp.com interview post, "破局思路" (写时共享).
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

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(u32x4* __restrict__ k_pool, u32x4* __restrict__ v_pool,
                                                               const int64_t* __restrict__ pairs,
                                                               int64_t block_vecs, int chunks) {
  const int chunk = blockIdx.x % chunks;
  const int which = (blockIdx.x / chunks) & 1;
  const int pair = blockIdx.x / (2 * chunks);
  const int64_t src = pairs[2 * pair];
  const int64_t dst = pairs[2 * pair + 1];
  u32x4* pool = which ? v_pool : k_pool;
  const u32x4* s = pool + src * block_vecs;
  u32x4* d = pool + dst * block_vecs;
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

int launch_copy_blocks(const pkv_pool_desc& pool, void* k_pool, void* v_pool, const int64_t* pairs,
                       int32_t num_pairs, void* stream) {
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
                       static_cast<u32x4*>(k_pool), static_cast<u32x4*>(v_pool), pairs + 2 * p0, block_vecs,
                       chunks);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return static_cast<int>(e);
  }
  return 0;
}

}  // namespace pkv
