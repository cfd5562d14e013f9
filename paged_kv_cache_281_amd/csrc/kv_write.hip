// KV write: each new token's K and V go into the slot the block manager reserved.
//
// Pages: agentalpha.top "Q32：vLLM PagedAttention 原理", answer part 2 (a new token
// fills the current block or opens a new one; stored data never moves);
// ohmygp.com interview post, "破局思路" (one slot per decoded token).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.h"
#include "kv_write_body.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

template <int EB>
__global__ __launch_bounds__(256) void kv_write_kernel(WriteArgs a) {
  kv_write_one<EB>(a, static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x);
}

}  // namespace

int launch_kv_write(const pkv_pool_desc& pool, void* k_pool, void* v_pool, const void* k_new,
                    const void* v_new, const int64_t* slots, int32_t num_tokens, void* stream) {
  const int eb = elem_bytes(pool.dtype);
  const int X = 16 / eb;
  const int64_t per_token = static_cast<int64_t>(pool.num_kv_heads) * (pool.head_dim / X);  // items per token
  // tokens per launch: a multiple of X, so every launch starts a whole V item
  const int64_t max_tokens = std::max<int64_t>(X, kMaxWriteItems / per_token / X * X);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t row_bytes = static_cast<int64_t>(pool.num_kv_heads) * pool.head_dim * eb;
  for (int64_t t0 = 0; t0 < num_tokens; t0 += max_tokens) {
    const int64_t nt = std::min<int64_t>(max_tokens, num_tokens - t0);
    WriteArgs a;
    a.k_pool = static_cast<char*>(k_pool);
    a.v_pool = static_cast<char*>(v_pool);
    a.k_new = static_cast<const char*>(k_new) + t0 * row_bytes;
    a.v_new = static_cast<const char*>(v_new) + t0 * row_bytes;
    a.slots = slots + t0;
    a.tokens = nt;
    a.total = eb == 4 ? kv_write_items<4>(nt, pool.num_kv_heads, pool.head_dim)
                      : kv_write_items<2>(nt, pool.num_kv_heads, pool.head_dim);
    a.H = pool.num_kv_heads;
    a.D = pool.head_dim;
    a.B = pool.block_size;
    const unsigned grid = static_cast<unsigned>((a.total + 255) / 256);
    if (eb == 4) {
      hipLaunchKernelGGL(kv_write_kernel<4>, dim3(grid), dim3(256), 0, s, a);
    } else {
      hipLaunchKernelGGL(kv_write_kernel<2>, dim3(grid), dim3(256), 0, s, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return static_cast<int>(e);
  }
  return 0;
}

}  // namespace pkv
