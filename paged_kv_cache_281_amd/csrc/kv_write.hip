// KV write: each new token's K and V go into the slot the block manager reserved.
//
// Pages: agentalpha.top "Q32：vLLM PagedAttention 原理", answer part 2 (a new token
// fills the current block or opens a new one; stored data never moves);
// ohmygp.com interview post, "破局思路" (one slot per decoded token).
//
// One thread per (token, kv head, 16-byte chunk of head_dim).  A K chunk is X
// consecutive d of one token, stored as one 16-byte vector at
// [block][head][d / X][offset][0..X).  The matching V elements go to X rows of
// the transposed V tile, [block][head][d][offset], one element per row.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

template <int EB>
__global__ __launch_bounds__(256) void kv_write_kernel(char* __restrict__ k_pool, char* __restrict__ v_pool,
                                                       const char* __restrict__ k_new,
                                                       const char* __restrict__ v_new,
                                                       const int64_t* __restrict__ slots, int64_t total,
                                                       int H, int D, int B) {
  constexpr int X = 16 / EB;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int nch = D / X;
  const int c = static_cast<int>(idx % nch);
  const int64_t th = idx / nch;
  const int h = static_cast<int>(th % H);
  const int64_t t = th / H;
  // the source vectors do not depend on the slot: issue all three loads together
  const int64_t src = ((t * H + h) * D + static_cast<int64_t>(c) * X) * EB;
  const u32x4 kv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k_new + src));
  const u32x4 vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v_new + src));
  const int64_t slot = slots[t];
  if (slot < 0) return;
  const int64_t blk = slot / B;
  const int off = static_cast<int>(slot % B);
  const int64_t tile = (blk * H + h) * static_cast<int64_t>(D) * B;  // elements
  *reinterpret_cast<u32x4*>(k_pool + (tile + (static_cast<int64_t>(c) * B + off) * X) * EB) = kv;
  const int64_t vrow = tile + static_cast<int64_t>(c) * X * B + off;  // element (d = c*X, off)
  if constexpr (EB == 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) reinterpret_cast<u32*>(v_pool)[vrow + static_cast<int64_t>(e) * B] = vv[e];
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const u32 w = vv[e >> 1];
      reinterpret_cast<uint16_t*>(v_pool)[vrow + static_cast<int64_t>(e) * B] =
          static_cast<uint16_t>((e & 1) ? (w >> 16) : (w & 0xffffu));
    }
  }
}

}  // namespace

int launch_kv_write(const pkv_pool_desc& pool, void* k_pool, void* v_pool, const void* k_new,
                    const void* v_new, const int64_t* slots, int32_t num_tokens, void* stream) {
  const int eb = elem_bytes(pool.dtype);
  const int X = 16 / eb;
  const int64_t per_token = static_cast<int64_t>(pool.num_kv_heads) * (pool.head_dim / X);
  // keep every launch under 2^31 work-items
  const int64_t max_tokens = std::max<int64_t>(1, (int64_t{1} << 31) / (256 * per_token) * 256);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t row_bytes = static_cast<int64_t>(pool.num_kv_heads) * pool.head_dim * eb;
  for (int64_t t0 = 0; t0 < num_tokens; t0 += max_tokens) {
    const int64_t nt = std::min<int64_t>(max_tokens, num_tokens - t0);
    const int64_t total = nt * per_token;
    const unsigned grid = static_cast<unsigned>((total + 255) / 256);
    const char* kn = static_cast<const char*>(k_new) + t0 * row_bytes;
    const char* vn = static_cast<const char*>(v_new) + t0 * row_bytes;
    if (eb == 4) {
      hipLaunchKernelGGL(kv_write_kernel<4>, dim3(grid), dim3(256), 0, s, static_cast<char*>(k_pool),
                         static_cast<char*>(v_pool), kn, vn, slots + t0, total, pool.num_kv_heads,
                         pool.head_dim, pool.block_size);
    } else {
      hipLaunchKernelGGL(kv_write_kernel<2>, dim3(grid), dim3(256), 0, s, static_cast<char*>(k_pool),
                         static_cast<char*>(v_pool), kn, vn, slots + t0, total, pool.num_kv_heads,
                         pool.head_dim, pool.block_size);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return static_cast<int>(e);
  }
  return 0;
}

}  // namespace pkv
