// Streaming-read probe: the HBM read rate a plain kernel reaches on this device, the
// ceiling the bandwidth-bound attention kernels are compared against (decode is bound
// by memory bandwidth: data.6616ai.com "PagedAttention 之外"; ohmygp.com "先搞清敌人").
//
// Each lane reads 16-byte chunks with non-temporal loads in a grid-stride loop, U
// chunks in flight per iteration; every wave folds what it read into one word (xor) and
// stores it, so no load can be dropped.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kReadThreads = 256;

template <int U>
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                                    u32* __restrict__ sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kReadThreads;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kReadThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  u32 x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) x ^= static_cast<u32>(__shfl_xor(static_cast<int>(x), d, 64));
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kReadThreads / 64) + threadIdx.x / 64] = x;
}

}  // namespace

int launch_stream_read(const void* src, size_t bytes, int32_t workgroups, int32_t unroll, void* sink, void* stream) {
  const auto* s = static_cast<const u32x4*>(src);
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  auto* k = static_cast<u32*>(sink);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(workgroups)), block(kReadThreads);
  switch (unroll) {
    case 1: hipLaunchKernelGGL(stream_read_kernel<1>, grid, block, 0, st, s, n16, k); break;
    case 2: hipLaunchKernelGGL(stream_read_kernel<2>, grid, block, 0, st, s, n16, k); break;
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, grid, block, 0, st, s, n16, k); break;
    case 8: hipLaunchKernelGGL(stream_read_kernel<8>, grid, block, 0, st, s, n16, k); break;
    default: return -1;
  }
  return static_cast<int>(hipGetLastError());
}

}  // namespace pkv
