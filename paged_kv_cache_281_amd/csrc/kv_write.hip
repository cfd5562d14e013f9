// KV write: each new token's K and V go into the slot the block manager reserved.
//
// Pages: agentalpha.top "Q32：vLLM PagedAttention 原理", answer part 2 (a new token
// fills the current block or opens a new one; stored data never moves);
// ohmygp.com interview post, "破局思路" (one slot per decoded token).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

// One workgroup per (group of B consecutive new tokens, KV head), heads varying fastest
// so that neighbouring workgroups read neighbouring bytes of the token rows.  When the group's
// slots are one whole block in order (prefill chunks fill whole blocks), the block's K
// tile [D/X][B][X] and V tile [D][B] are built in LDS from coalesced reads of the token
// rows and stored as contiguous 16-byte pieces.  Otherwise each token goes from LDS to
// its own slot (K as 16-byte pieces, V element by element; slot -1 is skipped).
#ifndef PKV_KV_WRITE_THREADS
#define PKV_KV_WRITE_THREADS 256
#endif
constexpr int kWriteThreads = PKV_KV_WRITE_THREADS;

template <int EB, int D, int B>
__global__ __launch_bounds__(kWriteThreads) void kv_write_tiles_kernel(const char* __restrict__ k_new,
                                                                       const char* __restrict__ v_new,
                                                                       const int64_t* __restrict__ slots,
                                                                       char* k_pool, char* v_pool, int64_t T, int H) {
  constexpr int X = 16 / EB;   // elements per 16-byte piece
  constexpr int CH = D / X;    // 16-byte pieces per token row of one head
  constexpr int NT = kWriteThreads;
  constexpr int NP = (B * CH + NT - 1) / NT;  // pieces per thread, of K and of V
  typedef typename std::conditional<EB == 2, uint16_t, u32>::type E;
  __shared__ u32x4 sk[CH][B + 1];                          // K pieces by (chunk, token), padded
  __shared__ __attribute__((aligned(16))) E sv[B][D + X];  // V rows by token, padded by 16 bytes
  const int h = static_cast<int>(blockIdx.x % static_cast<unsigned>(H));
  const int64_t t0 = static_cast<int64_t>(blockIdx.x / static_cast<unsigned>(H)) * B;
  const int n = static_cast<int>(min(static_cast<int64_t>(B), T - t0));
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int64_t row = static_cast<int64_t>(H) * D * EB;  // bytes per token in k_new / v_new
  const char* ksrc = k_new + t0 * row + static_cast<int64_t>(h) * D * EB;
  const char* vsrc = v_new + t0 * row + static_cast<int64_t>(h) * D * EB;
  const int64_t s0 = slots[t0];
  // whole-block test (uniform: every wave reaches the same answer)
  const int64_t si = lane < n ? slots[t0 + lane] : s0 + lane;
  const bool whole = n == B && s0 >= 0 && s0 % B == 0 &&
                     __builtin_amdgcn_ballot_w64(lane < B && si != s0 + lane) == 0;
  // the group's token rows into LDS, every load first: piece j = (token j / CH, chunk
  // j % CH); tokens past the end read the last token again (never stored)
  {
    u32x4 kr[NP], vr[NP];
#pragma unroll
    for (int x = 0; x < NP; ++x) {
      const int j = min(tid + NT * x, B * CH - 1);
      const int i = min(j / CH, n - 1), c = j - (j / CH) * CH;
      kr[x] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ksrc + i * row + c * 16));
      vr[x] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vsrc + i * row + c * 16));
    }
#pragma unroll
    for (int x = 0; x < NP; ++x) {
      const int j = min(tid + NT * x, B * CH - 1);
      const int i = j / CH, c = j - (j / CH) * CH;
      sk[c][i] = kr[x];
      *reinterpret_cast<u32x4*>(&sv[i][c * X]) = vr[x];
    }
  }
  __syncthreads();
  if (whole) {
    const int64_t tile = (s0 / B * H + h) * static_cast<int64_t>(D) * B * EB;  // bytes
    for (int j = tid; j < B * CH; j += NT) {  // K tile out: piece j = (chunk j / B, token j % B)
      const int c = j / B, i = j - (j / B) * B;
      *reinterpret_cast<u32x4*>(k_pool + tile + static_cast<int64_t>(j) * 16) = sk[c][i];
    }
    for (int q = tid; q < D * B / X; q += NT) {  // V tile out: row q / (B / X), tokens X (q % (B / X)) ..
      const int d = q / (B / X), i0 = (q - d * (B / X)) * X;
      u32x4 pk;
      if constexpr (EB == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          pk[e] = static_cast<u32>(sv[i0 + 2 * e][d]) | (static_cast<u32>(sv[i0 + 2 * e + 1][d]) << 16);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[e] = sv[i0 + e][d];
      }
      *reinterpret_cast<u32x4*>(v_pool + tile + static_cast<int64_t>(q) * 16) = pk;
    }
    return;
  }
  // Otherwise token by token, tokens varying fastest: runs of consecutive slots (a
  // chunk that starts inside a block) still give contiguous stores.
  for (int j = tid; j < n * CH; j += NT) {  // K: one 16-byte piece per (chunk j / n, token j % n)
    const int c = j / n, i = j - (j / n) * n;
    const int64_t s = slots[t0 + i];
    if (s < 0) continue;
    *reinterpret_cast<u32x4*>(k_pool + ((s / B * H + h) * static_cast<int64_t>(D) * B + (c * B + s % B) * X) * EB) =
        sk[c][i];
  }
  for (int j = tid; j < n * D; j += NT) {  // V: one element per (row j / n, token j % n)
    const int d = j / n, i = j - (j / n) * n;
    const int64_t s = slots[t0 + i];
    if (s < 0) continue;
    reinterpret_cast<E*>(v_pool)[(s / B * H + h) * static_cast<int64_t>(D) * B + static_cast<int64_t>(d) * B + s % B] =
        sv[i][d];
  }
}

template <int EB, int D>
int launch_tiles_d(const pkv_pool_desc& pool, void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                   const int64_t* slots, int64_t T, hipStream_t s) {
  const int H = pool.num_kv_heads, B = pool.block_size;
  const int64_t row = static_cast<int64_t>(H) * D * EB;
  // tokens per launch: whole groups, at most 2^31 - 1 workgroups
  const int64_t max_tokens = static_cast<int64_t>(0x7fffffff) / H * B;
  for (int64_t t0 = 0; t0 < T; t0 += max_tokens) {
    const int64_t nt = std::min(max_tokens, T - t0);
    const dim3 grid(static_cast<unsigned>((nt + B - 1) / B * H));
    auto* kn = static_cast<const char*>(k_new) + t0 * row;
    auto* vn = static_cast<const char*>(v_new) + t0 * row;
    auto* kp = static_cast<char*>(k_pool);
    auto* vp = static_cast<char*>(v_pool);
    if (B == 16)
      hipLaunchKernelGGL((kv_write_tiles_kernel<EB, D, 16>), grid, dim3(kWriteThreads), 0, s, kn, vn, slots + t0, kp,
                         vp, nt, H);
    else
      hipLaunchKernelGGL((kv_write_tiles_kernel<EB, D, 32>), grid, dim3(kWriteThreads), 0, s, kn, vn, slots + t0, kp,
                         vp, nt, H);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return static_cast<int>(e);
  }
  return 0;
}

}  // namespace

int launch_kv_write(const pkv_pool_desc& pool, void* k_pool, void* v_pool, const void* k_new,
                    const void* v_new, const int64_t* slots, int32_t num_tokens, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (elem_bytes(pool.dtype) == 4)
    return pool.head_dim == 64 ? launch_tiles_d<4, 64>(pool, k_pool, v_pool, k_new, v_new, slots, num_tokens, s)
                               : launch_tiles_d<4, 128>(pool, k_pool, v_pool, k_new, v_new, slots, num_tokens, s);
  return pool.head_dim == 64 ? launch_tiles_d<2, 64>(pool, k_pool, v_pool, k_new, v_new, slots, num_tokens, s)
                             : launch_tiles_d<2, 128>(pool, k_pool, v_pool, k_new, v_new, slots, num_tokens, s);
}

}  // namespace pkv
