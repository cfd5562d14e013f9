// Body of the KV write, shared by the stand-alone write kernel and the fused write +
// plan kernel.  Work item i is both a K item and a V item:
//   K item (token t, kv head h, chunk c): X consecutive d of one token, one 16-byte
//     vector at [block][h][d / X][offset][0..X);
//   V item (tokens X*g .. X*g+X-1, kv head h, row d): the X tokens' V[d] go to row d of
//     the transposed V tile, [block][h][d][offset].  When their slots are consecutive
//     and start on a multiple of X (a prefill writes whole runs of a block), that is
//     one 16-byte store; otherwise one element per token.
// There are ceil(T / X) * H * D items; items past T * H * D / X have no K part.
//
// Pages: agentalpha.top "Q32：vLLM PagedAttention 原理", answer part 2 (a new token
// fills the current block or opens a new one; stored data never moves);
// ohmygp.com interview post, "破局思路" (one slot per decoded token).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "device_common.h"

namespace pkv {

struct WriteArgs {
  char* k_pool;
  char* v_pool;
  const char* k_new;
  const char* v_new;
  const int64_t* slots;
  int64_t tokens;
  int64_t total;  // ceil(tokens / X) * heads * head_dim work items
  int H, D, B;
};

template <int EB>
__host__ __device__ inline int64_t kv_write_items(int64_t tokens, int H, int D) {
  constexpr int X = 16 / EB;
  return (tokens + X - 1) / X * H * D;
}

template <int EB>
__device__ __forceinline__ void kv_write_one(const WriteArgs& a, int64_t idx) {
  constexpr int X = 16 / EB;
  typedef typename std::conditional<EB == 2, uint16_t, u32>::type E;
  if (idx >= a.total) return;
  const int H = a.H, D = a.D, B = a.B;
  const int64_t T = a.tokens;
  // ---- K item
  const int nch = D / X;
  if (idx < T * H * nch) {
    const int c = static_cast<int>(idx % nch);
    const int64_t th = idx / nch;
    const int h = static_cast<int>(th % H);
    const int64_t t = th / H;
    const u32x4 kv = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(a.k_new + ((t * H + h) * D + static_cast<int64_t>(c) * X) * EB));
    const int64_t slot = a.slots[t];
    if (slot >= 0) {
      const int64_t tile = (slot / B * H + h) * static_cast<int64_t>(D) * B;  // elements
      *reinterpret_cast<u32x4*>(a.k_pool + (tile + (static_cast<int64_t>(c) * B + slot % B) * X) * EB) = kv;
    }
  }
  // ---- V item
  const int d = static_cast<int>(idx % D);
  const int64_t gh = idx / D;
  const int h = static_cast<int>(gh % H);
  const int64_t t0 = gh / H * X;
  E val[X];
  int64_t sl[X];
  bool run = t0 + X <= T;
#pragma unroll
  for (int i = 0; i < X; ++i) {
    const int64_t t = min(t0 + i, T - 1);  // clamped: tokens past T are not stored
    val[i] = __builtin_nontemporal_load(reinterpret_cast<const E*>(a.v_new + ((t * H + h) * D + d) * EB));
    sl[i] = a.slots[t];
  }
  run = run && sl[0] >= 0 && sl[0] % X == 0;
#pragma unroll
  for (int i = 1; i < X; ++i) run = run && sl[i] == sl[0] + i;
  if (run) {
    const int64_t row = (sl[0] / B * H + h) * static_cast<int64_t>(D) * B + static_cast<int64_t>(d) * B + sl[0] % B;
    u32x4 pk;
    if constexpr (EB == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) pk[e] = static_cast<u32>(val[2 * e]) | (static_cast<u32>(val[2 * e + 1]) << 16);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) pk[e] = val[e];
    }
    *reinterpret_cast<u32x4*>(a.v_pool + row * EB) = pk;
  } else {
#pragma unroll
    for (int i = 0; i < X; ++i) {
      if (t0 + i < T && sl[i] >= 0) {
        const int64_t row = (sl[i] / B * H + h) * static_cast<int64_t>(D) * B + static_cast<int64_t>(d) * B + sl[i] % B;
        reinterpret_cast<E*>(a.v_pool)[row] = val[i];
      }
    }
  }
}

// Largest number of work-items one write launch covers (the grid stays below 2^31).
constexpr int64_t kMaxWriteItems = int64_t{1} << 30;

}  // namespace pkv
