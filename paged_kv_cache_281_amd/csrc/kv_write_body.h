// Body of the KV write (one thread per (token, kv head, 16-byte chunk of head_dim)),
// shared by the stand-alone write kernel and the fused write + plan kernel.
//
// Pages: agentalpha.top "Q32：vLLM PagedAttention 原理", answer part 2 (a new token
// fills the current block or opens a new one; stored data never moves);
// ohmygp.com interview post, "破局思路" (one slot per decoded token).
//
// A K chunk is X consecutive d of one token, stored as one 16-byte vector at
// [block][head][d / X][offset][0..X).  The matching V elements go to X rows of the
// transposed V tile, [block][head][d][offset], one element per row.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"

namespace pkv {

struct WriteArgs {
  char* k_pool;
  char* v_pool;
  const char* k_new;
  const char* v_new;
  const int64_t* slots;
  int64_t total;  // tokens * heads * chunks
  int H, D, B;
};

template <int EB>
__device__ __forceinline__ void kv_write_one(const WriteArgs& a, int64_t idx) {
  constexpr int X = 16 / EB;
  if (idx >= a.total) return;
  const int H = a.H, D = a.D, B = a.B;
  const int nch = D / X;
  const int c = static_cast<int>(idx % nch);
  const int64_t th = idx / nch;
  const int h = static_cast<int>(th % H);
  const int64_t t = th / H;
  // the source vectors do not depend on the slot: issue all three loads together
  const int64_t src = ((t * H + h) * D + static_cast<int64_t>(c) * X) * EB;
  const u32x4 kv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.k_new + src));
  const u32x4 vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.v_new + src));
  const int64_t slot = a.slots[t];
  if (slot < 0) return;
  const int64_t blk = slot / B;
  const int off = static_cast<int>(slot % B);
  const int64_t tile = (blk * H + h) * static_cast<int64_t>(D) * B;  // elements
  *reinterpret_cast<u32x4*>(a.k_pool + (tile + (static_cast<int64_t>(c) * B + off) * X) * EB) = kv;
  const int64_t vrow = tile + static_cast<int64_t>(c) * X * B + off;  // element (d = c*X, off)
  if constexpr (EB == 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) reinterpret_cast<u32*>(a.v_pool)[vrow + static_cast<int64_t>(e) * B] = vv[e];
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const u32 w = vv[e >> 1];
      reinterpret_cast<uint16_t*>(a.v_pool)[vrow + static_cast<int64_t>(e) * B] =
          static_cast<uint16_t>((e & 1) ? (w >> 16) : (w & 0xffffu));
    }
  }
}

// Largest number of work-items one write launch covers (the grid stays below 2^31).
constexpr int64_t kMaxWriteItems = int64_t{1} << 30;

}  // namespace pkv
