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

// One workgroup per (range of B consecutive new tokens, KV head), heads varying fastest
// so that neighbouring workgroups read neighbouring bytes of the token rows.  The new
// tokens fall into segments: runs of consecutive slots inside one block (a token
// continues the previous token's segment when its slot is the next one and does not
// open a block; slot -1 is skipped and ends a segment).  A workgroup writes the
// segments that start in its range, which may reach up to B - 1 tokens into the next
// range, so a prefill chunk's whole blocks stay whole wherever they start in the token
// list.  A segment that is a whole block in order has its K tile [D/X][B][X] and V tile
// [D][B] built in LDS from coalesced reads of the token rows and stored as contiguous
// 16-byte pieces; the other tokens go from LDS to their own slots (K as 16-byte pieces,
// V element by element).
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
  constexpr int R = 2 * B - 1;                // token rows a workgroup may write
  constexpr int NP = (R * CH + NT - 1) / NT;  // pieces per thread, of K and of V
  static_assert(2 * B <= 64, "one wave holds the range and its continuation");
  typedef typename std::conditional<EB == 2, uint16_t, u32>::type E;
  __shared__ u32x4 sk[CH][R + 1];                          // K pieces by (chunk, row), padded
  __shared__ __attribute__((aligned(16))) E sv[R][D + X];  // V rows, padded by 16 bytes
  __shared__ int s_span[3];                                // first row, end, whole-block row or -1
  const int h = static_cast<int>(blockIdx.x % static_cast<unsigned>(H));
  const int64_t base = static_cast<int64_t>(blockIdx.x / static_cast<unsigned>(H)) * B;
  const int tid = threadIdx.x;
  const int64_t row = static_cast<int64_t>(H) * D * EB;  // bytes per token in k_new / v_new
  // the segments, by wave 0: lane p looks at token base + p (p < 2B) and its predecessor
  if (tid < 64) {
    const int p = tid;
    const int64_t t = base + p;
    const int64_t s = (p < 2 * B && t < T) ? slots[t] : -1;
    const int64_t sp = (p < 2 * B && t >= 1 && t - 1 < T && (p > 0 || base > 0)) ? slots[t - 1] : -1;
    const bool cont = s >= 0 && sp >= 0 && s == sp + 1 && s % B != 0;
    const bool start = s >= 0 && !cont;
    const unsigned long long starts = __builtin_amdgcn_ballot_w64(start && p < B);
    const unsigned long long conts = __builtin_amdgcn_ballot_w64(cont);
    if (p == 0) {
      if (starts == 0) {
        s_span[0] = s_span[1] = 0;
        s_span[2] = -1;
      } else {
        const int a = __builtin_ctzll(starts);
        const int last = 63 - __builtin_clzll(starts);
        // the last segment ends at the first token after it that does not continue it
        const unsigned long long after = ~conts & (~0ull << (last + 1));
        const int e = after ? __builtin_ctzll(after) : 2 * B;
        s_span[0] = a;
        s_span[1] = min(e, last + B);
        s_span[2] = -1;
      }
    }
    // a whole block in order: a start at block offset 0 followed by B - 1 continuations
    const unsigned long long need = ((1ull << (B - 1)) - 1) << (p + 1);
    const bool whole = start && p < B && s % B == 0 && (conts & need) == need;
    const unsigned long long w = __builtin_amdgcn_ballot_w64(whole);
    if (p == 0 && w) s_span[2] = __builtin_ctzll(w);
  }
  __syncthreads();
  const int a = s_span[0], e = s_span[1], tile = s_span[2];
  if (a >= e) return;  // workgroup-uniform: no segment starts in this range
  // the rows of tokens base + a .. base + e - 1 into LDS (row p - a), every load first
  const char* ksrc = k_new + base * row + static_cast<int64_t>(h) * D * EB;
  const char* vsrc = v_new + base * row + static_cast<int64_t>(h) * D * EB;
  const int n = e - a;
  {
    u32x4 kr[NP], vr[NP];
#pragma unroll
    for (int x = 0; x < NP; ++x) {
      const int j = tid + NT * x;
      if (x == 0 || j < n * CH) {  // (a range of one whole block needs one piece per thread)
        const int jj = min(j, n * CH - 1);
        const int i = a + jj / CH, c = jj - (jj / CH) * CH;
        kr[x] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ksrc + i * row + c * 16));
        vr[x] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vsrc + i * row + c * 16));
      }
    }
#pragma unroll
    for (int x = 0; x < NP; ++x) {
      const int j = tid + NT * x;
      if (j < n * CH) {
        const int i = j / CH, c = j - (j / CH) * CH;
        sk[c][i] = kr[x];
        *reinterpret_cast<u32x4*>(&sv[i][c * X]) = vr[x];
      }
    }
  }
  __syncthreads();
  const int64_t* sl = slots + base;
  int t0 = 0, t1 = 0;  // rows of the whole block, if any
  if (tile >= 0) {
    t0 = tile - a;
    t1 = t0 + B;
    const int64_t s0 = sl[tile];
    const int64_t dst = (s0 / B * H + h) * static_cast<int64_t>(D) * B * EB;  // bytes
    for (int j = tid; j < B * CH; j += NT) {  // K tile out: piece j = (chunk j / B, token j % B)
      const int c = j / B, i = j - (j / B) * B;
      *reinterpret_cast<u32x4*>(k_pool + dst + static_cast<int64_t>(j) * 16) = sk[c][t0 + i];
    }
    for (int q = tid; q < D * B / X; q += NT) {  // V tile out: row q / (B / X), tokens X (q % (B / X)) ..
      const int d = q / (B / X), i0 = t0 + (q - d * (B / X)) * X;
      u32x4 pk;
      if constexpr (EB == 2) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          pk[k] = static_cast<u32>(sv[i0 + 2 * k][d]) | (static_cast<u32>(sv[i0 + 2 * k + 1][d]) << 16);
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) pk[k] = sv[i0 + k][d];
      }
      *reinterpret_cast<u32x4*>(v_pool + dst + static_cast<int64_t>(q) * 16) = pk;
    }
  }
  // the other rows token by token, tokens varying fastest (a run of consecutive slots
  // still gives contiguous stores)
  const int m = n - (t1 - t0);
  if (m == 0) return;
  for (int j = tid; j < m * CH; j += NT) {  // K: one 16-byte piece per (chunk j / m, token j % m)
    const int c = j / m, k = j - (j / m) * m;
    const int i = k < t0 ? k : k + (t1 - t0);
    const int64_t s = sl[a + i];
    if (s < 0) continue;
    *reinterpret_cast<u32x4*>(k_pool + ((s / B * H + h) * static_cast<int64_t>(D) * B + (c * B + s % B) * X) * EB) =
        sk[c][i];
  }
  for (int j = tid; j < m * D; j += NT) {  // V: one element per (row j / m, token j % m)
    const int d = j / m, k = j - (j / m) * m;
    const int i = k < t0 ? k : k + (t1 - t0);
    const int64_t s = sl[a + i];
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
