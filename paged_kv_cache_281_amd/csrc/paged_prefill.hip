// Causal attention of chunks of new tokens over a paged KV pool (prefill and chunked
// prefill), for gfx950 (CDNA4).
//
// Pages: agentalpha.top "Q32：vLLM PagedAttention 原理", follow-up 3 (FlashAttention
// loads K/V block by block; over paged storage that loading goes through the block
// table, since the blocks are only logically contiguous); data.6616ai.com
// "可能的追问" (FlashAttention fused with paged reads).
//
// Sequence b appends a chunk of C_b tokens whose K/V are already in the pool, so its
// context holds L_b tokens including the chunk.  Query token t of the chunk sits at
// position p = L_b - C_b + t and attends to positions 0..p.
//
// Work split.  The rows of the problem are (query token, query head) pairs of one KV
// head, token-major: row = t * G + g.  A workgroup (4 waves) owns ROWS consecutive
// rows of one (sequence, KV head); each wave owns RG groups of 16 rows and walks the
// 16-token units of K/V from position 0 up to the last position its rows can see,
// with two register buffers (the next unit's loads are in flight while the current
// one is computed).  Waves are independent: no LDS, no barriers.
//
// Products (16x16x32 and 16x16x16 bf16/fp16 MFMA, fp32 accumulate), per 16 rows:
//   S^T[token][row] = K[token][:] . Q[row][:]   (K fragment as A, Q^T as B)
//   O^T[d][row]    += V^T[d][token] P^T[token][row]
// The score accumulator's register layout (lane (r, m) holds tokens 4r..4r+3 of row m)
// is the B operand of the P.V product as it stands, rounded to the pool type.  The
// fragments are the decode kernel's: K chunk (4i + r) of token m, and V row (16c + m)
// at tokens 4r..4r+3 of the transposed V tile.
//
// Masking: a score is kept when its token is <= the row's position (a select, so a
// NaN in a masked slot never propagates), and V elements of tokens past the context
// are zeroed before they meet p = 0.  Every row sees token 0, so each row's running
// max is finite after the first unit.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kPfWaves = 4;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr float kPfRescaleLog2 = 8.f;  // lazy rescale threshold (log2 units)

#ifndef PKV_PREFILL_RG
#define PKV_PREFILL_RG 2
#endif
constexpr int kRG = PKV_PREFILL_RG;              // 16-row groups per wave
constexpr int kTileRows = 16 * kRG * kPfWaves;   // rows per workgroup

struct PrefillParams {
  const char* q;
  const char* kp;
  const char* vp;
  char* out;
  const int* tables;
  const int* ctx;
  const int* qstart;
  int N, T, Hq, Hkv, G, W, Lmax, ntiles;
  float scale_log2;
};

template <class T, int D, int B, int RG>
__global__ __launch_bounds__(kPfThreads) void attn_prefill_mfma(PrefillParams P) {
  constexpr int EB = T::kBytes;
  static_assert(EB == 2, "MFMA path is for 16-bit pools");
  constexpr int KI = D / 32;   // 16x16x32 steps over head_dim
  constexpr int NC = D / 16;   // 16x16x16 products per unit (16 d each)
  constexpr int SUB = B / 16;  // 16-token units per block
  constexpr int64_t TILE = static_cast<int64_t>(B) * D * EB;
  typedef typename T::Bits Bits;
  struct Buf {
    u32x4 k[KI];
    u32x2 v[NC];
  };

  // Tiles holding the latest tokens (the most work) are launched first; KV heads
  // vary fastest, so with 8 KV heads each XCD serves one head's K/V from its L2.
  const int kvh = blockIdx.x % P.Hkv;
  const int rest = blockIdx.x / P.Hkv;
  const int b = rest % P.N;
  const int tile = P.ntiles - 1 - rest / P.N;
  const int q0 = P.qstart[b];
  const int C = P.qstart[b + 1] - q0;
  const int L = min(max(P.ctx[b], 0), P.Lmax);
  // a chunk must lie inside q and inside its context; anything else writes nothing
  if (C <= 0 || C > L || q0 < 0 || q0 > P.T - C) return;
  const int nrows = C * P.G;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wrow0 = tile * kTileRows + w * 16 * RG;
  if (wrow0 >= nrows) return;  // no barriers in this kernel: an idle wave may leave
  const int r = lane >> 4;
  const int m = lane & 15;
  const int prefix = L - C;
  const int t_last = min(nrows - 1, wrow0 + 16 * RG - 1) / P.G;
  const int nunits = (prefix + t_last + 1 + 15) >> 4;  // units up to the last visible position

  // this lane's row in each group (rows past the chunk compute on a valid row and are not stored)
  int pos[RG];
  int64_t orow[RG];
  bool store[RG];
  u32x4 qf[RG][KI];
#pragma unroll
  for (int k = 0; k < RG; ++k) {
    const int row = wrow0 + 16 * k + m;
    store[k] = row < nrows;
    const int rr = store[k] ? row : wrow0;
    const int t = rr / P.G;
    const int g = rr - t * P.G;
    pos[k] = prefix + t;
    orow[k] = static_cast<int64_t>(q0 + t) * P.Hq + kvh * P.G + g;
    const char* qrow = P.q + orow[k] * D * EB;
#pragma unroll
    for (int ki = 0; ki < KI; ++ki) qf[k][ki] = *reinterpret_cast<const u32x4*>(qrow + (4 * ki + r) * 16);
  }

  const int* trow = P.tables + static_cast<int64_t>(b) * P.W;
  const char* kbase = P.kp + kvh * TILE;
  const char* vbase = P.vp + kvh * TILE;
  const int64_t bstride = static_cast<int64_t>(P.Hkv) * TILE;
  const int koff = (r * B + m) * 16;      // + ki * 4 * B * 16 + sub * 256
  const int voff = (m * B + 4 * r) * EB;  // + c * 16 * B * EB + sub * 16 * EB

  // K/V are re-read by every tile of the sequence: ordinary (cached) loads
  auto load = [&](int u, Buf& f) {
    const int e = u / SUB;
    const int blk = trow[e];  // uniform: a scalar load
    const int sub = u - e * SUB;
    const char* kt = kbase + blk * bstride + sub * 256;
    const char* vt = vbase + blk * bstride + sub * 16 * EB;
#pragma unroll
    for (int ki = 0; ki < KI; ++ki) f.k[ki] = *reinterpret_cast<const u32x4*>(kt + koff + ki * 4 * B * 16);
#pragma unroll
    for (int c = 0; c < NC; ++c) f.v[c] = *reinterpret_cast<const u32x2*>(vt + voff + c * 16 * B * EB);
  };

  float m_run[RG], l_part[RG];
  f32x4 o[RG][NC];
#pragma unroll
  for (int k = 0; k < RG; ++k) {
    m_run[k] = kNegInf;
    l_part[k] = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) o[k][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto compute = [&](int u, Buf& f) {
    const int j0 = 16 * u + 4 * r;  // token of this lane's first score
    if (16 * u + 16 > L) {          // tokens past the context: zero V
      const u32 mlo = (j0 + 0 < L ? 0x0000ffffu : 0u) | (j0 + 1 < L ? 0xffff0000u : 0u);
      const u32 mhi = (j0 + 2 < L ? 0x0000ffffu : 0u) | (j0 + 3 < L ? 0xffff0000u : 0u);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        f.v[c][0] &= mlo;
        f.v[c][1] &= mhi;
      }
    }
#pragma unroll
    for (int k = 0; k < RG; ++k) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ki = 0; ki < KI; ++ki) acc = T::mfma_k32(f.k[ki], qf[k][ki], acc);
      float s[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) s[j] = (j0 + j <= pos[k]) ? acc[j] * P.scale_log2 : kNegInf;
      float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      mx = max_xor16(mx);
      mx = max_xor32(mx);
      if (wave_any(mx > m_run[k] + kPfRescaleLog2)) {
        const float mn = fmaxf(m_run[k], mx);
        const float alpha = fast_exp2(m_run[k] - mn);
        l_part[k] *= alpha;
#pragma unroll
        for (int c = 0; c < NC; ++c) o[k][c] *= alpha;
        m_run[k] = mn;
      }
      const u32 p01 = T::pack2(fast_exp2(s[0] - m_run[k]), fast_exp2(s[1] - m_run[k]));
      const u32 p23 = T::pack2(fast_exp2(s[2] - m_run[k]), fast_exp2(s[3] - m_run[k]));
      l_part[k] += (T::lo(p01) + T::hi(p01)) + (T::lo(p23) + T::hi(p23));
      const u32x2 pb = {p01, p23};
#pragma unroll
      for (int c = 0; c < NC; ++c) o[k][c] = T::mfma_k16(f.v[c], pb, o[k][c]);
    }
  };

  Buf first;
  load(0, first);
  PKV_FENCE();
  pipeline2<1, Buf>(0, nunits, first, load, compute);

  // lane (r, m) holds O^T[16c + 4r + j][row m]: four consecutive d per store
#pragma unroll
  for (int k = 0; k < RG; ++k) {
    float l = sum_xor16(l_part[k]);
    l = sum_xor32(l);
    const float inv = 1.f / l;
    if (store[k]) {
      Bits* orow_p = reinterpret_cast<Bits*>(P.out) + orow[k] * D;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        u32x2 pk;
        pk[0] = T::pack2(o[k][c][0] * inv, o[k][c][1] * inv);
        pk[1] = T::pack2(o[k][c][2] * inv, o[k][c][3] * inv);
        *reinterpret_cast<u32x2*>(orow_p + 16 * c + 4 * r) = pk;
      }
    }
  }
}

template <class T, int D, int B>
int launch_prefill_t(const PrefillArgs& a, hipStream_t s) {
  PrefillParams P;
  P.q = static_cast<const char*>(a.q);
  P.kp = static_cast<const char*>(a.k_pool);
  P.vp = static_cast<const char*>(a.v_pool);
  P.out = static_cast<char*>(a.out);
  P.tables = a.block_tables;
  P.ctx = a.context_lens;
  P.qstart = a.query_start;
  P.N = a.num_seqs;
  P.T = a.num_tokens;
  P.Hq = a.num_q_heads;
  P.Hkv = a.num_kv_heads;
  P.G = a.num_q_heads / a.num_kv_heads;
  P.W = a.max_blocks_per_seq;
  P.Lmax = a.max_blocks_per_seq * a.block_size;
  P.ntiles = static_cast<int>(prefill_tiles(a.max_query_len, P.G));
  P.scale_log2 = a.scale * kLog2e;
  const int64_t grid = static_cast<int64_t>(P.ntiles) * P.N * P.Hkv;
  hipLaunchKernelGGL((attn_prefill_mfma<T, D, B, kRG>), dim3(static_cast<unsigned>(grid)), dim3(kPfThreads), 0, s,
                     P);
  return static_cast<int>(hipGetLastError());
}

template <class T>
int launch_prefill_d(const PrefillArgs& a, hipStream_t s) {
  if (a.head_dim == 64) return a.block_size == 16 ? launch_prefill_t<T, 64, 16>(a, s) : launch_prefill_t<T, 64, 32>(a, s);
  return a.block_size == 16 ? launch_prefill_t<T, 128, 16>(a, s) : launch_prefill_t<T, 128, 32>(a, s);
}

}  // namespace

int64_t prefill_tiles(int64_t max_query_len, int64_t group) {
  return (max_query_len * group + kTileRows - 1) / kTileRows;
}

bool prefill_supported(int32_t dtype, int32_t head_dim, int32_t block_size) {
  return (dtype == PKV_F16 || dtype == PKV_BF16) && (head_dim == 64 || head_dim == 128) &&
         (block_size == 16 || block_size == 32);
}

int launch_prefill(const PrefillArgs& a, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (a.dtype) {
    case PKV_F16: return launch_prefill_d<F16>(a, s);
    case PKV_BF16: return launch_prefill_d<BF16>(a, s);
    default: return -1;
  }
}

}  // namespace pkv
