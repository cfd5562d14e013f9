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
// head, token-major: row = t * G + g.  A workgroup (4 waves) owns a tile of 64 * RG
// consecutive rows of one (sequence, KV head), RG = 2 for chunks that fill whole
// tiles and 1 for short ones.  A one-workgroup plan pass lists the (sequence, tile)
// tasks that exist, those reading the most K/V first.
// The workgroup walks 32-token units of K/V (one 32-token block or two 16-token
// blocks) from position 0 up to the last position its rows can see.  All 256 threads
// copy each unit from the pool into a ring of three LDS buffers, two units ahead of
// the one being computed, with one barrier per unit; each wave reads the unit's
// fragments once and uses them for all of its RG groups of 16 rows.
//
// Products (16x16x32 bf16/fp16 MFMA, fp32 accumulate), per 16 rows:
//   S^T[token][row] = K[token][:] . Q[row][:]   (K fragment as A, Q^T as B)
//   O^T[d][row]    += V^T[d][token] P^T[token][row]
// The scores come from two chains whose A rows are the tokens
// tau_s(i) = 8*(i/4) + 4*s + i%4 (s = 0, 1), so lane (r, m) holds the scores of
// tokens 8r..8r+7 of row m: after the softmax, rounded to the pool type, they are the
// B operand of the P.V product as they stand, and its A operand (V^T) is 16
// bytes of a V row (the 16 bytes of tokens 8r..8r+7, contiguous in LDS).
//
// Masking: a score is kept when its token is <= the row's position (a select, so a
// NaN in a masked slot never propagates; applied only on units that reach past a
// wave's first position), and V elements of tokens past the context are zeroed before
// they meet p = 0.  Every row sees token 0, so each row's running max is finite after
// the first unit.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kPfWaves = 4;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr float kPfRescaleLog2 = 8.f;  // lazy rescale threshold (log2 units)

// Row groups (16 rows each) per wave: kRGBig when the chunks fill whole workgroup
// tiles, 1 for short chunks (fewer idle rows).
#ifndef PKV_PREFILL_RG_BIG
#define PKV_PREFILL_RG_BIG 2
#endif
constexpr int kRGBig = PKV_PREFILL_RG_BIG;
constexpr int kRGSmall = 1;

struct PrefillParams {
  const char* q;
  const char* kp;
  const char* vp;
  char* out;
  const void* tables;  // int32 or uint16 entries, or two-level leaves (the kernel's Tab parameter)
  const int* dir;      // two-level tables: the leaf directory
  const int* ctx;
  const int* qstart;
  int2* tasks;    // (sequence, tile) tasks, most units first (plan pass)
  int* counters;  // counters[0] = number of tasks
  int N, T, Hq, Hkv, G, W, Lmax, rows, cap;
  float scale_log2;
};

// Chunk geometry of sequence b, or false when its chunk is empty or breaks the
// contract (longer than its context, or outside q).
__device__ __forceinline__ bool chunk_of(const PrefillParams& P, int b, int& q0, int& C, int& L) {
  q0 = P.qstart[b];
  C = P.qstart[b + 1] - q0;
  L = min(max(P.ctx[b], 0), P.Lmax);
  return C > 0 && C <= L && q0 >= 0 && q0 <= P.T - C;
}

// 32-token units a tile of `rows` rows reads: up to its last row's position.
__device__ __forceinline__ int tile_units(const PrefillParams& P, int C, int L, int tile) {
  const int last = (L - C) + min(C * P.G - 1, (tile + 1) * P.rows - 1) / P.G;
  return (last + 1 + 31) >> 5;
}

// ---------------------------------------------------------------------------------
// Plan (one workgroup): lists every (sequence, tile) task, most units first, so the
// long tiles start early and short ones fill in at the end; no task is listed for
// rows a chunk does not have.  Tasks are bucketed by unit count (counts of
// kPlanBuckets - 1 and more share the top bucket); the order within a bucket depends
// on timing, and no result depends on the order.
// ---------------------------------------------------------------------------------
constexpr int kPlanThreads = 1024;
constexpr int kPlanBuckets = 1024;
static_assert(kPlanBuckets == kPlanThreads, "one bucket per plan thread");

// Inclusive sum over the workgroup's threads in thread order: lane shuffles within each
// wave, then each thread adds the totals of the waves before its own (two barriers,
// where a step-by-step scan over the whole workgroup takes two per doubling).
__device__ __forceinline__ int plan_scan(int v, int* s_wsum) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(v, d, 64);
    v += lane >= d ? t : 0;
  }
  if (lane == 63) s_wsum[tid >> 6] = v;
  __syncthreads();
  for (int w = 0; w < (tid >> 6); ++w) v += s_wsum[w];
  __syncthreads();  // s_wsum is free again
  return v;
}

// Calls f(b, t, C, L) for every (sequence b, tile t) the chunks have.  Sequences are
// taken kPlanThreads at a time; their tiles are spread over all threads (a block-wide
// scan of the tile counts, then a binary search per tile), so a long chunk's many
// tiles do not fall on one thread.  With `loaded`, a batch of at most kPlanThreads
// sequences reuses the chunks and tile offsets an earlier call left in LDS.
template <class F>
__device__ __forceinline__ void plan_tiles(const PrefillParams& P, int* s_end, int* s_c, int* s_l, int* s_wsum,
                                           bool loaded, F&& f) {
  const int tid = threadIdx.x;
  for (int b0 = 0; b0 < P.N; b0 += kPlanThreads) {
    if (!loaded) {
      int q0, C = 0, L = 0, nt = 0;
      if (b0 + tid < P.N && chunk_of(P, b0 + tid, q0, C, L)) nt = (C * P.G + P.rows - 1) / P.rows;
      s_c[tid] = C;
      s_l[tid] = L;
      s_end[tid] = plan_scan(nt, s_wsum);  // inclusive: tiles of sequences b0 .. b0 + tid
      __syncthreads();
    }
    const int total = s_end[kPlanThreads - 1];
    for (int g = tid; g < total; g += kPlanThreads) {
      int lo = 0, hi = kPlanThreads - 1;  // first sequence whose range ends past g
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s_end[mid] > g) hi = mid; else lo = mid + 1;
      }
      f(b0 + lo, g - (lo ? s_end[lo - 1] : 0), s_c[lo], s_l[lo]);
    }
    __syncthreads();  // s_end, s_c, s_l are reused by the next batch
  }
}

__global__ __launch_bounds__(kPlanThreads) void prefill_plan(PrefillParams P) {
  __shared__ int cnt[kPlanBuckets];
  __shared__ int s_end[kPlanThreads], s_c[kPlanThreads], s_l[kPlanThreads];
  __shared__ int s_wsum[kPlanThreads / 64];
  const int tid = threadIdx.x;
  cnt[tid] = 0;
  __syncthreads();
  auto bucket = [&](int t, int C, int L) {
    return kPlanBuckets - 1 - min(tile_units(P, C, L, t), kPlanBuckets - 1);
  };
  plan_tiles(P, s_end, s_c, s_l, s_wsum, false,
             [&](int b, int t, int C, int L) { atomicAdd(&cnt[bucket(t, C, L)], 1); });
  // exclusive scan of the bucket counts (bucket 0 = most units)
  __syncthreads();
  const int v = cnt[tid];
  const int incl = plan_scan(v, s_wsum);
  if (tid == kPlanBuckets - 1) P.counters[0] = min(incl, P.cap);
  cnt[tid] = incl - v;  // exclusive offsets
  __syncthreads();
  plan_tiles(P, s_end, s_c, s_l, s_wsum, P.N <= kPlanThreads, [&](int b, int t, int C, int L) {
    const int slot = atomicAdd(&cnt[bucket(t, C, L)], 1);
    if (slot < P.cap) P.tasks[slot] = make_int2(b, t);  // overlapping chunks could overflow the bound
  });
}

// The 4 waves of a workgroup share each 32-token K/V unit.  The unit is copied from
// the pool straight into LDS (global_load_lds: every lane moves 16 bytes to its place in
// a 1 KiB run), in a ring of kPfStages buffers: unit u + 2 is in flight while unit u is
// computed, and one barrier per unit both publishes unit u + 1 and frees the buffer of
// unit u - 1.  Each half of K and of V holds the tokens of one 16-token half of the
// unit (one block at block size 16), so every 1 KiB copy run reads a single block: its
// tile address is the same for all lanes (scalar), and each lane only adds a fixed
// offset.  K half h: chunk c (8 elements of d), token t of the half at 16-byte piece
// c * 16 + (t ^ 4h); V half h: row d, tokens 8 q .. 8 q + 7 of the half (q = 0, 1) at
// piece d * 2 + (q ^ ((d / 8) % 2)).  The XORs put the 16 lanes of a fragment read
// (8 tokens from each half, or 16 rows) in distinct banks.  Each wave reads a fragment
// just before the products that use it, once for all RG of its 16-row groups.
template <int D>
struct PrefillLds {
  static constexpr int kKPieces = D / 8 * 32;  // 16-byte K pieces per unit
  static constexpr int kVPieces = D * 4;       // 16-byte V pieces per unit
  static constexpr int kKHalf = kKPieces / 2;  // pieces of one token half
  static constexpr int kVHalf = kVPieces / 2;
  static_assert(kKHalf % 64 == 0 && kVHalf % 64 == 0, "a copy run lies in one half");
  static constexpr int kKBytes = kKPieces * 16;
  static constexpr int kBytes = (kKPieces + kVPieces) * 16;
  static constexpr int kRuns = (kKPieces + kVPieces) / 64;  // 64-piece runs (one load instruction each)
};
constexpr int kPfStages = 3;

// s_waitcnt with only the vector-memory count limited (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt and lgkmcnt at their maxima)
constexpr int vmcnt_only(int n) { return (n & 0xf) | (((n >> 4) & 3) << 14) | (0x7 << 4) | (0xf << 8); }

template <class T, int D, int B, int RG, class Tab>
__global__ __launch_bounds__(kPfThreads) void attn_prefill_lds(PrefillParams P) {
  constexpr int EB = T::kBytes;
  static_assert(EB == 2, "MFMA path is for 16-bit pools");
  constexpr int KI = D / 32;
  constexpr int NC = D / 16;
  constexpr int BPU = 32 / B;
  constexpr int ROWS = 16 * RG * kPfWaves;
  constexpr int KB = PrefillLds<D>::kKBytes;
  constexpr int KRUNS = PrefillLds<D>::kKPieces / 64;
  constexpr int RUNS = PrefillLds<D>::kRuns;
  constexpr int NX = RUNS / kPfWaves;  // load instructions per thread per unit
  static_assert(RUNS % kPfWaves == 0 && KRUNS % kPfWaves == 0, "runs must divide over the waves");
  constexpr int64_t TILE = static_cast<int64_t>(B) * D * EB;
  typedef typename T::Bits Bits;
  __shared__ __align__(16) char s_kv[kPfStages][PrefillLds<D>::kBytes];

  // task t = blockIdx / Hkv from the plan's list (longest first); KV heads vary
  // fastest, so with 8 KV heads each XCD serves one head's K/V from its L2
  const int kvh = blockIdx.x % P.Hkv;
  const int t = blockIdx.x / P.Hkv;
  // workgroup-uniform exits only (the unit loop has barriers)
  if (t >= P.counters[0]) return;
  const int2 task = P.tasks[t];
  const int b = task.x;
  const int tile = task.y;
  if (b < 0 || b >= P.N || tile < 0) return;  // only a list left by the plan pass is valid
  int q0, C, L;
  if (!chunk_of(P, b, q0, C, L)) return;
  const int nrows = C * P.G;
  const int row0 = tile * ROWS;
  if (row0 >= nrows) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane >> 4;
  const int m = lane & 15;
  const int prefix = L - C;
  const int wg_last = prefix + min(nrows - 1, row0 + ROWS - 1) / P.G;
  const int nunits = (wg_last + 1 + 31) >> 5;
  const int nblk = (L + B - 1) / B;
  const int wrow0 = row0 + w * 16 * RG;
  const bool wave_rows = wrow0 < nrows;  // a wave past the chunk still copies and waits
  const int wrow_c = wave_rows ? wrow0 : row0;
  const int w_first = prefix + wrow_c / P.G;
  const int w_last = prefix + min(nrows - 1, wrow_c + 16 * RG - 1) / P.G;

  int pos[RG];
  int64_t orow[RG];
  bool store[RG];
  u32x4 qf[RG][KI];
#pragma unroll
  for (int k = 0; k < RG; ++k) {
    const int row = wrow0 + 16 * k + m;
    store[k] = row < nrows;
    const int rr = store[k] ? row : wrow_c;
    const int t = rr / P.G;
    const int g = rr - t * P.G;
    pos[k] = prefix + t;
    orow[k] = static_cast<int64_t>(q0 + t) * P.Hq + kvh * P.G + g;
    const char* qrow = P.q + orow[k] * D * EB;
#pragma unroll
    for (int ki = 0; ki < KI; ++ki) qf[k][ki] = *reinterpret_cast<const u32x4*>(qrow + (4 * ki + r) * 16);
  }

  // This thread's piece of each of its NX runs: run x*kPfWaves + w, piece (run * 64 + lane).
  // K piece i -> half h = i / KH, chunk c, token 16 h + t of the unit (layout above); V
  // piece j -> half h, row d, tokens 16 h + 8 q .. + 7.  The half of a run is the same for
  // all its lanes (g_hi: a scalar choice of the tile at block size 16).
  constexpr int KH = PrefillLds<D>::kKHalf;
  constexpr int VH = PrefillLds<D>::kVHalf;
  constexpr int LEAF = PKV_LEAF_TOKENS / B;  // two-level leaf entries
  const int64_t bstride = static_cast<int64_t>(P.Hkv) * TILE;
  const char* kbase = P.kp + kvh * TILE;
  const char* vbase = P.vp + kvh * TILE;
  int g_off[NX];
  bool g_hi[NX];  // (16-token blocks) the run comes from the unit's second block
#pragma unroll
  for (int x = 0; x < NX; ++x) {
    const int run = x * kPfWaves + w;
    if (run < KRUNS) {
      const int h = run * 64 / KH;
      const int wi = run * 64 - h * KH + lane;
      const int c = wi >> 4;
      const int t = (wi & 15) ^ (4 * h);
      g_hi[x] = BPU == 2 && h == 1;
      g_off[x] = (c * B + (BPU == 2 ? t : 16 * h + t)) * 16;
    } else {
      const int j0 = run * 64 - PrefillLds<D>::kKPieces;
      const int h = j0 / VH;
      const int wi = j0 - h * VH + lane;
      const int d = wi >> 1;
      const int q = (wi & 1) ^ ((d >> 3) & 1);
      g_hi[x] = BPU == 2 && h == 1;
      g_off[x] = (d * B + (BPU == 2 ? 8 * q : 16 * h + 8 * q)) * EB;
    }
  }
  auto fetch = [&](int u, int stage) {
    const int e0 = u * BPU;
    // block ids through the scalar cache (the waits for them leave the K/V loads in flight);
    // an absent second block reuses the first
    const int blk0 = table_entry_uniform<Tab, LEAF>(P.tables, P.dir, b, P.W, e0);
    const int blk1 = BPU == 2 ? table_entry_uniform<Tab, LEAF>(P.tables, P.dir, b, P.W, min(e0 + 1, nblk - 1)) : blk0;
    // the unit's tiles (scalar addresses); each run takes one of them (a scalar choice)
    // and each lane adds its fixed offset
    const char* kt0 = kbase + blk0 * bstride;
    const char* kt1 = kbase + blk1 * bstride;
    const char* vt0 = vbase + blk0 * bstride;
    const char* vt1 = vbase + blk1 * bstride;
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      const int run = x * kPfWaves + w;
      const char* src = (run < KRUNS ? (g_hi[x] ? kt1 : kt0) : (g_hi[x] ? vt1 : vt0)) + g_off[x];
      // (typed pointers: with char pointers the host pass drops the kernel's launch stub)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const u32x4*>(src),
                                       reinterpret_cast<u32x4*>(&s_kv[stage][run * 64 * 16]), 16, 0, 0);
    }
  };

  const float cs = P.scale_log2;
  const float inv_cs = 1.f / cs;
  // m_run: the row's running max of the scaled scores; lim: the raw score above which a
  // rescale is due, (m_run + threshold) / cs, kept beside it so that the common case
  // compares raw scores without scaling them
  float m_run[RG], lim[RG], l_run[RG];
  f32x4 o[RG][NC];
#pragma unroll
  for (int k = 0; k < RG; ++k) {
    m_run[k] = kNegInf;
    lim[k] = kNegInf;
    l_run[k] = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) o[k][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // this lane's pieces in the fragment reads (layout above): K fragment (ki, s2) reads
  // chunk 4 ki + r, token tau_s2(m) = 8 (m / 4) + 4 s2 + m % 4 of the unit, which lies in
  // half m / 8; V fragment c reads row 16 c + m, tokens 8 r .. 8 r + 7 (half r / 2)
  const int kh = m >> 3;
  const int kpiece = kh * KH + r * 16 + 8 * ((m >> 2) & 1) + (m & 3);
  const int kbyte[2] = {(kpiece + 4 * kh) * 16, (kpiece + 4 * (kh ^ 1)) * 16};  // s2 = 0, 1
  const int vbyte = (PrefillLds<D>::kKPieces + (r >> 1) * VH + m * 2 + ((r & 1) ^ ((m >> 3) & 1))) * 16;

  // LDS fragment reads are issued one step ahead of the products that use them (two
  // register buffers), so each read has a step of MFMAs to land.
  // (a lane offset per unit, the rest an immediate of the read)
  auto kfrag = [&](const char* base, int ki, int s2) {
    return *reinterpret_cast<const u32x4*>(base + kbyte[s2] + 1024 * ki);
  };
  auto vfrag = [&](const char* base, int c) {
    return *reinterpret_cast<const u32x4*>(base + vbyte + 512 * c);
  };
  // P.V over the unit (V of tokens past the context was zeroed in LDS)
  auto pv = [&](const char* base, const u32x4 (&pb)[RG]) {
    u32x4 vb[2];
    vb[0] = vfrag(base, 0);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (c + 1 < NC) vb[(c + 1) & 1] = vfrag(base, c + 1);
#pragma unroll
      for (int k = 0; k < RG; ++k) o[k][c] = T::mfma_k32(vb[c & 1], pb[k], o[k][c]);
    }
  };
  // V elements of tokens past the context (t >= L) in the unit of stage `stage` become 0
  // before they meet p = 0 (a NaN in an unused slot would survive 0 * NaN)
  auto zero_v_tail = [&](int u, int stage) {
    char* base = s_kv[stage] + KB;
    const int t0 = L - 32 * u;  // first local token past the context
    for (int i = tid; i < D * 4; i += kPfThreads) {
      const int h = i / VH;
      const int d = (i - h * VH) >> 1;
      const int q = 2 * h + ((i & 1) ^ ((d >> 3) & 1));  // tokens 8q .. 8q + 7 of the unit
      if (8 * q + 8 <= t0) continue;
      u32x4* pc = reinterpret_cast<u32x4*>(base + i * 16);
      u32x4 v = *pc;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        v[kk] &= (8 * q + 2 * kk < t0 ? 0x0000ffffu : 0u) | (8 * q + 2 * kk + 1 < t0 ? 0xffff0000u : 0u);
      *pc = v;
    }
  };

  auto compute = [&](int u, int stage) {
    const char* base = s_kv[stage];
    const int j0 = 32 * u + 8 * r;
    const bool diag = 32 * u + 31 > w_first;
    // scores of every group: independent MFMA chains, interleaved
    f32x4 acc[RG][2];
#pragma unroll
    for (int k = 0; k < RG; ++k) {
      acc[k][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc[k][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    u32x4 kb[2][2];
    kb[0][0] = kfrag(base, 0, 0);
    kb[0][1] = kfrag(base, 0, 1);
#pragma unroll
    for (int ki = 0; ki < KI; ++ki) {
      if (ki + 1 < KI) {
        kb[(ki + 1) & 1][0] = kfrag(base, ki + 1, 0);
        kb[(ki + 1) & 1][1] = kfrag(base, ki + 1, 1);
      }
#pragma unroll
      for (int k = 0; k < RG; ++k) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) acc[k][s2] = T::mfma_k32(kb[ki & 1][s2], qf[k][ki], acc[k][s2]);
      }
    }
    float sc[RG][8];  // raw scores of tokens 8r + e, e = 4 s + j
#pragma unroll
    for (int k = 0; k < RG; ++k) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sc[k][e] = acc[k][e >> 2][e & 3];
    }
    if (diag) {
#pragma unroll
      for (int k = 0; k < RG; ++k) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sc[k][e] = (j0 + e <= pos[k]) ? sc[k][e] : kNegInf;
      }
    }
    // This lane's max over its 8 raw scores first; a row's four lanes are combined only
    // when one of them is above the row's limit, since the row's max then is too.
    float mx[RG];
    unsigned long long grow = 0;
#pragma unroll
    for (int k = 0; k < RG; ++k) {
      // (nested pairs of fmaxf become v_max3: three of them and one v_max for 8 values)
      const float a = fmaxf(fmaxf(sc[k][0], sc[k][1]), sc[k][2]);
      const float bb = fmaxf(fmaxf(sc[k][3], sc[k][4]), sc[k][5]);
      mx[k] = fmaxf(fmaxf(fmaxf(a, bb), sc[k][6]), sc[k][7]);
      grow |= __builtin_amdgcn_ballot_w64(mx[k] > lim[k]);
    }
    if (grow != 0) {  // rare: some row's max passed its limit
#pragma unroll
      for (int k = 0; k < RG; ++k) {
        const float rmx = max_xor32(max_xor16(mx[k]));  // the row's max (raw)
        const bool raise = rmx > lim[k];                 // each row (lane m) on its own
        const float nm = rmx * cs;                       // scale > 0: the max of the scaled scores
        const float alpha = raise ? fast_exp2(m_run[k] - nm) : 1.f;
        l_run[k] *= alpha;
#pragma unroll
        for (int c = 0; c < NC; ++c) o[k][c] *= alpha;
        m_run[k] = raise ? nm : m_run[k];
        lim[k] = raise ? (nm + kPfRescaleLog2) * inv_cs : lim[k];
      }
    }
    u32x4 pb[RG];
#pragma unroll
    for (int k = 0; k < RG; ++k) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = fast_exp2(fmaf(sc[k][e], cs, -m_run[k]));
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) pb[k][kk] = T::pack2(p[2 * kk], p[2 * kk + 1]);
      // the row's sum gathers the probabilities as rounded for the P.V product (two per
      // dot2 with ones: half the VALU operations of separate adds)
      const u32 one2 = T::pack2(1.f, 1.f);
      float lk = T::dot2(pb[k][0], one2, l_run[k]);
      lk = T::dot2(pb[k][1], one2, lk);
      lk = T::dot2(pb[k][2], one2, lk);
      l_run[k] = T::dot2(pb[k][3], one2, lk);
    }
    pv(base, pb);
  };

  // Ring of kPfStages LDS buffers: unit u computed from buffer u % 3 while units u + 1
  // and u + 2 load.  Before unit u: this thread's loads of unit u have landed (its later
  // unit's NX loads may still be in flight), and the barrier makes every thread's
  // loads visible and ends every wave's use of buffer (u - 1) % 3, which unit u + 2 then fills.
  // (the barrier is s_barrier alone: a full __syncthreads would also wait for the loads
  // of unit u + 1; the signal fences keep the compiler from moving LDS reads across it)
  fetch(0, 0);
  if (nunits > 1) fetch(1, 1);
  // Everything issued so far has landed before the loop (the query fragments with the
  // first two units): with the queries known complete, the compiler has no reason to
  // wait for every copy in flight before each unit's first product.
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  for (int u = 0; u < nunits; ++u) {
    if (u + 1 < nunits) __builtin_amdgcn_s_waitcnt(vmcnt_only(NX));
    else __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (u + 2 < nunits) fetch(u + 2, (u + 2) % kPfStages);
    if (32 * u + 32 > L) {  // the unit holding the context's end (workgroup-uniform)
      zero_v_tail(u, u % kPfStages);
      __builtin_amdgcn_s_waitcnt(vmcnt_only(63) & ~(0xf << 8));  // (lgkmcnt 0: the LDS writes are done)
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_barrier();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
    if (wave_rows && 32 * u <= w_last) compute(u, u % kPfStages);  // units this wave's rows can see
  }

#pragma unroll
  for (int k = 0; k < RG; ++k) {
    float l = sum_xor16(l_run[k]);
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

template <class T, int D, int B, int RG, class Tab>
int launch_prefill_rg(const PrefillArgs& a, PrefillParams P, hipStream_t s) {
  P.rows = 16 * RG * kPfWaves;
  P.cap = static_cast<int>(prefill_task_bound(a.num_tokens, a.num_seqs, P.G, P.rows));
  hipLaunchKernelGGL(prefill_plan, dim3(1), dim3(kPlanThreads), 0, s, P);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return static_cast<int>(e);
  const int64_t grid = static_cast<int64_t>(P.cap) * P.Hkv;
  hipLaunchKernelGGL((attn_prefill_lds<T, D, B, RG, Tab>), dim3(static_cast<unsigned>(grid)), dim3(kPfThreads), 0, s,
                     P);
  return static_cast<int>(hipGetLastError());
}

template <class T, int D, int B, class Tab>
int launch_prefill_t(const PrefillArgs& a, hipStream_t s) {
  PrefillParams P;
  P.q = static_cast<const char*>(a.q);
  P.kp = static_cast<const char*>(a.k_pool);
  P.vp = static_cast<const char*>(a.v_pool);
  P.out = static_cast<char*>(a.out);
  P.tables = a.block_tables;
  P.dir = a.table_dir;
  P.ctx = a.context_lens;
  P.qstart = a.query_start;
  P.counters = static_cast<int*>(a.workspace);
  P.tasks = reinterpret_cast<int2*>(static_cast<char*>(a.workspace) + kPrefillCounterBytes);
  P.N = a.num_seqs;
  P.T = a.num_tokens;
  P.Hq = a.num_q_heads;
  P.Hkv = a.num_kv_heads;
  P.G = a.num_q_heads / a.num_kv_heads;
  P.W = a.max_blocks_per_seq;
  P.Lmax = a.max_blocks_per_seq * a.block_size;
  P.rows = 0;
  P.cap = 0;
  P.scale_log2 = a.scale * kLog2e;
  if (static_cast<int64_t>(a.max_query_len) * P.G >= 16 * kRGBig * kPfWaves)
    return launch_prefill_rg<T, D, B, kRGBig, Tab>(a, P, s);
  return launch_prefill_rg<T, D, B, kRGSmall, Tab>(a, P, s);
}

template <class T, class Tab>
int launch_prefill_tab(const PrefillArgs& a, hipStream_t s) {
  if (a.head_dim == 64)
    return a.block_size == 16 ? launch_prefill_t<T, 64, 16, Tab>(a, s) : launch_prefill_t<T, 64, 32, Tab>(a, s);
  return a.block_size == 16 ? launch_prefill_t<T, 128, 16, Tab>(a, s) : launch_prefill_t<T, 128, 32, Tab>(a, s);
}

template <class T>
int launch_prefill_d(const PrefillArgs& a, hipStream_t s) {
  if (a.table_dir) return launch_prefill_tab<T, TwoLevel>(a, s);
  return a.table_bytes == 2 ? launch_prefill_tab<T, uint16_t>(a, s) : launch_prefill_tab<T, int>(a, s);
}

}  // namespace

int64_t prefill_task_bound(int64_t num_tokens, int64_t num_seqs, int64_t group, int64_t tile_rows) {
  // sum_b ceil(C_b G / rows) <= T G / rows + N
  return (num_tokens * group + tile_rows - 1) / tile_rows + num_seqs;
}

size_t prefill_workspace_bytes(int64_t num_tokens, int64_t num_seqs, int64_t group) {
  return kPrefillCounterBytes +
         static_cast<size_t>(prefill_task_bound(num_tokens, num_seqs, group, 16 * kRGSmall * kPfWaves)) * 8;
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
