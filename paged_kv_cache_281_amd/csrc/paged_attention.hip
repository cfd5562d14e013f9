// Decode attention over a paged KV pool, for gfx950 (CDNA4).
//
// Pages: data.6616ai.com vLLM article, "PagedAttention：把虚拟内存搬进 KV Cache" (the
// attention kernel reads K/V by block index: logically contiguous, physically
// scattered); agentalpha.top "Q32：vLLM PagedAttention 原理", follow-up 3 (blockwise,
// FlashAttention-style loading adapted to scattered blocks through pointer
// indexing); data.6616ai.com "可能的追问" (the cost is table lookups and
// non-contiguous access); data.6616ai.com "PagedAttention 之外" and ohmygp.com
// "先搞清敌人" (decode is bound by memory, not compute).
//
// Work split.  A workgroup (4 waves) owns one (sequence, kv head [, group of up to
// 16 query heads], partition of 1024 or 2048 context tokens, chosen per launch).  It stages
// the partition's block-table entries in LDS, then each wave walks every 4th
// 16-token unit of the partition with a register double buffer (the next unit's K
// and V loads are in flight while the current unit is computed), keeping an online
// softmax (running max in log2 units, running sum, rescaled output).  Items are
// taken from a device-built task list ordered longest first (plan kernel).  The four
// waves' states are merged in LDS.  A sequence that fits in one partition gets its
// final output here; longer ones leave (max, sum, normalised output) per partition
// in the workspace, and the workgroup that completes a row's last partition merges
// them, weighting partition p by exp2(m_p - M) * l_p.
//
// Loads.  With the pool layout of pkv.h one (block, kv head) tile is contiguous:
// K as [D/X][B][X] 16-byte chunks, V as [D][B].  Lane (r = lane/16, m = lane%16)
// reads K chunk (4i + r) of token m of the unit, so every K load instruction covers
// four 256-byte runs; it reads V row (16c + m), tokens 4r..4r+3, so every V load
// instruction covers 512 contiguous bytes.  The physical block id comes from LDS and
// is made wave-uniform, so tile addresses are scalar.
//
// bf16/fp16 pools use MFMA (1..16 query heads per kv head): the scores
// S^T[token][head] of a 16-token unit are a 16x16x32 MFMA chain over D (K fragment as
// A, the item's queries zero-padded to 16 columns as B), and O^T[d][head] +=
// V^T[d][token] P^T[token][head] is a 16x16x16 MFMA per 16 d whose B operand is the
// score accumulator's own register layout, rounded to the pool type.  The columns a
// small query group leaves empty hold the query heads of other sequences that share
// the item's prefix.  fp32 pools use the vector ALU (FMAs).
//
// NaN safety: scores of tokens past the context are replaced by -inf (select, not
// arithmetic) and V elements of those tokens are zeroed before they meet p = 0.
// The per-token reduction order depends only on logical positions, so the result
// does not depend on where the blocks sit.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.h"
#include "kv_write_body.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kPTMax = PKV_PARTITION_TOKENS_MAX;  // largest partition (LDS table staging)
template <int B>
constexpr int kLeaf = PKV_LEAF_TOKENS / B;  // entries per two-level leaf
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

struct Params {
  const char* q;
  const char* kp;
  const char* vp;
  char* out;
  float* ws_o;
  float* ws_ml;
  const void* tables;   // int32 or uint16 entries, or two-level leaves (the kernels' Tab parameter)
  const int* dir;       // two-level tables: the leaf directory
  const int* ctx;
  int4* tasks;          // work items, longest first (written by the plan pass)
  int* counters;        // counters[0] = number of items, counters[1] = log2 of the partition size
  int* done;            // [N * Hq]: partitions finished per (sequence, first head of a group)
  int* seq_np;          // [N]: partial results of each sequence's rows
  int4* seq_grp;        // [N]: shared-prefix group of each sequence (plan pass)
  int* members;         // [N]: the sequences of each shared-prefix group, group by group
  int* member_own;      // [N]: beside members: each member's own tokens (fused items)
  int N, Hq, Hkv, G, NHG, W, Pmax, Lmax, B, D;
  float scale_log2;
  int tab_bytes;   // 4 or 2 (flat tables)
  int leaf_e;      // entries per two-level leaf
  int slots;       // resident partition workgroups (plan's size choice)
  int force_log2;  // 0, or the partition size fixed by the caller (log2)
  int cm;          // sequences per shared-prefix item (16 / G); below 2: no shared-prefix items
  int fuse_ok;     // the partition kernel runs fused items (16-token units, one unit per block)
};

// Work items (int4): x = the sequence (an ordinary item) or the offset of the item's
// sequences in the members list (a shared-prefix item), with the flags below; y = the
// first context token; z = the number of tokens (0: the zero output of an empty
// context); w = the partial-result slot of the item | (the partial count of the
// sequence's rows for an ordinary item, or the number of sequences of a shared-prefix
// item) << 16.
constexpr int kPrefixTask = 1 << 29;
// A shared-prefix item whose group needs several items (more sequences than one item's
// columns): its K/V loads are cached, so the group's other items, listed next to it,
// find the shared blocks in L2.
constexpr int kSharedTask = 1 << 30;
// A shared-prefix item that also computes every member's own tokens (after the prefix):
// its units are the prefix's, then each member's, and its rows are complete at the end.
constexpr int kFusedTask = 1 << 28;
constexpr int kTaskIndex = kFusedTask - 1;
// Units (16 tokens) of a fused item at most: the prefix and its members' own tokens.
constexpr int kFusedMaxUnits = 192;
// Parts a fused group's work is cut into at most (each part a workgroup of its own).
constexpr int kFusedMaxParts = 4;

// Context length of sequence b, clamped to what its table can address (longer
// values break the caller's contract; clamping keeps every access in bounds).
__device__ __forceinline__ int context_len(const Params& P, int b) { return min(max(P.ctx[b], 0), P.Lmax); }

// An item as the partition kernels use it.  `ok` is false for anything a plan pass
// cannot have written (a workspace without a preceding plan pass): such items do
// nothing, so every access stays inside the buffers.
struct Item {
  bool ok, prefix, shared, fused;
  int idx;   // sequence, or offset in the members list
  int tok0, ntok, p;
  int nm;    // sequences whose rows the item computes
  int np;    // partial count of an ordinary item's rows
  int parts; // a fused item: the parts of its group's work (it computes part p)
};
__device__ __forceinline__ Item decode_item(const Params& P, const int4 t, int unit, int cols_per_seq) {
  Item it;
  it.prefix = (t.x & kPrefixTask) != 0;
  it.shared = (t.x & kSharedTask) != 0;
  it.fused = it.prefix && (t.x & kFusedTask) != 0;
  it.idx = t.x & kTaskIndex;
  it.tok0 = t.y;
  it.ntok = t.z;
  it.p = t.w & 0xffff;
  const int hi = (t.w >> 16) & 0x7fff;
  it.nm = it.prefix ? (hi & 0xff) : 1;
  it.parts = it.prefix ? (hi >> 8) : 0;
  it.np = it.prefix ? 0 : hi;
  it.ok = t.x >= 0 && it.tok0 >= 0 && it.ntok >= 0 && it.tok0 + it.ntok <= P.Lmax && it.tok0 % unit == 0 &&
          it.p < P.Pmax && it.nm >= 1 && it.idx + it.nm <= P.N &&
          (it.prefix ? (it.nm * cols_per_seq <= 16 && it.ntok > 0) : (it.np >= 1 && it.np <= P.Pmax)) &&
          (it.fused ? (it.parts >= 1 && it.parts <= kFusedMaxParts && it.p < it.parts) : it.parts == 0);
  return it;
}

// ---------------------------------------------------------------------------------
// Plan kernel (one workgroup).  It finds sequences that share their leading blocks,
// picks this launch's partition size, and lists every work item, longest first so
// that the short tail items of a skewed batch run last.
//
// Shared prefixes.  Sequences whose first physical block is the same (forked samples,
// beams, requests on one cached prompt) form a group, inside aligned windows of
// kGroupWin sequences.  The group's shared prefix is the run of leading table entries
// that is equal in every member's row, cut to blocks that every member fills (found by
// comparing the rows entry by entry, so any table contents give the right result).
// When it holds at least kMinSharedTokens tokens, its attention is computed once for
// the group: a shared-prefix item puts the query heads of up to 16 / G members side by
// side as the columns of the MFMA products, so each prefix block is read once per item
// instead of once per member.  Each member's own tokens (after the prefix) are
// ordinary items.  A member's partials are those of the prefix partitions followed by
// those of its own partitions.  Only the MFMA kernels (16-bit pools, G <= 8) take
// shared-prefix items.  A group whose prefix fits one partition and whose members' own
// tokens are short is fused: one item per column set computes the prefix and every
// member's own tokens (masking each own unit to its member's columns), cut into parts
// when the batch has few such items (fused_parts); a member's partials are then one per
// part.
//
// Size: 2048 tokens unless the batch is too small to hide its longest 2048-token item
// (choose_partition_log2): fewer, longer partitions save each workgroup's fixed start
// and end, but a batch that cannot fill the chip ends when its longest item does.
//
// Order: items are bucketed into 64 classes by their number of tokens (classes of
// PT/64 tokens; full partitions first; an empty sequence gets one item in class 1,
// which writes its zero output).  Only the order within a class and which members an
// item of a large group takes depend on timing; no result depends on either (each
// column of a product, each row's partials and their merge order are fixed).
// ---------------------------------------------------------------------------------
// Sequences with more full partitions than this have their items written by the whole
// workgroup instead of one thread.
constexpr int kPlanSerialMax = 32;
constexpr int kPlanCoopMax = 256;
constexpr int kPlanClasses = 64;
constexpr int kGroupWin = 512;     // sequences are grouped within aligned windows of this many
constexpr int kGroupHash = 1024;   // hash slots for a window's first blocks (at most half used)
constexpr int kGroupWinWords = (65536 / kGroupWin + 31) / 32;  // one bit per window: it has groups
constexpr int kMinSharedTokens = 256;  // shortest prefix given shared-prefix items
static_assert((kGroupHash & (kGroupHash - 1)) == 0 && kGroupHash >= 2 * kGroupWin, "hash size");

// Entry j of sequence b's table, any format (only read below the sequence's length).
__device__ __forceinline__ int table_entry(const Params& P, int b, int j) {
  if (P.dir) {
    const int leaf = P.dir[static_cast<int64_t>(b) * (P.W / P.leaf_e) + j / P.leaf_e];
    return static_cast<const int*>(P.tables)[static_cast<int64_t>(leaf) * P.leaf_e + j % P.leaf_e];
  }
  if (P.tab_bytes == 2) return static_cast<const uint16_t*>(P.tables)[static_cast<int64_t>(b) * P.W + j];
  return static_cast<const int*>(P.tables)[static_cast<int64_t>(b) * P.W + j];
}

// Group rows are compared in segments of one entry per lane of a wave (64 consecutive
// entries, so each load instruction reads neighbouring words); a wave keeps kCmpBatch
// segments in flight.
constexpr int kCmpSeg = 64;
constexpr int kCmpBatch = 24;

// Entry j of row b in one table format, without branches (so that a batch of such loads
// is issued back to back): 0 = int32 rows, 1 = uint16 rows, 2 = two-level.
template <int F>
__device__ __forceinline__ int table_entry_fmt(const Params& P, int b, int j) {
  if constexpr (F == 2) {
    const int leaf = P.dir[static_cast<int64_t>(b) * (P.W / P.leaf_e) + j / P.leaf_e];
    return static_cast<const int*>(P.tables)[static_cast<int64_t>(leaf) * P.leaf_e + j % P.leaf_e];
  } else if constexpr (F == 1) {
    return static_cast<const uint16_t*>(P.tables)[static_cast<int64_t>(b) * P.W + j];
  } else {
    return static_cast<const int*>(P.tables)[static_cast<int64_t>(b) * P.W + j];
  }
}

// One batch of row segments of a window.  Lane i < kCmpBatch holds segment i: its
// member's index k in the window's list, first entry j0 (-1: none), the two rows (the
// member's and its group's first member's) and the number of entries to compare.  Every
// lane compares entry j0 + lane of the two rows; the first differing entry of each
// segment lowers `mis` of its member.  Addresses come from lane reads, so the loads of
// the whole batch are issued back to back.
template <int F>
__device__ __forceinline__ void compare_segments(const Params& P, int rk, int rj, int ra, int rb, int rc, int* mis) {
  const int lane = threadIdx.x & 63;
  int ea[kCmpBatch], eb[kCmpBatch];
  unsigned in = 0;  // bit i: this lane's entry of segment i exists
  static_assert(kCmpBatch <= 32, "one bit per segment");
  // the entry this lane reads for segment i: its own if it exists, else one that does
  // (entry 0 of both rows always exists)
  auto entry = [&](int i) {
    const int j0 = __builtin_amdgcn_readlane(rj, i);
    return j0 < 0 ? 0 : min(j0 + lane, __builtin_amdgcn_readlane(rc, i) - 1);
  };
#pragma unroll
  for (int i = 0; i < kCmpBatch; ++i) {
    const int j0 = __builtin_amdgcn_readlane(rj, i);
    in |= static_cast<unsigned>(j0 >= 0 && j0 + lane < __builtin_amdgcn_readlane(rc, i)) << i;
    const int a = __builtin_amdgcn_readlane(ra, i);
    const int b = __builtin_amdgcn_readlane(rb, i);
    const int jj = entry(i);
    if constexpr (F == 2) {  // the leaves first, then their entries
      const int64_t dw = P.W / P.leaf_e;
      ea[i] = P.dir[a * dw + jj / P.leaf_e];
      eb[i] = P.dir[b * dw + jj / P.leaf_e];
    } else {
      ea[i] = table_entry_fmt<F>(P, a, jj);
      eb[i] = table_entry_fmt<F>(P, b, jj);
    }
  }
  if constexpr (F == 2) {
    const int* leaves = static_cast<const int*>(P.tables);
#pragma unroll
    for (int i = 0; i < kCmpBatch; ++i) {
      const int e = entry(i) % P.leaf_e;
      ea[i] = leaves[static_cast<int64_t>(ea[i]) * P.leaf_e + e];
      eb[i] = leaves[static_cast<int64_t>(eb[i]) * P.leaf_e + e];
    }
  }
#pragma unroll
  for (int i = 0; i < kCmpBatch; ++i) {
    const unsigned long long m = __ballot(((in >> i) & 1u) && ea[i] != eb[i]);
    if (m && lane == 0) atomicMin(&mis[__builtin_amdgcn_readlane(rk, i)], __builtin_amdgcn_readlane(rj, i) + __builtin_ctzll(m));
  }
}

// The hash slot of first block `key` (inserted if new), or -1 if the table is full.
__device__ __forceinline__ int hash_slot(int* hkey, int key) {
  int slot = static_cast<int>((static_cast<unsigned>(key) * 2654435761u) >> 22) & (kGroupHash - 1);
  for (int probe = 0; probe < kGroupHash; ++probe) {
    const int prev = atomicCAS(&hkey[slot], -1, key);
    if (prev == -1 || prev == key) return slot;
    slot = (slot + 1) & (kGroupHash - 1);
  }
  return -1;
}

// Class of an item of `n` tokens at partition size 2^lg: 1..64 (64: more than 63/64 of
// a partition, with the full partitions).
__device__ __forceinline__ int item_class(int n, int lg) {
  const int sh = lg - 6;
  return n > 0 ? (n + (1 << sh) - 1) >> sh : 1;
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int mask) {
  const unsigned lo = static_cast<unsigned>(__shfl_xor(static_cast<int>(static_cast<unsigned>(v)), mask, 64));
  const unsigned hi = static_cast<unsigned>(__shfl_xor(static_cast<int>(static_cast<unsigned>(v >> 32)), mask, 64));
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}

// A sequence's shared-prefix group as the plan records it (seq_grp): prefix tokens, the
// sequence's rank in the group, the group's size, its longest context, and the offset of
// its members in the members list (-1: no group).
struct Grp {
  int sp, rank, cnt, maxl, base;
};
__device__ __forceinline__ Grp unpack_grp(int4 r) {
  return Grp{r.x, r.y & 0xffff, static_cast<int>(static_cast<unsigned>(r.y) >> 16), r.z, r.w};
}
__device__ __forceinline__ int4 pack_grp(const Grp& g) { return make_int4(g.sp, g.rank | (g.cnt << 16), g.maxl, g.base); }
__device__ constexpr Grp kNoGroup = {0, 0, 1, 0, -1};

// Whether a group's items are fused at partition size 2^lg: the prefix fits one partition
// and, with the own tokens of an item's members (at most maxl - sp each), at most
// kFusedMaxUnits units.
__device__ __forceinline__ bool fused_group(const Params& P, const Grp& g, int lg) {
  if (!P.fuse_ok || g.base < 0 || g.sp > (1 << lg)) return false;
  const int per = min(P.cm, g.cnt);
  return (g.sp >> 4) + per * ((g.maxl - g.sp + 15) >> 4) <= kFusedMaxUnits;
}

// The items of a shared-prefix group's partition-sized pieces: item k of a run covers
// prefix partition p0 + k / ncs for the group's column set k % ncs.
__device__ __forceinline__ int4 prefix_task(const Params& P, const Grp& g, int ncs, int k, int p0, int lg, int ntok) {
  const int p = p0 + k / ncs;
  const int cs = k - (k / ncs) * ncs;
  const int nm = min(P.cm, g.cnt - cs * P.cm);
  const int flag = kPrefixTask | (ncs > 1 ? kSharedTask : 0);
  return make_int4((g.base + cs * P.cm) | flag, p << lg, ntok, p | (nm << 16));
}

// Part s of `parts` of a fused group's column set cs.
__device__ __forceinline__ int4 fused_task(const Params& P, const Grp& g, int ncs, int cs, int s, int parts) {
  const int nm = min(P.cm, g.cnt - cs * P.cm);
  const int flag = kPrefixTask | (ncs > 1 ? kSharedTask : 0) | kFusedTask;
  return make_int4((g.base + cs * P.cm) | flag, 0, g.sp, s | (nm << 16) | (parts << 24));
}

// Parts per fused item.  A batch of few groups gives few workgroups, each a long chain
// of dependent loads; cutting each group's work into parts (merged like partitions) runs
// it on more of the device.  Measured on forked batches of 1020-token prompts (4 samples,
// 8 KV heads, 768 resident slots): 4 parts ran 15-22% faster with 32 or 64 workgroups,
// 2 parts about even with 128, and any split slower from 256 workgroups (each part then
// pays a dependent partial store and merge while the device is already busy).  So: one
// part per three resident slots' worth of workgroups, at most four, and at least one
// prefix unit per wave and part.
__device__ __forceinline__ int fused_parts(const Params& P, int fused_sets, int prefix_units) {
#ifdef PKV_FUSED_PARTS
  const int want = PKV_FUSED_PARTS;
#else
  const int wg = max(fused_sets, 1) * P.Hkv * P.NHG;
  const int want = P.slots / (3 * wg);
#endif
  return max(1, min(min(want, kFusedMaxParts), min(P.Pmax, prefix_units / kWaves)));
}

// The class of one part of a fused column set: its share of the prefix plus min(cm,
// members) times the group's longest own tokens, at most a partition.
__device__ __forceinline__ int fused_class(const Params& P, const Grp& g, int lg, int parts) {
  const int size = g.sp + min(P.cm, g.cnt) * (g.maxl - g.sp);
  return item_class(min(1 << lg, (size + parts - 1) / parts), lg);
}

__device__ __forceinline__ void plan_body(const Params& P) {
  const int N = P.N;
  constexpr int NB = kPlanClasses;
  __shared__ int cnt[2][NB + 1];
  __shared__ int off[NB + 1];
  __shared__ int n_coop, s_lmax, s_nmem, s_any, n_scan, s_fsets[2];
  __shared__ unsigned long long s_tokens;
  // items written cooperatively: (first slot, count, sequence or group, kind) and the
  // group state of a shared-prefix run
  __shared__ int coop_s[kPlanCoopMax], coop_n[kPlanCoopMax], coop_b[kPlanCoopMax], coop_k[kPlanCoopMax];
  __shared__ int4 coop_g[kPlanCoopMax];
  __shared__ int hkey[kGroupHash], hlead[kGroupHash], hcnt[kGroupHash], hS[kGroupHash], hrank[kGroupHash],
      hbase[kGroupHash], hmaxl[kGroupHash];
  __shared__ int wslot[kGroupWin], wrank[kGroupWin], wscan[kGroupWin], wlead[kGroupWin], wcap[kGroupWin],
      wmis[kGroupWin], wpre[kGroupWin + 1];
  __shared__ unsigned win_any[kGroupWinWords];
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  const int lane = tid & 63;
  // the context length of this thread's first sequence, kept for the passes below (a
  // batch of at most blockDim sequences is then read once)
  const int L_first = tid < N ? context_len(P, tid) : 0;
  auto len_of = [&](int b) { return b == tid ? L_first : context_len(P, b); };
  // and its first table entry, read together with the length (plain tables only: a
  // two-level row is followed only for a sequence long enough to be grouped)
  const int fb_first = (tid < N && P.cm >= 2 && P.tables && !P.dir) ? table_entry(P, tid, 0) : -1;
  Grp g_first = kNoGroup;  // this thread's first sequence's group, once known
  if (tid <= NB) {
    cnt[0][tid] = 0;
    cnt[1][tid] = 0;
  }
  if (tid < kGroupWinWords) win_any[tid] = 0;
  if (tid == 0) {
    n_coop = 0;
    s_lmax = 0;
    s_tokens = 0;
    s_nmem = 0;
    s_fsets[0] = 0;
    s_fsets[1] = 0;
  }
  for (int i = tid; i < N * P.Hq; i += nt) P.done[i] = 0;
  __syncthreads();

  // ---- shared-prefix groups, window by window ----
  if (P.cm >= 2 && P.tables) {
    for (int w0 = 0; w0 < N; w0 += kGroupWin) {
      for (int i = tid; i < kGroupHash; i += nt) {
        hkey[i] = -1;
        hlead[i] = 0x7fffffff;
        hcnt[i] = 0;
        hS[i] = 0x7fffffff;
        hrank[i] = 0;
        hmaxl[i] = 0;
      }
      if (tid == 0) {
        n_scan = 0;
        s_any = 0;
      }
      __syncthreads();
      for (int i = tid; i < kGroupWin; i += nt) {
        const int b = w0 + i;
        int slot = -1;
        if (b < N && len_of(b) >= kMinSharedTokens) {
          const int fb = (b == tid && !P.dir) ? fb_first : table_entry(P, b, 0);
          slot = fb >= 0 ? hash_slot(hkey, fb) : -1;
          if (slot >= 0) {
            atomicMin(&hlead[slot], b);
            atomicAdd(&hcnt[slot], 1);
            atomicMax(&hmaxl[slot], len_of(b));
          }
        }
        wslot[i] = slot;
      }
      __syncthreads();
      for (int i = tid; i < kGroupWin; i += nt) {
        const int slot = wslot[i];
        if (slot >= 0 && hcnt[slot] >= 2) {
          const int b = w0 + i;
          s_any = 1;
          const int a = hlead[slot];
          if (a == b) {
            atomicMin(&hS[slot], context_len(P, b) / P.B);
          } else {
            const int k = atomicAdd(&n_scan, 1);
            wscan[k] = b;
            wlead[k] = a;
            wcap[k] = min(context_len(P, a), context_len(P, b)) / P.B;
            wmis[k] = wcap[k];
          }
        }
      }
      __syncthreads();
      if (s_any) {
        // every member's row against the group's first member's, in segments of kCmpSeg
        // entries: wpre holds each member's first segment in the window's segment list
        if (tid < 64) {
          constexpr int PER = kGroupWin / 64;
          int c[PER], sum = 0;
#pragma unroll
          for (int e = 0; e < PER; ++e) {
            const int k = tid * PER + e;
            c[e] = k < n_scan ? (wcap[k] + kCmpSeg - 1) / kCmpSeg : 0;
            sum += c[e];
          }
          int v = sum;
#pragma unroll
          for (int d = 1; d < 64; d <<= 1) {
            const int t = __shfl_up(v, d, 64);
            v += tid >= d ? t : 0;
          }
          int run = v - sum;
#pragma unroll
          for (int e = 0; e < PER; ++e) {
            wpre[tid * PER + e] = run;
            run += c[e];
          }
          if (tid == 63) wpre[kGroupWin] = v;
        }
        __syncthreads();
        const int total = wpre[kGroupWin];
        const int wave = tid >> 6;
        const int nwaves = nt >> 6;
        for (int u0 = wave * kCmpBatch; u0 < total; u0 += nwaves * kCmpBatch) {
          // lane i < kCmpBatch resolves segment u0 + i: its member k and first entry
          int rk = 0, rj = -1, ra = 0, rb = 0, rc = 1;  // (rj = -1: no segment)
          if (lane < kCmpBatch && u0 + lane < total) {
            const int u = u0 + lane;
            int lo = 0, hi = n_scan - 1;  // the member: the last k with wpre[k] <= u
            while (lo < hi) {
              const int mid = (lo + hi + 1) >> 1;
              if (wpre[mid] <= u) lo = mid;
              else hi = mid - 1;
            }
            rk = lo;
            rj = (u - wpre[lo]) * kCmpSeg;
            if (rj >= wmis[lo]) rj = -1;  // an earlier segment already differs
            ra = wlead[lo];
            rb = wscan[lo];
            rc = wcap[lo];
          }
          if (P.dir) compare_segments<2>(P, rk, rj, ra, rb, rc, wmis);
          else if (P.tab_bytes == 2) compare_segments<1>(P, rk, rj, ra, rb, rc, wmis);
          else compare_segments<0>(P, rk, rj, ra, rb, rc, wmis);
        }
        __syncthreads();
        for (int k = tid; k < n_scan; k += nt) atomicMin(&hS[wslot[wscan[k] - w0]], wmis[k]);
        __syncthreads();
        for (int i = tid; i < kGroupWin; i += nt) {
          const int slot = wslot[i];
          int rank = -1;
          if (slot >= 0 && hcnt[slot] >= 2 && hS[slot] * P.B >= kMinSharedTokens) {
            rank = atomicAdd(&hrank[slot], 1);
            if (hlead[slot] == w0 + i) hbase[slot] = atomicAdd(&s_nmem, hcnt[slot]);
          }
          wrank[i] = rank;
        }
        __syncthreads();
        for (int i = tid; i < kGroupWin && w0 + i < N; i += nt) {
          const int b = w0 + i;
          const int slot = wslot[i];
          const int rank = wrank[i];
          Grp g = kNoGroup;
          if (rank >= 0) {
            g = Grp{hS[slot] * P.B, rank, hcnt[slot], hmaxl[slot], hbase[slot]};
            P.members[g.base + rank] = b;
            P.member_own[g.base + rank] = len_of(b) - g.sp;
          }
          P.seq_grp[b] = pack_grp(g);
          if (b == tid) g_first = g;
        }
        if (tid == 0) win_any[(w0 / kGroupWin) >> 5] |= 1u << ((w0 / kGroupWin) & 31);
      }
      __syncthreads();
    }
  }
  auto group_of = [&](int b) {
    const int win = b / kGroupWin;
    if (b == tid && tid < kGroupWin) return g_first;  // (sequence tid was this thread's in window 0)
    return (win_any[win >> 5] >> (win & 31)) & 1u ? unpack_grp(P.seq_grp[b]) : kNoGroup;
  };

  // ---- item counts per class at both candidate sizes, total tokens, longest length ----
  const int lg_lo = P.force_log2 ? P.force_log2 : kLgPartMin;
  const int lg_hi = P.force_log2 ? P.force_log2 : kLgPartMax;
  unsigned long long tokens = 0;
  int lmax = 0;
  for (int b = tid; b < N; b += nt) {
    const int L = len_of(b);
    const Grp g = group_of(b);
    const int ncs = (g.base >= 0 && g.rank == 0) ? (g.cnt + P.cm - 1) / P.cm : 0;  // the group's item writer
    tokens += static_cast<unsigned long long>(L);  // the size rule counts every sequence's context (as on the host)
    lmax = max(lmax, L);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int lg = c ? lg_hi : lg_lo;
      const bool fz = fused_group(P, g, lg);
      const int own = fz ? 0 : L - g.sp;  // (a fused group's own tokens are in its items)
      const int full = own >> lg;
      const int rem = own - (full << lg);
      int nfull = full;
      if ((rem || L == 0) && !fz) atomicAdd(&cnt[c][item_class(rem, lg)], 1);
      if (ncs && fz) {
        atomicAdd(&s_fsets[c], ncs);  // (counted by class once the number of parts is known)
      } else if (ncs) {
        const int fp = g.sp >> lg;
        const int rp = g.sp - (fp << lg);
        nfull += fp * ncs;
        if (rp) atomicAdd(&cnt[c][item_class(rp, lg)], ncs);
      }
      if (nfull) atomicAdd(&cnt[c][NB], nfull);
    }
  }
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    tokens += shfl_xor_u64(tokens, d);
    lmax = max(lmax, __shfl_xor(lmax, d, 64));
  }
  if (lane == 0) {
    atomicAdd(&s_tokens, tokens);
    atomicMax(&s_lmax, lmax);
  }
  __syncthreads();
  const int lg = choose_partition_log2(s_tokens, s_lmax, P.Hkv * P.NHG, P.D, P.B, P.slots, P.force_log2);
  const int csel = lg == lg_lo ? 0 : 1;
  const int* ccnt = cnt[csel];
  // fused groups: each column set's work in `parts` items, counted by class
  const int fsets = s_fsets[csel];
  if (fsets) {
    for (int b = tid; b < N; b += nt) {
      const Grp g = group_of(b);
      if (g.base >= 0 && g.rank == 0 && fused_group(P, g, lg)) {
        const int parts = fused_parts(P, fsets, g.sp >> 4);
        atomicAdd(&cnt[csel][fused_class(P, g, lg, parts)], ((g.cnt + P.cm - 1) / P.cm) * parts);
      }
    }
    __syncthreads();
  }
  // exclusive offsets of the classes, longest first (class NB, then NB - 1, ...): one
  // wave scans them with lane shuffles, lane i holding class NB - i
  static_assert(NB <= 64, "one wave scans the classes");
  if (tid < 64) {
    const int k = NB - tid;
    const int c = k >= 1 ? ccnt[k] : 0;
    int v = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(v, d, 64);
      v += tid >= d ? t : 0;
    }
    if (k >= 1) off[k] = v - c;
    if (tid == 63) {
      P.counters[0] = v;
      P.counters[1] = lg;
    }
  }
  __syncthreads();

  // ---- the items ----
  const int PT = 1 << lg;
  for (int b = tid; b < N; b += nt) {
    const int L = len_of(b);
    const Grp g = group_of(b);
    const bool fz = fused_group(P, g, lg);
    const int parts = fz ? fused_parts(P, fsets, g.sp >> 4) : 1;
    const int npp = g.base >= 0 ? (g.sp + PT - 1) >> lg : 0;
    const int own = fz ? 0 : L - g.sp;
    const int full = own >> lg;
    const int rem = own - (full << lg);
    const int np = fz ? parts : L == 0 ? 1 : npp + full + (rem > 0);
    P.seq_np[b] = np;
    if (full) {
      const int st = atomicAdd(&off[NB], full);
      const int k = full > kPlanSerialMax ? atomicAdd(&n_coop, 1) : kPlanCoopMax;
      if (k < kPlanCoopMax) {
        coop_s[k] = st;
        coop_n[k] = full;
        coop_b[k] = b;
        coop_k[k] = 0;
        coop_g[k] = make_int4(g.sp, npp, np, 0);
      } else {
        for (int q = 0; q < full; ++q) P.tasks[st + q] = make_int4(b, g.sp + (q << lg), PT, (npp + q) | (np << 16));
      }
    }
    if ((rem || L == 0) && !fz) {
      const int pos = atomicAdd(&off[item_class(rem, lg)], 1);
      P.tasks[pos] = make_int4(b, g.sp + (full << lg), rem, (npp + full) | (np << 16));
    }
    if (g.base >= 0 && g.rank == 0 && fz) {  // the group's fused items: parts per column set
      const int ncs = (g.cnt + P.cm - 1) / P.cm;
      const int st = atomicAdd(&off[fused_class(P, g, lg, parts)], ncs * parts);
      for (int q = 0; q < ncs * parts; ++q) P.tasks[st + q] = fused_task(P, g, ncs, q / parts, q % parts, parts);
    } else if (g.base >= 0 && g.rank == 0) {  // the group's shared-prefix items
      const int ncs = (g.cnt + P.cm - 1) / P.cm;
      const int fp = g.sp >> lg;
      const int rp = g.sp - (fp << lg);
      if (fp) {
        const int n = fp * ncs;
        const int st = atomicAdd(&off[NB], n);
        const int k = n > kPlanSerialMax ? atomicAdd(&n_coop, 1) : kPlanCoopMax;
        if (k < kPlanCoopMax) {
          coop_s[k] = st;
          coop_n[k] = n;
          coop_b[k] = ncs;
          coop_k[k] = 1;
          coop_g[k] = pack_grp(g);
        } else {
          for (int q = 0; q < n; ++q) P.tasks[st + q] = prefix_task(P, g, ncs, q, 0, lg, PT);
        }
      }
      if (rp) {
        const int st = atomicAdd(&off[item_class(rp, lg)], ncs);
        for (int q = 0; q < ncs; ++q) P.tasks[st + q] = prefix_task(P, g, ncs, q, fp, lg, rp);
      }
    }
  }
  __syncthreads();
  const int nc = min(n_coop, kPlanCoopMax);
  for (int k = 0; k < nc; ++k) {
    const int4 g = coop_g[k];
    for (int q = tid; q < coop_n[k]; q += nt) {
      P.tasks[coop_s[k] + q] = coop_k[k] ? prefix_task(P, unpack_grp(g), coop_b[k], q, 0, lg, PT)
                                         : make_int4(coop_b[k], g.x + (q << lg), PT, (g.y + q) | (g.z << 16));
    }
  }
}

__global__ __launch_bounds__(1024) void attn_plan(Params P) { plan_body(P); }

// The step's KV write and the attention plan in one launch: workgroup 0 plans, the
// others write (the two touch disjoint memory; the partition pass that follows in
// stream order sees both).
#ifndef PKV_PREP_THREADS
#define PKV_PREP_THREADS 1024
#endif
constexpr int kPrepThreads = PKV_PREP_THREADS;
#ifndef PKV_WRITE_THREADS
#define PKV_WRITE_THREADS 256
#endif
constexpr int kWriteThreads = PKV_WRITE_THREADS;

template <int EB>
__global__ __launch_bounds__(kPrepThreads) void decode_prepare_kernel(Params P, WriteArgs wa) {
  if (blockIdx.x == 0) {
    plan_body(P);
    return;
  }
  if (threadIdx.x >= kWriteThreads) return;
  kv_write_one<EB>(wa, static_cast<int64_t>(blockIdx.x - 1) * kWriteThreads + threadIdx.x);
}

// Device-scope (relaxed) stores and loads of the partition partials: coherent across
// the XCDs' separate L2 caches without a cache write-back or invalidation.
__device__ __forceinline__ void store_device(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_device(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class T, int D>
__device__ __forceinline__ void zero_rows(const Params& P, int b, int hq0, int nrows) {
  typedef typename T::Bits Bits;
  Bits* o = reinterpret_cast<Bits*>(P.out) + (static_cast<int64_t>(b) * P.Hq + hq0) * D;
  for (int i = threadIdx.x; i < nrows * D; i += kThreads) o[i] = T::from_float(0.f);
}

// The output row of each column of an item and that row's partial count.
template <int C>
struct ColSmem {
  int64_t row[C];
  int np[C];
  int member[C];  // the sequence of each of the item's sequences (by member index)
  int last[C];    // this workgroup merges that member's rows
};

// Merge the four waves' (max, sum, output) in LDS; store each column's final row (a row
// of one partial) or its partial in slot p.
template <class T, int D, int C>
__device__ __forceinline__ void combine_and_store(const Params& P, const float (*s_m)[C], const float (*s_l)[C],
                                                  const float (*s_o)[C][D + 4], const ColSmem<C>& cs, int ncols,
                                                  int p) {
  typedef typename T::Bits Bits;
  for (int idx = threadIdx.x; idx < ncols * D; idx += kThreads) {
    const int g = idx / D;
    const int d = idx - g * D;
    float M = s_m[0][g];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][g]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(s_m[w][g] - M);
      num += f * s_o[w][g][d];
      den += f * s_l[w][g];
    }
    const int64_t row = cs.row[g];
    if (cs.np[g] == 1) {
      reinterpret_cast<Bits*>(P.out)[row * D + d] = T::from_float(num / den);
    } else {
      // partials are read by whichever workgroup merges the row, possibly on another
      // XCD: device-scope stores write through to the coherent level
      const int64_t pr = row * P.Pmax + p;
      store_device(&P.ws_o[pr * D + d], num / den);
      if (d == 0) {
        store_device(&P.ws_ml[2 * pr], M);
        store_device(&P.ws_ml[2 * pr + 1], den);
      }
    }
  }
}

// Runs load/compute over this wave's units w, w+NW, w+2*NW, ... with three register
// buffers: while unit i is computed, units i+1 and i+2 are in flight.  Loads in the
// steady-state loop are unconditional, so each compute waits only for its own data.
// The caller has already issued the loads of the first unit into A.
template <int NW, class Buf, class Load, class Compute>
__device__ __forceinline__ void pipeline3(int w, int nunits, Buf& A, Load&& load, Compute&& compute) {
  const int n = nunits > w ? (nunits - w + NW - 1) / NW : 0;
  Buf B, C;
  if (n > 1) load(w + NW, B);
  int i = 0;
  for (; i + 4 < n; i += 3) {
    const int u = w + i * NW;
    load(u + 2 * NW, C);
    compute(u, A);
    load(u + 3 * NW, A);
    compute(u + NW, B);
    load(u + 4 * NW, B);
    compute(u + 2 * NW, C);
  }
  const int r = n - i;
  const int u = w + i * NW;
  if (r == 4) {
    load(u + 2 * NW, C);
    compute(u, A);
    load(u + 3 * NW, A);
    compute(u + NW, B);
    compute(u + 2 * NW, C);
    compute(u + 3 * NW, A);
  } else if (r == 3) {
    load(u + 2 * NW, C);
    compute(u, A);
    compute(u + NW, B);
    compute(u + 2 * NW, C);
  } else if (r == 2) {
    compute(u, A);
    compute(u + NW, B);
  } else if (r == 1) {
    compute(u, A);
  }
}

#ifndef PKV_STAGES
#define PKV_STAGES 2
#endif
template <int NW, class Buf, class Load, class Compute>
__device__ __forceinline__ void pipeline(int w, int nunits, Buf& first, Load&& load, Compute&& compute) {
  if constexpr (PKV_STAGES == 3) {
    pipeline3<NW, Buf>(w, nunits, first, load, compute);
  } else {
    pipeline2<NW, Buf>(w, nunits, first, load, compute);
  }
}

// Loads of K/V tiles: every byte is read once per decode step, so they are issued
// non-temporal (streamed through the caches without displacing the block tables,
// queries and partial results that are reused).
template <class V>
__device__ __forceinline__ V load_stream(const char* p) {
#ifdef PKV_CACHED_LOADS
  return *reinterpret_cast<const V*>(p);
#else
  return __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
#endif
}

// K/V tile loads of a workgroup whose sequence shares its first blocks with its
// neighbours (a task flagged by the plan) are cached loads instead: the group's other
// workgroups, listed next to it, read the same shared blocks from L2.  They are buffer
// loads from a resource over the tile (base: the tile's scalar address), so they stay
// distinct instructions from the streaming global loads on the other side of the
// workgroup-uniform branch (two loads that differ only in their cache hint would be
// merged into one plain load).
using Streamed = std::false_type;
using Cached = std::true_type;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* tile) {
  // raw (stride 0) resource; 0x00020000 is the gfx9 word-3 format for untyped access
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(tile), static_cast<short>(0), 0x7fffffff, 0x00020000);
}
template <class V>
__device__ __forceinline__ V load_cached(__amdgpu_buffer_rsrc_t r, int off) {
  static_assert(sizeof(V) == 16 || sizeof(V) == 8, "8- or 16-byte K/V fragments");
  if constexpr (sizeof(V) == 16) return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  else return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
// The same through a per-lane pointer (no tile base to build a resource from): plain
// loads when cached.
template <class V, class Temporal>
__device__ __forceinline__ V load_kv(const char* p) {
  if constexpr (Temporal::value) return *reinterpret_cast<const V*>(p);
  else return load_stream<V>(p);
}

// Rows split into at most this many partitions are merged inside the partition
// kernel by their last finisher; longer rows (long contexts) are merged by a separate
// kernel that spreads each row over a whole workgroup.
#ifndef PKV_FUSE_MAX_PARTS
#define PKV_FUSE_MAX_PARTS 32
#endif
constexpr int kFuseMaxParts = PKV_FUSE_MAX_PARTS;

// The query fragments of the MFMA path are kept in LDS (re-read per unit), which
// lowers register use enough for three waves per SIMD.
#ifndef PKV_Q_IN_REGS
#define PKV_Q_IN_LDS 1
#endif

// A running max is only raised (and the accumulators rescaled) when a new score
// exceeds it by more than this many log2 units; until then probabilities are taken
// against the stale max and stay below 2^kRescaleLog2 (no overflow in fp32/bf16/fp16).
constexpr float kRescaleLog2 = 8.f;

// ---------------------------------------------------------------------------------
// Log-sum-exp merge of the partition partials of one (sequence, query head) row, by
// the calling workgroup: M = max_p m_p, w_p = exp2(m_p - M) * l_p,
// out = sum_p w_p * o_p / sum_p w_p.
// ---------------------------------------------------------------------------------
template <int D>
struct MergeSmem {
  static constexpr int NCOL = D / 4;
  static constexpr int NG = kThreads / NCOL;
  float red[kWaves];
  float w[kThreads];  // weights of one chunk of kThreads partials
  f32x4 acc[NG][NCOL];
};

// Partials whose loads one thread of the merge keeps in flight together.
constexpr int kMergeUnroll = 8;

// (the partials were stored by an earlier kernel: plain loads)
template <class T, int D>
__device__ __forceinline__ void merge_row(const Params& P, int64_t row, int np, MergeSmem<D>& sm) {
  typedef typename T::Bits Bits;
  constexpr int NCOL = MergeSmem<D>::NCOL;
  constexpr int NG = MergeSmem<D>::NG;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const float* ml = P.ws_ml + row * P.Pmax * 2;
  const float* po = P.ws_o + row * P.Pmax * D;

  const int col = tid % NCOL;
  const int grp = tid / NCOL;
  // this thread's first partials (they do not depend on the max: their loads go out
  // with the (max, sum) loads) and its (max, sum) of the first chunk
  f32x4 v0[kMergeUnroll];
  {
    const int n0 = min(np, kThreads);
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const int j = min(grp + u * NG, n0 - 1);
      v0[u] = *reinterpret_cast<const f32x4*>(po + static_cast<int64_t>(j) * D + col * 4);
    }
  }
  float2 ml0 = make_float2(kNegInf, 0.f);
  if (tid < np) ml0 = *reinterpret_cast<const float2*>(&ml[2 * tid]);
  float mx = ml0.x;
  for (int i = tid + kThreads; i < np; i += kThreads) mx = fmaxf(mx, ml[2 * i]);
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) mx = fmaxf(mx, shfl_xor(mx, k));
  if (lane == 0) sm.red[w] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(sm.red[0], sm.red[1]), fmaxf(sm.red[2], sm.red[3]));
  __syncthreads();

  // chunks of kThreads partials: each thread's weight into LDS, then every thread adds
  // its partials (p = grp, grp + NG, ... in order), all of its loads issued together
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int c0 = 0; c0 < np; c0 += kThreads) {
    const int i = c0 + tid;
    float wi = 0.f;
    if (i < np) {
      const float2 v = c0 == 0 ? ml0 : *reinterpret_cast<const float2*>(&ml[2 * i]);
      wi = fast_exp2(v.x - M) * v.y;
    }
    den += wi;
    sm.w[tid] = wi;
    __syncthreads();
    const int n = min(np - c0, kThreads);
    int j0 = grp;
    if (c0 == 0) {  // the batch loaded up front
#pragma unroll
      for (int u = 0; u < kMergeUnroll; ++u) {
        if (j0 + u * NG < n) acc += sm.w[j0 + u * NG] * v0[u];
      }
      j0 += NG * kMergeUnroll;
    }
    for (; j0 < n; j0 += NG * kMergeUnroll) {
      f32x4 v[kMergeUnroll];
#pragma unroll
      for (int u = 0; u < kMergeUnroll; ++u) {
        const int j = min(j0 + u * NG, n - 1);  // (an existing partial; its weight is not used)
        v[u] = *reinterpret_cast<const f32x4*>(po + static_cast<int64_t>(c0 + j) * D + col * 4);
      }
#pragma unroll
      for (int u = 0; u < kMergeUnroll; ++u) {
        if (j0 + u * NG < n) acc += sm.w[j0 + u * NG] * v[u];
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) den += shfl_xor(den, k);
  if (lane == 0) sm.red[w] = den;
  __syncthreads();
  const float DEN = (sm.red[0] + sm.red[1]) + (sm.red[2] + sm.red[3]);

  sm.acc[grp][col] = acc;
  __syncthreads();
  if (tid < NCOL) {
    f32x4 sum = sm.acc[0][tid];
#pragma unroll
    for (int g = 1; g < NG; ++g) sum += sm.acc[g][tid];
    Bits* o = reinterpret_cast<Bits*>(P.out) + row * D + tid * 4;
    const float inv = 1.f / DEN;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = T::from_float(sum[e] * inv);
  }
  __syncthreads();
}

// (max, sum) of partial i of a row as one 8-byte device-scope load (the pair's two
// stores have completed before the row's count reaches its last partition).
__device__ __forceinline__ float2 load_ml(const float* ml, int i) {
  const unsigned long long v = __hip_atomic_load(
      reinterpret_cast<unsigned long long*>(const_cast<float*>(ml) + 2 * i), __ATOMIC_RELAXED,
      __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float(static_cast<unsigned>(v)), __uint_as_float(static_cast<unsigned>(v >> 32)));
}

// Merge of the rows row0 .. row0 + nrows - 1 (each of np <= kFuseMaxParts partials,
// stored by workgroups of the running kernel) by the calling workgroup, one thread per
// output element: M = max_p m_p, w_p = exp2(m_p - M) * l_p, out = sum_p w_p o_p / sum_p w_p,
// summed in partition order.  No barrier: each element is independent.  The loads of
// up to kMergeBatch partials are issued together (one round trip for short rows).
constexpr int kMergeBatch = 8;
template <class T, int D>
__device__ __forceinline__ void merge_rows_fused(const Params& P, int64_t row0, int nrows, int np) {
  typedef typename T::Bits Bits;
  for (int idx = threadIdx.x; idx < nrows * D; idx += kThreads) {
    const int g = idx / D;
    const int d = idx - g * D;
    const int64_t row = row0 + g;
    const float* ml = P.ws_ml + row * P.Pmax * 2;
    const float* po = P.ws_o + row * P.Pmax * D + d;
    float2 v[kMergeBatch];
    float o[kMergeBatch];
    float M = kNegInf;
    if (np > kMergeBatch) {
      for (int i0 = 0; i0 < np; i0 += kMergeBatch) {
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) v[k] = load_ml(ml, min(i0 + k, np - 1));
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) M = fmaxf(M, v[k].x);
      }
    }
    float num = 0.f, den = 0.f;
    for (int i0 = 0; i0 < np; i0 += kMergeBatch) {
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) {
        const int i = min(i0 + k, np - 1);
        v[k] = load_ml(ml, i);
        o[k] = load_device(&po[static_cast<int64_t>(i) * D]);
      }
      if (np <= kMergeBatch) {
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) M = fmaxf(M, v[k].x);
      }
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) {
        if (i0 + k < np) {
          const float w = fast_exp2(v[k].x - M) * v[k].y;
          num = fmaf(w, o[k], num);
          den += w;
        }
      }
    }
    reinterpret_cast<Bits*>(P.out)[row * D + d] = T::from_float(num / den);
  }
}

// After a partition's partials are stored: the workgroup that finishes a row's last
// partition (device-scope counter, zeroed by the plan pass) merges its query heads.
// Every thread waits until its device-scope partial stores have completed before the
// workgroup's count is added, so the merging workgroup, whose device-scope loads are
// issued after it has read the final count, sees every partition's partials.
//
// This ordering is the hardware's, not the language memory model's: the partials are
// relaxed agent-scope atomic stores (on gfx950 they write through the XCD's L2 to the
// coherent level, sc1), `s_waitcnt 0` holds the thread until they have completed, and
// the counter add and the merging loads are relaxed too.  A release add paired with an
// acquire load would be the portable form, but an agent-scope release writes back the
// whole L2 of the XCD: a __threadfence() version of this protocol was measured 5.5x
// slower.  The signal fences keep the compiler from moving the stores past the wait.
// An item covers `nm` sequences' rows hq0 .. hq0 + nrows - 1 (member i's partial count
// at cs.np[i * nrows]); each sequence's counter is advanced once per item.
template <class T, int D, int C>
__device__ __forceinline__ void finish_rows(const Params& P, ColSmem<C>& cs, int nm, int hq0, int nrows) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);  // all of this thread's memory operations have completed
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x < nm) {
    const int i = threadIdx.x;
    const int np = cs.np[i * nrows];
    cs.last[i] = np > 1 && np <= kFuseMaxParts &&
                 atomicAdd(&P.done[static_cast<int64_t>(cs.member[i]) * P.Hq + hq0], 1) == np - 1;
  }
  __syncthreads();
  for (int i = 0; i < nm; ++i) {
    if (cs.last[i]) merge_rows_fused<T, D>(P, static_cast<int64_t>(cs.member[i]) * P.Hq + hq0, nrows, cs.np[i * nrows]);
  }
}

// Columns of the MFMA kernels' products: lane m (of every 16-lane row) is column m,
// query head hq0 + m % gcur of the item's sequence m / gcur (an ordinary item has one
// sequence; a shared-prefix item up to 16 / gcur).  Lanes 0..15 record each column's
// output row and partial count, and each sequence's id, in LDS for the epilogue.
struct Cols {
  bool hv;           // lane's column is used
  int64_t qrow;      // query row of the lane's column (a used row for unused columns)
  bool need_finish;  // some covered sequence's rows are merged in this kernel
};
template <int C>
__device__ __forceinline__ Cols setup_columns(const Params& P, const Item& it, int hq0, int gcur, ColSmem<C>& cs) {
  const int m = threadIdx.x & 15;
  const int mi = m / gcur;
  Cols c;
  c.hv = mi < it.nm;
  int member = it.prefix ? P.members[it.idx + (c.hv ? mi : 0)] : it.idx;
  member = min(max(member, 0), P.N - 1);  // (a plan pass writes sequence ids only)
  const int np = min(max(it.prefix ? P.seq_np[member] : it.np, 1), P.Pmax);
  c.qrow = static_cast<int64_t>(member) * P.Hq + hq0 + (m - mi * gcur);
  if (threadIdx.x < 16) {
    cs.row[m] = c.qrow;
    cs.np[m] = np;
    if (c.hv && m == mi * gcur) cs.member[mi] = member;
  }
  c.need_finish = __builtin_amdgcn_ballot_w64(c.hv && np > 1 && np <= kFuseMaxParts) != 0;
  return c;
}

// ---------------------------------------------------------------------------------
// MFMA partition kernel: bf16/fp16 pools, 1..16 query heads per workgroup.
// grid = (num_kv_heads * head_groups, max_partitions, num_seqs)
// ---------------------------------------------------------------------------------
#ifndef PKV_MFMA_WAVES_PER_EU
#define PKV_MFMA_WAVES_PER_EU 1
#endif
template <class T, int D, int B, int GMAX, class Tab>
__global__ __launch_bounds__(kThreads, PKV_MFMA_WAVES_PER_EU) void attn_partition_mfma(Params P) {
  constexpr int EB = T::kBytes;
  static_assert(EB == 2, "MFMA path is for 16-bit pools");
  constexpr int KI = D / 32;   // 16x16x32 steps over head_dim
  constexpr int NC = D / 16;   // 16x16x16 products per unit (16 d each)
  constexpr int SUB = B / 16;  // 16-token units per block
  constexpr int BPP_MAX = kPTMax / B;  // table entries of the largest partition
  constexpr int64_t TILE = static_cast<int64_t>(B) * D * EB;
  struct Buf {
    u32x4 k[KI];
    u32x2 v[NC];
  };

  constexpr int C = 16;  // columns of the products
  constexpr int TABN = BPP_MAX > kFusedMaxUnits ? BPP_MAX : kFusedMaxUnits;
  __shared__ int s_tab[TABN];
  // fused items: per unit, its valid tokens | (1 + the member whose own tokens it holds) << 8,
  // and each wave's units in the order it takes them
  __shared__ int s_uinfo[kFusedMaxUnits];
  __shared__ int s_wlist[kWaves][kFusedMaxUnits];
  __shared__ float s_m[kWaves][C];
  __shared__ float s_l[kWaves][C];
  __shared__ float s_o[kWaves][C][D + 4];
  __shared__ ColSmem<C> s_cols;

  const int HY = P.Hkv * P.NHG;
  const int t = blockIdx.x / HY;
  const int hy = blockIdx.x - t * HY;
  if (t >= P.counters[0]) return;
  const int kvh = hy / P.NHG;
  const int hg = hy - kvh * P.NHG;
  const int hq0 = kvh * P.G + hg * 16;
  const int gcur = min(16, P.G - hg * 16);
  const Item it = decode_item(P, P.tasks[t], 16, gcur);
  if (!it.ok) return;  // only an item list left by the plan pass is valid
  // (fused items: one unit per block, at least one prefix unit per wave in every part)
  if (it.fused && (SUB != 1 || it.tok0 != 0 || it.ntok % 16 != 0 || it.parts * kWaves * 16 > it.ntok)) return;
  if (it.ntok == 0) {
    if (!it.prefix && it.p == 0) zero_rows<T, D>(P, it.idx, hq0, gcur);
    return;
  }
  const bool shared = it.shared;
  // whose table row the item reads (a shared-prefix item's sequences share these entries)
  const int lead = it.prefix ? min(max(P.members[it.idx], 0), P.N - 1) : it.idx;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane >> 4;
  const int m = lane & 15;
  const int ntok = it.ntok;
  const int pe = it.tok0 / B;  // the item's first table entry
  int nunits = (ntok + 15) >> 4;
  const int nblk = (ntok + B - 1) / B;
  // A fused item computes part it.p of its group's work: the prefix units [ps0, ps1) and
  // each member's own units [os0, os0 + f_units) (its share of them), listed locally as
  // the part's prefix units, then each member's own units; member k's start at local
  // index f_start (lane k of every wave holds a member's values).
  int f_own = 0, f_seq = 0, f_start = 0, f_units = 0, f_os0 = 0, f_off = 0;
  int ps0 = 0, ps1 = nblk;
  int wunits = nunits > w ? (nunits - w + kWaves - 1) / kWaves : 0;  // units this wave takes
  // A member's own unit j goes to wave (j + off) % kWaves, off a hash of the number of its
  // own units (and the prefix's unit u to u % kWaves), so every column meets its units in
  // the same waves and order whatever the other members; the hash spreads the members'
  // uneven last units over the waves instead of piling them on the first ones.
  auto wave_share = [](int n, int wv) { return n > wv ? (n - wv + kWaves - 1) / kWaves : 0; };
  auto wave_range = [&](int a, int b, int wv) { return wave_share(b, wv) - wave_share(a, wv); };
  if (it.fused) {
    const int S = it.parts, sp = it.p;
    ps0 = sp * nblk / S;
    ps1 = (sp + 1) * nblk / S;
    const int k = min(lane, it.nm - 1);
    f_seq = min(max(P.members[it.idx + k], 0), P.N - 1);
    f_own = min(max(P.member_own[it.idx + k], 0), P.Lmax - ntok);
    const int uk = (f_own + 15) >> 4;
    f_os0 = lane < it.nm ? sp * uk / S : 0;
    f_units = lane < it.nm ? (sp + 1) * uk / S - f_os0 : 0;
    f_off = static_cast<int>((static_cast<unsigned>(uk) * 2654435761u >> 7) & (kWaves - 1));
    // exclusive scan of the members' own units over lanes (nm <= 16)
    int v = f_units;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const int o2 = __shfl_up(v, d, 64);
      v += (lane & 63) >= d ? o2 : 0;
    }
    f_start = (ps1 - ps0) + v - f_units;
    const int total = __shfl(f_start + f_units, it.nm - 1, 64);
    int mine = wave_range(f_os0 + f_off, f_os0 + f_units + f_off, w);
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) mine += __shfl_xor(mine, d, 64);
    wunits = total > kFusedMaxUnits ? 0 : wave_range(ps0, ps1, w) + __shfl(mine, 0, 64);
    nunits = min(total, kFusedMaxUnits);
  }
  // the prefix entries staged from the lead's row: [ps0, ps1) of the item's blocks
  const int nloc = ps1 - ps0;

  // Preamble: issue every load first (the partition's table entries and the queries,
  // then the first unit's block id and its K/V), write LDS afterwards; vmcnt counts
  // in issue order, so the LDS writes wait only for the table and query loads.
  // (unconditional loads from clamped, always-valid addresses keep the waits exact; a
  // partition may span several two-level leaves, so each lane looks its entry up)
  const int tab_val = static_cast<int>(__builtin_nontemporal_load(
      table_row<Tab, kLeaf<B>>(P.tables, P.dir, lead, P.W, pe + ps0 + min(tid, nloc - 1))));
  const Cols col = setup_columns<C>(P, it, hq0, gcur, s_cols);
  const bool hv = col.hv;
  u32x4 qf[KI];
  {
    const char* qrow = P.q + col.qrow * D * EB;
#pragma unroll
    for (int ki = 0; ki < KI; ++ki) qf[ki] = load_stream<u32x4>(qrow + (4 * ki + r) * 16);
#pragma unroll
    for (int ki = 0; ki < KI; ++ki) qf[ki] = hv ? qf[ki] : u32x4{0u, 0u, 0u, 0u};
  }

  const char* kbase = P.kp + kvh * TILE;
  const char* vbase = P.vp + kvh * TILE;
  const int64_t bstride = static_cast<int64_t>(P.Hkv) * TILE;
  const int koff = (r * B + m) * 16;       // + ki * 4 * B * 16 + sub * 256
  const int voff = (m * B + 4 * r) * EB;   // + c * 16 * B * EB + sub * 16 * EB

  auto load_blk = [&](auto temporal, int u, int blk, Buf& f) {
    const int sub = u - (u / SUB) * SUB;
    const char* kt = kbase + blk * bstride + sub * 256;
    const char* vt = vbase + blk * bstride + sub * 16 * EB;
    if constexpr (decltype(temporal)::value) {
      const auto rk = tile_rsrc(kt);
      const auto rv = tile_rsrc(vt);
#pragma unroll
      for (int ki = 0; ki < KI; ++ki) f.k[ki] = load_cached<u32x4>(rk, koff + ki * 4 * B * 16);
#pragma unroll
      for (int c = 0; c < NC; ++c) f.v[c] = load_cached<u32x2>(rv, voff + c * 16 * B * EB);
    } else {
#pragma unroll
      for (int ki = 0; ki < KI; ++ki) f.k[ki] = load_stream<u32x4>(kt + koff + ki * 4 * B * 16);
#pragma unroll
      for (int c = 0; c < NC; ++c) f.v[c] = load_stream<u32x2>(vt + voff + c * 16 * B * EB);
    }
  };
  // `shared` is uniform over the workgroup: one scalar branch per unit picks the flavour
  // the unit of this wave's i-th step
  auto unit_of = [&](int i) { return it.fused ? __builtin_amdgcn_readfirstlane(s_wlist[w][i]) : w + kWaves * i; };
  auto load = [&](int i, Buf& f) {
    const int u = unit_of(i);
    const int blk = __builtin_amdgcn_readfirstlane(s_tab[u / SUB]);
    if (shared) load_blk(Cached{}, u, blk, f);
    else load_blk(Streamed{}, u, blk, f);
  };
  // a fused item's units after the prefix: thread u stages unit u (its block id and its
  // valid tokens | member), loaded before the first unit's K/V so the LDS writes wait
  // only for these table loads
  static_assert(kFusedMaxUnits <= kThreads, "one thread stages each unit of a fused item");
  int f_tab = 0, f_info = 16, f_wave = tid % kWaves, f_pos = tid / kWaves;
  if (it.fused) {
    int k = 0;
    for (int q = 1; q < it.nm; ++q) k = tid >= __shfl(f_start, q, 64) ? q : k;
    const int os0k = __shfl(f_os0, k, 64);
    const int j = os0k + tid - __shfl(f_start, k, 64);  // member k's own unit (of all its units)
    const int seq_k = __shfl(f_seq, k, 64);
    const int own_k = __shfl(f_own, k, 64);
    const int offk = __shfl(f_off, k, 64);
    // own unit j of member k: in wave (j + offk) % kWaves, after that wave's prefix units
    // of the part and its units of members 0 .. k-1 (the shuffles run in every lane)
    const int jw = (j + offk) % kWaves;
    int before = wave_range(ps0, ps1, jw) + wave_range(os0k + offk, j + offk, jw);
    for (int q = 0; q < it.nm; ++q) {
      const int o0 = __shfl(f_os0, q, 64) + __shfl(f_off, q, 64);
      const int uq = __shfl(f_units, q, 64);
      before += q < k ? wave_range(o0, o0 + uq, jw) : 0;
    }
    if (tid >= nloc) {
      f_wave = jw;
      f_pos = before;
    } else {  // the part's prefix unit ps0 + tid
      f_wave = (ps0 + tid) % kWaves;
      f_pos = wave_range(ps0, ps0 + tid, f_wave);
    }
    if (tid >= nloc && tid < nunits) {
      f_tab = static_cast<int>(*table_row<Tab, kLeaf<B>>(P.tables, P.dir, seq_k, P.W, nblk + j));
      f_info = min(16, own_k - 16 * j) | ((k + 1) << 8);
    }
  }
  // the wave's first unit takes its block id straight from the table (a scalar load);
  // a wave without units loads unit 0 (unused) so the load stays unconditional
  Buf first;
  {
    // (a fused part's wave w starts with its prefix unit ps0 + u0, the first one in wave w)
    const int u0 = it.fused ? (w - ps0 % kWaves + kWaves) % kWaves : w < nunits ? w : 0;
    const int blk = static_cast<int>(*table_row<Tab, kLeaf<B>>(P.tables, P.dir, lead, P.W, pe + ps0 + u0 / SUB));
    if (shared) load_blk(Cached{}, u0, blk, first);
    else load_blk(Streamed{}, u0, blk, first);
  }
  PKV_FENCE();
  if (tid < nloc) s_tab[tid] = tab_val;
  if (it.fused && tid < nunits) {
    if (tid >= nloc) s_tab[tid] = f_tab;
    s_uinfo[tid] = f_info;
    s_wlist[f_wave][f_pos] = tid;
  }
#ifdef PKV_Q_IN_LDS
  // query fragments live in LDS (lane-major, conflict-free) and are re-read per unit
  __shared__ u32x4 s_q[KI][64];
  if (w == 0) {
#pragma unroll
    for (int ki = 0; ki < KI; ++ki) s_q[ki][lane] = qf[ki];
  }
#endif
  __syncthreads();

  const int mcol = m / gcur;  // the member of this lane's column
  float m_run = kNegInf;
  float l_part = 0.f;
  f32x4 o[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int i, Buf& f) {
    const int u = unit_of(i);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ki = 0; ki < KI; ++ki) {
#ifdef PKV_Q_IN_LDS
      acc = T::mfma_k32(f.k[ki], s_q[ki][lane], acc);
#else
      acc = T::mfma_k32(f.k[ki], qf[ki], acc);
#endif
    }
    float s0 = acc[0] * P.scale_log2, s1 = acc[1] * P.scale_log2;
    float s2 = acc[2] * P.scale_log2, s3 = acc[3] * P.scale_log2;
    // valid tokens of the unit; a fused item's member unit also masks the other members' columns
    int valid = ntok - 16 * u;
    int seg = 0;
    if (it.fused) {
      const int info = __builtin_amdgcn_readfirstlane(s_uinfo[u]);
      valid = info & 0xff;
      seg = info >> 8;
    }
    if (valid < 16 || seg) {
      const int t0 = 4 * r;
      const bool colok = seg == 0 || mcol == seg - 1;
      s0 = (colok && t0 + 0 < valid) ? s0 : kNegInf;
      s1 = (colok && t0 + 1 < valid) ? s1 : kNegInf;
      s2 = (colok && t0 + 2 < valid) ? s2 : kNegInf;
      s3 = (colok && t0 + 3 < valid) ? s3 : kNegInf;
      const u32 mlo = (t0 + 0 < valid ? 0x0000ffffu : 0u) | (t0 + 1 < valid ? 0xffff0000u : 0u);
      const u32 mhi = (t0 + 2 < valid ? 0x0000ffffu : 0u) | (t0 + 3 < valid ? 0xffff0000u : 0u);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        f.v[c][0] &= mlo;
        f.v[c][1] &= mhi;
      }
    }
    // This lane's max over its scores; a column's four lanes are combined only when one
    // of them is above the threshold (the column's max then is too: the same decisions
    // and values as combining them on every unit).  Each column (lane m of every row)
    // decides its own rescale, so no column's result depends on the other columns.
    float mx = fmaxf(fmaxf(s0, s1), fmaxf(s2, s3));
    if (wave_any(mx > m_run + kRescaleLog2)) {
      mx = max_xor32(max_xor16(mx));
      const bool raise = mx > m_run + kRescaleLog2;
      const float alpha = raise ? fast_exp2(m_run - mx) : 1.f;
      l_part *= alpha;
#pragma unroll
      for (int c = 0; c < NC; ++c) o[c] *= alpha;
      m_run = raise ? mx : m_run;
    }
    const u32 p01 = T::pack2(fast_exp2(s0 - m_run), fast_exp2(s1 - m_run));
    const u32 p23 = T::pack2(fast_exp2(s2 - m_run), fast_exp2(s3 - m_run));
    l_part += (T::lo(p01) + T::hi(p01)) + (T::lo(p23) + T::hi(p23));
    const u32x2 pb = {p01, p23};
#pragma unroll
    for (int c = 0; c < NC; ++c) o[c] = T::mfma_k16(f.v[c], pb, o[c]);
  };

  pipeline2s(0, 1, wunits, first, load, compute);

  float l = sum_xor16(l_part);
  l = sum_xor32(l);
  if (hv) {
    if (r == 0) {
      s_m[w][m] = m_run;
      s_l[w][m] = l;
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int j = 0; j < 4; ++j) s_o[w][m][16 * c + 4 * r + j] = o[c][j];
    }
  }
  __syncthreads();
  combine_and_store<T, D, C>(P, s_m, s_l, s_o, s_cols, it.nm * gcur, it.p);
  if (col.need_finish) finish_rows<T, D, C>(P, s_cols, it.nm, hq0, gcur);
}

// ---------------------------------------------------------------------------------
// MFMA partition kernel with 32-token units (bf16/fp16, 1..16 query heads): one unit
// is one 32-token block, or two consecutive 16-token blocks.  The scores of a unit are
// two 16x16x32 MFMA chains over D whose rows are the tokens tau_s(i) =
// 8*(i/4) + 4*s + i%4 (s = 0, 1), so that lane (r, m) ends up holding the scores of
// tokens 8r..8r+7; P.V is then one 16x16x32 MFMA per 16 d whose V^T fragment is 16
// contiguous bytes of a V row (each V load instruction reads 1 KiB contiguously at
// block 32, two 512-byte runs at block 16).
// grid = (items * num_kv_heads * head_groups)
// ---------------------------------------------------------------------------------
template <class T, int D, int B, int GMAX, class Tab>
__global__ __launch_bounds__(kThreads, PKV_MFMA_WAVES_PER_EU) void attn_partition_mfma32(Params P) {
  constexpr int EB = T::kBytes;
  static_assert(EB == 2, "MFMA path is for 16-bit pools");
  constexpr int KI = D / 32;   // 16x16x32 steps over head_dim per 16-token sub-tile
  constexpr int NC = D / 16;   // 16x16x32 P.V products per unit (16 d each)
  constexpr int BPU = 32 / B;  // blocks per unit
  constexpr int BPP_MAX = kPTMax / B;  // table entries of the largest partition
  constexpr int64_t TILE = static_cast<int64_t>(B) * D * EB;
  struct Buf {
    u32x4 k[2][KI];
    u32x4 v[NC];
  };

  constexpr int C = 16;  // columns of the products
  __shared__ int s_tab[BPP_MAX];
  __shared__ float s_m[kWaves][C];
  __shared__ float s_l[kWaves][C];
  __shared__ float s_o[kWaves][C][D + 4];
  __shared__ ColSmem<C> s_cols;
  __shared__ u32x4 s_q[KI][64];

  const int HY = P.Hkv * P.NHG;
  const int t = blockIdx.x / HY;
  const int hy = blockIdx.x - t * HY;
  if (t >= P.counters[0]) return;
  const int kvh = hy / P.NHG;
  const int hg = hy - kvh * P.NHG;
  const int hq0 = kvh * P.G + hg * 16;
  const int gcur = min(16, P.G - hg * 16);
  const Item it = decode_item(P, P.tasks[t], 32, gcur);
  if (!it.ok || it.fused) return;  // only an item list left by the plan pass is valid (no fused items here)
  if (it.ntok == 0) {
    if (!it.prefix && it.p == 0) zero_rows<T, D>(P, it.idx, hq0, gcur);
    return;
  }
  const bool shared = it.shared;
  // whose table row the item reads (a shared-prefix item's sequences share these entries)
  const int lead = it.prefix ? min(max(P.members[it.idx], 0), P.N - 1) : it.idx;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane >> 4;
  const int m = lane & 15;
  const int ntok = it.ntok;
  const int pe = it.tok0 / B;  // the item's first table entry
  const int nunits = (ntok + 31) >> 5;
  const int nblk = (ntok + B - 1) / B;

  // preamble: all loads first (table entries, queries, first unit), LDS writes after
  const int tab_val = static_cast<int>(__builtin_nontemporal_load(
      table_row<Tab, kLeaf<B>>(P.tables, P.dir, lead, P.W, pe + min(tid, nblk - 1))));
  const Cols col = setup_columns<C>(P, it, hq0, gcur, s_cols);
  const bool hv = col.hv;
  u32x4 qf[KI];
  {
    const char* qrow = P.q + col.qrow * D * EB;
#pragma unroll
    for (int ki = 0; ki < KI; ++ki) qf[ki] = load_stream<u32x4>(qrow + (4 * ki + r) * 16);
#pragma unroll
    for (int ki = 0; ki < KI; ++ki) qf[ki] = hv ? qf[ki] : u32x4{0u, 0u, 0u, 0u};
  }

  const char* kbase = P.kp + kvh * TILE;
  const char* vbase = P.vp + kvh * TILE;
  const int64_t bstride = static_cast<int64_t>(P.Hkv) * TILE;
  // lane geometry: K rows of sub-tile s are tokens tau_s(m); V lanes read tokens 8r..8r+7
  const int tau0 = 8 * (m >> 2) + (m & 3);  // tau_s(m) = tau0 + 4 s, in 0..31
  int koff[2];
  int voff;
  bool k_second;  // (block 16) this lane's K rows are in the unit's second block
  bool v_second;
  if constexpr (BPU == 2) {
    k_second = m >= 8;
    v_second = r >= 2;
    koff[0] = (r * B + (tau0 & 15)) * 16;        // + ki * 4 * B * 16
    koff[1] = (r * B + ((tau0 + 4) & 15)) * 16;
    voff = (m * B + 8 * (r & 1)) * EB;           // + c * 16 * B * EB
  } else {
    k_second = false;
    v_second = false;
    koff[0] = (r * B + tau0) * 16;
    koff[1] = (r * B + tau0 + 4) * 16;
    voff = (m * B + 8 * r) * EB;
  }

  auto load_blk = [&](auto temporal, int blk0, int blk1, Buf& f) {
    // cached buffer loads need one tile base per wave: units of one 32-token block
    constexpr bool kBuf = decltype(temporal)::value && BPU == 1;
    using Tp = std::integral_constant<bool, decltype(temporal)::value && !kBuf>;
    const char* k0 = kbase + blk0 * bstride;
    const char* v0 = vbase + blk0 * bstride;
    const char* kt = k0;
    const char* vt = v0;
    if constexpr (BPU == 2) {
      const char* k1 = kbase + blk1 * bstride;
      const char* v1 = vbase + blk1 * bstride;
      kt = k_second ? k1 : k0;
      vt = v_second ? v1 : v0;
    }
    if constexpr (kBuf) {
      const auto rk = tile_rsrc(kt);
      const auto rv = tile_rsrc(vt);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int ki = 0; ki < KI; ++ki) f.k[s][ki] = load_cached<u32x4>(rk, koff[s] + ki * 4 * B * 16);
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) f.v[c] = load_cached<u32x4>(rv, voff + c * 16 * B * EB);
    } else {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int ki = 0; ki < KI; ++ki) f.k[s][ki] = load_kv<u32x4, Tp>(kt + koff[s] + ki * 4 * B * 16);
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) f.v[c] = load_kv<u32x4, Tp>(vt + voff + c * 16 * B * EB);
    }
  };
  // `shared` is uniform over the workgroup: one scalar branch per unit picks the flavour
  auto load = [&](int u, Buf& f) {
    const int blk0 = __builtin_amdgcn_readfirstlane(s_tab[u * BPU]);
    const int blk1 = BPU == 2 ? __builtin_amdgcn_readfirstlane(s_tab[min(u * BPU + 1, nblk - 1)]) : blk0;
    if (shared) load_blk(Cached{}, blk0, blk1, f);
    else load_blk(Streamed{}, blk0, blk1, f);
  };
  Buf first;
  {
    const int u0 = w < nunits ? w : 0;
    // (the unit's entries lie in one leaf: leaves hold an even number of entries)
    const auto* e0 = table_row<Tab, kLeaf<B>>(P.tables, P.dir, lead, P.W, pe + u0 * BPU);
    const int blk0 = static_cast<int>(e0[0]);
    const int blk1 = BPU == 2 ? static_cast<int>(e0[u0 * BPU + 1 < nblk ? 1 : 0]) : blk0;
    if (shared) load_blk(Cached{}, blk0, blk1, first);
    else load_blk(Streamed{}, blk0, blk1, first);
  }
  PKV_FENCE();
  if (tid < nblk) s_tab[tid] = tab_val;
  if (w == 0) {
#pragma unroll
    for (int ki = 0; ki < KI; ++ki) s_q[ki][lane] = qf[ki];
  }
  __syncthreads();

  float m_run = kNegInf;
  float l_part = 0.f;
  f32x4 o[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int u, Buf& f) {
    f32x4 acc[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ki = 0; ki < KI; ++ki) acc[s] = T::mfma_k32(f.k[s][ki], s_q[ki][lane], acc[s]);
    }
    float sc[8];  // tokens 8r + e of the unit, e = 4 s + j
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int j = 0; j < 4; ++j) sc[4 * s + j] = acc[s][j] * P.scale_log2;
    }
    if (32 * u + 32 > ntok) {
      const int t0 = 32 * u + 8 * r;
#pragma unroll
      for (int e = 0; e < 8; ++e) sc[e] = (t0 + e < ntok) ? sc[e] : kNegInf;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const u32 msk = (t0 + 2 * k < ntok ? 0x0000ffffu : 0u) | (t0 + 2 * k + 1 < ntok ? 0xffff0000u : 0u);
#pragma unroll
        for (int c = 0; c < NC; ++c) f.v[c][k] &= msk;
      }
    }
    // (a column's lanes are combined only when a rescale may be due, as in the 16-token
    // kernel; each column decides its own rescale)
    float mx = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
    if (wave_any(mx > m_run + kRescaleLog2)) {
      mx = max_xor32(max_xor16(mx));
      const bool raise = mx > m_run + kRescaleLog2;
      const float alpha = raise ? fast_exp2(m_run - mx) : 1.f;
      l_part *= alpha;
#pragma unroll
      for (int c = 0; c < NC; ++c) o[c] *= alpha;
      m_run = raise ? mx : m_run;
    }
    u32x4 pb;
#pragma unroll
    for (int k = 0; k < 4; ++k) pb[k] = T::pack2(fast_exp2(sc[2 * k] - m_run), fast_exp2(sc[2 * k + 1] - m_run));
    l_part += ((T::lo(pb[0]) + T::hi(pb[0])) + (T::lo(pb[1]) + T::hi(pb[1]))) +
              ((T::lo(pb[2]) + T::hi(pb[2])) + (T::lo(pb[3]) + T::hi(pb[3])));
#pragma unroll
    for (int c = 0; c < NC; ++c) o[c] = T::mfma_k32(f.v[c], pb, o[c]);
  };

  pipeline<kWaves, Buf>(w, nunits, first, load, compute);

  float l = sum_xor16(l_part);
  l = sum_xor32(l);
  if (hv) {
    if (r == 0) {
      s_m[w][m] = m_run;
      s_l[w][m] = l;
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int j = 0; j < 4; ++j) s_o[w][m][16 * c + 4 * r + j] = o[c][j];
    }
  }
  __syncthreads();
  combine_and_store<T, D, C>(P, s_m, s_l, s_o, s_cols, it.nm * gcur, it.p);
  if (col.need_finish) finish_rows<T, D, C>(P, s_cols, it.nm, hq0, gcur);
}

// ---------------------------------------------------------------------------------
// Vector-ALU partition kernel: one query head per kv head (any pool type), or fp32
// pools with G query heads per kv head.  grid = (num_kv_heads, max_partitions, num_seqs)
// ---------------------------------------------------------------------------------
template <class T, int D, int B, int G, class Tab>
__global__ __launch_bounds__(kThreads, T::kBytes == 2 ? 4 : 1) void attn_partition_valu(Params P) {
  constexpr int EB = T::kBytes;
  constexpr int X = 16 / EB;
  constexpr int NCH = D / X;
  constexpr int KL = NCH / 4;  // K chunks per lane per unit: r, r+4, r+8, ...
  constexpr int NV = D / 16;   // V rows per lane per unit: m, m+16, ...
  constexpr int SUB = B / 16;
  constexpr int BPP_MAX = kPTMax / B;  // table entries of the largest partition
  constexpr int64_t TILE = static_cast<int64_t>(B) * D * EB;
  typedef typename std::conditional<EB == 2, u32x2, u32x4>::type VVec;  // 4 tokens of one V row
  struct Buf {
    u32x4 k[KL];
    VVec v[NV];
  };

  __shared__ int s_tab[BPP_MAX];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
  __shared__ float s_o[kWaves][G][D + 4];
  __shared__ ColSmem<G> s_cols;

  const int t = blockIdx.x / P.Hkv;
  const int kvh = blockIdx.x - t * P.Hkv;
  if (t >= P.counters[0]) return;
  const Item it = decode_item(P, P.tasks[t], 16, G);
  // (the plan gives this kernel ordinary items only)
  if (!it.ok || it.prefix) return;  // only an item list left by the plan pass is valid
  const int b = it.idx;
  const int hq0 = kvh * G;
  if (it.ntok == 0) {
    if (it.p == 0) zero_rows<T, D>(P, b, hq0, G);
    return;
  }
  const int np = it.np;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane >> 4;
  const int m = lane & 15;
  const int ntok = it.ntok;
  const int pe = it.tok0 / B;  // the item's first table entry
  const int nunits = (ntok + 15) >> 4;
  const int nblk = (ntok + B - 1) / B;

  // Preamble: issue every load first (table entries, queries, then the first unit's
  // block id and K/V), write LDS afterwards.
  // (unconditional: exact waits)
  const int tab_val = static_cast<int>(__builtin_nontemporal_load(
      table_row<Tab, kLeaf<B>>(P.tables, P.dir, b, P.W, pe + min(tid, nblk - 1))));

  // queries: lane keeps chunks r + 4i of every head (fp32 pools: pre-scaled floats)
  u32x4 qw[G][KL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const char* qrow = P.q + (static_cast<int64_t>(b) * P.Hq + hq0 + g) * D * EB;
#pragma unroll
    for (int i = 0; i < KL; ++i) qw[g][i] = load_stream<u32x4>(qrow + (r + 4 * i) * 16);
  }

  const char* kbase = P.kp + kvh * TILE;
  const char* vbase = P.vp + kvh * TILE;
  const int64_t bstride = static_cast<int64_t>(P.Hkv) * TILE;
  const int koff = (r * B + m) * 16;      // + i * 4 * B * 16 + sub * 256
  const int voff = (m * B + 4 * r) * EB;  // + c * 16 * B * EB + sub * 16 * EB

  auto load_blk = [&](int u, int blk, Buf& f) {
    const int sub = u - (u / SUB) * SUB;
    const char* kt = kbase + blk * bstride + sub * 256;
    const char* vt = vbase + blk * bstride + sub * 16 * EB;
#pragma unroll
    for (int i = 0; i < KL; ++i) f.k[i] = load_stream<u32x4>(kt + koff + i * 4 * B * 16);
#pragma unroll
    for (int c = 0; c < NV; ++c) f.v[c] = load_stream<VVec>(vt + voff + c * 16 * B * EB);
  };
  auto load = [&](int u, Buf& f) { load_blk(u, __builtin_amdgcn_readfirstlane(s_tab[u / SUB]), f); };
  // the wave's first unit takes its block id straight from the table (a scalar load);
  // a wave without units loads unit 0 (unused) so the load stays unconditional
  Buf first;
  {
    const int u0 = w < nunits ? w : 0;
    load_blk(u0, static_cast<int>(*table_row<Tab, kLeaf<B>>(P.tables, P.dir, b, P.W, pe + u0 / SUB)), first);
  }
  PKV_FENCE();
  if (tid < nblk) s_tab[tid] = tab_val;
  if constexpr (EB == 4) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int i = 0; i < KL; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) qw[g][i][e] = __float_as_uint(__uint_as_float(qw[g][i][e]) * P.scale_log2);
      }
    }
  }
  __syncthreads();

  float m_run[G], l_part[G], o[G][NV];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = kNegInf;
    l_part[g] = 0.f;
#pragma unroll
    for (int c = 0; c < NV; ++c) o[g][c] = 0.f;
  }
  const int src_row = (lane & 48) | (4 * r);  // lane holding token 4r of this row

  auto compute = [&](int u, Buf& f) {
    float s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < KL; ++i) {
        if constexpr (EB == 2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) part = T::dot2(f.k[i][e], qw[g][i][e], part);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) part = fmaf(__uint_as_float(f.k[i][e]), __uint_as_float(qw[g][i][e]), part);
        }
      }
      part = sum_xor16(part);
      part = sum_xor32(part);
      s[g] = (EB == 2) ? part * P.scale_log2 : part;
    }
    if (16 * u + 16 > ntok) {
      const bool valid = 16 * u + m < ntok;
#pragma unroll
      for (int g = 0; g < G; ++g) s[g] = valid ? s[g] : kNegInf;
      const int t0 = 16 * u + 4 * r;
#pragma unroll
      for (int c = 0; c < NV; ++c) {
        if constexpr (EB == 2) {
          const u32 mlo = (t0 + 0 < ntok ? 0x0000ffffu : 0u) | (t0 + 1 < ntok ? 0xffff0000u : 0u);
          const u32 mhi = (t0 + 2 < ntok ? 0x0000ffffu : 0u) | (t0 + 3 < ntok ? 0xffff0000u : 0u);
          f.v[c][0] &= mlo;
          f.v[c][1] &= mhi;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) f.v[c][e] = (t0 + e < ntok) ? f.v[c][e] : 0u;
        }
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      // (the row's max only when a lane's score may call for a rescale: the row's max
      // is above the threshold exactly when one of its lanes is)
      if (wave_any(s[g] > m_run[g] + kRescaleLog2)) {
        const float mn = fmaxf(m_run[g], row_max16(s[g]));
        const float alpha = fast_exp2(m_run[g] - mn);
        l_part[g] *= alpha;
#pragma unroll
        for (int c = 0; c < NV; ++c) o[g][c] *= alpha;
        m_run[g] = mn;
      }
      float pr = fast_exp2(s[g] - m_run[g]);
      if constexpr (EB == 2) {
        pr = T::lo(T::pack2(pr, 0.f));  // probabilities in the pool type, as the product uses them
        const float other = dpp<0xB1>(pr);  // lane ^ 1
        const u32 pw = (m & 1) ? T::pack2(other, pr) : T::pack2(pr, other);  // (p[2k], p[2k+1])
        const u32 pp0 = shfl_idx_u(pw, src_row);
        const u32 pp1 = shfl_idx_u(pw, src_row + 2);
#pragma unroll
        for (int c = 0; c < NV; ++c) {
          float acc = T::dot2(f.v[c][0], pp0, o[g][c]);
          o[g][c] = T::dot2(f.v[c][1], pp1, acc);
        }
      } else {
        float pt[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pt[e] = shfl_idx(pr, src_row + e);
#pragma unroll
        for (int c = 0; c < NV; ++c) {
          float acc = o[g][c];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = fmaf(pt[e], __uint_as_float(f.v[c][e]), acc);
          o[g][c] = acc;
        }
      }
      l_part[g] += pr;
    }
  };

  pipeline<kWaves, Buf>(w, nunits, first, load, compute);

#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float l = row_sum16(l_part[g]);
#pragma unroll
    for (int c = 0; c < NV; ++c) o[g][c] = sum_xor32(sum_xor16(o[g][c]));
    if (lane < 16) {
      if (m == 0) {
        s_m[w][g] = m_run[g];
        s_l[w][g] = l;
      }
#pragma unroll
      for (int c = 0; c < NV; ++c) s_o[w][g][16 * c + m] = o[g][c];
    }
  }
  if (tid < G) {
    s_cols.row[tid] = static_cast<int64_t>(b) * P.Hq + hq0 + tid;
    s_cols.np[tid] = np;
    if (tid == 0) s_cols.member[0] = b;
  }
  __syncthreads();
  combine_and_store<T, D, G>(P, s_m, s_l, s_o, s_cols, G, it.p);
  if (np > 1 && np <= kFuseMaxParts) finish_rows<T, D, G>(P, s_cols, 1, hq0, G);
}

// Merge kernel for rows of more than kFuseMaxParts partitions.  grid = (Hq, N)
template <class T, int D>
__global__ __launch_bounds__(kThreads) void attn_merge_long(Params P) {
  __shared__ MergeSmem<D> s_merge;
  const int hq = blockIdx.x;
  const int b = blockIdx.y;
  const int np = min(P.seq_np[b], P.Pmax);
  if (np <= kFuseMaxParts) return;
  merge_row<T, D>(P, static_cast<int64_t>(b) * P.Hq + hq, np, s_merge);
}

// Which MFMA kernel a block size uses: 32-token units or 16-token units.
#ifndef PKV_UNIT32_B16
#define PKV_UNIT32_B16 0
#endif
#ifndef PKV_UNIT32_B32
#define PKV_UNIT32_B32 1
#endif
template <int B>
constexpr bool kUnit32 = (B == 16) ? PKV_UNIT32_B16 != 0 : PKV_UNIT32_B32 != 0;

Params make_params(const AttnArgs& a) {
  Params P;
  P.q = static_cast<const char*>(a.q);
  P.kp = static_cast<const char*>(a.k_pool);
  P.vp = static_cast<const char*>(a.v_pool);
  P.out = static_cast<char*>(a.out);
  P.ws_o = a.ws_o;
  P.ws_ml = a.ws_ml;
  P.tables = a.block_tables;
  P.dir = a.table_dir;
  P.ctx = a.context_lens;
  P.tasks = reinterpret_cast<int4*>(a.tasks);
  P.counters = a.counters;
  P.done = a.done;
  P.seq_np = a.seq_np;
  P.seq_grp = reinterpret_cast<int4*>(a.seq_grp);
  P.members = a.members;
  P.B = a.block_size;
  P.N = a.num_seqs;
  P.Hq = a.num_q_heads;
  P.Hkv = a.num_kv_heads;
  P.G = a.num_q_heads / a.num_kv_heads;
  P.NHG = (P.G + 15) / 16;
  P.W = a.max_blocks_per_seq;
  P.Pmax = a.max_parts;
  P.Lmax = a.max_blocks_per_seq * a.block_size;
  P.D = a.head_dim;
  P.scale_log2 = a.scale * kLog2e;
  P.tab_bytes = a.table_bytes;
  P.leaf_e = PKV_LEAF_TOKENS / a.block_size;
  P.slots = a.slots;
  P.force_log2 = a.force_log2;
  // shared-prefix items need the MFMA kernels (16-bit pools, 1..8 query heads per kv
  // head, so that an item holds at least two sequences)
  P.cm = (a.dtype != PKV_F32 && P.G >= 1 && P.G <= 8) ? 16 / P.G : 0;
  P.fuse_ok = (P.cm >= 2 && a.block_size == 16 && !kUnit32<16>) ? 1 : 0;
  P.member_own = a.member_own;
  return P;
}


template <class T, int D, int B, class Tab>
int launch_partitions_t(const AttnArgs& a, hipStream_t s) {
  const Params P = make_params(a);
  const dim3 block(kThreads);
  const int64_t items = static_cast<int64_t>(a.num_seqs) * (a.grid_parts > 0 ? a.grid_parts : a.max_parts);
  // fp32 pools run on the vector ALU; 16-bit pools on the MFMA kernel, MHA (one query
  // head per KV head) included: its idle product columns then hold the query heads of
  // forked sequences that share a prefix.  Measured: a forked MHA batch (64 prompts x 4
  // samples) 0.707 -> 0.273 ms for the partition pass; a batch without shared prefixes
  // 1.8% slower than on the vector-ALU kernel (3 waves/SIMD against 4).
  if constexpr (T::kBytes == 4) {
    const dim3 grid(static_cast<unsigned>(items * a.num_kv_heads));
    switch (P.G) {
      case 1: hipLaunchKernelGGL((attn_partition_valu<T, D, B, 1, Tab>), grid, block, 0, s, P); break;
      case 2: hipLaunchKernelGGL((attn_partition_valu<T, D, B, 2, Tab>), grid, block, 0, s, P); break;
      case 4: hipLaunchKernelGGL((attn_partition_valu<T, D, B, 4, Tab>), grid, block, 0, s, P); break;
      default: return -1;
    }
  } else if constexpr (T::kBytes == 2) {
    const dim3 grid(static_cast<unsigned>(items * a.num_kv_heads * P.NHG));
    if (kUnit32<B>) {
      if (P.G <= 4) {
        hipLaunchKernelGGL((attn_partition_mfma32<T, D, B, 4, Tab>), grid, block, 0, s, P);
      } else if (P.G <= 8) {
        hipLaunchKernelGGL((attn_partition_mfma32<T, D, B, 8, Tab>), grid, block, 0, s, P);
      } else {
        hipLaunchKernelGGL((attn_partition_mfma32<T, D, B, 16, Tab>), grid, block, 0, s, P);
      }
    } else if (P.G <= 4) {
      hipLaunchKernelGGL((attn_partition_mfma<T, D, B, 4, Tab>), grid, block, 0, s, P);
    } else if (P.G <= 8) {
      hipLaunchKernelGGL((attn_partition_mfma<T, D, B, 8, Tab>), grid, block, 0, s, P);
    } else {
      hipLaunchKernelGGL((attn_partition_mfma<T, D, B, 16, Tab>), grid, block, 0, s, P);
    }
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_parts <= kFuseMaxParts) return static_cast<int>(e);
  hipLaunchKernelGGL((attn_merge_long<T, D>), dim3(a.num_q_heads, a.num_seqs), block, 0, s, P);
  return static_cast<int>(hipGetLastError());
}

template <class T, class Tab>
int launch_partitions_tab(const AttnArgs& a, hipStream_t s) {
  if (a.head_dim == 64)
    return a.block_size == 16 ? launch_partitions_t<T, 64, 16, Tab>(a, s) : launch_partitions_t<T, 64, 32, Tab>(a, s);
  return a.block_size == 16 ? launch_partitions_t<T, 128, 16, Tab>(a, s) : launch_partitions_t<T, 128, 32, Tab>(a, s);
}

template <class T>
int launch_partitions_d(const AttnArgs& a, hipStream_t s) {
  if (a.table_dir) return launch_partitions_tab<T, TwoLevel>(a, s);
  return a.table_bytes == 2 ? launch_partitions_tab<T, uint16_t>(a, s) : launch_partitions_tab<T, int>(a, s);
}

}  // namespace

bool attn_supported(int32_t dtype, int32_t head_dim, int32_t block_size, int32_t group) {
  if (head_dim != 64 && head_dim != 128) return false;
  if (block_size != 16 && block_size != 32) return false;
  if (group < 1) return false;
  if (dtype == PKV_F32) return group == 1 || group == 2 || group == 4;
  return dtype == PKV_F16 || dtype == PKV_BF16;
}

int launch_decode_prepare(const AttnArgs& a, const pkv_pool_desc& pool, void* k_pool, void* v_pool,
                          const void* k_new, const void* v_new, const int64_t* slots, int32_t num_tokens,
                          void* stream) {
  const int eb = elem_bytes(pool.dtype);
  const int64_t total = eb == 4 ? kv_write_items<4>(num_tokens, pool.num_kv_heads, pool.head_dim)
                                : kv_write_items<2>(num_tokens, pool.num_kv_heads, pool.head_dim);
  if (total > kMaxWriteItems) {  // very large writes: two launches
    const int rc = launch_attn_plan(a, stream);
    return rc ? rc : launch_kv_write(pool, k_pool, v_pool, k_new, v_new, slots, num_tokens, stream);
  }
  const Params P = make_params(a);
  WriteArgs wa;
  wa.k_pool = static_cast<char*>(k_pool);
  wa.v_pool = static_cast<char*>(v_pool);
  wa.k_new = static_cast<const char*>(k_new);
  wa.v_new = static_cast<const char*>(v_new);
  wa.slots = slots;
  wa.tokens = num_tokens;
  wa.total = total;
  wa.H = pool.num_kv_heads;
  wa.D = pool.head_dim;
  wa.B = pool.block_size;
  const unsigned grid = 1 + static_cast<unsigned>((total + kWriteThreads - 1) / kWriteThreads);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (eb == 4) {
    hipLaunchKernelGGL(decode_prepare_kernel<4>, dim3(grid), dim3(kPrepThreads), 0, s, P, wa);
  } else {
    hipLaunchKernelGGL(decode_prepare_kernel<2>, dim3(grid), dim3(kPrepThreads), 0, s, P, wa);
  }
  return static_cast<int>(hipGetLastError());
}

int launch_attn_plan(const AttnArgs& a, void* stream) {
  const Params P = make_params(a);
  hipLaunchKernelGGL(attn_plan, dim3(1), dim3(1024), 0, static_cast<hipStream_t>(stream), P);
  return static_cast<int>(hipGetLastError());
}

int launch_attn_partitions(const AttnArgs& a, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (a.dtype) {
    case PKV_F32: return launch_partitions_d<F32>(a, s);
    case PKV_F16: return launch_partitions_d<F16>(a, s);
    case PKV_BF16: return launch_partitions_d<BF16>(a, s);
    default: return -1;
  }
}

}  // namespace pkv
