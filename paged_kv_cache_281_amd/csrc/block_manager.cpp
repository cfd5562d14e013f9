// Host-side block manager: block tables, on-demand allocation, fork, copy-on-write.
//
// Pages: agentalpha.top "Q32：vLLM PagedAttention 原理", answer part 2 (fixed-size
// blocks handed out on demand; a per-request table from logical to physical block)
// and part 3 (shared blocks are copied only when a sharer writes); data.6616ai.com
// vLLM article, "PagedAttention：把虚拟内存搬进 KV Cache" (blocks requested one at a
// time as a request grows; refcounted prefix sharing); ohmygp.com interview post,
// "破局思路" (one slot per decoded token, a new block only when the current one is
// full; copy on write into a shared block).
//
// The free list is a ring buffer over all block ids: allocation pops from the
// front, release pushes to the back.  Tables are per-sequence vectors.
//
// Prefix caching (optional; data.6616ai.com "PagedAttention 之外": the KV blocks of
// a prefix shared across requests, such as a system prompt, are cached and reused):
// every full block of a prompt is keyed by FNV-1a 64 over the key of the block
// before it (0 for the first) and its token ids; a new prompt reuses the cached
// blocks of its longest cached prefix of full blocks, never the block holding its
// last token.  Its other full blocks are registered when allocated (unless the key
// is taken); partial tails and blocks filled by decoding are not cached.  A cached
// block whose count drops to zero joins an evictable list in release order;
// allocation takes the free list first, then evicts the least recently released.
#include <cstdint>
#include <cstring>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pkv.h"
#include "pkv_internal.h"

struct pkv_bm {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> ring;      // free list storage, capacity num_blocks
  int64_t head = 0;               // index of the next block to hand out
  int64_t count = 0;              // number of free blocks
  std::vector<int32_t> refcount;  // per physical block
  struct Seq {
    std::vector<int32_t> table;
    int32_t len = 0;
  };
  std::unordered_map<int32_t, Seq> seqs;

  // prefix cache
  bool prefix_cache = false;
  std::unordered_map<uint64_t, int32_t> cached;  // key -> block
  std::vector<char> has_key;                      // per block: registered in `cached`
  std::vector<uint64_t> key, parent_key;
  std::vector<std::vector<int32_t>> key_tokens;
  std::vector<int32_t> ev_prev, ev_next;          // evictable list (release order)
  int32_t ev_head = -1, ev_tail = -1;
  int64_t ev_count = 0;

  int64_t available() const { return count + ev_count; }

  void ev_push(int32_t b) {
    ev_prev[b] = ev_tail;
    ev_next[b] = -1;
    if (ev_tail >= 0) ev_next[ev_tail] = b; else ev_head = b;
    ev_tail = b;
    ++ev_count;
  }
  void ev_remove(int32_t b) {
    if (ev_prev[b] >= 0) ev_next[ev_prev[b]] = ev_next[b]; else ev_head = ev_next[b];
    if (ev_next[b] >= 0) ev_prev[ev_next[b]] = ev_prev[b]; else ev_tail = ev_prev[b];
    --ev_count;
  }

  // callers check available() first
  int32_t take() {
    int32_t b;
    if (count > 0) {
      b = ring[head];
      head = (head + 1) % num_blocks;
      --count;
    } else {
      b = ev_head;
      ev_remove(b);
      cached.erase(key[b]);
      has_key[b] = 0;
      key_tokens[b].clear();
    }
    refcount[b] = 1;
    return b;
  }
  void give_back(int32_t b) {
    ring[(head + count) % num_blocks] = b;
    ++count;
  }
  // a block whose count reached zero
  void release(int32_t b) {
    if (prefix_cache && has_key[b]) ev_push(b); else give_back(b);
  }
};

namespace {

int32_t bad(const char* msg) { return pkv::set_error(PKV_ERR_INVALID_ARG, msg); }

pkv_bm::Seq* find(pkv_bm* bm, int32_t seq) {
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? nullptr : &it->second;
}
const pkv_bm::Seq* find(const pkv_bm* bm, int32_t seq) {
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? nullptr : &it->second;
}

int64_t div_up(int64_t a, int64_t b) { return (a + b - 1) / b; }

// FNV-1a, 64-bit: for each byte, h ^= byte, then h *= 1099511628211 (mod 2^64).
uint64_t fnv1a64_bytes(const unsigned char* p, size_t n, uint64_t h) {
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= 1099511628211ULL;
  }
  return h;
}

// Key of a full block: FNV-1a 64 over the parent key (8 bytes, little-endian) and the
// block's token ids (4 bytes each, little-endian two's complement).
uint64_t block_key(uint64_t parent, const int32_t* tokens, int32_t n) {
  unsigned char buf[8];
  for (int i = 0; i < 8; ++i) buf[i] = static_cast<unsigned char>(parent >> (8 * i));
  uint64_t h = fnv1a64_bytes(buf, 8, 14695981039346656037ULL);
  for (int32_t t = 0; t < n; ++t) {
    const uint32_t u = static_cast<uint32_t>(tokens[t]);
    for (int i = 0; i < 4; ++i) buf[i] = static_cast<unsigned char>(u >> (8 * i));
    h = fnv1a64_bytes(buf, 4, h);
  }
  return h;
}

}  // namespace

extern "C" {

int32_t pkv_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order, pkv_bm** out) {
  if (!out || !free_order) return bad("pkv_bm_create: null pointer");
  if (num_blocks <= 0 || block_size <= 0) return bad("pkv_bm_create: num_blocks and block_size must be positive");
  std::vector<char> seen(num_blocks, 0);
  for (int32_t i = 0; i < num_blocks; ++i) {
    int32_t b = free_order[i];
    if (b < 0 || b >= num_blocks || seen[b]) return bad("pkv_bm_create: free_order is not a permutation");
    seen[b] = 1;
  }
  auto* bm = new pkv_bm;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->ring.assign(free_order, free_order + num_blocks);
  bm->head = 0;
  bm->count = num_blocks;
  bm->refcount.assign(num_blocks, 0);
  *out = bm;
  return PKV_OK;
}

void pkv_bm_destroy(pkv_bm* bm) { delete bm; }

int32_t pkv_bm_add_seq(pkv_bm* bm, int32_t seq, int32_t num_tokens) {
  if (!bm) return bad("pkv_bm_add_seq: null manager");
  if (seq < 0 || num_tokens < 0) return bad("pkv_bm_add_seq: negative sequence id or token count");
  if (find(bm, seq)) return bad("pkv_bm_add_seq: sequence already exists");
  int64_t need = div_up(num_tokens, bm->block_size);
  if (need > bm->available())
    return pkv::set_error(PKV_ERR_OUT_OF_BLOCKS, "pkv_bm_add_seq: not enough free blocks");
  pkv_bm::Seq s;
  s.table.reserve(need);
  for (int64_t i = 0; i < need; ++i) s.table.push_back(bm->take());
  s.len = num_tokens;
  bm->seqs.emplace(seq, std::move(s));
  return PKV_OK;
}

int32_t pkv_bm_fork(pkv_bm* bm, int32_t parent, int32_t child) {
  if (!bm) return bad("pkv_bm_fork: null manager");
  if (child < 0) return bad("pkv_bm_fork: negative sequence id");
  const pkv_bm::Seq* p = find(bm, parent);
  if (!p) return bad("pkv_bm_fork: unknown parent");
  if (find(bm, child)) return bad("pkv_bm_fork: child already exists");
  pkv_bm::Seq c = *p;
  for (int32_t b : c.table) ++bm->refcount[b];
  bm->seqs.emplace(child, std::move(c));
  return PKV_OK;
}

int32_t pkv_bm_append_slot(pkv_bm* bm, int32_t seq, int64_t* slot, int32_t* cow_src, int32_t* cow_dst) {
  if (!bm || !slot || !cow_src || !cow_dst) return bad("pkv_bm_append_slot: null pointer");
  pkv_bm::Seq* s = find(bm, seq);
  if (!s) return bad("pkv_bm_append_slot: unknown sequence");
  const int32_t B = bm->block_size;
  const int32_t pos = s->len;
  *cow_src = -1;
  *cow_dst = -1;
  if (pos % B == 0) {
    if (bm->available() == 0) return pkv::set_error(PKV_ERR_OUT_OF_BLOCKS, "pkv_bm_append_slot: no free block");
    s->table.push_back(bm->take());
  } else {
    int32_t tail = s->table.back();
    if (bm->refcount[tail] > 1) {
      if (bm->available() == 0) return pkv::set_error(PKV_ERR_OUT_OF_BLOCKS, "pkv_bm_append_slot: no free block");
      int32_t fresh = bm->take();
      --bm->refcount[tail];
      s->table.back() = fresh;
      *cow_src = tail;
      *cow_dst = fresh;
    }
  }
  *slot = static_cast<int64_t>(s->table[pos / B]) * B + pos % B;
  s->len = pos + 1;
  return PKV_OK;
}

int32_t pkv_bm_step(pkv_bm* bm, const int32_t* seqs, int32_t n, int64_t* slots_out, int64_t* pairs_out,
                    int32_t* num_pairs) {
  if (!bm || !num_pairs || (n > 0 && (!seqs || !slots_out || !pairs_out))) return bad("pkv_bm_step: null pointer");
  if (n < 0) return bad("pkv_bm_step: negative count");
  *num_pairs = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t src, dst;
    int32_t st = pkv_bm_append_slot(bm, seqs[i], &slots_out[i], &src, &dst);
    if (st != PKV_OK) return st;
    if (src >= 0) {
      pairs_out[2 * *num_pairs] = src;
      pairs_out[2 * *num_pairs + 1] = dst;
      ++*num_pairs;
    }
  }
  return PKV_OK;
}

int32_t pkv_bm_free_seq(pkv_bm* bm, int32_t seq) {
  if (!bm) return bad("pkv_bm_free_seq: null manager");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return bad("pkv_bm_free_seq: unknown sequence");
  for (int32_t b : it->second.table) {
    if (--bm->refcount[b] == 0) bm->release(b);
  }
  bm->seqs.erase(it);
  return PKV_OK;
}

int32_t pkv_bm_move_seqs(pkv_bm* src, pkv_bm* dst, const int32_t* seqs, int32_t n, int64_t* pairs_out,
                         int32_t cap, int32_t* num_pairs) {
  if (!src || !dst || (n > 0 && !seqs) || !num_pairs) return bad("pkv_bm_move_seqs: null pointer");
  if (src == dst) return bad("pkv_bm_move_seqs: source and destination are the same manager");
  if (n < 0 || cap < 0) return bad("pkv_bm_move_seqs: negative count");
  if (src->block_size != dst->block_size) return bad("pkv_bm_move_seqs: block sizes differ");
  // validate everything first: the call is all or nothing
  std::unordered_map<int32_t, int32_t> mapping;  // source block -> destination block
  int64_t distinct = 0;
  for (int32_t i = 0; i < n; ++i) {
    const pkv_bm::Seq* s = find(src, seqs[i]);
    if (!s) return bad("pkv_bm_move_seqs: unknown sequence");
    if (find(dst, seqs[i])) return bad("pkv_bm_move_seqs: sequence exists in the destination");
    for (int32_t j = 0; j < i; ++j)
      if (seqs[j] == seqs[i]) return bad("pkv_bm_move_seqs: duplicate sequence");
    for (int32_t b : s->table)
      if (mapping.emplace(b, -1).second) ++distinct;
  }
  if (distinct > dst->available())
    return pkv::set_error(PKV_ERR_OUT_OF_BLOCKS, "pkv_bm_move_seqs: destination has too few free blocks");
  if (distinct > cap) return bad("pkv_bm_move_seqs: pairs_out capacity too small");
  int32_t np = 0;
  for (int32_t i = 0; i < n; ++i) {
    const pkv_bm::Seq& s = src->seqs[seqs[i]];
    pkv_bm::Seq d;
    d.table.reserve(s.table.size());
    for (int32_t b : s.table) {
      int32_t& c = mapping[b];
      if (c >= 0) {
        ++dst->refcount[c];
      } else {
        c = dst->take();
        pairs_out[2 * np] = b;
        pairs_out[2 * np + 1] = c;
        ++np;
      }
      d.table.push_back(c);
    }
    d.len = s.len;
    dst->seqs.emplace(seqs[i], std::move(d));
  }
  for (int32_t i = 0; i < n; ++i) pkv_bm_free_seq(src, seqs[i]);
  *num_pairs = np;
  return PKV_OK;
}

int32_t pkv_bm_seq_len(const pkv_bm* bm, int32_t seq, int32_t* len) {
  if (!bm || !len) return bad("pkv_bm_seq_len: null pointer");
  const pkv_bm::Seq* s = find(bm, seq);
  if (!s) return bad("pkv_bm_seq_len: unknown sequence");
  *len = s->len;
  return PKV_OK;
}

int32_t pkv_bm_slots(const pkv_bm* bm, int32_t seq, int32_t pos0, int32_t count, int64_t* out) {
  if (!bm || (count > 0 && !out)) return bad("pkv_bm_slots: null pointer");
  const pkv_bm::Seq* s = find(bm, seq);
  if (!s) return bad("pkv_bm_slots: unknown sequence");
  if (pos0 < 0 || count < 0 || static_cast<int64_t>(pos0) + count > s->len)
    return bad("pkv_bm_slots: positions outside the sequence");
  const int32_t B = bm->block_size;
  for (int32_t i = 0; i < count; ++i) {
    int32_t pos = pos0 + i;
    out[i] = static_cast<int64_t>(s->table[pos / B]) * B + pos % B;
  }
  return PKV_OK;
}

int32_t pkv_bm_block_table(const pkv_bm* bm, int32_t seq, int32_t* out, int32_t cap, int32_t* n) {
  if (!bm || !n || (cap > 0 && !out)) return bad("pkv_bm_block_table: null pointer");
  const pkv_bm::Seq* s = find(bm, seq);
  if (!s) return bad("pkv_bm_block_table: unknown sequence");
  *n = static_cast<int32_t>(s->table.size());
  if (*n > cap) return bad("pkv_bm_block_table: capacity too small");
  if (*n) std::memcpy(out, s->table.data(), sizeof(int32_t) * *n);
  return PKV_OK;
}

int32_t pkv_bm_block_tables(const pkv_bm* bm, const int32_t* seqs, int32_t n, int32_t width, int32_t pad,
                            int32_t* out) {
  if (!bm || (n > 0 && (!seqs || !out))) return bad("pkv_bm_block_tables: null pointer");
  if (n < 0 || width < 0) return bad("pkv_bm_block_tables: negative size");
  for (int32_t i = 0; i < n; ++i) {
    const pkv_bm::Seq* s = find(bm, seqs[i]);
    if (!s) return bad("pkv_bm_block_tables: unknown sequence");
    if (static_cast<int64_t>(s->table.size()) > width) return bad("pkv_bm_block_tables: table wider than width");
  }
  for (int32_t i = 0; i < n; ++i) {
    const pkv_bm::Seq* s = find(bm, seqs[i]);
    int32_t* row = out + static_cast<int64_t>(i) * width;
    int32_t k = static_cast<int32_t>(s->table.size());
    if (k) std::memcpy(row, s->table.data(), sizeof(int32_t) * k);
    for (int32_t j = k; j < width; ++j) row[j] = pad;
  }
  return PKV_OK;
}

int32_t pkv_bm_block_tables16(const pkv_bm* bm, const int32_t* seqs, int32_t n, int32_t width, int32_t pad,
                              uint16_t* out) {
  if (!bm || (n > 0 && (!seqs || !out))) return bad("pkv_bm_block_tables16: null pointer");
  if (n < 0 || width < 0) return bad("pkv_bm_block_tables16: negative size");
  if (pad < 0 || pad > 65535) return bad("pkv_bm_block_tables16: pad does not fit 16 bits");
  for (int32_t i = 0; i < n; ++i) {
    const pkv_bm::Seq* s = find(bm, seqs[i]);
    if (!s) return bad("pkv_bm_block_tables16: unknown sequence");
    if (static_cast<int64_t>(s->table.size()) > width) return bad("pkv_bm_block_tables16: table wider than width");
    for (int32_t b : s->table)
      if (b > 65535) return bad("pkv_bm_block_tables16: block id does not fit 16 bits");
  }
  for (int32_t i = 0; i < n; ++i) {
    const pkv_bm::Seq* s = find(bm, seqs[i]);
    uint16_t* row = out + static_cast<int64_t>(i) * width;
    const int32_t k = static_cast<int32_t>(s->table.size());
    for (int32_t j = 0; j < k; ++j) row[j] = static_cast<uint16_t>(s->table[j]);
    for (int32_t j = k; j < width; ++j) row[j] = static_cast<uint16_t>(pad);
  }
  return PKV_OK;
}

int32_t pkv_bm_block_tables_2l(const pkv_bm* bm, const int32_t* seqs, int32_t n, int32_t dir_width, int32_t pad,
                               int32_t* dir_out, int32_t* leaves_out, int32_t leaf_cap, int32_t* num_leaves) {
  if (!bm || !num_leaves || (n > 0 && (!seqs || !dir_out))) return bad("pkv_bm_block_tables_2l: null pointer");
  if (n < 0 || dir_width <= 0 || leaf_cap < 0) return bad("pkv_bm_block_tables_2l: bad size");
  if (PKV_LEAF_TOKENS % bm->block_size != 0)
    return bad("pkv_bm_block_tables_2l: the block size does not divide a leaf");
  const int64_t E = PKV_LEAF_TOKENS / bm->block_size;
  int64_t total = n > 0 ? 1 : 0;  // the shared padding leaf
  for (int32_t i = 0; i < n; ++i) {
    const pkv_bm::Seq* s = find(bm, seqs[i]);
    if (!s) return bad("pkv_bm_block_tables_2l: unknown sequence");
    const int64_t k = (static_cast<int64_t>(s->table.size()) + E - 1) / E;
    if (k > dir_width) return bad("pkv_bm_block_tables_2l: table needs more than dir_width leaves");
    total += k;
  }
  if (total > 0x7fffffff) return bad("pkv_bm_block_tables_2l: too many leaves");
  *num_leaves = static_cast<int32_t>(total);
  if (!leaves_out) return PKV_OK;  // count only
  if (total > leaf_cap) return bad("pkv_bm_block_tables_2l: leaves do not fit leaf_cap");
  if (n == 0) return PKV_OK;
  const int32_t pad_leaf = static_cast<int32_t>(total - 1);
  int32_t next = 0;
  for (int32_t i = 0; i < n; ++i) {
    const pkv_bm::Seq* s = find(bm, seqs[i]);
    const int64_t nb = static_cast<int64_t>(s->table.size());
    int32_t* drow = dir_out + static_cast<int64_t>(i) * dir_width;
    for (int64_t j = 0; j < dir_width; ++j) {
      if (j * E >= nb) {
        drow[j] = pad_leaf;
        continue;
      }
      drow[j] = next;
      int32_t* leaf = leaves_out + static_cast<int64_t>(next) * E;
      for (int64_t e = 0; e < E; ++e) leaf[e] = j * E + e < nb ? s->table[j * E + e] : pad;
      ++next;
    }
  }
  int32_t* leaf = leaves_out + static_cast<int64_t>(pad_leaf) * E;
  for (int64_t e = 0; e < E; ++e) leaf[e] = pad;
  return PKV_OK;
}

int32_t pkv_bm_refcount(const pkv_bm* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->refcount[block];
}

int32_t pkv_bm_num_free(const pkv_bm* bm) { return bm ? static_cast<int32_t>(bm->available()) : -1; }

int32_t pkv_bm_num_cached(const pkv_bm* bm) { return bm ? static_cast<int32_t>(bm->cached.size()) : -1; }

int32_t pkv_bm_set_prefix_cache(pkv_bm* bm, int32_t enable) {
  if (!bm) return bad("pkv_bm_set_prefix_cache: null manager");
  if (!bm->seqs.empty() || !bm->cached.empty())
    return bad("pkv_bm_set_prefix_cache: only a manager without sequences or cached blocks can switch");
  bm->prefix_cache = enable != 0;
  const size_t n = static_cast<size_t>(bm->num_blocks);
  bm->has_key.assign(n, 0);
  bm->key.assign(n, 0);
  bm->parent_key.assign(n, 0);
  bm->key_tokens.assign(n, {});
  bm->ev_prev.assign(n, -1);
  bm->ev_next.assign(n, -1);
  bm->ev_head = bm->ev_tail = -1;
  bm->ev_count = 0;
  return PKV_OK;
}

int32_t pkv_bm_add_seq_tokens(pkv_bm* bm, int32_t seq, const int32_t* tokens, int32_t n, int32_t* cached_tokens) {
  if (!bm || (n > 0 && !tokens) || !cached_tokens) return bad("pkv_bm_add_seq_tokens: null pointer");
  if (seq < 0 || n < 0) return bad("pkv_bm_add_seq_tokens: negative sequence id or token count");
  if (find(bm, seq)) return bad("pkv_bm_add_seq_tokens: sequence already exists");
  if (!bm->prefix_cache) {
    const int32_t st = pkv_bm_add_seq(bm, seq, n);
    if (st == PKV_OK) *cached_tokens = 0;
    return st;
  }
  const int32_t B = bm->block_size;
  const int64_t nblk = div_up(n, B);
  const int32_t nfull = n / B;
  const int32_t lookup = (n > 0 ? n - 1 : 0) / B;  // full blocks entirely before the last token
  std::vector<uint64_t> keys(nfull), parents(nfull);
  std::vector<int32_t> hits;
  uint64_t parent = 0;
  for (int32_t i = 0; i < nfull; ++i) {
    const int32_t* t = tokens + static_cast<int64_t>(i) * B;
    const uint64_t k = block_key(parent, t, B);
    keys[i] = k;
    parents[i] = parent;
    if (i < lookup && static_cast<int32_t>(hits.size()) == i) {
      auto it = bm->cached.find(k);
      if (it != bm->cached.end()) {
        const int32_t b = it->second;
        if (bm->parent_key[b] == parent && std::memcmp(bm->key_tokens[b].data(), t, sizeof(int32_t) * B) == 0)
          hits.push_back(b);
      }
    }
    parent = k;
  }
  int64_t pinned_evictable = 0;
  for (int32_t b : hits)
    if (bm->refcount[b] == 0) ++pinned_evictable;
  if (nblk - static_cast<int64_t>(hits.size()) > bm->available() - pinned_evictable)
    return pkv::set_error(PKV_ERR_OUT_OF_BLOCKS, "pkv_bm_add_seq_tokens: not enough free blocks");
  for (int32_t b : hits) {
    if (bm->refcount[b] == 0) bm->ev_remove(b);
    ++bm->refcount[b];
  }
  pkv_bm::Seq s;
  s.table = hits;
  s.table.reserve(nblk);
  for (int64_t i = static_cast<int64_t>(hits.size()); i < nblk; ++i) {
    const int32_t b = bm->take();
    if (i < nfull && bm->cached.find(keys[i]) == bm->cached.end()) {
      bm->cached.emplace(keys[i], b);
      bm->has_key[b] = 1;
      bm->key[b] = keys[i];
      bm->parent_key[b] = parents[i];
      bm->key_tokens[b].assign(tokens + i * B, tokens + (i + 1) * B);
    }
    s.table.push_back(b);
  }
  s.len = n;
  bm->seqs.emplace(seq, std::move(s));
  *cached_tokens = static_cast<int32_t>(hits.size()) * B;
  return PKV_OK;
}

}  // extern "C"
