// Host block manager: free pool, per-block reference counts, block tables,
// fork (prefix sharing) and copy-on-write.
//
// What the pages fix ("PagedAttention" robocikowo.com, Komponenty and Jak
// działa; "PagedAttention et RadixAttention : parlons de KV Cache", section
// on PagedAttention as an operating system, steps 1-4): a per-sequence table
// maps logical blocks to physical ones; a manager hands blocks out of a free
// pool as sequences grow, one block at a time; sequences with a common
// prefix point at the same physical blocks, counted by reference, and a
// write into a shared block first duplicates it; a finished sequence gives
// its blocks back individually for immediate reuse ("PagedAttention —
// Gestion mémoire pour LLM à long contexte", Pourquoi c'est important).
//
// The pages leave the policy open; this manager is deterministic:
//   * the free pool is a stack (vector back = top); the caller's initial
//     order hands out element 0 first; released blocks are pushed on top;
//   * a write at length L allocates at block boundaries, and copies the
//     block holding slot L only if it is shared; the batch is walked in
//     call order;
//   * every call validates and counts what it needs before mutating, so an
//     error leaves the state unchanged.
//
// Prefix caching by chained block digests ("PagedAttention et RadixAttention
// : parlons de KV Cache", on vLLM's automatic prefix caching and on cache
// salting): a full block whose token ids are known gets
// SHA-256(parent digest || salt || token ids) and is registered under it; a
// cached admission walks a prompt's full blocks and shares each registered
// one until the first miss; the salt keeps tenants apart.  Policy:
//   * a block registers when it fills, if its ids and its parent's digest are
//     known and the digest is not registered yet (else it is a duplicate and
//     stays unregistered);
//   * a registered block released to refcount 0 keeps its digest and joins an
//     eviction list (oldest first); a released sequence adds its registered
//     blocks from the last to the first, so chains lose their deepest blocks
//     first;
//   * allocation pops the free stack, and takes (and unregisters) the oldest
//     evictable block only when the stack is empty; a cache hit takes an
//     evictable block off the list;
//   * a registered block is immutable: a write into one (possible after a
//     fork inside it) copies it first even for its only holder; a block
//     released that way joins the eviction list after the whole call, so no
//     copy of the call reads a block the same call hands out again.
//
// Swapping to host memory ("PagedAttention — Gestion mémoire pour LLM à long
// contexte", Mode d'échec and the glossary's Page eviction: when GPU memory
// runs out even with paging, pages go to CPU RAM and come back on demand):
// a host pool with its own free stack; swap-out gives each block of a
// sequence, in logical order, a fresh host block and then drops the GPU
// references as a free would; swap-in takes fresh GPU blocks (free stack,
// then eviction list) and releases the host blocks.  Both are atomic.
#include <algorithm>
#include <cstdint>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pkv_status.h"
#include "sha256.h"

struct pkv_block_manager {
  struct Seq {
    std::vector<int32_t> table;
    int32_t len = 0;
    // Prefix cache: salt, the known leading token ids (they stop being
    // recorded once an append comes without ids) and the chain digests of
    // the leading full blocks.
    uint64_t salt = 0;
    std::vector<int32_t> tokens;
    std::vector<pkv::Digest> digests;
    // Swapped out: the table is empty and host_table holds the host blocks.
    bool swapped = false;
    std::vector<int32_t> host_table;
    // Device mirrors (pkv_bm_stage_step), one per tracked device table: row
    // of that table this sequence was last written to (-1: none), entries
    // written there, and the lowest entry changed since (a copy-on-write
    // replacement).
    int32_t mirror_row[2] = {-1, -1};
    int32_t mirror_blocks[2] = {0, 0};
    int32_t dirty_from[2] = {INT32_MAX, INT32_MAX};
  };
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_stack;  // back() is handed out next
  std::vector<int32_t> refcount;
  int32_t num_shared = 0;  // blocks with refcount >= 2
  std::unordered_map<int64_t, Seq> seqs;
  // Prefix cache: digest registry, each block's digest, and the eviction
  // list of registered blocks at refcount 0 (a doubly linked list over block
  // ids, head = oldest).
  std::unordered_map<pkv::Digest, int32_t, pkv::DigestHash> cached;
  std::vector<pkv::Digest> block_digest;
  std::vector<uint8_t> registered;
  std::vector<int32_t> lru_prev, lru_next;
  int32_t lru_head = -1, lru_tail = -1, lru_size = 0;
  // Host swap pool.
  int32_t num_host_blocks = 0;
  std::vector<int32_t> host_free;  // back() is handed out next
  // The device tables the mirror state refers to (a caller may alternate two,
  // e.g. to stage one step while the previous one still reads the other),
  // with the sequence whose entries each row last received, and the call
  // count of their last use (the least recently used one is replaced).
  struct DeviceTable {
    const void* table = nullptr;
    int32_t width = 0;
    std::vector<int64_t> row_owner;
    uint64_t last_use = 0;
  };
  DeviceTable mirrors[2];
  uint64_t stage_calls = 0;
  // Scratch reused by pkv_bm_stage_step and pkv_bm_append_slots.
  std::vector<int32_t> scratch_slots, scratch_pairs, scratch_released;
};

namespace {

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int32_t check_handle(const pkv_block_manager* bm) {
  if (!bm) return pkv::fail(PKV_ERR_INVALID_ARG, "null block manager handle");
  return PKV_OK;
}

using BM = pkv_block_manager;

void lru_push_back(BM* bm, int32_t b) {
  bm->lru_prev[b] = bm->lru_tail;
  bm->lru_next[b] = -1;
  if (bm->lru_tail >= 0) bm->lru_next[bm->lru_tail] = b;
  else bm->lru_head = b;
  bm->lru_tail = b;
  ++bm->lru_size;
}

void lru_remove(BM* bm, int32_t b) {
  const int32_t p = bm->lru_prev[b], n = bm->lru_next[b];
  if (p >= 0) bm->lru_next[p] = n;
  else bm->lru_head = n;
  if (n >= 0) bm->lru_prev[n] = p;
  else bm->lru_tail = p;
  bm->lru_prev[b] = bm->lru_next[b] = -1;
  --bm->lru_size;
}

int64_t available(const BM* bm) { return static_cast<int64_t>(bm->free_stack.size()) + bm->lru_size; }

// A fresh block: the free stack first, else the oldest evictable block,
// whose digest is forgotten.  The caller has checked availability.
int32_t take_block(BM* bm) {
  if (!bm->free_stack.empty()) {
    const int32_t b = bm->free_stack.back();
    bm->free_stack.pop_back();
    return b;
  }
  const int32_t b = bm->lru_head;
  lru_remove(bm, b);
  bm->cached.erase(bm->block_digest[b]);
  bm->registered[b] = 0;
  return b;
}

// Block i of s has just filled: give it its chain digest and register it.
void complete_block(BM* bm, BM::Seq& s, int32_t i) {
  const int32_t bs = bm->block_size;
  if (static_cast<int64_t>(s.tokens.size()) < static_cast<int64_t>(i + 1) * bs ||
      static_cast<int32_t>(s.digests.size()) != i)
    return;
  const pkv::Digest parent = i ? s.digests[i - 1] : pkv::Digest{};
  const pkv::Digest d = pkv::block_digest(parent, s.salt, s.tokens.data() + static_cast<size_t>(i) * bs, bs);
  s.digests.push_back(d);
  const int32_t b = s.table[i];
  if (bm->cached.emplace(d, b).second) {
    bm->block_digest[b] = d;
    bm->registered[b] = 1;
  }
}

// Refcount changes that keep num_shared (blocks held at least twice) exact.
inline void ref_inc(BM* bm, int32_t b) {
  if (++bm->refcount[b] == 2) ++bm->num_shared;
}
inline int32_t ref_dec(BM* bm, int32_t b) {
  if (bm->refcount[b]-- == 2) --bm->num_shared;
  return bm->refcount[b];
}

// Drops one reference from each block of a table: blocks reaching zero go
// to the free stack in logical order, registered ones to the eviction list
// from the last to the first.
void release_table(BM* bm, const std::vector<int32_t>& t) {
  for (int32_t b : t) {
    if (ref_dec(bm, b) == 0 && !bm->registered[b]) bm->free_stack.push_back(b);
  }
  for (auto r = t.rbegin(); r != t.rend(); ++r) {
    if (bm->refcount[*r] == 0 && bm->registered[*r]) lru_push_back(bm, *r);
  }
}

int32_t check_on_gpu(const BM::Seq& s, int64_t id) {
  if (s.swapped) return pkv::fail(PKV_ERR_INVALID_ARG, "sequence %lld is swapped out", (long long)id);
  return PKV_OK;
}

// Registered blocks for the leading full blocks of a prompt, up to the first miss.
void match_prefix(const BM* bm, const int32_t* tokens, int32_t n, uint64_t salt, std::vector<int32_t>* blocks,
                  std::vector<pkv::Digest>* digests) {
  const int32_t bs = bm->block_size;
  pkv::Digest d{};
  for (int32_t i = 0; i < n / bs; ++i) {
    d = pkv::block_digest(d, salt, tokens + static_cast<size_t>(i) * bs, bs);
    auto it = bm->cached.find(d);
    if (it == bm->cached.end()) break;
    blocks->push_back(it->second);
    if (digests) digests->push_back(d);
  }
}

}  // namespace

extern "C" {

int32_t pkv_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* initial_free_order,
                      pkv_block_manager** out) {
  if (!out) return pkv::fail(PKV_ERR_INVALID_ARG, "out handle pointer is null");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "num_blocks (%d) and block_size (%d) must be positive", num_blocks,
                     block_size);
  if (static_cast<int64_t>(num_blocks) * block_size > INT32_MAX)
    return pkv::fail(PKV_ERR_INVALID_ARG, "num_blocks * block_size exceeds the int32 slot range");
  auto* bm = new (std::nothrow) pkv_block_manager();
  if (!bm) return pkv::fail(PKV_ERR_INVALID_ARG, "out of host memory");
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->refcount.assign(num_blocks, 0);
  bm->block_digest.resize(num_blocks);
  bm->registered.assign(num_blocks, 0);
  bm->lru_prev.assign(num_blocks, -1);
  bm->lru_next.assign(num_blocks, -1);
  bm->free_stack.resize(num_blocks);
  if (initial_free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = initial_free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete bm;
        return pkv::fail(PKV_ERR_INVALID_ARG, "initial_free_order is not a permutation (entry %d = %d)", i, b);
      }
      seen[b] = 1;
      bm->free_stack[num_blocks - 1 - i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) bm->free_stack[num_blocks - 1 - i] = i;
  }
  *out = bm;
  return pkv::ok();
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

int32_t pkv_bm_add_seq_cached(pkv_block_manager* bm, int64_t seq_id, const int32_t* tokens, int32_t n_tokens,
                              uint64_t salt, int32_t* n_cached_out) {
  if (int32_t e = check_handle(bm)) return e;
  if (bm->seqs.count(seq_id)) return pkv::fail(PKV_ERR_INVALID_ARG, "sequence %lld already exists", (long long)seq_id);
  if (n_tokens < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "n_tokens < 0");
  if (n_tokens > 0 && !tokens) return pkv::fail(PKV_ERR_INVALID_ARG, "tokens is null");
  pkv_block_manager::Seq s;
  match_prefix(bm, tokens, n_tokens, salt, &s.table, &s.digests);
  for (int32_t b : s.table) {
    if (bm->refcount[b] == 0) lru_remove(bm, b);
    ref_inc(bm, b);
  }
  s.len = static_cast<int32_t>(s.table.size()) * bm->block_size;
  s.salt = salt;
  if (s.len > 0) s.tokens.assign(tokens, tokens + s.len);
  const int32_t n = s.len;
  bm->seqs.emplace(seq_id, std::move(s));
  if (n_cached_out) *n_cached_out = n;
  return pkv::ok();
}

int32_t pkv_bm_add_seq(pkv_block_manager* bm, int64_t seq_id) {
  return pkv_bm_add_seq_cached(bm, seq_id, nullptr, 0, 0, nullptr);
}

int32_t pkv_bm_match_prefix(const pkv_block_manager* bm, const int32_t* tokens, int32_t n_tokens, uint64_t salt) {
  if (int32_t e = check_handle(bm)) return e;
  if (n_tokens < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "n_tokens < 0");
  if (n_tokens > 0 && !tokens) return pkv::fail(PKV_ERR_INVALID_ARG, "tokens is null");
  std::vector<int32_t> blocks;
  match_prefix(bm, tokens, n_tokens, salt, &blocks, nullptr);
  pkv::ok();
  return static_cast<int32_t>(blocks.size()) * bm->block_size;
}

int32_t pkv_block_digest(const uint8_t* parent, uint64_t salt, const int32_t* tokens, int32_t n_tokens,
                         uint8_t* out) {
  if (!out) return pkv::fail(PKV_ERR_INVALID_ARG, "out is null");
  if (n_tokens < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "n_tokens < 0");
  if (n_tokens > 0 && !tokens) return pkv::fail(PKV_ERR_INVALID_ARG, "tokens is null");
  pkv::Digest p{};
  if (parent) std::copy(parent, parent + 32, p.begin());
  const pkv::Digest d = pkv::block_digest(p, salt, tokens, n_tokens);
  std::copy(d.begin(), d.end(), out);
  return pkv::ok();
}

int32_t pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child, int32_t num_tokens) {
  if (int32_t e = check_handle(bm)) return e;
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return pkv::fail(PKV_ERR_UNKNOWN_SEQ, "unknown parent sequence %lld", (long long)parent);
  if (int32_t e = check_on_gpu(it->second, parent)) return e;
  if (bm->seqs.count(child)) return pkv::fail(PKV_ERR_INVALID_ARG, "sequence %lld already exists", (long long)child);
  if (num_tokens < 0 || num_tokens > it->second.len)
    return pkv::fail(PKV_ERR_INVALID_ARG, "fork length %d outside the parent's context [0, %d]", num_tokens,
                     it->second.len);
  pkv_block_manager::Seq s;
  const int64_t nshared = cdiv(num_tokens, bm->block_size);
  s.table.assign(it->second.table.begin(), it->second.table.begin() + nshared);
  s.len = num_tokens;
  const auto& ps = it->second;
  s.salt = ps.salt;
  s.tokens.assign(ps.tokens.begin(), ps.tokens.begin() + std::min<size_t>(num_tokens, ps.tokens.size()));
  s.digests.assign(ps.digests.begin(),
                   ps.digests.begin() + std::min<size_t>(num_tokens / bm->block_size, ps.digests.size()));
  for (int32_t b : s.table) ref_inc(bm, b);
  bm->seqs.emplace(child, std::move(s));
  return pkv::ok();
}

int32_t pkv_bm_append_slots(pkv_block_manager* bm, const int64_t* seq_ids, int32_t n_seqs,
                            const int32_t* num_tokens, const int32_t* token_ids, int32_t* slot_mapping_out,
                            int32_t slot_capacity,
                            int32_t* n_slots_out, int32_t* cow_pairs_out, int32_t cow_capacity,
                            int32_t* n_cow_out) {
  if (int32_t e = check_handle(bm)) return e;
  if (n_seqs < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "n_seqs < 0");
  if (n_seqs > 0 && !seq_ids) return pkv::fail(PKV_ERR_INVALID_ARG, "seq_ids is null");
  if (slot_capacity < 0 || cow_capacity < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "negative capacity");
  const int32_t bs = bm->block_size;

  // Pass 1: validate and count, without touching the state.
  std::vector<pkv_block_manager::Seq*> seqp(n_seqs);
  std::unordered_set<int64_t> seen;
  seen.reserve(static_cast<size_t>(n_seqs) * 2);
  int64_t total_tokens = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return pkv::fail(PKV_ERR_UNKNOWN_SEQ, "unknown sequence %lld", (long long)seq_ids[i]);
    if (int32_t e = check_on_gpu(it->second, seq_ids[i])) return e;
    if (!seen.insert(seq_ids[i]).second)
      return pkv::fail(PKV_ERR_INVALID_ARG, "sequence %lld appears twice in one call", (long long)seq_ids[i]);
    const int32_t n = num_tokens ? num_tokens[i] : 1;
    if (n < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "negative token count for sequence %lld", (long long)seq_ids[i]);
    if (static_cast<int64_t>(it->second.len) + n > INT32_MAX)
      return pkv::fail(PKV_ERR_INVALID_ARG, "sequence %lld would exceed the int32 length range", (long long)seq_ids[i]);
    seqp[i] = &it->second;
    total_tokens += n;
  }
  if (total_tokens > slot_capacity)
    return pkv::fail(PKV_ERR_CAPACITY, "slot buffer holds %d slots, %lld needed", slot_capacity, (long long)total_tokens);
  if (total_tokens > 0 && !slot_mapping_out) return pkv::fail(PKV_ERR_INVALID_ARG, "slot_mapping_out is null");
  int64_t need_blocks = 0, need_cow = 0;
  std::unordered_map<int32_t, int32_t> dropped;  // simulated refcount drops on shared last blocks
  for (int32_t i = 0; i < n_seqs; ++i) {
    const int32_t n = num_tokens ? num_tokens[i] : 1;
    if (n == 0) continue;
    const int32_t L = seqp[i]->len;
    if (L % bs) {
      const int32_t last = seqp[i]->table[L / bs];
      int32_t& d = dropped[last];
      if (bm->registered[last] || bm->refcount[last] - d > 1) {
        ++need_cow;
        ++d;
      }
    }
    need_blocks += cdiv(static_cast<int64_t>(L) + n, bs) - cdiv(L, bs);
  }
  need_blocks += need_cow;
  if (need_cow > cow_capacity)
    return pkv::fail(PKV_ERR_CAPACITY, "copy-pair buffer holds %d pairs, %lld needed", cow_capacity, (long long)need_cow);
  if (need_cow > 0 && !cow_pairs_out) return pkv::fail(PKV_ERR_INVALID_ARG, "cow_pairs_out is null");
  if (need_blocks > available(bm))
    return pkv::fail(PKV_ERR_OUT_OF_BLOCKS, "%lld blocks needed, %lld free", (long long)need_blocks,
                     (long long)available(bm));

  // Pass 2: apply.  Cannot fail from here on.
  int32_t ns = 0, nc = 0;
  std::vector<int32_t>& released = bm->scratch_released;
  released.clear();
  for (int32_t i = 0; i < n_seqs; ++i) {
    pkv_block_manager::Seq& s = *seqp[i];
    const int32_t n = num_tokens ? num_tokens[i] : 1;
    for (int32_t t = 0; t < n; ++t) {
      const int32_t L = s.len;
      if (L % bs == 0) {
        const int32_t b = take_block(bm);
        bm->refcount[b] = 1;
        s.table.push_back(b);
      } else {
        const int32_t old = s.table[L / bs];
        if (bm->refcount[old] > 1 || bm->registered[old]) {
          const int32_t b = take_block(bm);
          cow_pairs_out[2 * nc] = old;
          cow_pairs_out[2 * nc + 1] = b;
          ++nc;
          if (ref_dec(bm, old) == 0) released.push_back(old);  // registered; last holder gone
          bm->refcount[b] = 1;
          s.table[L / bs] = b;
          for (int32_t& d : s.dirty_from)
            if (L / bs < d) d = L / bs;
        }
      }
      if (token_ids && static_cast<int64_t>(s.tokens.size()) == L) s.tokens.push_back(token_ids[ns]);
      slot_mapping_out[ns++] = s.table[L / bs] * bs + L % bs;
      s.len = L + 1;
      if ((L + 1) % bs == 0) complete_block(bm, s, L / bs);
    }
  }
  for (int32_t b : released) lru_push_back(bm, b);
  if (n_slots_out) *n_slots_out = ns;
  if (n_cow_out) *n_cow_out = nc;
  return pkv::ok();
}

int32_t pkv_bm_free_seq(pkv_block_manager* bm, int64_t seq_id) {
  if (int32_t e = check_handle(bm)) return e;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return pkv::fail(PKV_ERR_UNKNOWN_SEQ, "unknown sequence %lld", (long long)seq_id);
  if (it->second.swapped) {
    for (int32_t h : it->second.host_table) bm->host_free.push_back(h);
  } else {
    release_table(bm, it->second.table);
  }
  bm->seqs.erase(it);
  return pkv::ok();
}

int32_t pkv_bm_block_tables(const pkv_block_manager* bm, const int64_t* seq_ids, int32_t n_seqs,
                            int32_t max_blocks_per_seq, int32_t* tables_out, int32_t* context_lens_out) {
  if (int32_t e = check_handle(bm)) return e;
  if (n_seqs < 0 || max_blocks_per_seq < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "negative size");
  if (n_seqs > 0 && (!seq_ids || (!tables_out && max_blocks_per_seq > 0)))
    return pkv::fail(PKV_ERR_INVALID_ARG, "null seq_ids or tables_out");
  std::vector<const pkv_block_manager::Seq*> seqp(n_seqs);
  for (int32_t i = 0; i < n_seqs; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return pkv::fail(PKV_ERR_UNKNOWN_SEQ, "unknown sequence %lld", (long long)seq_ids[i]);
    if (int32_t e = check_on_gpu(it->second, seq_ids[i])) return e;
    if (static_cast<int64_t>(it->second.table.size()) > max_blocks_per_seq)
      return pkv::fail(PKV_ERR_CAPACITY, "sequence %lld holds %zu blocks > max_blocks_per_seq %d",
                       (long long)seq_ids[i], it->second.table.size(), max_blocks_per_seq);
    seqp[i] = &it->second;
  }
  for (int32_t i = 0; i < n_seqs; ++i) {
    int32_t* row = tables_out + static_cast<int64_t>(i) * max_blocks_per_seq;
    const auto& t = seqp[i]->table;
    std::copy(t.begin(), t.end(), row);
    std::fill(row + t.size(), row + max_blocks_per_seq, -1);
    if (context_lens_out) context_lens_out[i] = seqp[i]->len;
  }
  return pkv::ok();
}

int32_t pkv_bm_num_free(const pkv_block_manager* bm) {
  if (int32_t e = check_handle(bm)) return e;
  return static_cast<int32_t>(available(bm));
}

int32_t pkv_bm_num_cached(const pkv_block_manager* bm) {
  if (int32_t e = check_handle(bm)) return e;
  return static_cast<int32_t>(bm->cached.size());
}

int32_t pkv_bm_evictable(const pkv_block_manager* bm, int32_t* out, int32_t capacity) {
  if (int32_t e = check_handle(bm)) return e;
  if (capacity < bm->lru_size)
    return pkv::fail(PKV_ERR_CAPACITY, "capacity %d < %d evictable blocks", capacity, bm->lru_size);
  if (bm->lru_size > 0 && !out) return pkv::fail(PKV_ERR_INVALID_ARG, "out is null");
  int32_t n = 0;
  for (int32_t b = bm->lru_head; b >= 0; b = bm->lru_next[b]) out[n++] = b;
  return n;
}

int32_t pkv_bm_cached_digest(const pkv_block_manager* bm, int32_t block, uint8_t* out) {
  if (int32_t e = check_handle(bm)) return e;
  if (block < 0 || block >= bm->num_blocks)
    return pkv::fail(PKV_ERR_INVALID_ARG, "block %d outside [0, %d)", block, bm->num_blocks);
  if (!bm->registered[block]) return 0;
  if (!out) return pkv::fail(PKV_ERR_INVALID_ARG, "out is null");
  std::copy(bm->block_digest[block].begin(), bm->block_digest[block].end(), out);
  return 1;
}

int32_t pkv_bm_num_shared(const pkv_block_manager* bm) {
  if (int32_t e = check_handle(bm)) return e;
  pkv::ok();
  return bm->num_shared;
}

int32_t pkv_bm_refcount(const pkv_block_manager* bm, int32_t block) {
  if (int32_t e = check_handle(bm)) return e;
  if (block < 0 || block >= bm->num_blocks)
    return pkv::fail(PKV_ERR_INVALID_ARG, "block %d outside [0, %d)", block, bm->num_blocks);
  return bm->refcount[block];
}

int32_t pkv_bm_seq_len(const pkv_block_manager* bm, int64_t seq_id) {
  if (int32_t e = check_handle(bm)) return e;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return pkv::fail(PKV_ERR_UNKNOWN_SEQ, "unknown sequence %lld", (long long)seq_id);
  return it->second.len;
}

int32_t pkv_bm_num_seqs(const pkv_block_manager* bm) {
  if (int32_t e = check_handle(bm)) return e;
  return static_cast<int32_t>(bm->seqs.size());
}

int32_t pkv_bm_free_stack(const pkv_block_manager* bm, int32_t* out, int32_t capacity) {
  if (int32_t e = check_handle(bm)) return e;
  const int32_t n = static_cast<int32_t>(bm->free_stack.size());
  if (capacity < n) return pkv::fail(PKV_ERR_CAPACITY, "capacity %d < %d free blocks", capacity, n);
  if (n > 0 && !out) return pkv::fail(PKV_ERR_INVALID_ARG, "out is null");
  std::copy(bm->free_stack.begin(), bm->free_stack.end(), out);
  return n;
}


int32_t pkv_bm_add_host_pool(pkv_block_manager* bm, int32_t num_host_blocks) {
  if (int32_t e = check_handle(bm)) return e;
  if (bm->num_host_blocks) return pkv::fail(PKV_ERR_INVALID_ARG, "the host pool is already set");
  if (num_host_blocks <= 0) return pkv::fail(PKV_ERR_INVALID_ARG, "num_host_blocks must be positive");
  bm->num_host_blocks = num_host_blocks;
  bm->host_free.resize(num_host_blocks);
  for (int32_t i = 0; i < num_host_blocks; ++i) bm->host_free[num_host_blocks - 1 - i] = i;
  return pkv::ok();
}

int32_t pkv_bm_swap_out(pkv_block_manager* bm, int64_t seq_id, int32_t* pairs_out, int32_t capacity,
                        int32_t* n_pairs_out) {
  if (int32_t e = check_handle(bm)) return e;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return pkv::fail(PKV_ERR_UNKNOWN_SEQ, "unknown sequence %lld", (long long)seq_id);
  auto& q = it->second;
  if (int32_t e = check_on_gpu(q, seq_id)) return e;
  const int32_t n = static_cast<int32_t>(q.table.size());
  if (capacity < n) return pkv::fail(PKV_ERR_CAPACITY, "pair buffer holds %d pairs, %d needed", capacity, n);
  if (n > 0 && !pairs_out) return pkv::fail(PKV_ERR_INVALID_ARG, "pairs_out is null");
  if (static_cast<size_t>(n) > bm->host_free.size())
    return pkv::fail(PKV_ERR_OUT_OF_BLOCKS, "%d host blocks needed, %zu free", n, bm->host_free.size());
  q.host_table.resize(n);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t h = bm->host_free.back();
    bm->host_free.pop_back();
    pairs_out[2 * i] = q.table[i];
    pairs_out[2 * i + 1] = h;
    q.host_table[i] = h;
  }
  release_table(bm, q.table);
  q.table.clear();
  q.swapped = true;
  q.mirror_row[0] = q.mirror_row[1] = -1;  // its device-table rows are rewritten in full after swap-in
  if (n_pairs_out) *n_pairs_out = n;
  return pkv::ok();
}

int32_t pkv_bm_swap_in(pkv_block_manager* bm, int64_t seq_id, int32_t* pairs_out, int32_t capacity,
                       int32_t* n_pairs_out) {
  if (int32_t e = check_handle(bm)) return e;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return pkv::fail(PKV_ERR_UNKNOWN_SEQ, "unknown sequence %lld", (long long)seq_id);
  auto& q = it->second;
  if (!q.swapped) return pkv::fail(PKV_ERR_INVALID_ARG, "sequence %lld is not swapped out", (long long)seq_id);
  const int32_t n = static_cast<int32_t>(q.host_table.size());
  if (capacity < n) return pkv::fail(PKV_ERR_CAPACITY, "pair buffer holds %d pairs, %d needed", capacity, n);
  if (n > 0 && !pairs_out) return pkv::fail(PKV_ERR_INVALID_ARG, "pairs_out is null");
  if (n > available(bm))
    return pkv::fail(PKV_ERR_OUT_OF_BLOCKS, "%d blocks needed, %lld free", n, (long long)available(bm));
  q.table.resize(n);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = take_block(bm);
    bm->refcount[b] = 1;
    q.table[i] = b;
    pairs_out[2 * i] = q.host_table[i];
    pairs_out[2 * i + 1] = b;
  }
  for (int32_t h : q.host_table) bm->host_free.push_back(h);
  q.host_table.clear();
  q.swapped = false;
  q.mirror_row[0] = q.mirror_row[1] = -1;
  if (n_pairs_out) *n_pairs_out = n;
  return pkv::ok();
}

int32_t pkv_bm_num_free_host(const pkv_block_manager* bm) {
  if (int32_t e = check_handle(bm)) return e;
  return static_cast<int32_t>(bm->host_free.size());
}

int32_t pkv_bm_is_swapped(const pkv_block_manager* bm, int64_t seq_id) {
  if (int32_t e = check_handle(bm)) return e;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return pkv::fail(PKV_ERR_UNKNOWN_SEQ, "unknown sequence %lld", (long long)seq_id);
  return it->second.swapped ? 1 : 0;
}

int32_t pkv_bm_stage_capacity(int32_t n_seqs, int32_t max_blocks_per_seq) {
  if (n_seqs < 0 || max_blocks_per_seq < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "negative size");
  const int64_t need = 4 + 4 * static_cast<int64_t>(n_seqs) + 3 * static_cast<int64_t>(n_seqs) * max_blocks_per_seq;
  if (need > INT32_MAX) return pkv::fail(PKV_ERR_INVALID_ARG, "stage size exceeds the int32 range");
  pkv::ok();
  return static_cast<int32_t>(need);
}

int32_t pkv_bm_stage_step(pkv_block_manager* bm, const int64_t* seq_ids, int32_t n_seqs, const int32_t* token_ids,
                          int32_t* stage,
                          int32_t stage_capacity, int32_t* block_tables, int32_t max_blocks_per_seq,
                          int32_t* context_lens, int32_t* slot_mapping, int32_t* cow_pairs, int32_t cow_capacity,
                          int32_t full, int32_t* n_cow_out, int32_t* max_len_out, void* stream) {
  if (int32_t e = check_handle(bm)) return e;
  if (n_seqs < 0 || max_blocks_per_seq <= 0 || stage_capacity < 0 || cow_capacity < 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "bad sizes");
  if (n_seqs == 0) {
    if (n_cow_out) *n_cow_out = 0;
    if (max_len_out) *max_len_out = 0;
    return pkv::ok();
  }
  if (!seq_ids || !stage || !block_tables || !context_lens || !slot_mapping || !cow_pairs)
    return pkv::fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (cow_capacity < n_seqs)
    return pkv::fail(PKV_ERR_CAPACITY, "copy-pair buffer holds %d pairs; one per sequence (%d) is required",
                     cow_capacity, n_seqs);
  const int32_t* stage_dev = nullptr;
  if (int32_t e = pkv::stage_device_ptr(stage, &stage_dev)) return e;
  const int32_t bs = bm->block_size;
  // The mirror of this device table, or the least recently used one, which
  // is then rebuilt (every entry written).
  int m = -1;
  for (int k = 0; k < 2; ++k)
    if (bm->mirrors[k].table == block_tables && bm->mirrors[k].width == max_blocks_per_seq) m = k;
  bool remap = full || m < 0;
  if (m < 0) m = bm->mirrors[0].last_use <= bm->mirrors[1].last_use ? 0 : 1;
  auto& mt = bm->mirrors[m];

  // Bound the record before anything changes, so every failure leaves the
  // manager untouched (the append below validates ids and counts the rest).
  int64_t bound = 4 + 4 * static_cast<int64_t>(n_seqs);
  for (int32_t i = 0; i < n_seqs; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return pkv::fail(PKV_ERR_UNKNOWN_SEQ, "unknown sequence %lld", (long long)seq_ids[i]);
    if (int32_t e = check_on_gpu(it->second, seq_ids[i])) return e;
    const auto& q = it->second;
    const bool owned = !remap && q.mirror_row[m] == i && i < static_cast<int32_t>(mt.row_owner.size()) &&
                       mt.row_owner[i] == seq_ids[i];
    const int64_t nb_after = (static_cast<int64_t>(q.len) + 1 + bs - 1) / bs;
    if (nb_after > max_blocks_per_seq)
      return pkv::fail(PKV_ERR_CAPACITY, "sequence %lld would hold %lld blocks > max_blocks_per_seq %d",
                       (long long)seq_ids[i], (long long)nb_after, max_blocks_per_seq);
    int64_t from = 0;
    if (owned) {
      from = q.mirror_blocks[m];
      if (q.dirty_from[m] < from) from = q.dirty_from[m];
      const int64_t write_at = q.len / bs;  // a copy-on-write may replace this entry
      if (write_at < from) from = write_at;
    }
    bound += 3 * (nb_after - from);
  }
  if (bound > stage_capacity)
    return pkv::fail(PKV_ERR_CAPACITY, "stage buffer holds %d ints, up to %lld needed", stage_capacity,
                     (long long)bound);

  bm->scratch_slots.resize(n_seqs);
  bm->scratch_pairs.resize(2 * static_cast<size_t>(n_seqs));
  int32_t ns = 0, nc = 0;
  if (int32_t e = pkv_bm_append_slots(bm, seq_ids, n_seqs, nullptr, token_ids, bm->scratch_slots.data(), n_seqs, &ns,
                                      bm->scratch_pairs.data(), n_seqs, &nc))
    return e;

  // Record: [n, pairs, updates, width] slots[n] lens[n] pairs[2*pairs] updates[3*updates]
  int32_t* slots = stage + 4;
  int32_t* lens = slots + n_seqs;
  int32_t* pairs = lens + n_seqs;
  int32_t* upd = pairs + 2 * nc;
  int32_t nu = 0, max_len = 0;
  if (remap) mt.row_owner.clear();
  if (static_cast<int32_t>(mt.row_owner.size()) < n_seqs) mt.row_owner.resize(n_seqs, -1);
  for (int32_t i = 0; i < n_seqs; ++i) {
    auto& q = bm->seqs.find(seq_ids[i])->second;
    const bool owned = !remap && q.mirror_row[m] == i && mt.row_owner[i] == seq_ids[i];
    slots[i] = bm->scratch_slots[i];
    lens[i] = q.len;
    if (q.len > max_len) max_len = q.len;
    const int32_t nb = static_cast<int32_t>(q.table.size());
    int32_t from = 0;
    if (owned) {
      from = q.mirror_blocks[m] < q.dirty_from[m] ? q.mirror_blocks[m] : q.dirty_from[m];
      if (from > nb) from = nb;
    }
    for (int32_t c = from; c < nb; ++c) {
      upd[3 * nu] = i;
      upd[3 * nu + 1] = c;
      upd[3 * nu + 2] = q.table[c];
      ++nu;
    }
    q.mirror_row[m] = i;
    q.mirror_blocks[m] = nb;
    q.dirty_from[m] = INT32_MAX;
    mt.row_owner[i] = seq_ids[i];
  }
  for (int32_t k = 0; k < 2 * nc; ++k) pairs[k] = bm->scratch_pairs[k];
  stage[0] = n_seqs;
  stage[1] = nc;
  stage[2] = nu;
  stage[3] = max_blocks_per_seq;
  if (remap) {
    mt.table = block_tables;
    mt.width = max_blocks_per_seq;
  }
  mt.last_use = ++bm->stage_calls;
  if (int32_t e = pkv::launch_stage(stage_dev, n_seqs, nc, nu, max_blocks_per_seq, slot_mapping, context_lens,
                                    cow_pairs, block_tables, stream))
    return e;
  if (n_cow_out) *n_cow_out = nc;
  if (max_len_out) *max_len_out = max_len;
  return pkv::ok();
}

}  // extern "C"
