// Radix-tree prefix index over the block manager.
//
// "PagedAttention et RadixAttention : parlons de KV Cache", section
// RadixAttention : un arbre qui n'oublie pas, and the paragraph after it:
// a persistent compressed trie over token sequences in which every distinct
// prefix is stored once and requests with a common start share a branch
// that splits exactly where their tokens first differ; a new request walks
// it token by token for the longest prefix already present and reuses that
// K/V; when memory runs out the least recently used leaves go first, while
// internal nodes that requests depend on are protected; and the tree only
// points at blocks the paged allocator manages.
//
// Policy (deterministic, shared with the oracle's model):
//   * every node but the root is backed by a block-manager sequence, its
//     holder, whose first `depth` tokens are the node's path; holders are
//     forks (of the request, or of the node being split), so they only add
//     reference counts; a split inside a block shares the partial block,
//     which the block manager copies only if someone writes into it;
//   * holder ids are kHolderBase + k in creation order;
//   * admit locks the matched path for the request (stamping it with the
//     current time), insert adds the request's path, release unlocks;
//   * evict frees the holders of unlocked leaves, least recently stamped
//     first (ties: the older node), until enough pool blocks are free; a
//     parent left without children becomes a leaf;
//   * time is a counter advanced by every admit and insert.
// This file uses only the block manager's C entry points.
#include <algorithm>
#include <cstdint>
#include <map>
#include <new>
#include <unordered_map>
#include <vector>

#include "pkv_status.h"

namespace {

constexpr int64_t kHolderBase = int64_t(1) << 62;

struct Node {
  std::vector<int32_t> edge;
  int32_t parent = -1;
  std::map<int32_t, int32_t> children;  // first token -> node index
  int32_t depth = 0;
  int64_t holder = -1;
  int64_t stamp = 0;
  int32_t locks = 0;
  int64_t serial = 0;
  bool alive = true;
};

}  // namespace

struct pkv_radix {
  pkv_block_manager* bm = nullptr;
  std::vector<Node> nodes;         // [0] is the root; evicted slots are reused
  std::vector<int32_t> free_slots;  // evicted node slots
  int64_t clock = 0;
  int64_t next_holder = 0;
  int64_t next_serial = 1;
  std::unordered_map<int64_t, std::vector<int32_t>> locked;  // request -> locked path
};

namespace {

struct Walk {
  std::vector<int32_t> path;  // node indices, fully or partly matched
  int32_t matched = 0;
  int32_t used = 0;  // tokens of the last node's edge that matched
};

Walk walk(const pkv_radix* rx, const int32_t* tokens, int32_t n) {
  Walk w;
  int32_t node = 0, i = 0;
  while (i < n) {
    const auto& ch = rx->nodes[node].children;
    auto it = ch.find(tokens[i]);
    if (it == ch.end()) break;
    const Node& c = rx->nodes[it->second];
    int32_t k = 0;
    while (k < static_cast<int32_t>(c.edge.size()) && i + k < n && c.edge[k] == tokens[i + k]) ++k;
    w.path.push_back(it->second);
    i += k;
    w.used = k;
    if (k < static_cast<int32_t>(c.edge.size())) break;
    node = it->second;
  }
  w.matched = i;
  return w;
}

int32_t new_node(pkv_radix* rx, std::vector<int32_t> edge, int32_t parent, int32_t depth) {
  Node nd;
  nd.edge = std::move(edge);
  nd.parent = parent;
  nd.depth = depth;
  nd.holder = kHolderBase + rx->next_holder++;
  nd.stamp = rx->clock;
  nd.serial = rx->next_serial++;
  if (!rx->free_slots.empty()) {
    const int32_t i = rx->free_slots.back();
    rx->free_slots.pop_back();
    rx->nodes[i] = std::move(nd);
    return i;
  }
  rx->nodes.push_back(std::move(nd));
  return static_cast<int32_t>(rx->nodes.size()) - 1;
}

int32_t check_tokens(const int32_t* tokens, int32_t n) {
  if (n < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "n_tokens < 0");
  if (n > 0 && !tokens) return pkv::fail(PKV_ERR_INVALID_ARG, "tokens is null");
  return PKV_OK;
}

// Depth-first node order, children by first token (the export order).
void dfs(const pkv_radix* rx, std::vector<int32_t>* out) {
  std::vector<int32_t> stack = {0};
  while (!stack.empty()) {
    const int32_t n = stack.back();
    stack.pop_back();
    if (n != 0) out->push_back(n);
    const auto& ch = rx->nodes[n].children;
    for (auto it = ch.rbegin(); it != ch.rend(); ++it) stack.push_back(it->second);
  }
}

}  // namespace

extern "C" {

int32_t pkv_radix_create(pkv_block_manager* bm, pkv_radix** out) {
  if (!out) return pkv::fail(PKV_ERR_INVALID_ARG, "out handle pointer is null");
  *out = nullptr;
  if (!bm) return pkv::fail(PKV_ERR_INVALID_ARG, "null block manager handle");
  auto* rx = new (std::nothrow) pkv_radix();
  if (!rx) return pkv::fail(PKV_ERR_INVALID_ARG, "out of host memory");
  rx->bm = bm;
  rx->nodes.emplace_back();  // root
  *out = rx;
  return pkv::ok();
}

void pkv_radix_destroy(pkv_radix* rx) {
  if (!rx) return;
  for (const Node& n : rx->nodes)
    if (n.alive && n.holder >= 0) pkv_bm_free_seq(rx->bm, n.holder);
  delete rx;
}

int32_t pkv_radix_match(const pkv_radix* rx, const int32_t* tokens, int32_t n_tokens) {
  if (!rx) return pkv::fail(PKV_ERR_INVALID_ARG, "null radix handle");
  if (int32_t e = check_tokens(tokens, n_tokens)) return e;
  pkv::ok();
  return walk(rx, tokens, n_tokens).matched;
}

int32_t pkv_radix_admit(pkv_radix* rx, int64_t seq_id, const int32_t* tokens, int32_t n_tokens,
                        int32_t* n_cached_out) {
  if (!rx) return pkv::fail(PKV_ERR_INVALID_ARG, "null radix handle");
  if (int32_t e = check_tokens(tokens, n_tokens)) return e;
  if (rx->locked.count(seq_id) || pkv_bm_seq_len(rx->bm, seq_id) >= 0)
    return pkv::fail(PKV_ERR_INVALID_ARG, "sequence %lld exists", (long long)seq_id);
  const Walk w = walk(rx, tokens, n_tokens);
  const int32_t e = w.matched ? pkv_bm_fork(rx->bm, rx->nodes[w.path.back()].holder, seq_id, w.matched)
                              : pkv_bm_add_seq(rx->bm, seq_id);
  if (e) return e;
  rx->clock += 1;
  for (int32_t n : w.path) {
    rx->nodes[n].locks += 1;
    rx->nodes[n].stamp = rx->clock;
  }
  rx->locked[seq_id] = w.path;
  if (n_cached_out) *n_cached_out = w.matched;
  return pkv::ok();
}

int32_t pkv_radix_release(pkv_radix* rx, int64_t seq_id) {
  if (!rx) return pkv::fail(PKV_ERR_INVALID_ARG, "null radix handle");
  auto it = rx->locked.find(seq_id);
  if (it == rx->locked.end()) return pkv::fail(PKV_ERR_UNKNOWN_SEQ, "sequence %lld holds no locks", (long long)seq_id);
  for (int32_t n : it->second) rx->nodes[n].locks -= 1;
  rx->locked.erase(it);
  return pkv::ok();
}

int32_t pkv_radix_insert(pkv_radix* rx, int64_t seq_id, const int32_t* tokens, int32_t n_tokens,
                         int32_t* n_added_out) {
  if (!rx) return pkv::fail(PKV_ERR_INVALID_ARG, "null radix handle");
  if (int32_t e = check_tokens(tokens, n_tokens)) return e;
  const int32_t len = pkv_bm_seq_len(rx->bm, seq_id);
  if (len < 0) return pkv::fail(PKV_ERR_UNKNOWN_SEQ, "unknown sequence %lld", (long long)seq_id);
  if (n_tokens > len) return pkv::fail(PKV_ERR_INVALID_ARG, "more tokens than the sequence holds");
  if (pkv_bm_is_swapped(rx->bm, seq_id) == 1)
    return pkv::fail(PKV_ERR_INVALID_ARG, "sequence %lld is swapped out", (long long)seq_id);
  const Walk w = walk(rx, tokens, n_tokens);
  rx->clock += 1;
  for (int32_t n : w.path) rx->nodes[n].stamp = rx->clock;
  int32_t parent = 0;
  if (!w.path.empty()) {
    const int32_t last = w.path.back();
    if (w.used < static_cast<int32_t>(rx->nodes[last].edge.size())) {
      // Split the edge where the tokens diverge (or end).
      const int32_t lp = rx->nodes[last].parent;
      const int32_t inner_depth =
          rx->nodes[last].depth - static_cast<int32_t>(rx->nodes[last].edge.size()) + w.used;
      std::vector<int32_t> head(rx->nodes[last].edge.begin(), rx->nodes[last].edge.begin() + w.used);
      const int32_t inner = new_node(rx, std::move(head), lp, inner_depth);  // may move rx->nodes
      if (int32_t e = pkv_bm_fork(rx->bm, rx->nodes[last].holder, rx->nodes[inner].holder, inner_depth)) return e;
      Node& L = rx->nodes[last];
      Node& I = rx->nodes[inner];
      I.locks = L.locks;
      rx->nodes[lp].children[I.edge[0]] = inner;
      L.edge.erase(L.edge.begin(), L.edge.begin() + w.used);
      L.parent = inner;
      I.children[L.edge[0]] = last;
      for (auto& kv : rx->locked) {  // requests depending on `last` also depend on `inner`
        auto& p = kv.second;
        auto pos = std::find(p.begin(), p.end(), last);
        if (pos != p.end()) p.insert(pos, inner);
      }
      parent = inner;
    } else {
      parent = last;
    }
  }
  int32_t added = 0;
  if (w.matched < n_tokens) {
    std::vector<int32_t> rest(tokens + w.matched, tokens + n_tokens);
    const int32_t leaf = new_node(rx, std::move(rest), parent, n_tokens);
    if (int32_t e = pkv_bm_fork(rx->bm, seq_id, rx->nodes[leaf].holder, n_tokens)) return e;
    rx->nodes[parent].children[rx->nodes[leaf].edge[0]] = leaf;
    added = n_tokens - w.matched;
  }
  if (n_added_out) *n_added_out = added;
  return pkv::ok();
}

int32_t pkv_radix_evict(pkv_radix* rx, int32_t num_free_blocks, int32_t* n_evicted_out) {
  if (!rx) return pkv::fail(PKV_ERR_INVALID_ARG, "null radix handle");
  int32_t n = 0;
  std::vector<int32_t> order;
  while (pkv_bm_num_free(rx->bm) < num_free_blocks) {
    order.clear();
    dfs(rx, &order);
    int32_t victim = -1;
    for (int32_t i : order) {
      const Node& c = rx->nodes[i];
      if (!c.children.empty() || c.locks) continue;
      if (victim < 0 || c.stamp < rx->nodes[victim].stamp ||
          (c.stamp == rx->nodes[victim].stamp && c.serial < rx->nodes[victim].serial))
        victim = i;
    }
    if (victim < 0) break;
    Node& v = rx->nodes[victim];
    pkv_bm_free_seq(rx->bm, v.holder);
    rx->nodes[v.parent].children.erase(v.edge[0]);
    v.alive = false;
    v.children.clear();
    v.edge.clear();
    rx->free_slots.push_back(victim);
    ++n;
  }
  if (n_evicted_out) *n_evicted_out = n;
  return pkv::ok();
}

int32_t pkv_radix_num_nodes(const pkv_radix* rx) {
  if (!rx) return pkv::fail(PKV_ERR_INVALID_ARG, "null radix handle");
  std::vector<int32_t> order;
  dfs(rx, &order);
  return static_cast<int32_t>(order.size());
}

int32_t pkv_radix_nodes(const pkv_radix* rx, int64_t* holders, int32_t* depths, int32_t* edge_lens, int32_t* locks,
                        int64_t* stamps, int32_t capacity) {
  if (!rx) return pkv::fail(PKV_ERR_INVALID_ARG, "null radix handle");
  std::vector<int32_t> order;
  dfs(rx, &order);
  const int32_t n = static_cast<int32_t>(order.size());
  if (capacity < n) return pkv::fail(PKV_ERR_CAPACITY, "capacity %d < %d nodes", capacity, n);
  if (n > 0 && (!holders || !depths || !edge_lens || !locks || !stamps))
    return pkv::fail(PKV_ERR_INVALID_ARG, "null output array");
  for (int32_t i = 0; i < n; ++i) {
    const Node& c = rx->nodes[order[i]];
    holders[i] = c.holder;
    depths[i] = c.depth;
    edge_lens[i] = static_cast<int32_t>(c.edge.size());
    locks[i] = c.locks;
    stamps[i] = c.stamp;
  }
  pkv::ok();
  return n;
}

}  // extern "C"
