#include "block_manager.hpp"

#include <algorithm>

namespace pa {

BlockManager::BlockManager(int32_t num_blocks, int32_t block_size)
    : num_blocks_(num_blocks),
      block_size_(block_size),
      next_(static_cast<size_t>(num_blocks), -1),
      prev_(static_cast<size_t>(num_blocks), -1),
      in_free_(static_cast<size_t>(num_blocks), 0),
      block_node_(static_cast<size_t>(num_blocks), -1),
      ref_(static_cast<size_t>(num_blocks), 0) {
  for (int32_t b = 0; b < num_blocks; ++b) push_free(b);
}

BmStatus BlockManager::set_free_order(const int32_t* perm, int32_t n) {
  if (touched_ || n != num_blocks_ || perm == nullptr) return BmStatus::kInvalid;
  std::vector<char> seen(static_cast<size_t>(num_blocks_), 0);
  for (int32_t i = 0; i < n; ++i) {
    if (perm[i] < 0 || perm[i] >= num_blocks_ || seen[perm[i]]) return BmStatus::kInvalid;
    seen[perm[i]] = 1;
  }
  head_ = tail_ = -1;
  free_count_ = 0;
  std::fill(in_free_.begin(), in_free_.end(), 0);
  for (int32_t i = 0; i < n; ++i) push_free(perm[i]);
  return BmStatus::kOk;
}

void BlockManager::unlink_free(int32_t b) {
  const int32_t p = prev_[b], q = next_[b];
  if (p >= 0) next_[p] = q; else head_ = q;
  if (q >= 0) prev_[q] = p; else tail_ = p;
  prev_[b] = next_[b] = -1;
  in_free_[b] = 0;
  --free_count_;
}

int32_t BlockManager::pop_free() {
  const int32_t b = head_;
  unlink_free(b);
  if (block_node_[b] >= 0) {  // the cached prefix block is reused: its entry goes
    clear_entry(b);
    ++cache_evictions_;
  }
  return b;
}

void BlockManager::push_free(int32_t b) {
  prev_[b] = tail_;
  next_[b] = -1;
  if (tail_ >= 0) next_[tail_] = b; else head_ = b;
  tail_ = b;
  in_free_[b] = 1;
  ++free_count_;
}

// Bucket of a trie node: FNV-1a over the parent node and the block's token
// ids, then the splitmix64 finalizer.  Only the bucket depends on it: a lookup
// compares the parent and the ids exactly.  Tests build a variant whose hash
// is constant (every key in one bucket) to show that.
uint64_t BlockManager::node_hash(int32_t parent, const int32_t* tokens) const {
#ifdef PA_PREFIX_HASH_CONSTANT
  (void)parent;
  (void)tokens;
  return 0;
#else
  uint64_t h = 0xCBF29CE484222325ull;
  h ^= static_cast<uint32_t>(parent);
  h *= 0x100000001B3ull;
  for (int32_t i = 0; i < block_size_; ++i) {
    h ^= static_cast<uint32_t>(tokens[i]);
    h *= 0x100000001B3ull;
  }
  h ^= h >> 30;
  h *= 0xBF58476D1CE4E5B9ull;
  h ^= h >> 27;
  h *= 0x94D049BB133111EBull;
  h ^= h >> 31;
  return h;
#endif
}

int32_t BlockManager::find_node(int32_t parent, const int32_t* tokens) const {
  const auto range = index_.equal_range(node_hash(parent, tokens));
  for (auto it = range.first; it != range.second; ++it) {
    const int32_t id = it->second;
    if (nodes_[id].parent == parent &&
        std::equal(tokens, tokens + block_size_, node_tokens_.begin() + static_cast<int64_t>(id) * block_size_))
      return id;
  }
  return -1;
}

// The node (parent, tokens), created if absent (a new node holds a reference
// on its parent).
int32_t BlockManager::get_node(int32_t parent, const int32_t* tokens) {
  int32_t id = find_node(parent, tokens);
  if (id >= 0) return id;
  if (!free_nodes_.empty()) {
    id = free_nodes_.back();
    free_nodes_.pop_back();
  } else {
    id = static_cast<int32_t>(nodes_.size());
    nodes_.emplace_back();
    node_tokens_.resize(node_tokens_.size() + block_size_);
  }
  PrefixNode& nd = nodes_[id];
  nd.parent = parent;
  nd.block = -1;
  nd.refs = 0;
  nd.hash = node_hash(parent, tokens);
  std::copy(tokens, tokens + block_size_, node_tokens_.begin() + static_cast<int64_t>(id) * block_size_);
  index_.emplace(nd.hash, id);
  if (parent >= 0) ++nodes_[parent].refs;
  return id;
}

void BlockManager::pin(int32_t node) {
  if (node >= 0) ++nodes_[node].refs;
}

// Drops one reference; a node left with none leaves the trie and releases its
// parent in turn.
void BlockManager::release(int32_t node) {
  while (node >= 0) {
    PrefixNode& nd = nodes_[node];
    if (--nd.refs > 0) return;
    const auto range = index_.equal_range(nd.hash);
    for (auto it = range.first; it != range.second; ++it) {
      if (it->second == node) {
        index_.erase(it);
        break;
      }
    }
    free_nodes_.push_back(node);
    node = nd.parent;
  }
}

// Enters block b under the node's prefix, replacing an entry with the same key.
void BlockManager::set_entry(int32_t node, int32_t b) {
  PrefixNode& nd = nodes_[node];
  if (nd.block >= 0) {
    block_node_[nd.block] = -1;  // replaced entry
  } else {
    ++nd.refs;
    ++cached_count_;
  }
  nd.block = b;
  block_node_[b] = node;
}

void BlockManager::clear_entry(int32_t b) {
  const int32_t node = block_node_[b];
  block_node_[b] = -1;
  nodes_[node].block = -1;
  --cached_count_;
  release(node);
}

// Token ids of n tokens appended to s from position first_token (the table
// already holds their blocks): each block they fill is entered under the
// sequence's prefix.
void BlockManager::append_ids(Seq& s, int64_t first_token, int32_t n, const int32_t* tokens) {
  const int64_t bs = block_size_;
  for (int32_t j = 0; j < n; ++j) {
    s.tail.push_back(tokens[j]);
    if (static_cast<int64_t>(s.tail.size()) == bs) {
      const int64_t i = (first_token + j) / bs;  // the block this token fills
      const int32_t nd = get_node(s.node, s.tail.data());
      set_entry(nd, s.table[i]);
      pin(nd);
      release(s.node);
      s.node = nd;
      s.tail.clear();
    }
  }
}

BmStatus BlockManager::seq_create_cached(const int32_t* tokens, int32_t n, int32_t* seq,
                                         int32_t* cached, int32_t* slots) {
  if (n < 0 || (n > 0 && (tokens == nullptr || slots == nullptr)) || seq == nullptr || cached == nullptr)
    return BmStatus::kInvalid;
  const int64_t bs = block_size_;
  const int64_t full = n / bs;
  // Look up the prompt's full blocks until the first miss.
  std::vector<int32_t> hits;
  int32_t parent = -1;
  for (int64_t i = 0; i < full; ++i) {
    const int32_t nd = find_node(parent, tokens + i * bs);
    if (nd < 0 || nodes_[nd].block < 0) break;
    hits.push_back(nodes_[nd].block);
    parent = nd;
  }
  const int64_t h = static_cast<int64_t>(hits.size());
  const int64_t need = (n - h * bs + bs - 1) / bs;
  int64_t revived = 0;
  for (int32_t b : hits) revived += ref_[b] == 0;
  if (need > free_count_ - revived) {
    ++alloc_failures_;
    return BmStatus::kNoBlocks;
  }
  touched_ = true;
  const int32_t s_id = seq_create();
  Seq& s = seqs_[s_id];
  for (int32_t b : hits) {
    if (ref_[b] == 0) unlink_free(b);
    ++ref_[b];
    s.table.push_back(b);
  }
  cache_hits_ += h;
  cache_misses_ += full - h;
  // The hit chain's last node holds its ancestors; it stays in the trie while
  // the allocations below evict other entries.
  pin(parent);
  for (int64_t i = 0; i < need; ++i) {
    const int32_t b = pop_free();
    ref_[b] = 1;
    s.table.push_back(b);
  }
  table_entries_ += static_cast<int64_t>(s.table.size());
  s.node = parent;  // pinned above
  s.len = static_cast<int32_t>(h * bs);
  append_ids(s, h * bs, static_cast<int32_t>(n - h * bs), tokens + h * bs);
  s.len = n;
  for (int64_t t = h * bs; t < n; ++t)
    slots[t - h * bs] = static_cast<int32_t>(static_cast<int64_t>(s.table[t / bs]) * bs + t % bs);
  *seq = s_id;
  *cached = static_cast<int32_t>(h * bs);
  return BmStatus::kOk;
}

int32_t BlockManager::seq_create() {
  seqs_.emplace_back();
  seqs_.back().alive = true;
  ++live_seqs_;
  return static_cast<int32_t>(seqs_.size() - 1);
}

BmStatus BlockManager::alloc(int32_t seq, int32_t n, int32_t* slots, int32_t* cow_src,
                             int32_t* cow_dst, const int32_t* tokens) {
  if (cow_src) *cow_src = -1;
  if (cow_dst) *cow_dst = -1;
  if (!valid_seq(seq)) return BmStatus::kBadSeq;
  if (n < 0 || (n > 0 && slots == nullptr)) return BmStatus::kInvalid;
  Seq& s = seqs_[seq];
  const int64_t bs = block_size_;
  const int64_t len = s.len;
  const int64_t new_len = len + n;
  const int64_t need = (new_len + bs - 1) / bs - static_cast<int64_t>(s.table.size());
  const bool cow = n > 0 && (len % bs) != 0 && ref_[s.table.back()] > 1;
  if (need + (cow ? 1 : 0) > free_count_) {
    ++alloc_failures_;
    return BmStatus::kNoBlocks;
  }
  touched_ = true;
  if (cow) {
    const int32_t old_b = s.table.back();
    const int32_t new_b = pop_free();
    ref_[new_b] = 1;
    --ref_[old_b];
    s.table.back() = new_b;
    ++cow_copies_;
    if (cow_src) *cow_src = old_b;
    if (cow_dst) *cow_dst = new_b;
  }
  for (int64_t i = 0; i < need; ++i) {
    const int32_t b = pop_free();
    ref_[b] = 1;
    s.table.push_back(b);
  }
  table_entries_ += need;
  for (int64_t j = 0; j < n; ++j) {
    const int64_t t = len + j;
    slots[j] = static_cast<int32_t>(static_cast<int64_t>(s.table[t / bs]) * bs + t % bs);
  }
  s.len = static_cast<int32_t>(new_len);
  if (n > 0 && s.known) {
    if (tokens) {
      append_ids(s, len, n, tokens);
    } else {  // ids unknown from here on: nothing more of this sequence is cached
      release(s.node);
      s.node = -1;
      s.known = false;
      s.tail.clear();
    }
  }
  return BmStatus::kOk;
}

BmStatus BlockManager::fork(int32_t parent, int32_t* child) {
  if (!valid_seq(parent)) return BmStatus::kBadSeq;
  if (child == nullptr) return BmStatus::kInvalid;
  const int32_t c = seq_create();
  Seq& p = seqs_[parent];  // seq_create may reallocate seqs_: take the reference after it
  Seq& k = seqs_[c];
  k.table = p.table;
  k.len = p.len;
  k.known = p.known;
  k.node = p.node;
  k.tail = p.tail;
  if (k.known) pin(k.node);
  for (int32_t b : k.table) ++ref_[b];
  table_entries_ += static_cast<int64_t>(k.table.size());
  *child = c;
  return BmStatus::kOk;
}

BmStatus BlockManager::free_seq(int32_t seq) {
  if (!valid_seq(seq)) return BmStatus::kBadSeq;
  Seq& s = seqs_[seq];
  for (auto it = s.table.rbegin(); it != s.table.rend(); ++it) {
    if (--ref_[*it] == 0) push_free(*it);
  }
  table_entries_ -= static_cast<int64_t>(s.table.size());
  s.table.clear();
  s.table.shrink_to_fit();
  if (s.known) release(s.node);
  s.node = -1;
  s.tail.clear();
  s.tail.shrink_to_fit();
  s.len = 0;
  s.alive = false;
  --live_seqs_;
  return BmStatus::kOk;
}

BmStatus BlockManager::seq_len(int32_t seq, int32_t* len, int32_t* nblocks) const {
  if (!valid_seq(seq)) return BmStatus::kBadSeq;
  if (len) *len = seqs_[seq].len;
  if (nblocks) *nblocks = static_cast<int32_t>(seqs_[seq].table.size());
  return BmStatus::kOk;
}

BmStatus BlockManager::table_row(int32_t seq, int32_t max_blocks, int32_t* row,
                                 int32_t* len) const {
  if (!valid_seq(seq)) return BmStatus::kBadSeq;
  const Seq& s = seqs_[seq];
  if (static_cast<int64_t>(s.table.size()) > max_blocks) return BmStatus::kInvalid;
  int32_t i = 0;
  for (; i < static_cast<int32_t>(s.table.size()); ++i) row[i] = s.table[i];
  for (; i < max_blocks; ++i) row[i] = -1;
  if (len) *len = s.len;
  return BmStatus::kOk;
}

int64_t BlockManager::shared_blocks() const {
  int64_t n = 0;
  for (int32_t r : ref_) n += r > 1;
  return n;
}

void BlockManager::free_queue(int32_t* out) const {
  int64_t i = 0;
  for (int32_t b = head_; b >= 0; b = next_[b]) out[i++] = b;
}

}  // namespace pa
