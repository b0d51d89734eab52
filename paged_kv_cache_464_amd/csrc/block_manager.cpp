#include "block_manager.hpp"

#include <algorithm>

namespace pa {

BlockManager::BlockManager(int32_t num_blocks, int32_t block_size)
    : num_blocks_(num_blocks),
      block_size_(block_size),
      next_(static_cast<size_t>(num_blocks), -1),
      prev_(static_cast<size_t>(num_blocks), -1),
      in_free_(static_cast<size_t>(num_blocks), 0),
      key_(static_cast<size_t>(num_blocks), 0),
      parent_key_(static_cast<size_t>(num_blocks), 0),
      has_key_(static_cast<size_t>(num_blocks), 0),
      key_tokens_(static_cast<size_t>(num_blocks) * block_size, 0),
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
  if (has_key_[b]) {  // the cached prefix block is reused: its entry goes
    auto it = cache_.find(key_[b]);
    if (it != cache_.end() && it->second == b) cache_.erase(it);
    has_key_[b] = 0;
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

// 64-bit key of a full block given its parent's key: FNV-1a over the token
// ids, then the splitmix64 finalizer to spread the bits.
uint64_t BlockManager::block_key(uint64_t parent, const int32_t* tokens) const {
  uint64_t h = parent ^ 0xCBF29CE484222325ull;
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
}

void BlockManager::register_block(int32_t b, uint64_t key, uint64_t parent, const int32_t* tokens) {
  auto it = cache_.find(key);
  if (it != cache_.end()) has_key_[it->second] = 0;  // replaced entry
  cache_[key] = b;
  key_[b] = key;
  parent_key_[b] = parent;
  has_key_[b] = 1;
  std::copy(tokens, tokens + block_size_, key_tokens_.begin() + static_cast<int64_t>(b) * block_size_);
}

BmStatus BlockManager::seq_create_cached(const int32_t* tokens, int32_t n, int32_t* seq,
                                         int32_t* cached, int32_t* slots) {
  if (n < 0 || (n > 0 && (tokens == nullptr || slots == nullptr)) || seq == nullptr || cached == nullptr)
    return BmStatus::kInvalid;
  const int64_t bs = block_size_;
  const int64_t full = n / bs;
  // Look up the prompt's full blocks until the first miss.
  std::vector<int32_t> hits;
  std::vector<uint64_t> keys;
  uint64_t parent = 0;
  for (int64_t i = 0; i < full; ++i) {
    const int32_t* tk = tokens + i * bs;
    const uint64_t k = block_key(parent, tk);
    keys.push_back(k);
    auto it = cache_.find(k);
    if (it == cache_.end()) break;
    const int32_t b = it->second;
    if (!has_key_[b] || key_[b] != k || parent_key_[b] != parent ||
        !std::equal(tk, tk + bs, key_tokens_.begin() + static_cast<int64_t>(b) * bs))
      break;
    hits.push_back(b);
    parent = k;
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
  for (int64_t i = 0; i < need; ++i) {
    const int32_t b = pop_free();
    ref_[b] = 1;
    s.table.push_back(b);
  }
  for (int64_t i = h; i < full; ++i) {
    if (i >= static_cast<int64_t>(keys.size())) keys.push_back(block_key(keys[i - 1], tokens + i * bs));
    register_block(s.table[i], keys[i], i == 0 ? 0 : keys[i - 1], tokens + i * bs);
  }
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
                             int32_t* cow_dst) {
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
  for (int64_t j = 0; j < n; ++j) {
    const int64_t t = len + j;
    slots[j] = static_cast<int32_t>(static_cast<int64_t>(s.table[t / bs]) * bs + t % bs);
  }
  s.len = static_cast<int32_t>(new_len);
  return BmStatus::kOk;
}

BmStatus BlockManager::fork(int32_t parent, int32_t* child) {
  if (!valid_seq(parent)) return BmStatus::kBadSeq;
  if (child == nullptr) return BmStatus::kInvalid;
  const int32_t c = seq_create();
  Seq& p = seqs_[parent];  // seq_create may reallocate seqs_: take the reference after it
  seqs_[c].table = p.table;
  seqs_[c].len = p.len;
  for (int32_t b : seqs_[c].table) ++ref_[b];
  *child = c;
  return BmStatus::kOk;
}

BmStatus BlockManager::free_seq(int32_t seq) {
  if (!valid_seq(seq)) return BmStatus::kBadSeq;
  Seq& s = seqs_[seq];
  for (auto it = s.table.rbegin(); it != s.table.rend(); ++it) {
    if (--ref_[*it] == 0) push_free(*it);
  }
  s.table.clear();
  s.table.shrink_to_fit();
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
