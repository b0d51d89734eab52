#include "block_manager.hpp"

namespace pa {

BlockManager::BlockManager(int32_t num_blocks, int32_t block_size)
    : num_blocks_(num_blocks),
      block_size_(block_size),
      ring_(static_cast<size_t>(num_blocks)),
      ref_(static_cast<size_t>(num_blocks), 0) {
  for (int32_t b = 0; b < num_blocks; ++b) ring_[b] = b;
  free_count_ = num_blocks;
}

BmStatus BlockManager::set_free_order(const int32_t* perm, int32_t n) {
  if (touched_ || n != num_blocks_ || perm == nullptr) return BmStatus::kInvalid;
  std::vector<char> seen(static_cast<size_t>(num_blocks_), 0);
  for (int32_t i = 0; i < n; ++i) {
    if (perm[i] < 0 || perm[i] >= num_blocks_ || seen[perm[i]]) return BmStatus::kInvalid;
    seen[perm[i]] = 1;
  }
  for (int32_t i = 0; i < n; ++i) ring_[i] = perm[i];
  head_ = 0;
  free_count_ = num_blocks_;
  return BmStatus::kOk;
}

int32_t BlockManager::pop_free() {
  int32_t b = ring_[head_];
  head_ = (head_ + 1) % num_blocks_;
  --free_count_;
  return b;
}

void BlockManager::push_free(int32_t b) {
  ring_[(head_ + free_count_) % num_blocks_] = b;
  ++free_count_;
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
  for (int64_t i = 0; i < free_count_; ++i) out[i] = ring_[(head_ + i) % num_blocks_];
}

}  // namespace pa
