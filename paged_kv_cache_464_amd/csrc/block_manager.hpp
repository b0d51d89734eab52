// Host-side block manager of the paged KV cache.
//
// Blocks of B tokens come from one physical pool; each sequence owns a block
// table (logical block -> physical block) that grows on demand (youngju.dev
// "KV cache and paged attention", section "PagedAttention: OS 가상 메모리식
// 관리"; iq-blog ch.4, section "OS Paging에서 가져온 해법").  Free blocks
// wait in a FIFO queue; an append that needs more blocks than are free fails
// and changes nothing (openakashic KV-cache failure-modes note, Key Points).
// Forked sequences share physical blocks with reference counts; appending into
// a shared, partly filled last block first copies it for the writer
// (youngju.dev page, section "prefix 공유와 copy-on-write"; iq-blog ch.4,
// section "Prefix Caching").
//
// Policy details the pages leave open, fixed here:
//  * the free queue pops from its head; freed blocks are appended at its tail,
//    visiting the freed sequence's table from last block to first;
//  * the block a copy-on-write needs counts toward an append's requirement;
//  * copy-on-write happens only for an append of >= 1 token into a partly
//    filled last block whose reference count exceeds one;
//  * sequence ids are 0, 1, 2, ... in creation order and never reused.
//
// Automatic prefix caching (iq-blog ch.4, section "Prefix Caching": identical
// prefixes found by a hash and shared by reference count; youngju.dev page,
// section "prefix 캐시의 수명과 무효화": hits reuse blocks, least recently used
// prefixes are evicted first; openakashic note, Key Points: a cached block
// taken from the free queue for a new allocation loses its entry; section
// "prefix 공유와 copy-on-write": multi-turn history is a shared prefix):
//  * the key of a cached block is its sequence's whole token prefix up to the
//    block's end, held exactly in a trie: node = (node of the prefix one
//    block shorter, the block's B token ids).  Lookup compares the ids and
//    the parent node, so two different prefixes never share a block whatever
//    the hash does (the hash only picks the bucket);
//  * every full block of a sequence whose token ids are known is cached: a
//    prompt's full blocks at creation, and each block an append with token
//    ids fills; a tokenless append makes the sequence's ids unknown for good;
//    forks inherit the ids;
//  * lookup stops at the first miss; hits leave the free queue if they sat
//    there; the rest of the prompt is allocated like an append and its full
//    blocks are registered (replacing an entry with the same key);
//  * freed cached blocks keep their entry at the free-queue tail, so the least
//    recently freed is evicted first; the free queue is a doubly linked list
//    so that a hit can take a block out of its middle;
//  * a trie node lives while it has an entry, a child node or a sequence
//    whose prefix ends there.
#pragma once

#include <cstdint>
#include <unordered_map>
#include <vector>

namespace pa {

enum class BmStatus { kOk, kInvalid, kNoBlocks, kBadSeq };

class BlockManager {
 public:
  BlockManager(int32_t num_blocks, int32_t block_size);

  int32_t num_blocks() const { return num_blocks_; }
  int32_t block_size() const { return block_size_; }

  // Permutation of 0..N-1 as the initial free-queue order; only before any allocation.
  BmStatus set_free_order(const int32_t* perm, int32_t n);

  int32_t seq_create();

  // Append n tokens.  slots[n] receive the new tokens' slots; *cow_src/*cow_dst the
  // copied block pair or -1.  tokens: the n appended token ids, or null.
  BmStatus alloc(int32_t seq, int32_t n, int32_t* slots, int32_t* cow_src, int32_t* cow_dst,
                 const int32_t* tokens = nullptr);
  // New sequence holding the prompt tokens[n]: *cached leading tokens come from
  // the prefix cache; slots[0 .. n - *cached) receive the rest's slots.
  BmStatus seq_create_cached(const int32_t* tokens, int32_t n, int32_t* seq, int32_t* cached,
                             int32_t* slots);
  BmStatus fork(int32_t parent, int32_t* child);
  BmStatus free_seq(int32_t seq);

  BmStatus seq_len(int32_t seq, int32_t* len, int32_t* nblocks) const;
  // Row of `max_blocks` entries padded with -1.
  BmStatus table_row(int32_t seq, int32_t max_blocks, int32_t* row, int32_t* len) const;

  int64_t free_count() const { return free_count_; }
  int64_t live_seqs() const { return live_seqs_; }
  int64_t cow_copies() const { return cow_copies_; }
  int64_t alloc_failures() const { return alloc_failures_; }
  int64_t shared_blocks() const;
  // Block-table entries of the live sequences (the sum of all reference
  // counts): over the used blocks, the mean number of holders of a block.
  int64_t table_entries() const { return table_entries_; }
  int64_t cache_hits() const { return cache_hits_; }
  int64_t cache_misses() const { return cache_misses_; }
  int64_t cache_evictions() const { return cache_evictions_; }
  int64_t cached_blocks() const { return cached_count_; }
  int64_t prefix_nodes() const { return static_cast<int64_t>(nodes_.size() - free_nodes_.size()); }
  const std::vector<int32_t>& refcounts() const { return ref_; }
  void free_queue(int32_t* out) const;  // head to tail, free_count() entries

 private:
  struct Seq {
    std::vector<int32_t> table;
    int32_t len = 0;
    bool alive = false;
    bool known = true;          // its token ids are known (prefix caching)
    int32_t node = -1;          // trie node of its full blocks' prefix (-1: empty prefix)
    std::vector<int32_t> tail;  // ids of the tokens in its partly filled last block
  };
  // A trie node: the prefix of its parent plus one block of B token ids.
  struct PrefixNode {
    int32_t parent = -1;  // -1: the empty prefix
    int32_t block = -1;   // cached block whose key this prefix is, or -1
    int32_t refs = 0;     // child nodes + sequences ending here + (block >= 0)
    uint64_t hash = 0;
  };
  bool valid_seq(int32_t s) const {
    return s >= 0 && s < static_cast<int32_t>(seqs_.size()) && seqs_[s].alive;
  }
  int32_t pop_free();  // head of the free queue; drops its cache entry, if any
  void push_free(int32_t b);
  void unlink_free(int32_t b);
  uint64_t node_hash(int32_t parent, const int32_t* tokens) const;
  int32_t find_node(int32_t parent, const int32_t* tokens) const;
  int32_t get_node(int32_t parent, const int32_t* tokens);
  void pin(int32_t node);
  void release(int32_t node);
  void set_entry(int32_t node, int32_t b);
  void clear_entry(int32_t b);
  void append_ids(Seq& s, int64_t first_token, int32_t n, const int32_t* tokens);

  int32_t num_blocks_;
  int32_t block_size_;
  // Free queue: doubly linked list over block ids (-1 ends).
  std::vector<int32_t> next_, prev_;
  std::vector<char> in_free_;
  int32_t head_ = -1, tail_ = -1;
  int64_t free_count_ = 0;
  // Prefix cache: the trie, its index by (parent, ids) hash, and each block's entry.
  std::vector<PrefixNode> nodes_;
  std::vector<int32_t> node_tokens_;  // B token ids per node
  std::vector<int32_t> free_nodes_;
  std::unordered_multimap<uint64_t, int32_t> index_;
  std::vector<int32_t> block_node_;  // node whose entry the block is, or -1
  int64_t cached_count_ = 0;
  int64_t cache_hits_ = 0, cache_misses_ = 0, cache_evictions_ = 0;
  std::vector<int32_t> ref_;
  std::vector<Seq> seqs_;
  int64_t live_seqs_ = 0;
  int64_t cow_copies_ = 0;
  int64_t alloc_failures_ = 0;
  int64_t table_entries_ = 0;
  bool touched_ = false;  // any allocation happened
};

}  // namespace pa
