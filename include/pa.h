/*
 * pa.h - C ABI of the paged KV-cache decode library (libpa.so, gfx950 / MI355X).
 *
 * What the library implements, and where each piece is defined:
 *
 *  - A KV cache split into fixed-size blocks of `block_size` tokens held in
 *    one physical pool; a per-sequence block table maps logical blocks to
 *    physical ones; blocks are handed out on demand from a free queue
 *    (youngju.dev "KV cache and paged attention", section "PagedAttention:
 *    OS 가상 메모리식 관리"; opsoai "vLLM PagedAttention은 KV 캐시를 어떻게
 *    관리할까", section "PagedAttention은 논리 블록과 물리 블록을 분리한다").
 *  - Allocation gives up when too few free blocks remain (openakashic
 *    KV-cache failure-modes note, Key Points).
 *  - Sequences sharing a prefix point at the same physical blocks with a
 *    reference count, and a shared block is copied when one sharer writes
 *    into it (youngju.dev page, section "prefix 공유와 copy-on-write";
 *    iq-blog ch.4 "Why PagedAttention cuts GPU memory waste", section
 *    "Prefix Caching").
 *  - Decode attention softmax(q K^T / sqrt(d)) V for one new query token per
 *    sequence (youngju.dev page, section "핵심 원리: KV 캐시란 무엇인가"),
 *    computed by a kernel that follows the block table to gather
 *    non-contiguous K/V blocks (iq-blog ch.4, section "PagedAttention
 *    알고리즘"), with query heads grouped onto fewer KV heads (GQA / MQA;
 *    youngju.dev page, section "GQA와 MQA").
 *  - fp8 KV storage at one byte per element (youngju.dev page, section
 *    "KV 양자화: FP8과 INT8"), as OCP E4M3FN with one fp32 scale per
 *    (layer, KV head) for K and one for V.
 *  - int8 KV storage at one byte per element with a scale and a zero point
 *    (same section): code c in [-128, 127], value (c - z) * s, one fp32
 *    scale s and one integer zero point z per (layer, KV head) for K and for
 *    V; a new token is encoded as clamp(rint(x * f32(1/s)) + z, -128, 127)
 *    (ties to even; NaN gives z).
 *
 * Conventions shared by every call:
 *  - Every call returns an int status: PA_OK (0) or a negative PA_ERR_*.
 *    Nothing throws across the ABI.  pa_last_error() returns a thread-local
 *    message describing the most recent failure on the calling thread.
 *  - "host" pointers are ordinary CPU memory; "device" pointers are GPU
 *    memory on the device that was current when the pool was bound.
 *    All device memory (the pool itself, q, out, tables, slot mappings,
 *    workspaces) is owned by the caller; the library keeps raw pointers only
 *    and frees nothing it did not allocate.  Host metadata (free queue,
 *    reference counts, block tables) is owned by the library and released by
 *    pa_pool_destroy.
 *  - `stream` is a hipStream_t (0 = the null stream).  Device work is
 *    enqueued asynchronously on that stream; host-only calls are synchronous.
 *  - A pool is not thread-safe; serialise calls on one pool.
 *  - Integer sizes are int32; byte sizes are uint64.
 *
 * Pool byte layout (device buffer given to pa_pool_bind, 256-byte aligned):
 *    [layers][2 (K, V)][num_blocks][kv_heads][tile]  then a metadata tail
 *    (fp32 scales, inverse scales and int8 zero points, a device status
 *    word).
 *  A tile holds one (block, KV head): block_size x head_dim elements in a
 *  kernel-specific order (K in 16-byte chunks of consecutive dims, V with
 *  4-token x 16-dim sub-tiles).  Use pa_gather_kv to read tokens back in
 *  logical [token][kv_head][dim] order.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes -------------------------------------------------------- */
#define PA_OK 0
#define PA_ERR_INVALID (-1)   /* bad argument, shape or state                  */
#define PA_ERR_NO_BLOCKS (-2) /* not enough free blocks; nothing was changed    */
#define PA_ERR_BAD_SEQ (-3)   /* unknown or freed sequence id                   */
#define PA_ERR_HIP (-4)       /* a HIP runtime call failed                      */
#define PA_ERR_UNBOUND (-5)   /* device call on a pool with no device memory    */

/* ---- KV element types ---------------------------------------------------- */
#define PA_DTYPE_FP16 0     /* IEEE binary16                                   */
#define PA_DTYPE_FP8_E4M3 1 /* OCP E4M3FN: value = decode(code) * scale        */
#define PA_DTYPE_INT8 2     /* int8 code c: value = (c - zero) * scale         */

/* ---- device status bits (pa_device_status) -------------------------------- */
#define PA_DEV_BAD_SLOT 1u  /* a slot >= num_blocks*block_size was skipped      */
#define PA_DEV_BAD_BLOCK 2u /* a table entry outside [0, num_blocks) was read as block 0 */
#define PA_DEV_BAD_LEN 4u   /* a context length < 1 or > max_blocks*block_size  */
#define PA_DEV_BAD_ORDER 8u /* a seq_order entry outside [0, num_seqs) was skipped */

/* ---- K/V load policy of the decode kernels (pa_pool_set_load_policy) -------- */
#define PA_LOADS_AUTO 0      /* cached when used blocks average >= 1.5 holders    */
#define PA_LOADS_STREAMING 1 /* nontemporal loads: every tile read once            */
#define PA_LOADS_CACHED 2    /* ordinary loads: sharers' reads of a tile hit in L2 */

/* ---- pa_decode_noalloc ------------------------------------------------------ */
#define PA_NOALLOC_SCRATCH_BYTES 33554432 /* 32 MiB of static device scratch per GPU */

typedef struct pa_pool pa_pool; /* opaque */

typedef struct pa_pool_info {
  int32_t layers, kv_heads, head_dim, block_size, dtype, num_blocks;
  int32_t elem_bytes; /* 2 (fp16) or 1 (fp8, int8)                            */
  int32_t bound;      /* 1 once pa_pool_bind succeeded                        */
  uint64_t tile_bytes;  /* block_size * head_dim * elem_bytes                  */
  uint64_t kv_bytes;    /* 2 * layers * kv_heads * head_dim * elem_bytes *
                           num_blocks * block_size: the pages' KV-size formula
                           (openakashic note, Key Points; youngju.dev page,
                           section "KV 캐시는 왜 메모리를 먹는가") at full pool */
  uint64_t total_bytes; /* kv_bytes + metadata tail: what pa_pool_bind needs   */
  float softmax_scale;  /* 1/sqrt(head_dim) in fp32, the temperature of
                           softmax(q K^T / sqrt(d)) V (youngju.dev page, section
                           "핵심 원리: KV 캐시란 무엇인가"): the scale to pass to
                           the attention calls when the caller has no other   */
  int32_t reserved;     /* 0                                                    */
} pa_pool_info;

typedef struct pa_stats {
  int64_t num_blocks, free_blocks, used_blocks, shared_blocks;
  int64_t num_seqs, cow_copies, alloc_failures;
  /* prefix cache (pa_seq_create_cached): full prompt blocks served from and
   * missed by the cache, entries dropped because their block was reused, and
   * entries held now */
  int64_t cache_hits, cache_misses, cache_evictions, cached_blocks;
} pa_stats;

typedef struct pa_profile {
  int32_t decode_launches, reduce_launches;
  double decode_ms, reduce_ms; /* summed HIP-event durations on the launch stream */
} pa_profile;

/* ---- pool ------------------------------------------------------------------ */

/* Create a pool descriptor: per layer, K and V pools of `num_blocks` blocks of
 * `block_size` tokens x `kv_heads` x `head_dim` (the fixed-size blocks of one
 * physical pool: youngju.dev page, section "PagedAttention: OS 가상 메모리식
 * 관리"; their bytes are the KV-size formula of section "KV 캐시는 왜 메모리를
 * 먹는가").  Supported: head_dim 64 or 128, block_size 8/16/32, dtype PA_DTYPE_*,
 * num_blocks*block_size < 2^31.  Anything else: PA_ERR_INVALID, *out = NULL.
 * No device memory is touched; host-side block management works unbound. */
int pa_pool_create(int32_t layers, int32_t kv_heads, int32_t head_dim, int32_t block_size,
                   int32_t dtype, int32_t num_blocks, pa_pool** out);

/* Release the host metadata (the caller frees the device buffer). NULL is a no-op.
 * (Library housekeeping; not a step of the method.) */
int pa_pool_destroy(pa_pool* pool);

/* Geometry, byte sizes and default softmax scale of a pool (pa_pool_info);
 * PA_ERR_INVALID for NULL arguments. */
int pa_pool_info_get(const pa_pool* pool, pa_pool_info* out);

/* How the decode kernels load K/V tiles (not a step of the method; results do
 * not depend on it).  Sequences that share a prefix read identical blocks
 * (youngju.dev page, section "prefix 공유와 copy-on-write"): with ordinary
 * loads their reads of a shared tile are served by L2, with nontemporal
 * loads a tile read once streams past the caches at a higher rate.
 * PA_LOADS_AUTO (the default) takes ordinary loads when the pool's used
 * blocks are named by at least 1.5 block-table entries on average, else
 * nontemporal ones.  PA_ERR_INVALID for an unknown policy.
 * pa_pool_load_policy returns the policy and (cached_now_out, may be NULL)
 * whether a decode launched now would use ordinary loads. */
int pa_pool_set_load_policy(pa_pool* pool, int32_t policy);
int pa_pool_load_policy(const pa_pool* pool, int32_t* policy_out, int32_t* cached_now_out);

/* Replace the initial free-queue order by a permutation of 0..num_blocks-1
 * (host int32[n], n == num_blocks).  Only valid before the first allocation,
 * else PA_ERR_INVALID.  The queue is the pool's free list (openakashic note,
 * Key Points: "free queue"; iq-blog ch.4, section "OS Paging에서 가져온 해법");
 * a seeded permutation places blocks at random physical positions. */
int pa_pool_set_free_order(pa_pool* pool, const int32_t* perm, int32_t n);

/* Attach caller-owned device memory of info.total_bytes, 256-byte aligned
 * (the physical pool of youngju.dev page, section "PagedAttention: OS 가상
 * 메모리식 관리"; fp8 scales: section "KV 양자화: FP8과 INT8").
 * fp8 pools need host fp32 scales k_scales[layers*kv_heads] and v_scales[...]
 * (layer-major); fp16 pools pass NULL.  The library writes the scales, their
 * fp32 reciprocals and a zeroed status word into the tail (synchronously). */
int pa_pool_bind(pa_pool* pool, void* dev_base, const float* k_scales, const float* v_scales);

/* The same for int8 pools (pa_pool_bind refuses them; youngju.dev page,
 * section "KV 양자화: FP8과 INT8": one byte per element needs a scale and a
 * zero point): host fp32 scales and
 * host int32 zero points in [-128, 127], each [layers*kv_heads] layer-major,
 * for K and for V.  Scales must be positive and finite; otherwise, or for a
 * zero point out of range, PA_ERR_INVALID and nothing is bound.  Inside the
 * pool an int8 code c is kept as the byte c + 128; pa_gather_kv returns c. */
int pa_pool_bind_int8(pa_pool* pool, void* dev_base, const float* k_scales, const float* v_scales,
                      const int32_t* k_zeros, const int32_t* v_zeros);

/* ---- block manager (host) ------------------------------------------------------ */

/* New empty sequence with an empty block table (youngju.dev page, section
 * "PagedAttention: OS 가상 메모리식 관리": one block table per request); ids
 * are 0, 1, 2, ... in creation order, never reused.  PA_ERR_INVALID for NULL. */
int pa_seq_create(pa_pool* pool, int32_t* seq_out);

/* Automatic prefix caching (iq-blog ch.4, section "Prefix Caching";
 * youngju.dev page, section "prefix 캐시의 수명과 무효화"; openakashic note,
 * Key Points).  New sequence holding the prompt tokens[n] (host int32 token
 * ids): its leading full blocks are taken from the prefix cache as far as the
 * prompt matches a cached prefix block by block (reference count + 1; a block
 * that sat in the free queue leaves it), the rest is allocated like
 * pa_alloc, and the prompt's newly allocated full blocks are entered in the
 * cache (later appends with ids enter the blocks they fill: pa_alloc_tokens).  *cached_out = tokens whose K/V the pool already holds (a multiple
 * of block_size); slots_out (host int32[n]) receives the slots of tokens
 * cached_out .. n-1, which the caller writes with pa_write_kv.  Freed cached
 * blocks keep their entry at the free-queue tail and lose it when the queue
 * hands them out again (least recently freed first).  The key of a block is
 * the whole token prefix up to its end, compared exactly (a trie of blocks:
 * the parent prefix and the block's ids), so different prefixes never share.
 * PA_ERR_NO_BLOCKS if the rest does not fit: nothing changes, no id is used. */
int pa_seq_create_cached(pa_pool* pool, const int32_t* tokens, int32_t n, int32_t* seq_out,
                         int32_t* cached_out, int32_t* slots_out);

/* Blocks on demand as a sequence grows (youngju.dev page, section
 * "PagedAttention: OS 가상 메모리식 관리"; copy-on-write: section "prefix 공유와
 * copy-on-write"; failure: openakashic note, Key Points).
 * Append n_tokens >= 0 tokens to `seq`.  slots_out (host int32[n_tokens]):
 * slot of the j-th new token = table[t / B] * B + t % B, t = old_len + j.
 * If the append lands in a partly filled last block shared with another
 * sequence, that block is copied first into a fresh block which replaces it
 * in this sequence's table (copy-on-write, the writer receives the copy);
 * cow_out (host int32[2], may be NULL) receives {src, dst} or {-1, -1}.  On a
 * bound pool the copy (all layers, K and V) is enqueued on `stream` before
 * returning, so later pa_write_kv calls on that stream see it.
 * Atomic: on PA_ERR_NO_BLOCKS (the copy's block counts toward the need)
 * nothing changes. */
int pa_alloc(pa_pool* pool, int32_t seq, int32_t n_tokens, int32_t* slots_out,
             int32_t* cow_out, void* stream);

/* pa_alloc with the appended tokens' ids (host int32[n_tokens]; NULL makes it
 * pa_alloc).  While a sequence's ids are known (it was created empty or with
 * a prompt, and every append gave ids; a fork inherits its parent's), every
 * block an append fills is entered in the prefix cache under the sequence's
 * whole token prefix, so a later prompt that extends it (the next turn of a
 * conversation: youngju.dev page, section "prefix 공유와 copy-on-write") is
 * served from the cache (pa_seq_create_cached).  An append without ids ends
 * that for the sequence.  Errors as pa_alloc. */
int pa_alloc_tokens(pa_pool* pool, int32_t seq, int32_t n_tokens, const int32_t* tokens,
                    int32_t* slots_out, int32_t* cow_out, void* stream);

/* Batched appends (the same pages as pa_alloc): for k = 0 .. count-1 in order,
 * append n_tokens[k] >= 0
 * tokens to seqs[k] exactly as pa_alloc_tokens would (the same allocator state
 * and slots), the slots back to back in slots_out (host int32[sum of n_tokens]).
 * tokens: the appended ids back to back (host int32[sum of n_tokens]), or NULL
 * for appends without ids.
 * The copy-on-write copies of the whole batch are enqueued on `stream` in one
 * launch (per 64 copies) after the appends, instead of one launch per copy:
 * every copy's destination is a fresh block private to its sequence, so the
 * copies do not depend on one another.  cow_out (host int32[2*count], may be
 * NULL): each append's {src, dst} or {-1, -1}.  done_out (may be NULL): the
 * number of appends made.  On a failing append k the appends before it stay
 * made (their copies enqueued), append k changes nothing, and its status is
 * returned (PA_ERR_NO_BLOCKS when the pool runs out). */
int pa_alloc_batch(pa_pool* pool, const int32_t* seqs, const int32_t* n_tokens, int32_t count,
                   const int32_t* tokens, int32_t* slots_out, int32_t* cow_out, int32_t* done_out,
                   void* stream);

/* New sequence sharing every block of `parent` (each reference count + 1):
 * sequences with a common prefix point at the same physical blocks
 * (youngju.dev page, section "prefix 공유와 copy-on-write"; opsoai page,
 * section "KV 캐시는 왜 요청이 늘수록 서빙 병목이 되는가": beams share their
 * prefix).  PA_ERR_BAD_SEQ for an unknown or freed parent. */
int pa_fork(pa_pool* pool, int32_t parent, int32_t* child_out);

/* Drop `seq`: its blocks are visited last to first, and each one whose
 * reference count reaches zero is appended to the free-queue tail (blocks
 * return to the free list when a request ends: iq-blog ch.4, section "OS
 * Paging에서 가져온 해법"; openakashic note, Key Points).  PA_ERR_BAD_SEQ for an
 * unknown or freed sequence. */
int pa_free(pa_pool* pool, int32_t seq);

/* Tokens and blocks of `seq` (either out pointer may be NULL); PA_ERR_BAD_SEQ
 * for an unknown or freed sequence. */
int pa_seq_len(const pa_pool* pool, int32_t seq, int32_t* len_out, int32_t* num_blocks_out);

/* Export block tables (logical block -> physical block, youngju.dev page,
 * section "PagedAttention: OS 가상 메모리식 관리"; int32 entries, iq-blog ch.4,
 * section "vLLM의 4-Layer 통합 아키텍처"): tables_out host int32[n][max_blocks]
 * (rows padded with -1), lens_out host int32[n].  PA_ERR_INVALID if a table is
 * longer than max_blocks, PA_ERR_BAD_SEQ for an unknown sequence. */
int pa_block_tables(const pa_pool* pool, const int32_t* seqs, int32_t n, int32_t max_blocks,
                    int32_t* tables_out, int32_t* lens_out);

/* The pool's block, sequence, copy-on-write and prefix-cache counters
 * (pa_stats; inspection, not a step of the method). */
int pa_pool_stats(const pa_pool* pool, pa_stats* out);

/* Allocator state for inspection (the reference counts of youngju.dev page,
 * section "prefix 공유와 copy-on-write", and the free queue of the openakashic
 * note, Key Points): reference count of every block (host
 * int32[num_blocks]); the free queue head to tail (host int32[num_blocks],
 * *n_out = number of free blocks). */
int pa_refcounts(const pa_pool* pool, int32_t* out);
int pa_free_queue(const pa_pool* pool, int32_t* out, int32_t* n_out);

/* ---- device operations ---------------------------------------------------------- */

/* Reshape-and-cache scatter (slot = block * block_size + offset: youngju.dev
 * page, section "PagedAttention: OS 가상 메모리식 관리"; one-byte elements:
 * section "KV 양자화: FP8과 INT8"): token t's K and V (device fp16 [n][kv_heads][head_dim],
 * 16-byte aligned) go to slot slot_mapping[t] (device int32[n]) of `layer`; negative slots are
 * skipped.  fp8 pools store encode(f32(x) * f32(1/scale)) with saturation to
 * +-448 and round-to-nearest-even; int8 pools store
 * clamp(rint(f32(x) * f32(1/scale)) + zero, -128, 127). */
int pa_write_kv(pa_pool* pool, int32_t layer, const void* k_new, const void* v_new,
                const int32_t* slot_mapping, int32_t n_tokens, void* stream);

/* Inverse of pa_write_kv (for tests and inspection; slot arithmetic as there):
 * read the stored K/V of each slot into device
 * k_out/v_out [n][kv_heads][head_dim] (fp16 values, raw uint8 codes for fp8,
 * int8 codes c for int8).
 * Negative slots leave their rows untouched. */
int pa_gather_kv(const pa_pool* pool, int32_t layer, const int32_t* slot_mapping,
                 int32_t n_tokens, void* k_out, void* v_out, void* stream);

/* Measurement reference, not part of the method: a kernel that only reads
 * `bytes` (a multiple of 16) of device memory at `buf` (16-byte aligned) with
 * 16-byte nontemporal loads, the best plain streaming read found on MI355X;
 * `sink` is a device uint32 it may write.  Its rate is the practical read
 * ceiling the decode kernel is compared with. */
int pa_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, void* stream);

/* Copy whole blocks src[i] -> dst[i] (host int32[n]) across all layers, K and V:
 * the copy of copy-on-write (youngju.dev page, section "prefix 공유와
 * copy-on-write").  PA_ERR_INVALID for a block id outside the pool. */
int pa_copy_blocks(pa_pool* pool, const int32_t* src, const int32_t* dst, int32_t n, void* stream);

/* Device bytes of the workspace pa_decode needs for this launch shape
 * (0 when it runs in a single pass).  partition_tokens as in pa_decode.
 * (Split-context partials are not on the pages: a softmax over a union of
 * disjoint chunks, merged by log-sum-exp.) */
int pa_decode_workspace_bytes(const pa_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                              int32_t max_blocks, int32_t partition_tokens, uint64_t* bytes_out);

/* Paged decode attention for one layer: softmax(q K^T * scale) V over each
 * sequence's cached tokens (youngju.dev page, section "핵심 원리: KV 캐시란
 * 무엇인가"), K/V gathered through the block table (iq-blog ch.4, section
 * "PagedAttention 알고리즘"), query heads grouped onto KV heads (youngju.dev
 * page, section "GQA와 MQA").
 *   q            device fp16 [num_seqs][num_q_heads][head_dim], 16-byte aligned
 *   block_tables device int32 [num_seqs][max_blocks] (entries past a sequence's
 *                last block are ignored)
 *   context_lens device int32 [num_seqs], 1 <= T_i <= max_blocks*block_size,
 *                the tokens each query attends to (the new one included)
 *   scale        softmax temperature, normally 1/sqrt(head_dim)
 *   out          device fp16 [num_seqs][num_q_heads][head_dim], 8-byte aligned
 * Query head h reads KV head h / (num_q_heads / kv_heads); num_q_heads must
 * be a multiple of kv_heads with a group of at most 32.
 * partition_tokens: 0 lets the library choose (one pass per (sequence, KV
 * head) when num_seqs * kv_heads >= U or max_blocks * block_size <= 1024;
 * otherwise ceil(U / (num_seqs * kv_heads)) chunks per context, where U is the
 * device's CU count, doubled when a KV head serves more than 16 query
 * heads); -1 forces one pass per (sequence, KV head); P > 0 (a
 * multiple of 16 and of block_size) splits each context into chunks of P
 * tokens whose partials are merged by log-sum-exp.
 * seq_order: NULL, or device int32 [num_seqs], a permutation of 0..num_seqs-1
 * giving the order in which workgroups take the sequences.  Results do not
 * depend on it; with uneven lengths, longest first (pa_order_longest_first)
 * keeps long sequences from starting last and idling the other CUs.  An entry
 * outside [0, num_seqs) sets PA_DEV_BAD_ORDER and is skipped; a repeated entry
 * leaves some sequence's output unwritten.
 * workspace: device memory of pa_decode_workspace_bytes() bytes, 16-byte
 * aligned (may be NULL when that is 0).  Out-of-range table entries or lengths never cause an
 * out-of-bounds access; they set PA_DEV_* bits instead.  num_seqs = 0 launches
 * nothing (q, block_tables, context_lens, out and workspace may then be NULL). */
int pa_decode(pa_pool* pool, int32_t layer, const void* q, int32_t num_q_heads,
              const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
              int32_t num_seqs, const int32_t* seq_order, float scale, int32_t partition_tokens,
              void* out, void* workspace, uint64_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): pa_decode
 * with the same arguments and results, minus the workspace.  When the plan
 * splits contexts, the chunk partials go to a static device array of
 * PA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends; a launch whose partials need more
 * (pa_decode_workspace_bytes > PA_NOALLOC_SCRATCH_BYTES) fails with
 * PA_ERR_INVALID and launches nothing.  The call allocates nothing (no
 * hipMalloc, no host allocation).  Every call on one GPU shares that array,
 * written before it is read within a call (nothing needs clearing): calls
 * that overlap on one GPU (several streams or host threads at once) race.
 * The current device must be the pool's. */
int pa_decode_noalloc(pa_pool* pool, int32_t layer, const void* q, int32_t num_q_heads,
                      const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                      int32_t num_seqs, const int32_t* seq_order, float scale, int32_t partition_tokens,
                      void* out, void* stream);

/* One decode step fused (passages as for pa_write_kv and pa_decode): the
 * scatter of pa_write_kv and the attention of pa_decode in one launch.  k_new, v_new: device fp16 [num_seqs][kv_heads]
 * [head_dim], 16-byte aligned, the new token of every sequence; slot_mapping: device int32
 * [num_seqs].  Each sequence's new token must be its last one, T_i - 1, at
 * the slot its block table gives that token (what pa_alloc returned for it);
 * then the result equals pa_write_kv(layer, k_new, v_new, slot_mapping,
 * num_seqs) followed by pa_decode(...) with the same arguments, pool contents
 * included.  A negative slot skips the store (the pool's copy of token
 * T_i - 1 is used); any other slot sets PA_DEV_BAD_SLOT and is skipped too.
 * The wave that attends over token T_i - 1 takes it from k_new / v_new (as the
 * pool will hold it: fp16, or its E4M3FN or int8 code) and then stores it. */
int pa_write_kv_decode(pa_pool* pool, int32_t layer, const void* k_new, const void* v_new,
                       const int32_t* slot_mapping, const void* q, int32_t num_q_heads,
                       const int32_t* block_tables, int32_t max_blocks,
                       const int32_t* context_lens, int32_t num_seqs, const int32_t* seq_order,
                       float scale, int32_t partition_tokens, void* out, void* workspace,
                       uint64_t workspace_bytes, void* stream);

/* Shared-prefix decode.  Sequences whose block tables begin with the same
 * blocks (beams of one search, requests on one cached system prompt) read
 * identical K/V there (youngju.dev page, section "prefix 공유와 copy-on-write";
 * iq-blog ch.4, section "Prefix Caching"): the attention of each sequence is
 * split at the end of the shared blocks.  In one launch, some workgroups read
 * chunks of a group's shared blocks once for all its members' query heads
 * while others attend to each sequence's own remaining tokens; a second,
 * short launch merges each grouped sequence's pieces by log-sum-exp.  The
 * result is that of pa_decode (pa_write_kv_decode when k_new, v_new and
 * slot_mapping are given) up to rounding.
 *
 * pa_shared_prefix_groups (host only) finds groups from host block tables
 * (host int32 [n][max_blocks], lens [n]): sequences with the same first
 * block, sharing the longest common run of block ids that lies before every
 * member's last token, rounded down to whole 16-token steps; a run shorter
 * than min_shared_tokens leaves its sequences alone.  Outputs: members_out
 * (host int32 [n]) the sequences group by group, group_start_out (host int32
 * [n + 1]) each group's first member, shared_blocks_out (host int32 [n]) the
 * group's shared blocks (0: no shared pass), *num_groups_out.
 *
 * pa_shared_prefix_plan checks such groups (host arrays; members a
 * permutation of 0..num_seqs-1, group_start non-decreasing from
 * group_start[0] = 0 to group_start[num_groups] = num_seqs, each
 * shared_blocks[g] at most max_blocks and times block_size a multiple of
 * 16) for a batch of num_seqs sequences with num_q_heads query heads
 * and block tables max_blocks wide, and uploads on `stream` the group list
 * into `workspace` (device memory of
 * pa_decode_shared_prefix_workspace_bytes() bytes for the same groups and
 * chunk_tokens, 16-byte aligned, owned by the caller, which keeps it alive
 * while the plan is used).  chunk_tokens: shared tokens per workgroup, a
 * multiple of 64, or 0 for the library's choice (about one shared
 * workgroup per CU, at least 256 tokens).  lens: the host context lengths
 * (int32 [num_seqs]) or NULL; with them, a group whose members all have at
 * most 128 tokens past the shared run is folded: one workgroup per member
 * run streams the shared tokens and then each member's own tokens, with no
 * partials and no merge (beams of one search).  They only steer the plan;
 * the launch reads the device lengths.  It fills *plan; bad group arrays
 * give PA_ERR_INVALID and upload nothing.  One plan serves every layer of a
 * step: the group list is uploaded once.
 *
 * pa_decode_shared_prefix runs one layer on a plan: q, block_tables,
 * context_lens, scale and out as in pa_decode with the plan's num_seqs,
 * num_q_heads and max_blocks.  The caller guarantees what the plan cannot
 * see on the host: every member's table holds its group's shared blocks
 * first, and its context has more tokens than them (a context at or below
 * them sets PA_DEV_BAD_LEN and gives the shared tokens' attention alone).
 * k_new, v_new, slot_mapping: all NULL, or the fused scatter of
 * pa_write_kv_decode (the new token lies past the shared blocks, in the
 * sequence's own piece).  The partials live in the plan's workspace: calls
 * on one plan must be on one stream, in order, and a later
 * plan on the same workspace replaces it (the kernels check every index they
 * take from the workspace: a stale plan can give wrong rows, never an access
 * outside the batch or the workspace). */
int pa_shared_prefix_groups(const pa_pool* pool, const int32_t* tables, const int32_t* lens, int32_t n,
                            int32_t max_blocks, int32_t min_shared_tokens, int32_t* members_out,
                            int32_t* group_start_out, int32_t* shared_blocks_out, int32_t* num_groups_out);
int pa_decode_shared_prefix_workspace_bytes(const pa_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                                            const int32_t* members, const int32_t* group_start,
                                            const int32_t* shared_blocks, int32_t num_groups,
                                            int32_t max_blocks, int32_t chunk_tokens, const int32_t* lens,
                                            uint64_t* bytes_out);
#define PA_SHARED_REREAD 1 /* pa_shared_plan.flags: several items read one shared chunk */
typedef struct pa_shared_plan {
  const pa_pool* pool;       /* the pool the plan was made for */
  int32_t num_seqs, num_q_heads, max_blocks;
  int32_t num_items;         /* shared work items (each a workgroup per KV head) */
  int32_t num_slots;         /* partial slots: shared chunks + 1 for every grouped sequence */
  int32_t chunk_tokens;      /* shared tokens per work item */
  int32_t num_private;       /* sequences with a private piece (not in a folded group) */
  int32_t flags;             /* PA_SHARED_REREAD: several items read one chunk (ordinary loads) */
  void* workspace;           /* the caller's workspace, as passed to the plan */
  uint64_t workspace_bytes;
} pa_shared_plan;
int pa_shared_prefix_plan(pa_pool* pool, int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks,
                          const int32_t* members, const int32_t* group_start, const int32_t* shared_blocks,
                          int32_t num_groups, int32_t chunk_tokens, const int32_t* lens, void* workspace,
                          uint64_t workspace_bytes, void* stream, pa_shared_plan* plan);
int pa_decode_shared_prefix(pa_pool* pool, int32_t layer, const pa_shared_plan* plan, const void* q,
                            const int32_t* block_tables, const int32_t* context_lens, const void* k_new,
                            const void* v_new, const int32_t* slot_mapping, float scale, void* out,
                            void* stream);

/* Multi-token paged attention: causal attention for several new query
 * tokens per sequence, i.e. prefill chunks and decode tokens mixed in one
 * batch (youngju.dev page, section "핵심 원리: KV 캐시란 무엇인가": a token's
 * query meets the keys and values of itself and all earlier tokens; iq-blog
 * ch.4: the scheduler mixes prefill and decode requests in one batch).
 *   query_start  HOST int32 [num_seqs + 1], query_start[0] = 0, non-decreasing:
 *                sequence i owns query rows query_start[i] .. query_start[i+1]-1,
 *                its last n_i = query_start[i+1] - query_start[i] tokens
 *                (n_i = 0: nothing; 1: a decode token; more: a prefill chunk)
 *   q, out       device fp16 [query_start[num_seqs]][num_q_heads][head_dim]
 *                (16- and 8-byte aligned)
 *   block_tables, max_blocks, context_lens, scale  as in pa_decode (scale
 *                nonzero); the K/V of every query token must already be in
 *                the pool (pa_write_kv), and T_i >= n_i
 * Row j of sequence i (0-based) sits at position T_i - n_i + j and attends
 * to tokens 0 .. T_i - n_i + j through the block table.  A sequence with
 * T_i < n_i or T_i > max_blocks*block_size sets PA_DEV_BAD_LEN and its rows
 * are zeros.  workspace: device memory of pa_multi_token_workspace_bytes()
 * bytes (16 per tile of query tokens), 16-byte aligned; the library uploads
 * its work list there on `stream` from pinned host memory it owns (a ring of
 * 16 buffers: a call waits only for the upload made 16 calls earlier).  Calls
 * that share a workspace must be on the same stream.  With no query rows
 * (query_start[num_seqs] = 0) nothing is launched, and q, out and workspace
 * may be NULL. */
int pa_multi_token_workspace_bytes(const pa_pool* pool, const int32_t* query_start, int32_t num_seqs,
                                   int32_t num_q_heads, uint64_t* bytes_out);
int pa_multi_token_attention(pa_pool* pool, int32_t layer, const void* q, int32_t num_q_heads,
                             const int32_t* query_start, const int32_t* block_tables, int32_t max_blocks,
                             const int32_t* context_lens, int32_t num_seqs, float scale, void* out,
                             void* workspace, uint64_t workspace_bytes, void* stream);

/* Host helper (scheduling, not a step of the method): order_out[0..n) =
 * indices of lens[0..n) by decreasing length,
 * equal lengths in increasing index (a stable sort), for pa_decode's seq_order. */
int pa_order_longest_first(const int32_t* lens, int32_t n, int32_t* order_out);

/* The two halves of a partitioned pa_decode, callable separately (not on the
 * pages: the chunked softmax and its log-sum-exp merge).
 * pa_decode_partials writes, for chunk c of every (sequence, query head), into
 * the workspace laid out as three consecutive fp32 arrays of C = ceil(max_blocks
 * * block_size / P) chunks each:
 *    m[num_seqs][num_q_heads][C]   max score of the chunk in base-2 units,
 *                                  max_t (q.k_t * scale * log2 e)
 *    l[num_seqs][num_q_heads][C]   sum_t 2^(s_t - m)
 *    o[num_seqs][num_q_heads][C][head_dim]  sum_t 2^(s_t - m) v_t / l
 * Chunks at or past ceil(T_i / P) are not written.
 * pa_lse_reduce merges chunks 0 .. ceil(T_i/P)-1 into out:
 *    out = sum_c w_c o_c / sum_c w_c,  w_c = l_c * 2^(m_c - max_c m_c).
 * Both take the workspace 16-byte aligned and out 8-byte aligned, as
 * pa_decode does (PA_ERR_INVALID otherwise). */
int pa_decode_partials(pa_pool* pool, int32_t layer, const void* q, int32_t num_q_heads,
                       const int32_t* block_tables, int32_t max_blocks,
                       const int32_t* context_lens, int32_t num_seqs, const int32_t* seq_order,
                       float scale, int32_t partition_tokens, void* workspace,
                       uint64_t workspace_bytes, void* stream);
int pa_lse_reduce(pa_pool* pool, const void* workspace, uint64_t workspace_bytes,
                  const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                  int32_t max_blocks, int32_t partition_tokens, void* out, void* stream);

/* Read (and optionally clear) the pool's device status word (PA_DEV_* bits:
 * contract violations the kernels detected and skipped); synchronises `stream`. */
int pa_device_status(pa_pool* pool, uint32_t* flags_out, int32_t clear, void* stream);

/* Kernel timing (measurement, not a step of the method): while enabled, the
 * pa_decode / pa_decode_partials launches
 * numbered 0, every, 2*every, ... since pa_profile_begin (up to max_launches of
 * them; every >= 1, 1 = all) are dispatched with HIP start/stop events that
 * the dispatch itself stamps at the kernel's start and end on the launch
 * stream (hipExtLaunchKernel), for the attention kernel and for the reduce
 * kernel; no extra packets are enqueued.  pa_profile_end synchronises those
 * events, returns the summed durations and disables timing. */
int pa_profile_begin(pa_pool* pool, int32_t max_launches, int32_t every);
int pa_profile_end(pa_pool* pool, pa_profile* out);

/* Message of the last failure on this thread ("" if none). */
const char* pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
