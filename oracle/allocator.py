"""Reference block manager (integers only; the GPU library must match it bit for bit).

What the pages fix:

* KV is split into fixed-size blocks; each request keeps a block table from
  logical block index to physical block, and blocks are handed out on demand
  as tokens accumulate (youngju.dev "KV cache and paged attention", section
  "PagedAttention: OS 가상 메모리식 관리"; opsoai "vLLM PagedAttention은 KV
  캐시를 어떻게 관리할까", section "PagedAttention은 논리 블록과 물리 블록을
  분리한다"; iq-blog ch.4, sections "OS Paging에서 가져온 해법" and
  "PagedAttention 알고리즘").
* Free blocks live in a free list / free queue, and an allocation is given up
  when not enough free blocks remain (openakashic KV-cache failure-modes note,
  Key Points; iq-blog ch.4, "OS Paging에서 가져온 해법").
* Sequences with a common prefix point at the same physical blocks with a
  reference count; a shared block is copied at the moment one sharer writes
  into it (copy-on-write) (youngju.dev page, section "prefix 공유와
  copy-on-write"; iq-blog ch.4, "Prefix Caching").

Readings where the pages are silent (each also listed in the design notes):

* The free queue is FIFO; its initial order is the caller's permutation (or
  0..N-1).  Allocation pops from the head.  When a sequence is freed, its
  blocks are visited last-to-first and every block whose count drops to zero
  is pushed to the tail.
* An append that needs more blocks than are free fails with no state change;
  the block a copy-on-write needs counts toward the requirement.
* Copy-on-write triggers only when the append lands in a partly filled last
  block whose count exceeds one; the appending sequence receives the copy.
* Sequence ids are 0, 1, 2, ... in creation order and are never reused.

Automatic prefix caching (iq-blog ch.4, section "Prefix Caching": identical
prefixes are found by a hash of the prefix and their blocks shared with a
reference count; youngju.dev page, section "prefix 캐시의 수명과 무효화": hits
reuse blocks, old prefixes are evicted least recently used first; openakashic
note, Key Points: a cached block taken from the free queue for a new
allocation loses its prefix entry).  Readings:

* A sequence's token ids are known when it was created with a prompt (or
  empty) and every append gave its token ids; a tokenless append makes them
  unknown for good.  Every full block of a sequence with known ids is
  cached: the prompt's full blocks at creation, and each block an append
  fills, when it fills (so a later turn of a conversation hits on the blocks
  generated in an earlier one: youngju.dev page, section "prefix 공유와
  copy-on-write", names multi-turn history as a shared prefix).  A fork
  inherits its parent's ids.  The key of a block is the whole token prefix
  up to its end (here the tuple itself, so the oracle is exact; the library
  compares the same prefixes exactly, block by block).
* Lookup walks the prompt's full blocks in order and stops at the first miss;
  a hit takes the block (count + 1), out of the free queue if it sat there.
* The rest of the prompt is allocated like an append; its full blocks are then
  registered (replacing an entry with the same key).
* Freed cached blocks keep their entry at the free-queue tail, so the least
  recently freed is reused (and evicted) first.
* A creation that needs more free blocks than remain (hits taken out of the
  queue do not count as free) fails and changes nothing; no id is used.
"""
from __future__ import annotations

from collections import deque


class NoBlocks(Exception):
    """Raised when an append needs more free blocks than the pool holds."""


class BadSeq(Exception):
    """Raised for an unknown or already-freed sequence id."""


class OracleAllocator:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = list(range(self.num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(self.num_blocks)):
            raise ValueError("free_order must be a permutation of range(num_blocks)")
        self.free = deque(order)
        self.ref = [0] * self.num_blocks
        self.tables = {}  # seq id -> list of physical block ids
        self.lens = {}  # seq id -> number of tokens
        self.tokens = {}  # seq id -> its token ids, or None when unknown
        self.next_id = 0
        self.cow_log = []  # (src, dst) in the order they happened
        self.failures = 0
        self.cache = {}  # prefix token tuple -> block
        self.block_key = [None] * self.num_blocks  # block -> its prefix key, if cached
        self.cache_hits = 0
        self.cache_misses = 0
        self.evictions = 0

    # -- sequence lifecycle ------------------------------------------------
    def seq_create(self) -> int:
        sid = self.next_id
        self.next_id += 1
        self.tables[sid] = []
        self.lens[sid] = 0
        self.tokens[sid] = []
        return sid

    def _check(self, sid):
        if sid not in self.tables:
            raise BadSeq(sid)

    def alloc(self, sid: int, n: int, tokens=None):
        """Append ``n`` tokens to ``sid``; return (slots, cow) where cow is (src, dst) or None.

        Slot of logical token t is table[t // B] * B + t % B (the block table maps
        the logical block to its physical block; the offset within the block is kept).
        ``tokens``: the appended token ids (``n`` of them), or None; with ids,
        every block the append fills is entered in the prefix cache.
        """
        self._check(sid)
        if n < 0:
            raise ValueError("n must be >= 0")
        if tokens is not None:
            tokens = [int(t) for t in tokens]
            if len(tokens) != n:
                raise ValueError("tokens must hold n ids")
        bs = self.block_size
        table = self.tables[sid]
        length = self.lens[sid]
        need = -(-(length + n) // bs) - len(table)
        cow = n > 0 and length % bs != 0 and self.ref[table[-1]] > 1
        if need + int(cow) > len(self.free):
            self.failures += 1
            raise NoBlocks(sid)
        cow_pair = None
        if cow:
            old = table[-1]
            new = self._take_free()
            self.ref[new] = 1
            self.ref[old] -= 1
            table[-1] = new
            cow_pair = (old, new)
            self.cow_log.append(cow_pair)
        for _ in range(need):
            b = self._take_free()
            self.ref[b] = 1
            table.append(b)
        slots = [table[(length + j) // bs] * bs + (length + j) % bs for j in range(n)]
        self.lens[sid] = length + n
        if n > 0:
            if tokens is None or self.tokens[sid] is None:
                self.tokens[sid] = None
            else:
                ids = self.tokens[sid]
                ids.extend(tokens)
                for i in range(length // bs, (length + n) // bs):  # the blocks this append filled
                    self._register(tuple(ids[:(i + 1) * bs]), table[i])
        return slots, cow_pair

    def _register(self, key, b):
        """Enter block ``b`` under the prefix ``key`` (replacing an entry with the same key)."""
        old = self.cache.get(key)
        if old is not None:
            self.block_key[old] = None
        self.cache[key] = b
        self.block_key[b] = key

    def _take_free(self) -> int:
        """Pop the free-queue head; a cached block loses its prefix entry."""
        b = self.free.popleft()
        key = self.block_key[b]
        if key is not None:
            if self.cache.get(key) == b:
                del self.cache[key]
            self.block_key[b] = None
            self.evictions += 1
        return b

    def seq_create_cached(self, tokens):
        """New sequence holding the prompt ``tokens``; returns (sid, cached, slots).

        ``cached`` tokens (whole leading blocks) already have their K/V in the
        pool; ``slots`` are the slots of the remaining tokens, to be written.
        """
        tokens = [int(t) for t in tokens]
        bs = self.block_size
        n = len(tokens)
        full = n // bs
        hits = []
        for i in range(full):
            b = self.cache.get(tuple(tokens[:(i + 1) * bs]))
            if b is None:
                break
            hits.append(b)
        h = len(hits)
        need = -(-(n - h * bs) // bs)
        revived = sum(1 for b in hits if self.ref[b] == 0)
        if need > len(self.free) - revived:
            self.failures += 1
            raise NoBlocks(tokens[:8])
        sid = self.seq_create()
        table = self.tables[sid]
        for b in hits:
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1
            table.append(b)
        self.cache_hits += h
        self.cache_misses += full - h
        for _ in range(need):
            b = self._take_free()
            self.ref[b] = 1
            table.append(b)
        for i in range(h, full):
            self._register(tuple(tokens[:(i + 1) * bs]), table[i])
        self.lens[sid] = n
        self.tokens[sid] = list(tokens)
        slots = [table[t // bs] * bs + t % bs for t in range(h * bs, n)]
        return sid, h * bs, slots

    def fork(self, parent: int) -> int:
        """New sequence sharing every block of ``parent`` (each count +1)."""
        self._check(parent)
        sid = self.seq_create()
        self.tables[sid] = list(self.tables[parent])
        self.lens[sid] = self.lens[parent]
        self.tokens[sid] = None if self.tokens[parent] is None else list(self.tokens[parent])
        for b in self.tables[sid]:
            self.ref[b] += 1
        return sid

    def free_seq(self, sid: int) -> None:
        """Drop ``sid``; blocks whose count reaches zero go to the free-queue tail."""
        self._check(sid)
        for b in reversed(self.tables[sid]):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.tables[sid]
        del self.lens[sid]
        del self.tokens[sid]

    # -- views ---------------------------------------------------------------
    def block_tables(self, seqs, max_blocks: int):
        """Rows of physical ids padded with -1, and the lengths."""
        rows, lens = [], []
        for s in seqs:
            self._check(s)
            t = self.tables[s]
            if len(t) > max_blocks:
                raise ValueError("table longer than max_blocks")
            rows.append(t + [-1] * (max_blocks - len(t)))
            lens.append(self.lens[s])
        return rows, lens

    def stats(self):
        used = sum(1 for r in self.ref if r > 0)
        shared = sum(1 for r in self.ref if r > 1)
        return {
            "num_blocks": self.num_blocks,
            "free_blocks": len(self.free),
            "used_blocks": used,
            "shared_blocks": shared,
            "num_seqs": len(self.tables),
            "cow_copies": len(self.cow_log),
            "alloc_failures": self.failures,
            "cache_hits": self.cache_hits,
            "cache_misses": self.cache_misses,
            "cache_evictions": self.evictions,
            "cached_blocks": len(self.cache),
        }

    def check_invariants(self) -> None:
        """Structural invariants that must hold after every operation."""
        total_refs = sum(self.ref)
        total_entries = sum(len(t) for t in self.tables.values())
        assert total_refs == total_entries, (total_refs, total_entries)
        free_set = set(self.free)
        assert len(free_set) == len(self.free), "duplicate block in free queue"
        zero = {b for b, r in enumerate(self.ref) if r == 0}
        assert zero == free_set, "free queue != blocks with zero references"
        assert all(r >= 0 for r in self.ref)
        bs = self.block_size
        for s, t in self.tables.items():
            assert len(t) == -(-self.lens[s] // bs), (s, len(t), self.lens[s])
        assert len(self.free) + sum(1 for r in self.ref if r > 0) == self.num_blocks
        for key, b in self.cache.items():
            assert self.block_key[b] == key, (key, b)
        assert sum(1 for k in self.block_key if k is not None) == len(self.cache)
