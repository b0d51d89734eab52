"""Pins of the oracle block manager: the page's worked block-table example,
the pages' closed forms, content round trips through forks and copy-on-write,
structural invariants under random operation sequences, atomic failure."""
import copy
import json
import os

import numpy as np
import pytest
from hypothesis import settings, strategies as st
from hypothesis.stateful import RuleBasedStateMachine, invariant, precondition, rule

from oracle import formulas
from oracle.allocator import BadSeq, NoBlocks, OracleAllocator
from oracle.kvstore import OracleKVStore
from workloads import cb_prefix_script
from workloads.configs import PAGE_EXAMPLE_FREE_ORDER

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_page_block_table_example():
    g = _golden("block_table_example.json")
    bs = g["block_size"]
    a = OracleAllocator(8, bs, PAGE_EXAMPLE_FREE_ORDER)
    req = {}
    for r in g["requests"]:
        s = a.seq_create()
        slots, cow = a.alloc(s, r["tokens"])
        assert cow is None
        req[r["name"]] = (s, slots)
        assert a.tables[s] == r["table"]
    # 16 + 16 + 8 tokens in A's three blocks; only the last one is partly used.
    sa, slots_a = req["A"]
    per_block = [sum(1 for x in slots_a if x // bs == b) for b in a.tables[sa]]
    assert per_block == g["requests"][0]["tokens_per_block"]
    assert slots_a[39] == 5 * 16 + 7 and req["B"][1][19] == 2 * 16 + 3
    a.check_invariants()
    # Tail waste: 8 + 12 empty slots of 80 allocated, under the Theorem 1 bound 16 / 20.
    waste = sum(formulas.tail_waste_tokens(r["tokens"], bs) for r in g["requests"])
    assert waste == 20 and waste / 80 < formulas.paged_waste_bound(bs, 20)


def test_slot_mapping_content_round_trip_through_fork_and_cow():
    """Write each token's logical index into its slot and read every sequence
    back contiguously through its table: must give 0..T-1 for every sequence."""
    bs, nb = 8, 64
    a = OracleAllocator(nb, bs, list(np.random.default_rng(3).permutation(nb)))
    store = OracleKVStore(2, nb, 1, bs, 4)

    def append(s, n):
        start = a.lens[s]
        slots, cow = a.alloc(s, n)
        if cow:
            store.copy_block(*cow)
        vals = np.arange(start, start + n, dtype=np.float16)[:, None, None] * np.ones((1, 1, 4), np.float16)
        for layer in range(2):
            store.write(layer, vals + layer, vals + 1000 + layer, slots)

    s0 = a.seq_create()
    append(s0, 13)
    s1 = a.fork(s0)
    s2 = a.fork(s1)
    append(s1, 5)   # copy-on-write of the shared partial block
    append(s2, 20)  # again (still shared with s0)
    append(s0, 3)   # s0 now owns its last block alone: no copy
    s3 = a.fork(s2)
    append(s3, 9)   # shared with s2: copied
    a.free_seq(s2)
    append(s3, 4)   # s3 is now the only holder: no copy
    assert len(a.cow_log) == 3
    for s in a.tables:
        t = a.lens[s]
        for layer in range(2):
            ks, vs = [], []
            for j, b in enumerate(a.tables[s]):
                kb, vb = store.block_values(layer, b)
                ks.append(kb[0, :, 0])
                vs.append(vb[0, :, 0])
            k = np.concatenate(ks)[:t]
            v = np.concatenate(vs)[:t]
            np.testing.assert_array_equal(k, np.arange(t) + layer)
            np.testing.assert_array_equal(v, np.arange(t) + 1000 + layer)
    a.check_invariants()


def test_allocation_failure_is_atomic():
    a = OracleAllocator(4, 16, [2, 0, 3, 1])
    s = a.seq_create()
    a.alloc(s, 40)  # 3 blocks
    t = a.fork(s)
    before = copy.deepcopy((list(a.free), a.ref, a.tables, a.lens))
    with pytest.raises(NoBlocks):
        a.alloc(t, 40)  # needs copy-on-write block + 2 new blocks, only 1 free
    assert (list(a.free), a.ref, a.tables, a.lens) == before
    assert a.stats()["alloc_failures"] == 1
    a.alloc(t, 8)  # the copy only: fits
    assert a.free == type(a.free)() and a.cow_log == [(a.tables[s][2], a.tables[t][2])]
    with pytest.raises(BadSeq):
        a.alloc(99, 1)


def test_free_returns_blocks_to_tail_in_reverse_order():
    a = OracleAllocator(6, 4, None)
    s = a.seq_create()
    a.alloc(s, 10)  # blocks 0, 1, 2
    a.free_seq(s)
    assert list(a.free) == [3, 4, 5, 2, 1, 0]


def test_kv_memory_arithmetic_matches_page():
    g = _golden("kv_memory_arithmetic.json")
    per_tok = formulas.kv_bytes(g["layers"], g["kv_heads"], g["head_dim"], g["dtype_bytes"], 1)
    assert per_tok == g["bytes_per_token_per_request"]
    assert per_tok * g["request_tokens"] == g["bytes_per_request"]
    assert per_tok * g["request_tokens"] * g["requests"] == g["bytes_for_all_requests"]


def test_closed_forms_match_page_numbers():
    g = _golden("closed_forms.json")
    c = g["internal_fragmentation"]
    assert formulas.internal_fragmentation(c["tokens"], c["max_tokens"]) * 100 == c["printed_percent"]
    c = g["reservation_waste"]
    assert abs(formulas.reservation_waste(c["used"], c["reserved"]) * 100 - c["printed_percent"]) <= c["printed_rounding"]
    c = g["paged_waste_bound"]
    assert abs(formulas.paged_waste_bound(c["block_size"], c["min_tokens"]) * 100 - c["printed_percent_upper"]) <= c["printed_rounding"]
    c = g["shared_copy_savings"]
    assert round(formulas.shared_copy_savings(c["requests"]) * 100, 9) == c["printed_percent"]
    c = g["prefix_savings"]
    assert round(formulas.prefix_savings(c["requests"], c["prefix"], c["mean_suffix"]) * 100, 9) == c["printed_percent"]
    c = g["kv_head_ratio"]
    for case in c["cases"]:
        r = formulas.kv_head_ratio(case["kv_heads"], c["reference_heads"]) * 100
        assert abs(r - case["printed_percent"]) <= case["printed_rounding"]
    c = g["fp8_bytes"]
    assert (1 - c["fp8_bytes"] / c["fp16_bytes"]) * 100 == c["printed_percent_saving"]
    c = g["block_table_overhead"]
    assert abs(formulas.block_table_bytes(c["requests"], 128) / 1000 - c["printed_kb"]) <= c["printed_rounding_kb"]


@pytest.mark.parametrize("seed", range(5))
def test_theorem1_waste_bound(seed):
    rng = np.random.default_rng(seed)
    for bs in (8, 16, 32):
        lens = rng.integers(64, 4096, size=50)
        a = OracleAllocator(int(sum(-(-int(t) // bs) for t in lens)), bs)
        for t in lens:
            a.alloc(a.seq_create(), int(t))
        allocated = sum(len(tb) for tb in a.tables.values()) * bs
        waste = allocated - int(lens.sum())
        for s, t in a.lens.items():
            assert 0 <= formulas.tail_waste_tokens(t, bs) <= bs - 1
        assert waste / allocated < formulas.paged_waste_bound(bs, int(lens.min()))


def _stored_tokens(a):
    """Distinct physical slots holding data: each block counted once, filled up to
    the longest sharer's offset in it."""
    fill = {}
    for s, tb in a.tables.items():
        for j, b in enumerate(tb):
            n = min(a.block_size, a.lens[s] - j * a.block_size)
            fill[b] = max(fill.get(b, 0), n)
    return sum(fill.values())


def test_prefix_sharing_savings_formula_exact_for_block_aligned_prefix():
    r, p, s_bar, bs = 100, 208, 50, 16
    a = OracleAllocator(2000, bs)
    parent = a.seq_create()
    a.alloc(parent, p)
    kids = [a.fork(parent) for _ in range(r)]
    a.free_seq(parent)
    for k in kids:
        a.alloc(k, s_bar)
    stored = _stored_tokens(a)
    logical = sum(a.lens.values())
    assert stored == p + r * s_bar and logical == r * (p + s_bar)
    assert abs((1 - stored / logical) - formulas.prefix_savings(r, p, s_bar)) < 1e-15
    # The same workload with the page's unaligned p = 200 shares 12 full blocks;
    # the partial 13th block is copied by every writer but the last one.
    a = OracleAllocator(2000, bs)
    parent = a.seq_create()
    a.alloc(parent, 200)
    kids = [a.fork(parent) for _ in range(r)]
    a.free_seq(parent)
    for k in kids:
        a.alloc(k, s_bar)
    assert len(a.cow_log) == r - 1
    assert _stored_tokens(a) == 192 + r * (8 + s_bar)


def test_cb_prefix_script_replays_cleanly():
    ops, rows = cb_prefix_script(464_003)
    a = OracleAllocator(16384, 16)
    n_rows = 0
    for op in ops:
        if op[0] == "create":
            a.seq_create()
        elif op[0] == "alloc":
            a.alloc(op[1], op[2])
            n_rows += op[2]
        elif op[0] == "fork":
            a.fork(op[1])
        elif op[0] == "free":
            a.free_seq(op[1])
    a.check_invariants()
    assert n_rows == rows and len(a.tables) == 256
    assert len(a.cow_log) == 99  # every fork but the last one to write copies the partial block
    assert 128 + 1 <= min(a.lens.values()) and max(a.lens.values()) <= 2048 + 512


class AllocatorMachine(RuleBasedStateMachine):
    def __init__(self):
        super().__init__()
        self.a = OracleAllocator(24, 4, list(np.random.default_rng(0).permutation(24)))
        self.live = []

    @rule()
    def create(self):
        self.live.append(self.a.seq_create())

    @precondition(lambda self: self.live)
    @rule(i=st.integers(0, 1000), n=st.integers(0, 13))
    def alloc(self, i, n):
        s = self.live[i % len(self.live)]
        before = copy.deepcopy((list(self.a.free), self.a.ref, self.a.tables, self.a.lens))
        try:
            slots, cow = self.a.alloc(s, n)
        except NoBlocks:
            assert (list(self.a.free), self.a.ref, self.a.tables, self.a.lens) == before
            return
        assert len(slots) == n and len(set(slots)) == n
        for x in slots:
            assert self.a.ref[x // 4] == 1  # an appended slot is never in a shared block

    @precondition(lambda self: self.live)
    @rule(i=st.integers(0, 1000))
    def fork(self, i):
        self.live.append(self.a.fork(self.live[i % len(self.live)]))

    @precondition(lambda self: self.live)
    @rule(i=st.integers(0, 1000))
    def free(self, i):
        self.a.free_seq(self.live.pop(i % len(self.live)))

    @invariant()
    def invariants(self):
        self.a.check_invariants()


TestAllocatorMachine = AllocatorMachine.TestCase
TestAllocatorMachine.settings = settings(max_examples=60, stateful_step_count=40, deadline=None)


# ---- automatic prefix caching -------------------------------------------------

def test_prefix_cache_savings_match_the_page_example():
    """R = 100 prompts sharing a 200-token system prompt with 50-token suffixes
    save 79.2% of the KV (iq-blog ch.4, "Prefix Caching"): with 2-token blocks
    both lengths are block aligned, so the cached pool holds exactly the
    formula's share."""
    r, p, s_bar, bs = 100, 200, 50, 2
    a = OracleAllocator(20000, bs)
    system = list(range(7, 7 + p))
    cached = []
    for i in range(r):
        _, c, slots = a.seq_create_cached(system + [10_000 + 1000 * i + j for j in range(s_bar)])
        cached.append(c)
        assert len(slots) == p + s_bar - c
    assert cached == [0] + [p] * (r - 1)
    used = a.stats()["used_blocks"]
    assert used * bs == p + r * s_bar
    savings = 1 - used * bs / (r * (p + s_bar))
    assert abs(savings - formulas.prefix_savings(r, p, s_bar)) < 1e-15
    assert round(100 * savings, 1) == 79.2
    st_ = a.stats()
    assert st_["cache_hits"] == (r - 1) * (p // bs) and st_["cache_evictions"] == 0
    a.check_invariants()


def test_prefix_cache_hits_stop_at_first_difference_and_skip_partial_blocks():
    a = OracleAllocator(32, 8)
    s0, c0, sl0 = a.seq_create_cached(list(range(20)))   # 2 full blocks + 4 tokens
    assert c0 == 0 and len(sl0) == 20 and len(a.cache) == 2
    s1, c1, sl1 = a.seq_create_cached(list(range(20)))   # same prompt: 2 blocks hit
    assert c1 == 16 and len(sl1) == 4
    assert a.tables[s1][:2] == a.tables[s0][:2] and a.tables[s1][2] != a.tables[s0][2]
    s2, c2, _ = a.seq_create_cached(list(range(8)) + [99] + list(range(9, 20)))  # differs in block 1
    assert c2 == 8 and a.tables[s2][0] == a.tables[s0][0] and a.tables[s2][1] != a.tables[s0][1]
    s3, c3, _ = a.seq_create_cached([5] + list(range(1, 24)))  # differs in block 0: block 1 not looked up
    assert c3 == 0
    assert a.ref[a.tables[s0][0]] == 3 and a.ref[a.tables[s0][1]] == 2
    a.check_invariants()


def test_prefix_cache_lru_eviction_and_revival_through_the_free_queue():
    """Freed cached blocks wait at the free-queue tail with their entries; a hit
    revives one from the middle of the queue; allocation takes the head and
    evicts the least recently freed first."""
    a = OracleAllocator(6, 8, free_order=[0, 1, 2, 3, 4, 5])
    s_a, _, _ = a.seq_create_cached([1] * 8)           # block 0, cached
    s_b, _, _ = a.seq_create_cached([2] * 8)           # block 1, cached
    s_c, _, _ = a.seq_create_cached([3] * 8)           # block 2, cached
    a.free_seq(s_a)
    a.free_seq(s_b)
    a.free_seq(s_c)
    assert list(a.free) == [3, 4, 5, 0, 1, 2] and len(a.cache) == 3
    s_b2, c, _ = a.seq_create_cached([2] * 8)          # revival of block 1 from the middle
    assert c == 8 and a.tables[s_b2] == [1] and list(a.free) == [3, 4, 5, 0, 2]
    x = a.seq_create()
    a.alloc(x, 32)                                      # takes 3, 4, 5, 0: evicts [1]*8's entry
    assert a.tables[x] == [3, 4, 5, 0] and a.evictions == 1 and list(a.free) == [2]
    _, c_a, _ = a.seq_create_cached([1] * 8)           # evicted: miss, takes block 2 (evicts [3]*8)
    assert c_a == 0 and a.evictions == 2 and len(a.cache) == 2
    with pytest.raises(NoBlocks):                        # nothing free: atomic failure, no id used
        a.seq_create_cached([9] * 8)
    nid = a.next_id
    assert a.stats()["alloc_failures"] == 1 and a.next_id == nid
    a.check_invariants()


def test_prefix_cached_sequences_read_the_right_content():
    """Content round trip: the K/V a cached sequence reads through its table
    is its own prompt's, whichever sequence wrote the shared blocks."""
    rng = np.random.default_rng(5)
    bs, d = 8, 4
    a = OracleAllocator(64, bs)
    store = OracleKVStore(1, 64, 1, bs, d)
    system = list(range(40))
    value = lambda tok: np.full((1, d), float(tok), np.float16)  # K/V of a token = its id
    seqs = {}
    for i in range(12):
        toks = system[:int(rng.integers(0, 41))] + [100 + i] * int(rng.integers(1, 9))
        s, c, slots = a.seq_create_cached(toks)
        kv = np.concatenate([value(t) for t in toks[c:]])[:, None, :] if len(toks) > c else np.zeros((0, 1, d), np.float16)
        store.write(0, kv, kv, slots)
        seqs[s] = toks
        if i % 3 == 2:
            a.free_seq(list(seqs)[0])
            del seqs[list(seqs)[0]]
    for s, toks in seqs.items():
        t = np.arange(len(toks))
        slots = np.asarray(a.tables[s])[t // bs] * bs + t % bs
        k, _ = store.read_slots(0, slots)
        np.testing.assert_array_equal(k[:, 0, 0], np.asarray(toks, np.float16))


def test_a_second_turn_hits_on_the_blocks_generated_in_the_first():
    """Multi-turn history is a shared prefix (youngju.dev page, "prefix 공유와
    copy-on-write"): appends with token ids enter every block they fill, so
    the next turn's prompt (first prompt + answer + new question) is served
    from the cache up to the last full block of prompt + answer."""
    bs = 8
    a = OracleAllocator(64, bs)
    prompt = list(range(100, 120))                      # 2 full blocks + 4 tokens
    s, c, _ = a.seq_create_cached(prompt)
    assert c == 0 and len(a.cache) == 2
    answer = list(range(500, 513))                      # 13 generated tokens, one at a time
    for t in answer:
        a.alloc(s, 1, [t])
    assert a.lens[s] == 33 and len(a.cache) == 4       # blocks 2 and 3 filled and entered
    turn1_blocks = list(a.tables[s][:4])
    a.free_seq(s)
    s2, c2, slots2 = a.seq_create_cached(prompt + answer + list(range(900, 910)))
    assert c2 == 32 and a.tables[s2][:4] == turn1_blocks and len(slots2) == 43 - 32
    st_ = a.stats()
    assert st_["cache_hits"] == 4 and st_["cache_misses"] == 2 + 1
    a.check_invariants()


def test_a_tokenless_append_ends_caching_for_its_sequence():
    bs = 4
    a = OracleAllocator(32, bs)
    s, _, _ = a.seq_create_cached([1, 2, 3, 4, 5, 6])  # 1 full block cached
    a.alloc(s, 2, [7, 8])                               # fills block 1: cached
    a.alloc(s, 3)                                       # no ids: the sequence's ids are unknown now
    a.alloc(s, 5, [1, 1, 1, 1, 1])                      # fills blocks: not cached
    assert a.tokens[s] is None and len(a.cache) == 2
    t = a.seq_create()                                  # empty sequence, appends with ids
    a.alloc(t, 4, [9, 9, 9, 9])
    assert len(a.cache) == 3 and a.cache[(9, 9, 9, 9)] == a.tables[t][0]
    _, c, _ = a.seq_create_cached([1, 2, 3, 4, 5, 6, 7, 8, 0])
    assert c == 8
    a.check_invariants()


def test_forks_inherit_token_ids_and_cache_their_own_continuations():
    """Two forks of a prompt with a partial last block: each append copies the
    shared block (copy-on-write) and, when the copy fills, enters it under
    that fork's own prefix."""
    bs = 4
    a = OracleAllocator(32, bs)
    p, _, _ = a.seq_create_cached([1, 2, 3, 4, 5, 6])
    f = a.fork(p)
    _, cow_f = a.alloc(f, 2, [7, 8])                    # f copies the shared block, fills it
    _, cow_p = a.alloc(p, 2, [70, 80])                  # p is now the block's only owner: no copy
    assert cow_f is not None and cow_p is None
    assert a.cache[(1, 2, 3, 4, 5, 6, 7, 8)] == a.tables[f][1] == cow_f[1]
    assert a.cache[(1, 2, 3, 4, 5, 6, 70, 80)] == a.tables[p][1] == cow_f[0]
    _, c1, _ = a.seq_create_cached([1, 2, 3, 4, 5, 6, 7, 8, 11])
    _, c2, _ = a.seq_create_cached([1, 2, 3, 4, 5, 6, 70, 80])
    assert c1 == 8 and c2 == 8
    a.check_invariants()


def test_evictions_take_the_entries_of_reused_blocks_only():
    """Freed cached blocks keep their entries until the free queue hands them
    out (child block first: a freed sequence's blocks join the queue last to
    first); then the prefixes miss and are entered again."""
    bs = 2
    a = OracleAllocator(4, bs, free_order=[0, 1, 2, 3])
    x, _, _ = a.seq_create_cached([1, 1, 2, 2])        # blocks 0 ([1,1]) and 1 ([1,1,2,2]) cached
    a.free_seq(x)                                       # free queue: 2, 3, 1, 0
    assert list(a.free) == [2, 3, 1, 0]
    y = a.seq_create()
    a.alloc(y, 6)                                       # takes 2, 3, 1: evicts [1,1,2,2]'s entry
    assert a.evictions == 1 and len(a.cache) == 1
    a.free_seq(y)                                       # free queue: 0, 1, 3, 2
    z = a.seq_create()
    a.alloc(z, 2)                                       # takes 0: evicts [1,1]
    assert a.evictions == 2 and len(a.cache) == 0
    a.free_seq(z)
    w, _, _ = a.seq_create_cached([5, 5, 6, 6])        # misses; enters two new blocks
    v, c, _ = a.seq_create_cached([5, 5, 6, 6, 7])
    assert c == 4 and len(a.cache) == 2
    a.check_invariants()


# ---- beam-style fork trees ------------------------------------------------------

@pytest.mark.parametrize("bs", [1, 4, 16])
def test_beam_fork_tree_matches_an_explicit_token_tree(bs):
    """Beam search keeps candidates that share their common prefix (opsoai
    page, "KV 캐시는 왜 요청이 늘수록 서빙 병목이 되는가"; iq-blog ch.4,
    "Prefix Caching").  Model the search as a tree of token nodes: every beam is
    a root-to-leaf path.  Reading each beam back through its table (with the
    copy-on-write copies applied to the stored contents) must give exactly its
    path; with one-token blocks nothing is ever copied and the pool holds
    exactly the tree's live nodes."""
    from workloads import beam_parents
    groups, k, prompt, steps = 3, 5, 21, 30
    a = OracleAllocator(4000, bs)
    content = {}  # slot -> token node held there

    def append(s, node):
        slots, cow = a.alloc(s, 1)
        if cow is not None:
            src, dst = cow
            for o in range(bs):
                if src * bs + o in content:
                    content[dst * bs + o] = content[src * bs + o]
        content[slots[0]] = node

    beams, paths = [], []
    for g in range(groups):
        s = a.seq_create()
        slots, _ = a.alloc(s, prompt)
        for i, sl in enumerate(slots):
            content[sl] = ("prompt", g, i)
        kids = [s] + [a.fork(s) for _ in range(k - 1)]
        beams.append(kids)
        paths.append([[("prompt", g, i) for i in range(prompt)] for _ in range(k)])
    for step in range(steps):
        for g, parents in enumerate(beam_parents(464_021, step, groups, k)):
            old, new, used = beams[g], [], set()
            for p in parents:
                if p in used:
                    new.append(a.fork(old[p]))
                else:
                    used.add(p)
                    new.append(old[p])
            for b in range(k):
                if b not in used:
                    a.free_seq(old[b])
            paths[g] = [paths[g][p] + [(step, g, j)] for j, p in enumerate(parents)]
            for j, s in enumerate(new):
                append(s, (step, g, j))
            beams[g] = new
        a.check_invariants()
        live = set()
        for g in range(groups):
            for s, path in zip(beams[g], paths[g]):
                t = a.tables[s]
                got = [content[t[i // bs] * bs + i % bs] for i in range(a.lens[s])]
                assert got == path
                live.update(path)
        if bs == 1:
            assert not a.cow_log
            assert a.stats()["used_blocks"] == len(live)
    if bs > 1:
        assert len(a.cow_log) > 0
