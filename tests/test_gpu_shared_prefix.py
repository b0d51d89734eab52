"""GPU parity of the shared-prefix decode (pa_decode_shared_prefix) against
the oracle's decode.  One launch: chunks of each group's shared tokens and
every sequence's own tokens run as separate pieces, and the last piece of a
sequence merges their partials; small chunk lengths make many pieces per
sequence at these sizes.

Sequences are built the way the pages share blocks: a prompt written once
and forked into several members (beams, parallel samples), each member then
appending its own tokens (copy-on-write of the prompt's last, partly filled
block on the first append); requests on one cached system prompt; and
unrelated sequences.  The batch interleaves the groups.  K/V of member m at
position t: the group prompt's row t for t < P, else the member's own row
t - P; the oracle store holds each sequence's whole context at the slots its
table gives, so shared slots are written with equal values."""
import numpy as np
import pytest
import torch

from oracle import attention
from oracle.kvstore import OracleKVStore
from paged_kv_cache_464_amd import pa
from tests.gpu_helpers import assert_close, say
from workloads import amax_scales, free_order, head_offsets, minmax_int8_params, normal_fp16

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


class Tree:
    def refresh(self):
        """Block tables and lengths of the batch, on the host and the device."""
        self.mb = max(self.pool.seq_len(s)[1] for s in self.batch)
        self.tables_np, self.lens_np = self.pool.block_tables(self.batch, self.mb)
        self.tables = torch.from_numpy(self.tables_np).cuda()
        self.lens = torch.from_numpy(self.lens_np).cuda()


def build_tree(groups, singles, hq, hkv, bs, dtype="fp16", head_dim=128, seed=464_200, num_blocks=None):
    """groups: list of (prompt_tokens, [tail tokens of each member]);
    singles: lengths of unrelated sequences.  Returns the pool, the batch
    (the groups' members and the singles in a seeded shuffle), the K/V rows
    of every sequence's context and the calibration of the quantised kinds."""
    D = head_dim
    t = Tree()
    t.bs, t.hq, t.hkv, t.dtype, t.D = bs, hq, hkv, dtype, D
    rng = np.random.default_rng(seed)
    pk = [normal_fp16((p, hkv, D), seed, 10 + g, "cuda") for g, (p, _) in enumerate(groups)]
    pv = [normal_fp16((p, hkv, D), seed, 40 + g, "cuda") for g, (p, _) in enumerate(groups)]
    tails = [n for _, ms in groups for n in ms] + list(singles)
    tk = [normal_fp16((n, hkv, D), seed, 100 + i, "cuda") for i, n in enumerate(tails)]
    tv = [normal_fp16((n, hkv, D), seed, 400 + i, "cuda") for i, n in enumerate(tails)]
    if dtype == "int8":
        off = torch.from_numpy(head_offsets(hkv)).cuda()[None, :, None]
        pk = [(x.float() + off).half() for x in pk]
        tk = [(x.float() + off).half() for x in tk]
    allk = torch.cat(pk + tk)
    allv = torch.cat(pv + tv)
    ks = vs = kz = vz = None
    t.scales = {}
    if dtype == "fp8":
        ks, vs = amax_scales(allk)[None], amax_scales(allv)[None]
    if dtype == "int8":
        a, b = minmax_int8_params(allk)
        c, d = minmax_int8_params(allv)
        ks, kz, vs, vz = a[None], b[None], c[None], d[None]
    t.scales = dict(k_scales=ks, v_scales=vs, k_zeros=kz, v_zeros=vz)
    need = sum(-(-(p + max(ms)) // bs) * len(ms) + 1 for p, ms in groups) + sum(-(-n // bs) for n in singles)
    nb = num_blocks or need + 16
    t.nb = nb
    t.pool = pa.PagedKVPool(1, hkv, D, bs, nb, dtype, free_order=free_order(seed, nb), **t.scales)
    t.pool.pool_bytes().fill_(0xFF)
    t.rows = {}  # seq -> (k rows, v rows) of its whole context, fp16 on the device
    batch = []
    ti = 0
    for g, (p, ms) in enumerate(groups):
        s = t.pool.seq_create()
        sl, _ = t.pool.alloc(s, p)
        t.pool.write_kv(0, pk[g], pv[g], torch.from_numpy(sl).cuda())
        mem = [s] + [t.pool.fork(s) for _ in range(len(ms) - 1)]
        for m, n in zip(mem, ms):
            sl, _ = t.pool.alloc(m, n)  # copy-on-write copies are enqueued by the library
            t.pool.write_kv(0, tk[ti], tv[ti], torch.from_numpy(sl).cuda())
            t.rows[m] = (torch.cat([pk[g], tk[ti]]), torch.cat([pv[g], tv[ti]]))
            ti += 1
        batch += mem
    for n in singles:
        s = t.pool.seq_create()
        sl, _ = t.pool.alloc(s, n)
        t.pool.write_kv(0, tk[ti], tv[ti], torch.from_numpy(sl).cuda())
        t.rows[s] = (tk[ti], tv[ti])
        ti += 1
        batch.append(s)
    t.batch = [batch[i] for i in rng.permutation(len(batch))]
    t.refresh()
    return t


def oracle_store(t):
    sc = t.scales
    st = OracleKVStore(1, t.nb, t.hkv, t.bs, t.D, t.dtype, sc["k_scales"], sc["v_scales"], sc["k_zeros"],
                       sc["v_zeros"])
    for i, s in enumerate(t.batch):
        k, v = t.rows[s]
        n = int(t.lens_np[i])
        pos = np.arange(n)
        st.write(0, k[:n].cpu().numpy(), v[:n].cpu().numpy(), t.tables_np[i][pos // t.bs] * t.bs + pos % t.bs)
    return st


def _check_groups_cover(t, groups, expect_shared):
    members, gstart, shared = groups
    assert sorted(members.tolist()) == list(range(len(t.batch)))
    assert sum(1 for k in shared if k > 0) == expect_shared


CASES = [
    # (dtype, bs, hq, hkv, head_dim)
    ("fp16", 16, 32, 8, 128),
    ("fp16", 8, 32, 8, 128),
    ("fp16", 32, 32, 8, 128),
    ("fp8", 16, 32, 8, 128),
    ("int8", 16, 32, 8, 128),
    ("fp16", 16, 32, 32, 128),  # one head per group: 32 members per item
    ("fp16", 16, 32, 1, 128),   # 32 heads per group: one member per item
    ("fp16", 16, 16, 2, 64),
    ("fp8", 32, 16, 2, 64),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_shared_prefix_decode_matches_the_oracle(case):
    dtype, bs, hq, hkv, D = CASES[case]
    say("shared prefix", dtype, bs, hq, hkv, D)
    rng = np.random.default_rng(464_200 + case)
    groups = [
        (300, [int(x) for x in rng.integers(1, 40, 5)]),        # beam-like: 5 members, short tails
        (1037, [int(x) for x in rng.integers(1, 300, 20)]),     # 20 members (several items each)
        (16, [3, 9]),                                          # below the 256-token minimum
        (2048, [1, 700]),                                      # long prompt, uneven tails
    ]
    singles = [int(x) for x in rng.integers(1, 900, 6)]
    t = build_tree(groups, singles, hq, hkv, bs, dtype, D)
    st = oracle_store(t)
    q = normal_fp16((len(t.batch), hq, D), 464_200, 3, "cuda")
    ref = attention.decode(st, 0, q.cpu().numpy(), t.tables_np, t.lens_np)
    # With the host lengths the plan folds the groups whose members have at
    # most 128 tokens of their own (the 5-member group, the 2-member groups
    # when their tails are short) and chunks the others, in one launch.
    for min_tokens, chunk, fold in ((256, 0, False), (16, 0, False), (256, 64, False), (16, 192, False),
                                    (256, 0, True), (16, 128, True)):
        g = t.pool.shared_prefix_groups(t.tables_np, t.lens_np, min_tokens)
        _check_groups_cover(t, g, 3 if min_tokens == 256 else 3 + (bs <= 16))
        lens = t.lens_np if fold else None
        plan = t.pool.shared_prefix_plan(len(t.batch), hq, t.mb, g, chunk_tokens=chunk, lens=lens)
        if fold:
            assert plan.plan.num_private < len(t.batch)  # the 5-member group at least is folded
        out = t.pool.decode_shared_prefix(0, q, t.tables, t.lens, plan)
        assert_close(out, ref, dtype, f"shared prefix min={min_tokens} chunk={chunk} fold={fold}")
        assert t.pool.device_status() == 0
    # Every group a singleton: the private pass alone over every token.
    n = len(t.batch)
    none = (np.arange(n, dtype=np.int32), np.arange(n + 1, dtype=np.int32), np.zeros(n, dtype=np.int32))
    out0 = t.pool.decode_shared_prefix(0, q, t.tables, t.lens, none)
    assert_close(out0, ref, dtype, "shared prefix, no groups")
    assert t.pool.device_status() == 0


@pytest.mark.parametrize("fold", [False, True])
@pytest.mark.parametrize("dtype,bs", [("fp16", 16), ("fp8", 8), ("int8", 32)])
def test_fused_shared_prefix_step_writes_like_write_kv_decode(dtype, bs, fold):
    """One generation step of every member: the new token appended (slots
    from the allocator), written and attended in the fused call (fold: by
    the folded items, whose waves take each member's own tokens; else by the
    private pieces); the pool's bytes equal those pa_write_kv_decode leaves,
    and both outputs match the oracle."""
    say("fused shared prefix", dtype, bs, "folded" if fold else "pieces")
    hq, hkv, D = 32, 8, 128
    rng = np.random.default_rng(464_201 + bs)
    groups = [(513, [int(x) for x in rng.integers(1, 60, 6)]), (777, [int(x) for x in rng.integers(1, 90, 9)])]
    t = build_tree(groups, [5, 300], hq, hkv, bs, dtype, D, seed=464_201)
    kn = normal_fp16((len(t.batch), hkv, D), 464_201, 7, "cuda")
    vn = normal_fp16((len(t.batch), hkv, D), 464_201, 8, "cuda")
    if dtype == "int8":
        kn = (kn.float() + torch.from_numpy(head_offsets(hkv)).cuda()[None, :, None]).half()
    slots, cow = t.pool.alloc_batch(t.batch, [1] * len(t.batch))
    assert all(c[0] < 0 for c in cow)  # the tails' blocks are private already
    for i, s in enumerate(t.batch):
        k, v = t.rows[s]
        t.rows[s] = (torch.cat([k, kn[i:i + 1]]), torch.cat([v, vn[i:i + 1]]))
    t.refresh()
    sl = torch.from_numpy(np.asarray(slots, dtype=np.int32)).cuda()
    q = normal_fp16((len(t.batch), hq, D), 464_201, 9, "cuda")
    g = t.pool.shared_prefix_groups(t.tables_np, t.lens_np, 256)
    assert sum(1 for k in g[2] if k > 0) == 2
    before = t.pool.pool_bytes().clone()
    plan = t.pool.shared_prefix_plan(len(t.batch), hq, t.mb, g, chunk_tokens=128,
                                     lens=t.lens_np if fold else None)
    assert plan.plan.num_private == (2 if fold else len(t.batch))  # the two singletons
    out_sp = t.pool.decode_shared_prefix(0, q, t.tables, t.lens, plan, k_new=kn, v_new=vn, slot_mapping=sl)
    after_sp = t.pool.pool_bytes().clone()
    t.pool.pool_bytes().copy_(before)
    out_wd = t.pool.write_kv_decode(0, kn, vn, sl, q, t.tables, t.lens)
    torch.cuda.synchronize()
    assert torch.equal(after_sp, t.pool.pool_bytes()), "pool bytes differ from pa_write_kv_decode's"
    ref = attention.decode(oracle_store(t), 0, q.cpu().numpy(), t.tables_np, t.lens_np)
    assert_close(out_sp, ref, dtype, "fused shared prefix")
    assert_close(out_wd, ref, dtype, "fused write + decode")
    assert t.pool.device_status() == 0


def test_requests_on_cached_system_prompts():
    """Requests built through the prefix cache on two system prompts (hits
    on their full blocks), decoded with the groups the helper finds."""
    say("cached system prompts")
    bs, hq, hkv, D, nb = 16, 32, 8, 128, 512
    rng = np.random.default_rng(464_202)
    systems = [list(rng.integers(0, 5000, 700)), list(rng.integers(0, 5000, 333))]
    table = normal_fp16((4096, hkv, D), 464_202, 1, "cuda")
    table_v = normal_fp16((4096, hkv, D), 464_202, 2, "cuda")
    pool = pa.PagedKVPool(1, hkv, D, bs, nb, free_order=free_order(464_202, nb))
    pool.pool_bytes().fill_(0xFF)

    def rows(toks, start):
        idx = torch.tensor([(int(x) * 131 + start + i) % 4096 for i, x in enumerate(toks)], device="cuda")
        return table[idx].contiguous(), table_v[idx].contiguous()

    seqs, prompts = [], {}
    for i in range(24):
        toks = systems[i % 2] + list(rng.integers(5000, 6000, int(rng.integers(1, 120))))
        s, cached, slots = pool.seq_create_cached(toks)
        if i >= 2:
            assert cached == len(systems[i % 2]) // bs * bs
        if len(slots):
            k, v = rows(toks[cached:], cached)
            pool.write_kv(0, k, v, torch.from_numpy(slots).cuda())
        seqs.append(s)
        prompts[s] = toks
    mb = max(-(-len(prompts[s]) // bs) for s in seqs)
    tables, lens = pool.block_tables(seqs, mb)
    st = OracleKVStore(1, nb, hkv, bs, D)
    for i, s in enumerate(seqs):
        pos = np.arange(lens[i])
        k, v = rows(prompts[s], 0)
        st.write(0, k.cpu().numpy(), v.cpu().numpy(), tables[i][pos // bs] * bs + pos % bs)
    q = normal_fp16((len(seqs), hq, D), 464_202, 3, "cuda")
    g = pool.shared_prefix_groups(tables, lens, 256)
    assert sorted(int(k) for k in g[2] if k > 0) == [333 // 16, 700 // 16]
    out = pool.decode_shared_prefix(0, q, torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(), g)
    assert_close(out, attention.decode(st, 0, q.cpu().numpy(), tables, lens), "fp16", "cached system prompts")
    assert pool.device_status() == 0


def test_shared_prefix_workspace_reuse_plans_and_empty_batch():
    """Two calls on one workspace (the second with fewer sequences and other
    groups), one plan serving several launches, then an empty batch."""
    say("workspace reuse")
    t = build_tree([(400, [3, 50, 7, 90]), (260, [2, 2, 2])], [40], 32, 8, 16)
    st = oracle_store(t)
    q = normal_fp16((len(t.batch), 32, 128), 464_203, 3, "cuda")
    g = t.pool.shared_prefix_groups(t.tables_np, t.lens_np, 16)
    need = [pa.pa_decode_shared_prefix_workspace_bytes(t.pool.handle, len(t.batch), 32, g, t.mb, c) for c in (0, 64)]
    ws = torch.empty(max(need), dtype=torch.uint8, device="cuda")
    out = t.pool.decode_shared_prefix(0, q, t.tables, t.lens, g, workspace=ws)
    assert_close(out, attention.decode(st, 0, q.cpu().numpy(), t.tables_np, t.lens_np), "fp16", "first call")
    keep = [i for i, s in enumerate(t.batch) if i % 2 == 0]
    tb, ln = t.tables_np[keep], t.lens_np[keep]
    g2 = t.pool.shared_prefix_groups(tb, ln, 16)
    q2 = q[keep].contiguous()
    out2 = t.pool.decode_shared_prefix(0, q2, torch.from_numpy(tb).cuda(), torch.from_numpy(ln).cuda(), g2,
                                       workspace=ws)
    assert_close(out2, attention.decode(st, 0, q2.cpu().numpy(), tb, ln), "fp16", "second call")
    # One plan, several launches (the layers of a step): the group list and
    # the zeroed counters are uploaded once, and each launch leaves the
    # counters at zero for the next; each launch matches the oracle.
    plan = t.pool.shared_prefix_plan(len(t.batch), 32, t.mb, g, workspace=ws, chunk_tokens=64)
    assert plan.plan.num_items > len(t.batch) // 4 and plan.plan.chunk_tokens == 64
    for rep in range(3):
        qr = normal_fp16((len(t.batch), 32, 128), 464_203, 10 + rep, "cuda")
        o = t.pool.decode_shared_prefix(0, qr, t.tables, t.lens, plan)
        assert_close(o, attention.decode(st, 0, qr.cpu().numpy(), t.tables_np, t.lens_np), "fp16",
                     f"planned launch {rep}")
    with pytest.raises(ValueError):  # a plan for another batch shape
        t.pool.decode_shared_prefix(0, q2, torch.from_numpy(tb).cuda(), torch.from_numpy(ln).cuda(), plan)
    e = torch.empty((0, 32, 128), dtype=torch.float16, device="cuda")
    empty = (np.zeros(0, np.int32), np.zeros(1, np.int32), np.zeros(0, np.int32))
    t.pool.decode_shared_prefix(0, e, torch.zeros((0, 1), dtype=torch.int32, device="cuda"),
                                torch.zeros(0, dtype=torch.int32, device="cuda"), empty)
    assert t.pool.device_status() == 0


def test_beam_k5_full_size_in_the_benchmark_configuration():
    """The benchmark's beam_k5 step at full size: 32 groups of 5 beams over a
    2040-token prompt, 16-token blocks, 32 query / 8 KV heads; each search
    step re-selects the survivors (forks, frees), appends one token per beam
    in one batch (copy-on-write copies enqueued), plans the groups found on
    the host tables with the host lengths (every group folds: the beams have
    a few tokens of their own) and runs the fused shared-prefix call.  After the last step, 10 sampled beams (every query
    head) match the oracle, whose store holds each sampled beam's whole
    context at the slots its table gives."""
    from workloads import beam_parents, workload
    w = workload("beam_k5")
    e = w.extra
    groups, k, prompt = e["groups"], e["k"], e["prompt"]
    hq, hkv, bs, D = w.q_heads, w.kv_heads, w.block_size, w.head_dim
    say("beam_k5 full size, shared-prefix decode")
    steps = 6
    nb = w.num_blocks + groups * k * (steps // bs + 2)
    pool = pa.PagedKVPool(1, hkv, D, bs, nb, free_order=free_order(w.seed, nb))
    pool.pool_bytes().fill_(0xFF)
    rows = {}  # seq -> (k rows, v rows) of its context, fp16 on the device
    beams = []
    for g in range(groups):
        s = pool.seq_create()
        sl, _ = pool.alloc(s, prompt)
        kp = normal_fp16((prompt, hkv, D), w.seed, 500 + g, "cuda")
        vp = normal_fp16((prompt, hkv, D), w.seed, 600 + g, "cuda")
        pool.write_kv(0, kp, vp, torch.from_numpy(sl).cuda())
        kids = [s] + [pool.fork(s) for _ in range(k - 1)]
        for c in kids:
            rows[c] = (kp, vp)
        beams.append(kids)
    q = None
    for step in range(steps):
        for g, parents in enumerate(beam_parents(w.seed, step, groups, k)):
            old, new, used = beams[g], [], set()
            for par in parents:
                if par in used:
                    c = pool.fork(old[par])
                    rows[c] = rows[old[par]]
                    new.append(c)
                else:
                    used.add(par)
                    new.append(old[par])
            for b in range(k):
                if b not in used:
                    pool.free(old[b])
                    del rows[old[b]]
            beams[g] = new
        seqs = [s for b in beams for s in b]
        slots, _ = pool.alloc_batch(seqs, [1] * len(seqs))
        kn = normal_fp16((len(seqs), hkv, D), w.seed, 1000 + step, "cuda")
        vn = normal_fp16((len(seqs), hkv, D), w.seed, 2000 + step, "cuda")
        for i, s in enumerate(seqs):
            rows[s] = (torch.cat([rows[s][0], kn[i:i + 1]]), torch.cat([rows[s][1], vn[i:i + 1]]))
        mb = max(pool.seq_len(s)[1] for s in seqs)
        tables, lens = pool.block_tables(seqs, mb)
        grp = pool.shared_prefix_groups(tables, lens, 256)
        assert sum(1 for x in grp[2] if x > 0) == groups
        q = normal_fp16((len(seqs), hq, D), w.seed, 3000 + step, "cuda")
        plan = pool.shared_prefix_plan(len(seqs), hq, mb, grp, lens=lens)  # as the benchmark plans it
        assert plan.plan.num_private == 0 and plan.plan.num_slots == 0  # every group folded
        out = pool.decode_shared_prefix(0, q, torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(), plan,
                                        k_new=kn, v_new=vn,
                                        slot_mapping=torch.from_numpy(np.asarray(slots, np.int32)).cuda())
    sample = list(range(0, len(seqs), len(seqs) // 10))[:10]
    st = OracleKVStore(1, nb, hkv, bs, D)
    for i in sample:
        s = seqs[i]
        n = int(lens[i])
        pos = np.arange(n)
        st.write(0, rows[s][0][:n].cpu().numpy(), rows[s][1][:n].cpu().numpy(), tables[i][pos // bs] * bs + pos % bs)
    ref = attention.decode(st, 0, q.cpu().numpy()[sample], tables[sample], lens[sample])
    assert_close(out[sample], ref, "fp16", "beam_k5 full size, sampled beams")
    assert pool.device_status() == 0


def test_prefix_cache_full_size_in_the_benchmark_configuration():
    """The benchmark's prefix_cache step at full size: 256 requests on four
    1024-token system prompts with 64-1024-token suffixes, created through the
    prefix cache (only uncached tokens written), one appended token per
    request, groups planned with the host lengths (the private pieces longest
    first) and the fused shared-prefix call; 12 sampled requests (every query
    head) match the oracle.  K/V of token id x at position t: row
    (131 x + t) of a seeded table, so equal prefixes carry equal K/V."""
    from workloads import prefix_cache_prompts, workload
    w = workload("prefix_cache")
    e = w.extra
    hq, hkv, bs, D = w.q_heads, w.kv_heads, w.block_size, w.head_dim
    say("prefix_cache full size, shared-prefix decode")
    prompts = prefix_cache_prompts(w.seed, w.num_seqs, e["systems"], e["system_tokens"], e["suffix"])
    rows_n = 8192
    table_k = normal_fp16((rows_n, hkv, D), w.seed, 700, "cuda")
    table_v = normal_fp16((rows_n, hkv, D), w.seed, 701, "cuda")
    nb = w.num_blocks + 2 * w.num_seqs
    pool = pa.PagedKVPool(1, hkv, D, bs, nb, free_order=free_order(w.seed, nb))
    pool.pool_bytes().fill_(0xFF)

    def rows(toks, start):
        idx = torch.tensor([(int(x) * 131 + start + i) % rows_n for i, x in enumerate(toks)], device="cuda")
        return table_k[idx].contiguous(), table_v[idx].contiguous()

    seqs = []
    for toks in prompts:
        s, cached, slots = pool.seq_create_cached(toks)
        if len(slots):
            k, v = rows(toks[cached:], cached)
            pool.write_kv(0, k, v, torch.from_numpy(slots).cuda())
        seqs.append(s)
    assert pool.stats()["cache_hits"] > 0
    new_ids = [90_000 + i for i in range(len(seqs))]
    slots, _ = pool.alloc_batch(seqs, [1] * len(seqs))
    ctx = [list(p) + [t] for p, t in zip(prompts, new_ids)]
    kn = torch.stack([rows([t], len(c) - 1)[0][0] for t, c in zip(new_ids, ctx)]).contiguous()
    vn = torch.stack([rows([t], len(c) - 1)[1][0] for t, c in zip(new_ids, ctx)]).contiguous()
    mb = max(pool.seq_len(s)[1] for s in seqs)
    tables, lens = pool.block_tables(seqs, mb)
    grp = pool.shared_prefix_groups(tables, lens, 256)
    assert sum(1 for x in grp[2] if x > 0) == e["systems"]
    plan = pool.shared_prefix_plan(len(seqs), hq, mb, grp, lens=lens)
    assert plan.plan.num_private == len(seqs) and plan.plan.num_items > 0
    q = normal_fp16((len(seqs), hq, D), w.seed, 702, "cuda")
    out = pool.decode_shared_prefix(0, q, torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(), plan,
                                    k_new=kn, v_new=vn,
                                    slot_mapping=torch.from_numpy(np.asarray(slots, np.int32)).cuda())
    sample = list(range(0, len(seqs), len(seqs) // 12))[:12]
    st = OracleKVStore(1, nb, hkv, bs, D)
    for i in sample:
        pos = np.arange(int(lens[i]))
        k, v = rows(ctx[i], 0)
        st.write(0, k.cpu().numpy(), v.cpu().numpy(), tables[i][pos // bs] * bs + pos % bs)
    ref = attention.decode(st, 0, q.cpu().numpy()[sample], tables[sample], lens[sample])
    assert_close(out[sample], ref, "fp16", "prefix_cache full size, sampled requests")
    assert pool.device_status() == 0


@pytest.mark.parametrize("fold", [False, True])
def test_shared_run_past_a_context_is_flagged(fold):
    """Host-forced contract violation: a group claims more shared blocks
    than one member's context holds (the plan cannot see device lengths;
    with fold, stale host lengths make the plan fold the group).  The launch
    flags PA_DEV_BAD_LEN (the shared pieces read the padding entries of the
    shortest member's table as block 0, flagged too, so that group's rows
    are undefined), and the other groups and the singletons still match the
    oracle."""
    say("shared run past a context", "folded" if fold else "pieces")
    t = build_tree([(640, [3, 40, 17]), (300, [5, 9])], [100, 900], 32, 8, 16, seed=464_400)
    g = t.pool.shared_prefix_groups(t.tables_np, t.lens_np, 256)
    members, gstart, shared = [a.copy() for a in g]
    gi = int(np.argmax(shared))  # the 640-token group: 40 shared blocks
    mem = members[gstart[gi]:gstart[gi + 1]]
    shortest = min(int(t.lens_np[m]) for m in mem)
    shared[gi] = (shortest + 15) // 16 + 1  # past the shortest member's last token
    assert shared[gi] <= t.mb
    lens_host = t.lens_np.copy()
    if fold:
        lens_host[mem] = shared[gi] * 16 + 8  # stale lengths: the plan folds the group
    plan = t.pool.shared_prefix_plan(len(t.batch), 32, t.mb, (members, gstart, shared), lens=lens_host if fold else None)
    q = normal_fp16((len(t.batch), 32, 128), 464_400, 3, "cuda")
    t.pool.device_status(clear=True)
    out = t.pool.decode_shared_prefix(0, q, t.tables, t.lens, plan)
    torch.cuda.synchronize()
    status = t.pool.device_status(clear=True)
    assert status & pa.PA_DEV_BAD_LEN
    ok = [i for i, s in enumerate(t.batch) if i not in set(int(m) for m in mem)]
    st = oracle_store(t)
    ref = attention.decode(st, 0, q.cpu().numpy()[ok], t.tables_np[ok], t.lens_np[ok])
    assert_close(out[ok], ref, "fp16", "sequences outside the broken group")
