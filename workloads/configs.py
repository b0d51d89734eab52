"""The five synthetic workloads of the paged-decode path, as plain data.

Shapes follow the pages' examples: 32 layers / 8 KV heads / head_dim 128 /
fp16 (youngju.dev "KV cache and paged attention", section on memory
arithmetic), 16-token blocks (same page, PagedAttention section), GQA and MQA
head layouts (same page, GQA/MQA section), fp8 KV (same page, KV quantisation
section), a shared 200-token prefix with ~50-token suffixes over 100 requests
(iq-blog ch.4 "Why PagedAttention cuts GPU memory waste", Prefix Caching
section).  All values are N(0,1); no dataset is involved.
"""
from __future__ import annotations

from dataclasses import dataclass, field

from .generators import seed_for, uniform_ints


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    layers: int
    q_heads: int
    kv_heads: int
    head_dim: int
    block_size: int
    dtype: str  # "fp16" or "fp8"
    num_blocks: int
    num_seqs: int
    context: tuple = ()  # per-sequence context lengths when fixed
    partition_tokens: int = 0  # 0: library default
    repeats: int = 1  # "1 layer timed xR"
    extra: dict = field(default_factory=dict)

    @property
    def seed(self) -> int:
        return seed_for(self.index)

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads


def _fp8_variants():
    out = {}
    for hkv in (8, 1):
        for bs in (8, 16, 32):
            n = 64 * 8192 // bs
            key = f"fp8_{'gqa' if hkv == 8 else 'mqa'}_bs{bs}"
            out[key] = Workload(5, key, 1, 32, hkv, 128, bs, "fp8", n, 64,
                                context=(8192,) * 64, repeats=32)
    return out


WORKLOADS = {
    "tiny": Workload(1, "tiny", 1, 8, 2, 128, 16, "fp16", 8, 2, context=(40, 20)),
    "gqa_32x4096": Workload(2, "gqa_32x4096", 32, 32, 8, 128, 16, "fp16", 8192, 32,
                            context=(4096,) * 32),
    # One GPU's share of gqa_32x4096 when its KV heads are split over 8 GPUs
    # (tensor parallelism): every layer's one KV head and its 4 query heads.
    "gqa_32x4096_tp8": Workload(2, "gqa_32x4096_tp8", 32, 4, 1, 128, 16, "fp16", 8192, 32,
                                context=(4096,) * 32),
    "cb_prefix": Workload(3, "cb_prefix", 1, 32, 8, 128, 16, "fp16", 16384, 256, repeats=32),
    "long_ctx": Workload(4, "long_ctx", 1, 64, 8, 128, 16, "fp16", 65536, 8,
                         context=(131072,) * 8, partition_tokens=512, repeats=80),
    **_fp8_variants(),
    # The fp8 shapes with int8 codes (per-(layer, KV head) scale and zero
    # point from each head's min/max; keys shifted by a per-head mean).
    "int8_gqa_bs16": Workload(8, "int8_gqa_bs16", 1, 32, 8, 128, 16, "int8", 64 * 8192 // 16, 64,
                              context=(8192,) * 64, repeats=32),
    "int8_mqa_bs16": Workload(8, "int8_mqa_bs16", 1, 32, 1, 128, 16, "int8", 64 * 8192 // 16, 64,
                              context=(8192,) * 64, repeats=32),
    # Requests built through the prefix cache: 4 system prompts of 1024 tokens,
    # request i takes system prompt i mod 4 plus its own U{64..1024} tokens.
    "prefix_cache": Workload(6, "prefix_cache", 1, 32, 8, 128, 16, "fp16", 16384, 256, repeats=32,
                             extra={"systems": 4, "system_tokens": 1024, "suffix": (64, 1024)}),
    # Multi-token attention: 16 prompts of 2048 tokens whose last 512 form a
    # prefill chunk (positions 1536..2047); and a mixed batch of 4 such chunks
    # with 60 decode tokens at 2048-token contexts.
    "prefill_chunks": Workload(9, "prefill_chunks", 1, 32, 8, 128, 16, "fp16", 16 * 2048 // 16, 16,
                               context=(2048,) * 16, repeats=32, extra={"queries": (512,) * 16}),
    "mixed_batch": Workload(10, "mixed_batch", 1, 32, 8, 128, 16, "fp16", 64 * 2048 // 16, 64,
                            context=(2048,) * 64, repeats=32, extra={"queries": (512,) * 4 + (1,) * 60}),
    # Beam search, width 5: 32 prompts of 2040 tokens, each with 5 beams that
    # every step re-fork from the survivors (beam_parents) and append a token.
    "beam_k5": Workload(7, "beam_k5", 1, 32, 8, 128, 16, "fp16", 8192, 160, repeats=32,
                        extra={"groups": 32, "k": 5, "prompt": 2040}),
}

# The page's own worked example of a block table: free blocks handed out in
# this order make request A (40 tokens) own blocks 0, 3, 5 and request B
# (20 tokens) own blocks 1, 2 (youngju.dev page, PagedAttention section).
PAGE_EXAMPLE_FREE_ORDER = (0, 3, 5, 1, 2, 4, 6, 7)


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def prefix_cache_prompts(seed: int, n: int, systems: int, system_tokens: int, suffix):
    """Token ids of ``n`` prompts: system prompt ``i % systems`` (ids below
    100000) followed by the request's own ``U{suffix}`` tokens (ids unique to
    it, from 100000 up)."""
    sys_ids = [list(uniform_ints(seed, 10 + k, 0, 99_999, system_tokens)) for k in range(systems)]
    lens = uniform_ints(seed, 20, suffix[0], suffix[1], n)
    prompts, nxt = [], 100_000
    for i in range(n):
        own = list(range(nxt, nxt + int(lens[i])))
        nxt += int(lens[i])
        prompts.append([int(t) for t in sys_ids[i % systems]] + own)
    return prompts


def beam_parents(seed: int, step: int, groups: int, k: int):
    """Beam survivor choice of one search step: for every group, ``k`` sorted
    indices (with repeats) of the old beams the new beams descend from."""
    out = []
    for g in range(groups):
        draws = uniform_ints(seed, 100_000 + step * 4096 + g, 0, k - 1, k)
        out.append(sorted(int(x) for x in draws))
    return out


def cb_prefix_script(seed: int, n_shared: int = 100, prefix: int = 200,
                     n_other: int = 156, suffix=(40, 60), prompt=(128, 2048),
                     gen=(1, 512)):
    """Operation script of the continuous-batching + shared-prefix workload.

    Returns ``(ops, n_rows)``.  Each op is a tuple:

    * ``("create",)``            new sequence; ids are 0, 1, 2, ... in creation order
    * ``("alloc", seq, n)``      append ``n`` tokens to ``seq``; their K/V are the next
                                 ``n`` rows of the workload's dense token-data tensor
    * ``("fork", parent)``       new sequence sharing ``parent``'s blocks
    * ``("free", seq)``
    * ``("flush",)``             write all K/V rows appended so far into the cache
                                 (needed before a copy-on-write can copy them)

    Order: one parent of ``prefix`` tokens, flush, ``n_shared`` forks, parent freed,
    ``n_other`` fresh prompts, then round-robin single-token appends across the
    unfinished sequences (forks append their suffix, the others their generated
    tokens), then a final flush.
    """
    ops = []
    rows = 0
    ops.append(("create",))
    parent = 0
    ops.append(("alloc", parent, prefix))
    rows += prefix
    ops.append(("flush",))
    children = list(range(1, n_shared + 1))
    for _ in children:
        ops.append(("fork", parent))
    ops.append(("free", parent))
    others = list(range(n_shared + 1, n_shared + 1 + n_other))
    prompts = uniform_ints(seed, 1, prompt[0], prompt[1], n_other)
    for sid, p in zip(others, prompts):
        ops.append(("create",))
        ops.append(("alloc", sid, int(p)))
        rows += int(p)
    remaining = {}
    for sid, s in zip(children, uniform_ints(seed, 2, suffix[0], suffix[1], n_shared)):
        remaining[sid] = int(s)
    for sid, g in zip(others, uniform_ints(seed, 3, gen[0], gen[1], n_other)):
        remaining[sid] = int(g)
    live = children + others
    while any(remaining[s] > 0 for s in live):
        for s in live:
            if remaining[s] > 0:
                ops.append(("alloc", s, 1))
                rows += 1
                remaining[s] -= 1
    ops.append(("flush",))
    return ops, rows
