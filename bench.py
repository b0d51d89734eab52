"""Paged decode attention benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload: 32 layers, 32 query / 8 KV heads, head_dim 128, fp16 K/V,
16-token blocks, 32 sequences with 4095 prefilled tokens, block placement a
seeded permutation of the pool.  One step = for every sequence append one
token (block manager), upload slot mapping / block tables / lengths, then for
each of the 32 layers scatter the new tokens' K/V into the cache and run paged
decode attention over the whole context (the first timed step attends to 4096
tokens).  The timed region holds exactly K steps; inputs are resident in HBM.

Prints one JSON line.  ``roofline`` is for the decode attention kernel: its
algorithmic KV bytes (each sequence's K and V, every KV head once) divided by
its average duration from HIP events recorded around every launch on the
launch stream during the timed steps.  ``cpu_baseline`` is the fp64 CPU
oracle timed on this host on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention: KV GB/s read + % HBM peak; tokens/s at 32×4096 GQA"
HBM_PEAK_GBPS = 8000.0
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "traffic_decode_gqa_32x4096.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "paged_kv_cache_464_amd", "csrc", f)
                  for f in ("decode_kernels.hip", "layout.hpp", "kernels.hpp")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel sources; else None."""
    if not os.path.exists(TRAFFIC_PROFILE):
        return None
    text = open(TRAFFIC_PROFILE).read()
    m_hash = re.search(r"kernel_source_sha256:\s*(\w+)", text)
    m_val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_hash and m_val) or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_val.group(1))


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return int(os.environ.get("OMP_NUM_THREADS", "1"))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---------------------------------------------------------------------------
# GQA decode step: 32 layers x 32 sequences x 4096 tokens
# ---------------------------------------------------------------------------

class GqaStep:
    def __init__(self, args):
        import torch

        from paged_kv_cache_464_amd import pa
        from workloads import free_order, normal_fp16, workload

        self.torch, self.pa = torch, pa
        w = workload("gqa_32x4096")
        self.w = w
        self.dev = "cuda"
        self.L, self.S, self.hq, self.hkv, self.bs = w.layers, w.num_seqs, w.q_heads, w.kv_heads, w.block_size
        self.prefill = w.context[0] - 1
        total_steps = args.warmup + args.steps
        # Exactly the 4096-token working set plus room for the appended tokens.
        extra_blocks = self.S * (-(-(self.prefill + total_steps) // self.bs) - w.context[0] // self.bs)
        self.num_blocks = w.num_blocks + max(extra_blocks, 0)
        self.order = free_order(w.seed, self.num_blocks)
        self.pool = pa.PagedKVPool(self.L, self.hkv, 128, self.bs, self.num_blocks, "fp16",
                                   free_order=self.order)
        self.partition = args.partition
        self.seqs = [self.pool.seq_create() for _ in range(self.S)]
        slots = [self.pool.alloc(s, self.prefill)[0] for s in self.seqs]
        slot_all = torch.from_numpy(np.concatenate(slots)).to(self.dev)
        self.prefill_slots = slots
        n_tok = self.S * self.prefill
        self.sample_kv = None
        for layer in range(self.L):
            k = normal_fp16((n_tok, self.hkv, 128), w.seed, 10_000 + 2 * layer, self.dev)
            v = normal_fp16((n_tok, self.hkv, 128), w.seed, 10_001 + 2 * layer, self.dev)
            self.pool.write_kv(layer, k, v, slot_all)
            if layer == 0 and not args.no_cpu_baseline:
                self.sample_kv = (k.cpu().numpy(), v.cpu().numpy())
            del k, v
        # Per-layer step inputs, resident for the whole run.
        self.q = normal_fp16((self.L, self.S, self.hq, 128), w.seed, 1, self.dev)
        self.k_new = normal_fp16((self.L, self.S, self.hkv, 128), w.seed, 2, self.dev)
        self.v_new = normal_fp16((self.L, self.S, self.hkv, 128), w.seed, 3, self.dev)
        self.out = torch.empty((self.L, self.S, self.hq, 128), dtype=torch.float16, device=self.dev)
        # Block tables are uploaded at a fixed width with room for every appended token.
        self.mb_cap = -(-(self.prefill + total_steps) // self.bs)
        ws = pa.pa_decode_workspace_bytes(self.pool.handle, self.S, self.hq, self.mb_cap,
                                          self.partition)
        self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=self.dev)
        # Step metadata (slot mapping, lengths, block tables) is packed into one
        # int32 buffer so that each step makes a single upload: two pinned host
        # copies used alternately (each guarded by the event of the upload that
        # last read it) and one device copy.
        n_meta = self.S * (2 + self.mb_cap)
        self.pinned = [torch.empty(n_meta, dtype=torch.int32, pin_memory=True) for _ in range(2)]
        self.uploaded = [torch.cuda.Event(), torch.cuda.Event()]
        self.meta_d = torch.empty(n_meta, dtype=torch.int32, device=self.dev)
        self.slots_d = self.meta_d[:self.S]
        self.lens_d = self.meta_d[self.S:2 * self.S]
        self.tables_d = self.meta_d[2 * self.S:].view(self.S, self.mb_cap)
        self.n_step = 0
        self.stream = torch.cuda.current_stream().cuda_stream  # every launch goes here
        self.kv_bytes_log = []
        self.first_step_slots = None
        torch.cuda.synchronize()

    def step(self):
        pa = self.pa
        k = self.n_step % 2
        self.n_step += 1
        self.uploaded[k].synchronize()  # the upload that last read this pinned set is done
        meta = self.pinned[k].numpy()
        slots = meta[:self.S]
        for i, s in enumerate(self.seqs):
            slots[i] = self.pool.alloc(s, 1)[0][0]
        if self.first_step_slots is None:
            self.first_step_slots = slots.copy()
        tables, lens = self.pool.block_tables(self.seqs, self.mb_cap)
        meta[self.S:2 * self.S] = lens
        meta[2 * self.S:] = tables.reshape(-1)
        self.meta_d.copy_(self.pinned[k], non_blocking=True)
        self.uploaded[k].record()
        h, st = self.pool.handle, self.stream
        for layer in range(self.L):
            pa.pa_write_kv(h, layer, self.k_new[layer], self.v_new[layer], self.slots_d, stream=st)
            pa.pa_decode(h, layer, self.q[layer], self.tables_d, self.lens_d, out=self.out[layer],
                         partition_tokens=self.partition, workspace=self.workspace, stream=st)
        self.kv_bytes_log.append(int(lens.astype(np.int64).sum()) * 2 * self.hkv * 128 * 2)
        return lens

    def cpu_baseline(self, budget_s):
        """fp64 oracle on layer 0 of this workload at the first step's context
        (4096 tokens), whole sequences, repeated over sequences until about
        ``budget_s`` seconds of attention math; scaled to all 32 layers."""
        from oracle import attention
        from oracle.kvstore import OracleKVStore

        k_all, v_all = self.sample_kv
        st = OracleKVStore(1, self.num_blocks, self.hkv, self.bs, 128)
        for i in range(self.S):
            a, b = i * self.prefill, (i + 1) * self.prefill
            st.write(0, k_all[a:b], v_all[a:b], self.prefill_slots[i])
        st.write(0, self.k_new[0].cpu().numpy(), self.v_new[0].cpu().numpy(), self.first_step_slots)
        ctx = self.prefill + 1
        nb = -(-ctx // self.bs)
        tables, _ = self.pool.block_tables(self.seqs, self.pool.seq_len(self.seqs[0])[1])
        tables = tables[:, :nb]
        q0 = self.q[0].cpu().numpy()
        done, t_total = 0, 0.0
        while t_total < budget_s and done < self.S:
            t0 = time.perf_counter()
            attention.decode(st, 0, q0[done:done + 1], tables[done:done + 1], [ctx])
            t_total += time.perf_counter() - t0
            done += 1
        per_seq_layer = t_total / done
        step_s = per_seq_layer * self.S * self.L
        return {
            "value": self.S / step_s,
            "unit": "tokens/s",
            "cores": blas_threads(),
            "kind": "oracle",
            "sample": (f"layer 0, {done} of {self.S} sequences x {ctx} tokens x {self.hq} query heads "
                       f"({t_total:.1f} s of attention math, numpy fp64); scaled x{self.S}/{done} "
                       f"sequences x {self.L} layers to one decode step"),
            "kv_gbps": (ctx * 2 * self.hkv * 128 * 2) / per_seq_layer / 1e9,
            "host_cpus": len(os.sched_getaffinity(0)),
            "cpu_count": os.cpu_count(),
            "cpu_model": cpu_model(),
        }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gqa_32x4096", choices=["gqa_32x4096"])
    ap.add_argument("--partition", type=int, default=0,
                    help="partition_tokens for pa_decode (0: library default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after the run, copy a buffer of this many MiB once (HBM counter calibration)")
    args = ap.parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the paged decode path has no multi-GPU mode)", file=sys.stderr)
        return 2

    import torch

    from paged_kv_cache_464_amd import _lib, pa

    if not os.path.exists(_lib.LIB_PATH):
        from paged_kv_cache_464_amd import build as _build
        _build.build()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)

    bench = GqaStep(args)
    for _ in range(args.warmup):
        bench.step()
    torch.cuda.synchronize()
    bench.kv_bytes_log.clear()
    pa.pa_profile_begin(bench.pool.handle, args.steps * bench.L)
    lens_seen = []
    gc.collect()
    gc.disable()  # no collector pauses inside the timed steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        lens_seen.append(int(bench.step()[0]))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gc.enable()
    prof = pa.pa_profile_end(bench.pool.handle)
    status = bench.pool.device_status()
    if status:
        print(f"device status flags {status:#x}", file=sys.stderr)
        return 1
    # The CPU oracle runs after the timed steps so that its BLAS threads cannot
    # compete with the host side of the step.
    cpu = None
    if not args.no_cpu_baseline:
        cpu = bench.cpu_baseline(args.cpu_budget)

    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_s = bench.S * args.steps / elapsed
    kv_bytes = float(sum(bench.kv_bytes_log)) * bench.L  # over all timed decode launches
    decode_s = prof["decode_ms"] / 1e3
    reduce_s = prof["reduce_ms"] / 1e3
    achieved = kv_bytes / decode_s / 1e9
    kv_gbps = kv_bytes / (decode_s + reduce_s) / 1e9
    traffic = stored_traffic()
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
    result = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": "gqa_32x4096",
            "layers": bench.L, "num_seqs": bench.S, "q_heads": bench.hq, "kv_heads": bench.hkv,
            "head_dim": 128, "block_size": bench.bs, "kv_dtype": "fp16", "accumulate": "fp32",
            "context_first_timed_step": lens_seen[0], "context_last_timed_step": lens_seen[-1],
            "num_blocks": bench.num_blocks, "partition_tokens": args.partition,
            "step": "alloc 1 token/seq + 32 x (write_kv + paged decode); attention only",
        },
        "kv_gbps": kv_gbps,
        "hbm_frac": kv_gbps / HBM_PEAK_GBPS,
        "decode_kernel_us": prof["decode_ms"] * 1e3 / max(prof["decode_launches"], 1),
        "reduce_kernel_us": prof["reduce_ms"] * 1e3 / max(prof["reduce_launches"], 1),
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
            "kernel": "paged decode attention (per launch: 32 seqs x T x 8 KV heads x 128 x 2 B x K,V)",
            "algorithmic_bytes_per_launch": kv_bytes / max(prof["decode_launches"], 1),
            "kernel_source": kernel_source_hash(),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
