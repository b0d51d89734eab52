"""Decode launches captured in a HIP graph (torch.cuda.CUDAGraph), as a
serving loop that replays a whole step would: the split fused write + decode
with its reduce, the no-allocation decode and a planned shared-prefix
decode (plans and workspaces made before the capture; the launches
themselves only launch kernels).  Every replay, with new queries and eager
work in between, equals the eager calls bit for bit, and the eager outputs
match the oracle."""
import numpy as np
import pytest
import torch

from oracle import attention
from paged_kv_cache_464_amd import pa
from tests.gpu_helpers import assert_close, say
from tests.test_gpu_shared_prefix import build_tree, oracle_store
from workloads import normal_fp16

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_decode_step_replays_in_a_hip_graph():
    say("graph capture of a decode step")
    hq, hkv, D = 32, 8, 128
    t = build_tree([(600, [3, 40, 17, 90, 5]), (1030, [64, 2, 30])], [2000, 77, 513], hq, hkv, 16, seed=464_300)
    S = len(t.batch)
    h = t.pool.handle
    # The new token of every sequence is its last one, written again at its
    # own slot (the same bytes: the replays leave the pool unchanged).
    last = np.asarray([int(x) - 1 for x in t.lens_np])
    kn = torch.stack([t.rows[s][0][last[i]] for i, s in enumerate(t.batch)]).contiguous()
    vn = torch.stack([t.rows[s][1][last[i]] for i, s in enumerate(t.batch)]).contiguous()
    sl = torch.from_numpy((t.tables_np[np.arange(S), last // 16] * 16 + last % 16).astype(np.int32)).cuda()
    P = 256
    ws = torch.empty(max(pa.pa_decode_workspace_bytes(h, S, hq, t.mb, P), 256), dtype=torch.uint8, device="cuda")
    g = t.pool.shared_prefix_groups(t.tables_np, t.lens_np, 256)
    plan_fold = t.pool.shared_prefix_plan(S, hq, t.mb, g, lens=t.lens_np)
    plan_pieces = t.pool.shared_prefix_plan(S, hq, t.mb, g, chunk_tokens=256)
    assert plan_fold.plan.num_items > 0 and plan_pieces.plan.num_slots > 0
    q = normal_fp16((S, hq, D), 464_300, 3, "cuda")

    def step(outs):
        pa.pa_write_kv_decode(h, 0, kn, vn, sl, q, t.tables, t.lens, out=outs[0], partition_tokens=P, workspace=ws)
        pa.pa_decode_noalloc(h, 0, q, t.tables, t.lens, outs[1], partition_tokens=512)
        pa.pa_decode_shared_prefix(h, 0, q, t.tables, t.lens, plan_fold, out=outs[2], k_new=kn, v_new=vn,
                                   slot_mapping=sl)
        pa.pa_decode_shared_prefix(h, 0, q, t.tables, t.lens, plan_pieces, out=outs[3])

    outs_e = [torch.empty_like(q) for _ in range(4)]
    outs_g = [torch.empty_like(q) for _ in range(4)]
    step(outs_e)  # eager warm-up before the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(outs_g)
    torch.cuda.synchronize()
    st = oracle_store(t)
    for rep in range(3):
        q.copy_(normal_fp16((S, hq, D), 464_300, 10 + rep, "cuda"))
        step(outs_e)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs_g, outs_e)):
            assert torch.equal(a, b), f"replay {rep}, launch {i} differs from the eager call"
        ref = attention.decode(st, 0, q.cpu().numpy(), t.tables_np, t.lens_np)
        for i in range(4):
            assert_close(outs_e[i], ref, "fp16", f"graph step replay {rep}, launch {i}")
    assert t.pool.device_status() == 0
