"""Edge cases of the device path: empty batches, a one-block pool, tables
wider than the contexts, and lengths or table entries outside the contract
(flagged in the device status word and read safely: the kernels clamp them,
so every launch still completes)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from paged_kv_cache_464_amd import pa
from tests.gpu_helpers import assert_close, build_case, oracle_decode, say

pytestmark = pytest.mark.gpu

MODES = (-1, 0, 64, 48)


def test_empty_batch_writes_and_decodes_nothing():
    say("empty batch")
    c = build_case([40, 20], 8, 2, 16, 8, 6001)
    k0 = c.k[:0].contiguous()
    slots0 = c.slot_all[:0].contiguous()
    c.pool.write_kv(0, k0, k0, slots0)
    for mode in MODES:
        out = c.pool.decode(0, c.q[:0].contiguous(), c.tables[:0].contiguous(), c.lens_dev[:0].contiguous(),
                            partition_tokens=mode)
        assert tuple(out.shape) == (0, 8, 128)
        out = c.pool.write_kv_decode(0, c.k[:0].contiguous(), c.v[:0].contiguous(), slots0,
                                     c.q[:0].contiguous(), c.tables[:0].contiguous(),
                                     c.lens_dev[:0].contiguous(), partition_tokens=mode)
        assert tuple(out.shape) == (0, 8, 128)
    # Multi-token attention with no query rows at all (every n_i = 0).
    q0 = c.q[:0].contiguous()
    out = c.pool.multi_token_attention(0, q0, [0, 0, 0], c.tables, c.lens_dev)
    assert tuple(out.shape) == (0, 8, 128)
    torch.cuda.synchronize()
    assert c.pool.device_status() == 0
    # The pool is unchanged by the empty calls.
    ref = oracle_decode(c, [0, 1])
    assert_close(c.pool.decode(0, c.q, c.tables, c.lens_dev), ref, "fp16", "after empty calls")


@pytest.mark.parametrize("dtype", ["fp16", "fp8", "int8"])
@pytest.mark.parametrize("t", [1, 9, 16])
def test_one_block_pool(dtype, t):
    say("one-block pool", dtype, t)
    c = build_case([t], 32, 8, 16, 1, 6100 + t, dtype)
    ref = oracle_decode(c, [0])
    for mode in (-1, 0, 16):
        assert_close(c.pool.decode(0, c.q, c.tables, c.lens_dev, partition_tokens=mode), ref, dtype,
                     f"{dtype}/T={t}/P={mode}")
    assert c.pool.device_status() == 0


def test_table_wider_than_the_contexts():
    """Entries past a sequence's last block (-1 padding) are never read."""
    say("wide table")
    c = build_case([40, 20, 1], 16, 2, 16, 12, 6200)
    wide = np.full((3, 40), -1, dtype=np.int32)
    wide[:, : c.tables_np.shape[1]] = c.tables_np
    tables = torch.from_numpy(wide).cuda()
    ref = oracle_decode(c, [0, 1, 2])
    for mode in MODES:
        assert_close(c.pool.decode(0, c.q, tables, c.lens_dev, partition_tokens=mode), ref, "fp16",
                     f"P={mode}")
    assert c.pool.device_status() == 0


def test_out_of_contract_lengths_are_flagged_and_read_safely():
    """T = 0 gives a row of zeros; T beyond the table's width is clamped to
    it; both set PA_DEV_BAD_LEN while the other sequences stay exact."""
    say("bad lengths")
    c = build_case([40, 20, 33], 8, 2, 16, 10, 6300)
    ref = oracle_decode(c, [0, 1, 2])
    t_cap = c.tables_np.shape[1] * 16
    for mode in MODES:
        lens = torch.tensor([40, 0, t_cap + 7], dtype=torch.int32, device="cuda")
        out = c.pool.decode(0, c.q, c.tables, lens, partition_tokens=mode)
        torch.cuda.synchronize()
        flags = c.pool.device_status(clear=True)
        assert flags & pa.PA_DEV_BAD_LEN, (mode, flags)
        got = out.double().cpu().numpy()
        assert_close(got[:1], ref[:1], "fp16", f"bad lengths, valid row, P={mode}")
        assert (got[1] == 0).all(), mode
    assert c.pool.device_status() == 0


def test_out_of_range_table_entry_is_flagged_and_read_as_block_zero():
    say("bad table entry")
    c = build_case([40, 20], 8, 2, 16, 8, 6400)
    bad = c.tables_np.copy()
    bad[1, 0] = 8 + 5  # past the pool
    tables = torch.from_numpy(bad).cuda()
    ref = oracle_decode(c, [0, 1])
    for mode in (-1, 0, 16):
        out = c.pool.decode(0, c.q, tables, c.lens_dev, partition_tokens=mode)
        torch.cuda.synchronize()
        assert c.pool.device_status(clear=True) & pa.PA_DEV_BAD_BLOCK, mode
        assert_close(out[:1], ref[:1], "fp16", f"bad table entry, valid row, P={mode}")
    assert c.pool.device_status() == 0


@pytest.mark.parametrize("dtype", ["fp16", "fp8", "int8"])
@pytest.mark.parametrize("hq,hkv", [(6, 2), (12, 2), (24, 2), (20, 1), (24, 1)])
def test_decode_group_sizes_that_are_not_powers_of_two(dtype, hq, hkv):
    """Groups of 3, 6, 12, 20 and 24 query heads per KV head: the column tile
    is padded (and a second tile partly filled above 16) in every schedule."""
    seed = 6500 + 7 * hq + hkv + {"fp16": 0, "fp8": 1, "int8": 2}[dtype]
    lens = [1, 37, 700, 16, 1100]
    nb = int(sum(-(-t // 16) for t in lens)) + 4
    say("odd group", dtype, hq, hkv)
    c = build_case(lens, hq, hkv, 16, nb, seed, dtype)
    ref = oracle_decode(c, list(range(len(lens))))
    for mode in (-1, 0, 32, 64, 256):
        assert_close(c.pool.decode(0, c.q, c.tables, c.lens_dev, partition_tokens=mode), ref, dtype,
                     f"{dtype}/{hq}x{hkv}/P={mode}")
    assert c.pool.device_status() == 0


@pytest.mark.parametrize("hq,hkv", [(6, 2), (12, 2), (20, 1)])
def test_multi_token_group_sizes_that_are_not_powers_of_two(hq, hkv):
    from oracle import attention
    from tests.gpu_helpers import oracle_for
    from workloads import normal_fp16

    lens = [1, 37, 300, 1000, 129, 700]
    n = [1, 37, 45, 1, 17, 64]
    nb = int(sum(-(-t // 16) for t in lens)) + 4
    say("odd group multi-token", hq, hkv)
    c = build_case(lens, hq, hkv, 16, nb, 6600 + hq + hkv)
    qs = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    q = normal_fp16((int(qs[-1]), hq, 128), 6600 + hq, 77, "cuda")
    out = c.pool.multi_token_attention(0, q, qs, c.tables, c.lens_dev)
    st = oracle_for(c, range(len(lens)))
    ref = attention.multi_token(st, 0, q.cpu().numpy(), qs, c.tables_np, lens)
    assert_close(out, ref, "fp16", f"multi {hq}x{hkv}")
    assert c.pool.device_status() == 0
