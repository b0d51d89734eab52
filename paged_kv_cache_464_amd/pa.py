"""Python binding of libpa with the C ABI's names (argument marshalling only).

Every function here converts Python/torch arguments to the plain pointers and
sizes of include/pa.h, checks that device tensors have the shapes, dtypes and
devices the kernels assume (so a wrong shape is an exception on the host, not
an out-of-bounds access on the GPU), calls the C function and raises on a
non-zero status.  All computation happens in libpa.so.
"""
from __future__ import annotations

import ctypes as C

import numpy as np
import torch

from . import _lib
from ._lib import (PA_DTYPE_FP16, PA_DTYPE_FP8_E4M3, PA_DTYPE_INT8, PA_ERR_BAD_SEQ, PA_ERR_NO_BLOCKS,  # noqa: F401
                   PA_DEV_BAD_BLOCK, PA_DEV_BAD_LEN, PA_DEV_BAD_ORDER, PA_DEV_BAD_SLOT,
                   PA_LOADS_AUTO, PA_LOADS_CACHED, PA_LOADS_STREAMING, PA_NOALLOC_SCRATCH_BYTES,
                   PA_SHARED_REREAD)


class PAError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libpa error {code}: {msg}")
        self.code = code


class NoBlocksError(PAError):
    pass


class BadSeqError(PAError):
    pass


def _check(rc):
    if rc != 0:
        msg = _lib.load().pa_last_error().decode()
        cls = {PA_ERR_NO_BLOCKS: NoBlocksError, PA_ERR_BAD_SEQ: BadSeqError}.get(rc, PAError)
        raise cls(rc, msg)


def _L():
    return _lib.load()


def _i32_host(a):
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return arr, arr.ctypes.data_as(C.POINTER(C.c_int32))


def _stream(stream):
    if stream is None:
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return C.c_void_p(stream.cuda_stream)
    return C.c_void_p(int(stream))


def _dev(t, dtype, shape=None, name="tensor"):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return C.c_void_p(t.data_ptr())


# ---- pool ------------------------------------------------------------------

def pa_pool_create(layers, kv_heads, head_dim, block_size, dtype, num_blocks) -> int:
    h = C.c_void_p()
    _check(_L().pa_pool_create(layers, kv_heads, head_dim, block_size, dtype, num_blocks, C.byref(h)))
    return h.value


# Per-handle caches of values that cannot change once a pool is bound (its
# geometry, and the workspace size of a launch shape), so that the per-launch
# wrappers below make one library call instead of three.
_BOUND_INFO = {}
_WS_BYTES = {}


def _forget(h):
    _BOUND_INFO.pop(h, None)
    for key in [k for k in _WS_BYTES if k[0] == h]:
        del _WS_BYTES[key]


def pa_pool_destroy(h):
    _forget(h)
    _check(_L().pa_pool_destroy(C.c_void_p(h)))


def pa_pool_info_get(h) -> dict:
    info = _lib.pa_pool_info()
    _check(_L().pa_pool_info_get(C.c_void_p(h), C.byref(info)))
    return {f: getattr(info, f) for f, _ in info._fields_}


def _info(h) -> dict:
    info = _BOUND_INFO.get(h)
    if info is None:
        info = pa_pool_info_get(h)
        if info["bound"]:
            _BOUND_INFO[h] = info
    return info


def pa_pool_set_free_order(h, perm):
    arr, ptr = _i32_host(perm)
    _check(_L().pa_pool_set_free_order(C.c_void_p(h), ptr, len(arr)))


def pa_pool_set_load_policy(h, policy):
    """PA_LOADS_AUTO, PA_LOADS_STREAMING or PA_LOADS_CACHED (K/V loads of decode)."""
    _check(_L().pa_pool_set_load_policy(C.c_void_p(h), int(policy)))


def pa_pool_load_policy(h):
    """(policy, whether a decode launched now would use ordinary loads)."""
    pol, now = C.c_int32(), C.c_int32()
    _check(_L().pa_pool_load_policy(C.c_void_p(h), C.byref(pol), C.byref(now)))
    return pol.value, bool(now.value)


def pa_pool_bind(h, dev_ptr: int, k_scales=None, v_scales=None):
    def fp(a):
        if a is None:
            return None, None
        arr = np.ascontiguousarray(np.asarray(a, dtype=np.float32).reshape(-1))
        return arr, arr.ctypes.data_as(C.POINTER(C.c_float))
    ka, kp = fp(k_scales)
    va, vp = fp(v_scales)
    _forget(h)
    _check(_L().pa_pool_bind(C.c_void_p(h), C.c_void_p(dev_ptr), kp, vp))


def pa_pool_bind_int8(h, dev_ptr: int, k_scales, v_scales, k_zeros, v_zeros):
    """Bind an int8 pool: fp32 scales and int32 zero points, each [layers*kv_heads]."""
    arrs = [np.ascontiguousarray(np.asarray(a, dtype=dt).reshape(-1))
            for a, dt in ((k_scales, np.float32), (v_scales, np.float32),
                          (k_zeros, np.int32), (v_zeros, np.int32))]
    ptrs = [a.ctypes.data_as(C.POINTER(C.c_float if a.dtype == np.float32 else C.c_int32)) for a in arrs]
    _forget(h)
    _check(_L().pa_pool_bind_int8(C.c_void_p(h), C.c_void_p(dev_ptr), *ptrs))


# ---- block manager ---------------------------------------------------------

def pa_seq_create(h) -> int:
    s = C.c_int32()
    _check(_L().pa_seq_create(C.c_void_p(h), C.byref(s)))
    return s.value


def pa_seq_create_cached(h, tokens):
    """Returns (seq, cached_tokens, slots of the uncached tokens)."""
    t, tp = _i32_host(tokens)
    slots = np.empty(max(len(t), 1), dtype=np.int32)
    s, c = C.c_int32(), C.c_int32()
    _check(_L().pa_seq_create_cached(C.c_void_p(h), tp, len(t), C.byref(s), C.byref(c),
                                     slots.ctypes.data_as(C.POINTER(C.c_int32))))
    return s.value, c.value, slots[:len(t) - c.value].copy()


def pa_alloc(h, seq, n_tokens, stream=0, tokens=None):
    """Returns (slots int32[n_tokens], (src, dst) or None).  ``tokens``: the
    appended token ids (pa_alloc_tokens), or None."""
    slots = np.empty(max(int(n_tokens), 0), dtype=np.int32)
    cow = np.full(2, -1, dtype=np.int32)
    st = C.c_void_p(0) if stream == 0 else _stream(stream)
    tp = None
    if tokens is not None:
        t_arr, tp = _i32_host(tokens)
        if len(t_arr) != int(n_tokens):
            raise ValueError("tokens must hold n_tokens ids")
    _check(_L().pa_alloc_tokens(C.c_void_p(h), int(seq), int(n_tokens), tp,
                                slots.ctypes.data_as(C.POINTER(C.c_int32)),
                                cow.ctypes.data_as(C.POINTER(C.c_int32)), st))
    return slots, (None if cow[0] < 0 else (int(cow[0]), int(cow[1])))


def pa_alloc_batch(h, seqs, n_tokens, stream=0, tokens=None):
    """Appends n_tokens[k] tokens to seqs[k] for every k in order, with one
    launch for all copy-on-write copies.  Returns (slots int32[sum n_tokens],
    cow int32[count][2] with -1 where an append copied nothing).  ``tokens``:
    the appended ids back to back, or None.

    If append k fails, appends 0 .. k-1 stay made (their copies enqueued): the
    raised error carries ``done`` = k and the ``slots`` and ``cow`` of those
    appends, so that the caller can still write their K/V."""
    s_arr, s_ptr = _i32_host(seqs)
    n_arr, n_ptr = _i32_host(n_tokens)
    if len(s_arr) != len(n_arr):
        raise ValueError("seqs and n_tokens differ in length")
    total = int(n_arr.sum()) if len(n_arr) else 0
    slots = np.empty(max(total, 0), dtype=np.int32)
    cow = np.full((len(s_arr), 2), -1, dtype=np.int32)
    tp = None
    if tokens is not None:
        t_arr, tp = _i32_host(tokens)
        if len(t_arr) != total:
            raise ValueError("tokens must hold sum(n_tokens) ids")
    done = C.c_int32()
    st = C.c_void_p(0) if stream == 0 else _stream(stream)
    rc = _L().pa_alloc_batch(C.c_void_p(h), s_ptr, n_ptr, len(s_arr), tp,
                             slots.ctypes.data_as(C.POINTER(C.c_int32)),
                             cow.ctypes.data_as(C.POINTER(C.c_int32)), C.byref(done), st)
    try:
        _check(rc)
    except PAError as e:
        k = done.value
        e.done = k
        e.slots = slots[:int(n_arr[:k].sum()) if k else 0].copy()
        e.cow = cow[:k].copy()
        raise
    return slots, cow


def pa_fork(h, parent) -> int:
    c = C.c_int32()
    _check(_L().pa_fork(C.c_void_p(h), int(parent), C.byref(c)))
    return c.value


def pa_free(h, seq):
    _check(_L().pa_free(C.c_void_p(h), int(seq)))


def pa_seq_len(h, seq):
    ln, nb = C.c_int32(), C.c_int32()
    _check(_L().pa_seq_len(C.c_void_p(h), int(seq), C.byref(ln), C.byref(nb)))
    return ln.value, nb.value


def pa_block_tables(h, seqs, max_blocks):
    s, sp = _i32_host(seqs)
    tables = np.empty((len(s), int(max_blocks)), dtype=np.int32)
    lens = np.empty(len(s), dtype=np.int32)
    _check(_L().pa_block_tables(C.c_void_p(h), sp, len(s), int(max_blocks),
                                tables.ctypes.data_as(C.POINTER(C.c_int32)),
                                lens.ctypes.data_as(C.POINTER(C.c_int32))))
    return tables, lens


def pa_pool_stats(h) -> dict:
    st = _lib.pa_stats()
    _check(_L().pa_pool_stats(C.c_void_p(h), C.byref(st)))
    return {f: getattr(st, f) for f, _ in st._fields_}


def pa_refcounts(h):
    n = pa_pool_info_get(h)["num_blocks"]
    out = np.empty(n, dtype=np.int32)
    _check(_L().pa_refcounts(C.c_void_p(h), out.ctypes.data_as(C.POINTER(C.c_int32))))
    return out


def pa_free_queue(h):
    n = pa_pool_info_get(h)["num_blocks"]
    out = np.empty(n, dtype=np.int32)
    cnt = C.c_int32()
    _check(_L().pa_free_queue(C.c_void_p(h), out.ctypes.data_as(C.POINTER(C.c_int32)), C.byref(cnt)))
    return out[:cnt.value].copy()


# ---- device operations ------------------------------------------------------

def pa_write_kv(h, layer, k_new, v_new, slot_mapping, stream=None):
    info = _info(h)
    n = slot_mapping.numel()
    shape = (n, info["kv_heads"], info["head_dim"])
    kp = _dev(k_new, torch.float16, shape, "k_new")
    vp = _dev(v_new, torch.float16, shape, "v_new")
    sp = _dev(slot_mapping, torch.int32, (n,), "slot_mapping")
    _check(_L().pa_write_kv(C.c_void_p(h), int(layer), kp, vp, sp, n, _stream(stream)))


def pa_gather_kv(h, layer, slot_mapping, k_out, v_out, stream=None):
    info = _info(h)
    n = slot_mapping.numel()
    dt = {PA_DTYPE_FP16: torch.float16, PA_DTYPE_FP8_E4M3: torch.uint8, PA_DTYPE_INT8: torch.int8}[info["dtype"]]
    shape = (n, info["kv_heads"], info["head_dim"])
    sp = _dev(slot_mapping, torch.int32, (n,), "slot_mapping")
    kp = _dev(k_out, dt, shape, "k_out")
    vp = _dev(v_out, dt, shape, "v_out")
    _check(_L().pa_gather_kv(C.c_void_p(h), int(layer), sp, n, kp, vp, _stream(stream)))


def pa_copy_blocks(h, src, dst, stream=None):
    s, sp = _i32_host(src)
    d, dp = _i32_host(dst)
    if len(s) != len(d):
        raise ValueError("src and dst differ in length")
    _check(_L().pa_copy_blocks(C.c_void_p(h), sp, dp, len(s), _stream(stream)))


def pa_decode_workspace_bytes(h, num_seqs, num_q_heads, max_blocks, partition_tokens=0) -> int:
    out = C.c_uint64()
    _check(_L().pa_decode_workspace_bytes(C.c_void_p(h), int(num_seqs), int(num_q_heads),
                                          int(max_blocks), int(partition_tokens), C.byref(out)))
    return out.value


def _decode_args(h, q, block_tables, context_lens):
    info = _info(h)
    if q.dim() != 3 or q.shape[2] != info["head_dim"]:
        raise ValueError(f"q must be [num_seqs][num_q_heads][{info['head_dim']}]")
    s, hq = int(q.shape[0]), int(q.shape[1])
    if block_tables.dim() != 2 or block_tables.shape[0] != s:
        raise ValueError("block_tables must be [num_seqs][max_blocks]")
    mb = int(block_tables.shape[1])
    qp = _dev(q, torch.float16, None, "q")
    tp = _dev(block_tables, torch.int32, None, "block_tables")
    lp = _dev(context_lens, torch.int32, (s,), "context_lens")
    return info, s, hq, mb, qp, tp, lp


def _workspace(h, s, hq, mb, partition_tokens, workspace, device):
    key = (h, s, hq, mb, int(partition_tokens))
    need = _WS_BYTES.get(key)
    if need is None:
        need = pa_decode_workspace_bytes(h, s, hq, mb, partition_tokens)
        if _info(h)["bound"]:
            _WS_BYTES[key] = need
    if need == 0:
        return C.c_void_p(0), 0, workspace
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    return C.c_void_p(workspace.data_ptr()), need, workspace


def pa_stream_read(buf, sink, stream=None):
    """Streaming-read reference kernel over a device tensor (its whole storage)."""
    n = buf.numel() * buf.element_size()
    n -= n % 16
    _check(_L().pa_stream_read(C.c_void_p(buf.data_ptr()), n, C.c_void_p(sink.data_ptr()), _stream(stream)))


def pa_order_longest_first(lens):
    """Indices of lens by decreasing length, ties in increasing index (host int32)."""
    a, ap = _i32_host(lens)
    order = np.empty(len(a), dtype=np.int32)
    _check(_L().pa_order_longest_first(ap, len(a), order.ctypes.data_as(C.POINTER(C.c_int32))))
    return order


def _order_arg(seq_order, s):
    if seq_order is None:
        return C.c_void_p(0)
    return _dev(seq_order, torch.int32, (s,), "seq_order")


def pa_decode(h, layer, q, block_tables, context_lens, out=None, scale=None, partition_tokens=0,
              workspace=None, stream=None, seq_order=None):
    info, s, hq, mb, qp, tp, lp = _decode_args(h, q, block_tables, context_lens)
    orp = _order_arg(seq_order, s)
    if out is None:
        out = torch.empty_like(q)
    op = _dev(out, torch.float16, tuple(q.shape), "out")
    wp, wb, workspace = _workspace(h, s, hq, mb, partition_tokens, workspace, q.device)
    if scale is None:
        scale = info["softmax_scale"]
    _check(_L().pa_decode(C.c_void_p(h), int(layer), qp, hq, tp, mb, lp, s, orp, float(scale),
                          int(partition_tokens), op, wp, wb, _stream(stream)))
    return out


def pa_decode_noalloc(h, layer, q, block_tables, context_lens, out, scale=None, partition_tokens=0,
                      stream=None, seq_order=None):
    """pa_decode without a workspace: split-context partials live in the
    library's static device scratch.  ``out`` is required (no allocation)."""
    info, s, hq, mb, qp, tp, lp = _decode_args(h, q, block_tables, context_lens)
    orp = _order_arg(seq_order, s)
    op = _dev(out, torch.float16, tuple(q.shape), "out")
    if scale is None:
        scale = info["softmax_scale"]
    _check(_L().pa_decode_noalloc(C.c_void_p(h), int(layer), qp, hq, tp, mb, lp, s, orp, float(scale),
                                  int(partition_tokens), op, _stream(stream)))
    return out


def pa_write_kv_decode(h, layer, k_new, v_new, slot_mapping, q, block_tables, context_lens,
                       out=None, scale=None, partition_tokens=0, workspace=None, stream=None,
                       seq_order=None):
    """pa_write_kv of each sequence's new (last) token fused into pa_decode."""
    info, s, hq, mb, qp, tp, lp = _decode_args(h, q, block_tables, context_lens)
    shape = (s, info["kv_heads"], info["head_dim"])
    kp = _dev(k_new, torch.float16, shape, "k_new")
    vp = _dev(v_new, torch.float16, shape, "v_new")
    sp = _dev(slot_mapping, torch.int32, (s,), "slot_mapping")
    orp = _order_arg(seq_order, s)
    if out is None:
        out = torch.empty_like(q)
    op = _dev(out, torch.float16, tuple(q.shape), "out")
    wp, wb, workspace = _workspace(h, s, hq, mb, partition_tokens, workspace, q.device)
    if scale is None:
        scale = info["softmax_scale"]
    _check(_L().pa_write_kv_decode(C.c_void_p(h), int(layer), kp, vp, sp, qp, hq, tp, mb, lp, s, orp,
                                   float(scale), int(partition_tokens), op, wp, wb, _stream(stream)))
    return out


def pa_shared_prefix_groups(h, tables, lens, min_shared_tokens=256):
    """Groups of sequences sharing leading blocks, from host block tables
    [n][max_blocks] and lengths: (members, group_start, shared_blocks) host
    int32 arrays (see pa_decode_shared_prefix)."""
    t = np.ascontiguousarray(np.asarray(tables, dtype=np.int32))
    ln, lp = _i32_host(lens)
    n, mb = t.shape
    if len(ln) != n:
        raise ValueError("lens and tables differ in length")
    members = np.empty(max(n, 1), dtype=np.int32)
    gstart = np.empty(n + 1, dtype=np.int32)
    shared = np.empty(max(n, 1), dtype=np.int32)
    ng = C.c_int32()
    ip = lambda a: a.ctypes.data_as(C.POINTER(C.c_int32))
    _check(_L().pa_shared_prefix_groups(C.c_void_p(h), ip(t), lp, n, mb, int(min_shared_tokens), ip(members),
                                        ip(gstart), ip(shared), C.byref(ng)))
    g = ng.value
    return members[:n].copy(), gstart[:g + 1].copy(), shared[:g].copy()


def _groups_args(groups, num_seqs):
    members, gstart, shared = (np.ascontiguousarray(np.asarray(a, dtype=np.int32).reshape(-1)) for a in groups)
    if len(members) != num_seqs or len(gstart) != len(shared) + 1:
        raise ValueError("groups must be (members[num_seqs], group_start[num_groups + 1], shared_blocks[num_groups])")
    ip = lambda a: a.ctypes.data_as(C.POINTER(C.c_int32))
    return (members, gstart, shared), ip(members), ip(gstart), ip(shared), len(shared)


def _lens_arg(lens, num_seqs):
    if lens is None:
        return None, None
    arr, ptr = _i32_host(lens)
    if len(arr) != num_seqs:
        raise ValueError("lens must hold one length per sequence")
    return arr, ptr


def pa_decode_shared_prefix_workspace_bytes(h, num_seqs, num_q_heads, groups, max_blocks, chunk_tokens=0,
                                            lens=None):
    keep, mp, gp, sp, ng = _groups_args(groups, num_seqs)
    la, lp = _lens_arg(lens, num_seqs)
    b = C.c_uint64()
    _check(_L().pa_decode_shared_prefix_workspace_bytes(C.c_void_p(h), int(num_seqs), int(num_q_heads), mp, gp,
                                                        sp, ng, int(max_blocks), int(chunk_tokens), lp,
                                                        C.byref(b)))
    return b.value


class SharedPlan:
    """A checked, uploaded group list (pa_shared_prefix_plan) and the
    workspace it lives in; one plan serves every layer of a step."""

    def __init__(self, plan, workspace, groups):
        self.plan, self.workspace, self.groups = plan, workspace, groups


def pa_shared_prefix_plan(h, num_seqs, num_q_heads, max_blocks, groups, workspace=None, stream=None,
                          device="cuda", chunk_tokens=0, lens=None):
    """Checks and uploads the groups (see pa_decode_shared_prefix).  ``lens``:
    host context lengths, which let the plan fold groups whose members have
    few tokens of their own (None: no folding)."""
    keep, mp, gp, sp, ng = _groups_args(groups, num_seqs)
    la, lp = _lens_arg(lens, num_seqs)
    need = pa_decode_shared_prefix_workspace_bytes(h, num_seqs, num_q_heads, keep, max_blocks, chunk_tokens, la)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    nbytes = workspace.numel() * workspace.element_size()
    if nbytes < need:
        raise ValueError(f"workspace needs {need} bytes")
    plan = _lib.pa_shared_plan()
    _check(_L().pa_shared_prefix_plan(C.c_void_p(h), int(num_seqs), int(num_q_heads), int(max_blocks), mp, gp,
                                      sp, ng, int(chunk_tokens), lp, C.c_void_p(workspace.data_ptr()), nbytes,
                                      _stream(stream), C.byref(plan)))
    return SharedPlan(plan, workspace, keep)


def pa_decode_shared_prefix(h, layer, q, block_tables, context_lens, groups, out=None, scale=None,
                            workspace=None, stream=None, k_new=None, v_new=None, slot_mapping=None,
                            chunk_tokens=0, lens=None):
    """Decode where groups of sequences share leading blocks.  ``groups`` is a
    SharedPlan (pa_shared_prefix_plan) or the (members, group_start,
    shared_blocks) arrays of pa_shared_prefix_groups, planned here on the
    call's stream (``lens``: host context lengths for the plan's folding).
    With k_new, v_new and slot_mapping, the new tokens are scattered as in
    pa_write_kv_decode."""
    info, s, hq, mb, qp, tp, lp = _decode_args(h, q, block_tables, context_lens)
    if not isinstance(groups, SharedPlan):
        groups = pa_shared_prefix_plan(h, s, hq, mb, groups, workspace, stream, q.device, chunk_tokens, lens)
    p = groups.plan
    if (p.num_seqs, p.num_q_heads, p.max_blocks) != (s, hq, mb):
        raise ValueError(f"the plan is for {p.num_seqs} sequences, {p.num_q_heads} query heads and tables "
                         f"{p.max_blocks} wide; got {s}, {hq}, {mb}")
    if out is None:
        out = torch.empty_like(q)
    op = _dev(out, torch.float16, tuple(q.shape), "out")
    kp = vp = slp = C.c_void_p(0)
    if k_new is not None or v_new is not None or slot_mapping is not None:
        shape = (s, info["kv_heads"], info["head_dim"])
        kp = _dev(k_new, torch.float16, shape, "k_new")
        vp = _dev(v_new, torch.float16, shape, "v_new")
        slp = _dev(slot_mapping, torch.int32, (s,), "slot_mapping")
    if scale is None:
        scale = info["softmax_scale"]
    _check(_L().pa_decode_shared_prefix(C.c_void_p(h), int(layer), C.byref(p), qp, tp, lp, kp, vp, slp,
                                        float(scale), op, _stream(stream)))
    return out


def pa_multi_token_workspace_bytes(h, query_start, num_q_heads):
    qs, qsp = _i32_host(query_start)
    b = C.c_uint64()
    _check(_L().pa_multi_token_workspace_bytes(C.c_void_p(h), qsp, len(qs) - 1, int(num_q_heads), C.byref(b)))
    return b.value


def pa_multi_token_attention(h, layer, q, query_start, block_tables, context_lens, out=None, scale=None,
                             workspace=None, stream=None):
    """Causal attention of query rows q [N][Hq][d]: sequence i owns rows
    query_start[i] .. query_start[i+1]-1 (host ints), its last tokens."""
    info = _info(h)
    qs, qsp = _i32_host(query_start)
    s = len(qs) - 1
    if q.dim() != 3 or q.shape[2] != info["head_dim"] or q.shape[0] != int(qs[-1]):
        raise ValueError(f"q must be [query_start[-1]][num_q_heads][{info['head_dim']}]")
    if block_tables.dim() != 2 or block_tables.shape[0] != s:
        raise ValueError("block_tables must be [num_seqs][max_blocks]")
    hq, mb = int(q.shape[1]), int(block_tables.shape[1])
    qp = _dev(q, torch.float16, None, "q")
    tp = _dev(block_tables, torch.int32, None, "block_tables")
    lp = _dev(context_lens, torch.int32, (s,), "context_lens")
    if out is None:
        out = torch.empty_like(q)
    op = _dev(out, torch.float16, tuple(q.shape), "out")
    need = pa_multi_token_workspace_bytes(h, qs, hq)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    wp = _dev(workspace, torch.uint8, None, "workspace")
    if scale is None:
        scale = info["softmax_scale"]
    _check(_L().pa_multi_token_attention(C.c_void_p(h), int(layer), qp, hq, qsp, tp, mb, lp, s, float(scale),
                                         op, wp, workspace.numel(), _stream(stream)))
    return out


def pa_decode_partials(h, layer, q, block_tables, context_lens, partition_tokens, scale=None,
                       workspace=None, stream=None, seq_order=None):
    """Returns (m, l, o) views into the workspace: [S][Hq][C], [S][Hq][C], [S][Hq][C][d]."""
    info, s, hq, mb, qp, tp, lp = _decode_args(h, q, block_tables, context_lens)
    orp = _order_arg(seq_order, s)
    wp, wb, workspace = _workspace(h, s, hq, mb, partition_tokens, workspace, q.device)
    if scale is None:
        scale = info["softmax_scale"]
    _check(_L().pa_decode_partials(C.c_void_p(h), int(layer), qp, hq, tp, mb, lp, s, orp, float(scale),
                                   int(partition_tokens), wp, wb, _stream(stream)))
    return workspace_views(workspace, s, hq, mb * info["block_size"], partition_tokens, info["head_dim"])


def workspace_views(workspace, num_seqs, num_q_heads, max_tokens, partition_tokens, head_dim):
    """(m, l, o) float32 views of a partitioned-decode workspace (layout of include/pa.h)."""
    c = -(-int(max_tokens) // int(partition_tokens))
    rows = num_seqs * num_q_heads * c

    def up(x):
        return (x + 255) // 256 * 256
    off_l = up(rows * 4)
    off_o = off_l + up(rows * 4)
    f = workspace.view(torch.uint8)
    m = f[:rows * 4].view(torch.float32).view(num_seqs, num_q_heads, c)
    l = f[off_l:off_l + rows * 4].view(torch.float32).view(num_seqs, num_q_heads, c)
    o = f[off_o:off_o + rows * head_dim * 4].view(torch.float32).view(num_seqs, num_q_heads, c, head_dim)
    return m, l, o


def pa_lse_reduce(h, workspace, context_lens, num_q_heads, max_blocks, partition_tokens, out,
                  stream=None):
    s = int(context_lens.numel())
    lp = _dev(context_lens, torch.int32, (s,), "context_lens")
    info = pa_pool_info_get(h)
    op = _dev(out, torch.float16, (s, num_q_heads, info["head_dim"]), "out")
    need = pa_decode_workspace_bytes(h, s, num_q_heads, max_blocks, partition_tokens)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    _check(_L().pa_lse_reduce(C.c_void_p(h), C.c_void_p(workspace.data_ptr()), need, lp, s,
                              int(num_q_heads), int(max_blocks), int(partition_tokens), op,
                              _stream(stream)))
    return out


def pa_device_status(h, clear=False, stream=None) -> int:
    v = C.c_uint32()
    _check(_L().pa_device_status(C.c_void_p(h), C.byref(v), 1 if clear else 0, _stream(stream)))
    return v.value


def pa_profile_begin(h, max_launches, every=1):
    _check(_L().pa_profile_begin(C.c_void_p(h), int(max_launches), int(every)))


def pa_profile_end(h) -> dict:
    p = _lib.pa_profile()
    _check(_L().pa_profile_end(C.c_void_p(h), C.byref(p)))
    return {f: getattr(p, f) for f, _ in p._fields_}


# ---- convenience owner of a bound pool ------------------------------------------

class PagedKVPool:
    """A pool descriptor plus the torch-allocated device buffer it is bound to."""

    def __init__(self, layers, kv_heads, head_dim, block_size, num_blocks, dtype="fp16",
                 device="cuda", free_order=None, k_scales=None, v_scales=None, bind=True,
                 k_zeros=None, v_zeros=None):
        code = {"fp16": PA_DTYPE_FP16, "fp8": PA_DTYPE_FP8_E4M3, "int8": PA_DTYPE_INT8}[dtype]
        self.handle = pa_pool_create(layers, kv_heads, head_dim, block_size, code, num_blocks)
        self.dtype = dtype
        self.buffer = None
        try:
            if free_order is not None:
                pa_pool_set_free_order(self.handle, free_order)
            self.info = pa_pool_info_get(self.handle)
            if bind:
                total = self.info["total_bytes"]
                self.buffer = torch.empty(total + 256, dtype=torch.uint8, device=device)
                base = self.buffer.data_ptr()
                aligned = (base + 255) // 256 * 256
                self.base_ptr = aligned
                if dtype == "int8":
                    pa_pool_bind_int8(self.handle, aligned, k_scales, v_scales, k_zeros, v_zeros)
                else:
                    pa_pool_bind(self.handle, aligned, k_scales, v_scales)
                self.info = pa_pool_info_get(self.handle)
        except Exception:
            pa_pool_destroy(self.handle)
            self.handle = None
            raise

    def __del__(self):
        if getattr(self, "handle", None):
            try:
                pa_pool_destroy(self.handle)
            except Exception:
                pass
            self.handle = None

    @property
    def block_size(self):
        return self.info["block_size"]

    def pool_bytes(self):
        """The pool's data region (K and V of every layer) as a uint8 tensor view."""
        off = self.base_ptr - self.buffer.data_ptr()
        return self.buffer[off:off + self.info["kv_bytes"]]

    def seq_create(self):
        return pa_seq_create(self.handle)

    def seq_create_cached(self, tokens):
        return pa_seq_create_cached(self.handle, tokens)

    def alloc(self, seq, n, stream=None, tokens=None):
        return pa_alloc(self.handle, seq, n, stream if self.buffer is not None else 0, tokens)

    def alloc_batch(self, seqs, n_tokens, stream=None, tokens=None):
        return pa_alloc_batch(self.handle, seqs, n_tokens, stream if self.buffer is not None else 0, tokens)

    def fork(self, parent):
        return pa_fork(self.handle, parent)

    def free(self, seq):
        pa_free(self.handle, seq)

    def seq_len(self, seq):
        return pa_seq_len(self.handle, seq)

    def block_tables(self, seqs, max_blocks):
        return pa_block_tables(self.handle, seqs, max_blocks)

    def stats(self):
        return pa_pool_stats(self.handle)

    def refcounts(self):
        return pa_refcounts(self.handle)

    def free_queue(self):
        return pa_free_queue(self.handle)

    def write_kv(self, layer, k_new, v_new, slot_mapping, stream=None):
        pa_write_kv(self.handle, layer, k_new, v_new, slot_mapping, stream)

    def gather_kv(self, layer, slot_mapping, stream=None):
        dt = {"fp16": torch.float16, "fp8": torch.uint8, "int8": torch.int8}[self.dtype]
        n = slot_mapping.numel()
        shape = (n, self.info["kv_heads"], self.info["head_dim"])
        k = torch.zeros(shape, dtype=dt, device=slot_mapping.device)
        v = torch.zeros(shape, dtype=dt, device=slot_mapping.device)
        pa_gather_kv(self.handle, layer, slot_mapping, k, v, stream)
        return k, v

    def copy_blocks(self, src, dst, stream=None):
        pa_copy_blocks(self.handle, src, dst, stream)

    def decode(self, layer, q, block_tables, context_lens, **kw):
        return pa_decode(self.handle, layer, q, block_tables, context_lens, **kw)

    def decode_noalloc(self, layer, q, block_tables, context_lens, out, **kw):
        return pa_decode_noalloc(self.handle, layer, q, block_tables, context_lens, out, **kw)

    def multi_token_attention(self, layer, q, query_start, block_tables, context_lens, **kw):
        return pa_multi_token_attention(self.handle, layer, q, query_start, block_tables, context_lens, **kw)

    def write_kv_decode(self, layer, k_new, v_new, slot_mapping, q, block_tables, context_lens, **kw):
        return pa_write_kv_decode(self.handle, layer, k_new, v_new, slot_mapping, q, block_tables,
                                  context_lens, **kw)

    def shared_prefix_groups(self, tables, lens, min_shared_tokens=256):
        return pa_shared_prefix_groups(self.handle, tables, lens, min_shared_tokens)

    def shared_prefix_plan(self, num_seqs, num_q_heads, max_blocks, groups, **kw):
        return pa_shared_prefix_plan(self.handle, num_seqs, num_q_heads, max_blocks, groups, **kw)

    def decode_shared_prefix(self, layer, q, block_tables, context_lens, groups, **kw):
        return pa_decode_shared_prefix(self.handle, layer, q, block_tables, context_lens, groups, **kw)

    def device_status(self, clear=False):
        return pa_device_status(self.handle, clear)
