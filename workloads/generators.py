"""Counter-free seeded generators.

Host-side integers (block placement permutations, lengths) come from numpy's
PCG64 via ``SeedSequence(seed).spawn``; bulk K/V/q tensors come from a torch
generator on the requested device, so that a 16 GiB pool can be filled on
the GPU without a host round trip.  The same tensor object is handed to both
the GPU path and (after a copy to host) the oracle, so the two sides always
see identical inputs even though CPU and GPU torch generators produce
different streams.
"""
from __future__ import annotations

import numpy as np
import torch

SEED_BASE = 464_000

# Largest finite magnitude of the OCP E4M3FN format.  Used only to derive
# calibration scales for synthetic data (amax / 448), an input convention.
FP8_E4M3_MAX = 448.0


def seed_for(config_index: int) -> int:
    """Seed of workload ``config_index`` (1-based)."""
    return SEED_BASE + int(config_index)


def _rng(seed: int, stream: int) -> np.random.Generator:
    child = np.random.SeedSequence([int(seed), int(stream)])
    return np.random.Generator(np.random.PCG64(child))


def free_order(seed: int, num_blocks: int, stream: int = 0) -> np.ndarray:
    """Seeded permutation of ``range(num_blocks)`` as int32 (initial free-queue order)."""
    return _rng(seed, 1000 + stream).permutation(num_blocks).astype(np.int32)


def uniform_ints(seed: int, stream: int, lo: int, hi: int, n: int) -> np.ndarray:
    """``n`` integers uniform on the closed range [lo, hi], int64."""
    return _rng(seed, 2000 + stream).integers(lo, hi + 1, size=n, dtype=np.int64)


def _torch_seed(seed: int, tag: int) -> int:
    # Mix (seed, tag) into one 63-bit torch seed deterministically.
    ss = np.random.SeedSequence([int(seed), 77, int(tag)])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64(0x7FFF_FFFF_FFFF_FFFF))


def normal_fp16(shape, seed: int, tag: int, device="cpu") -> torch.Tensor:
    """Standard-normal fp16 tensor: N(0,1) drawn in fp32, rounded to fp16 (RNE)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(_torch_seed(seed, tag))
    x = torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.float32)
    return x.to(torch.float16)


def amax_scales(x: torch.Tensor) -> np.ndarray:
    """Per-KV-head fp32 calibration scales ``amax|x| / 448`` for ``x[..., Hkv, d]``.

    Returned on the host as float32 of shape [Hkv].  This is how the
    synthetic fp8 workload picks its per-(layer, kv_head) scales.
    """
    hkv = x.shape[-2]
    a = x.reshape(-1, hkv, x.shape[-1]).abs().amax(dim=(0, 2)).to(torch.float32).cpu().numpy()
    a = np.maximum(a, np.float32(1e-6))
    return (a / np.float32(FP8_E4M3_MAX)).astype(np.float32)


def minmax_int8_params(x: torch.Tensor):
    """Per-KV-head int8 calibration of ``x[..., Hkv, d]``: the scale maps the
    head's [min, max] onto the 255 steps of [-128, 127] and the zero point is
    the code of 0, ``s = (max - min) / 255``, ``z = clamp(rint(-128 - min / s))``.

    Returned on the host: float32 scales and int32 zero points of shape [Hkv].
    This is how the synthetic int8 workloads pick their per-(layer, kv_head)
    parameters (an input convention, like ``amax_scales`` for fp8).
    """
    hkv = x.shape[-2]
    y = x.reshape(-1, hkv, x.shape[-1]).to(torch.float32)
    lo = y.amin(dim=(0, 2)).cpu().numpy().astype(np.float64)
    hi = y.amax(dim=(0, 2)).cpu().numpy().astype(np.float64)
    s = np.maximum((hi - lo) / 255.0, 1e-6).astype(np.float32)
    z = np.clip(np.rint(-128.0 - lo / s.astype(np.float64)), -128, 127).astype(np.int32)
    return s, z


def head_offsets(hkv: int) -> np.ndarray:
    """Per-KV-head mean shifts for the int8 workloads' keys (-1 .. 1.5), so
    that zero points differ from head to head."""
    return np.linspace(-1.0, 1.5, hkv).astype(np.float32)
