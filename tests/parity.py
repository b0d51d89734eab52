"""Parity criteria of the GPU attention outputs against the fp64 oracle.

No GPU is needed here: the criteria are plain numpy, so CPU tests can show
what they accept and what they reject.

Stated tolerances (the problem statement): max-abs error <= 2e-3 for fp16
K/V, and 2e-2 "relative" for fp8 K/V, read per (sequence, head) row as
max_j |out - ref| <= 2e-2 * max_j |ref|.

Derived tolerance, every element kind: per (sequence, head) row,
max_j |out - ref| <= 4e-3 * max_j |ref|.  The kernel computes on the exact
stored values (fp16 bits, E4M3 codes widened exactly to fp16, int8 codes as
the exact fp16 integers c - z), with fp32 score and output accumulation; its
rounding steps are each about 2^-11 relative: the fp16 output (at most
2^-11 * max|ref| per element), the fp16 probabilities fed to the P.V product
(independent, mean-zero errors whose sum grows like the square root of the
tokens that carry weight, far below 2^-11 of the row at T >= 16), and fp32
accumulation.  4e-3 is 8x the output rounding.  It matters at long context:
outputs shrink like 1/sqrt(T) (about 0.012 at most per row for N(0,1) data
at T = 131072), so the stated 2e-3 max-abs alone cannot see a lost 512-token
chunk there; the row-relative bound can (tests/test_parity_criterion.py).
"""
from __future__ import annotations

import json
import os

import numpy as np

FP16_ATOL = 2e-3       # stated: max-abs, fp16 K/V
FP8_RTOL_STATED = 2e-2  # stated: per-row relative, fp8 K/V
ROW_RTOL = 4e-3        # derived: per-row relative, every element kind

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MARGINS_PATH = os.path.join(ROOT, "gpurun_out", "parity_margins.jsonl")


def errors(got, ref):
    """(max-abs error, largest per-row relative error) over the last axis."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    row_err = err.max(axis=-1)
    row_ref = np.abs(ref).max(axis=-1)
    return float(err.max()), float((row_err / np.maximum(row_ref, 1e-30)).max())


def failures(got, ref, dtype):
    """Names of the criteria ``got`` fails for KV element kind ``dtype``
    (an empty list: it passes), and the two error figures."""
    got = np.asarray(got, dtype=np.float64)
    bad = []
    if not np.isfinite(got).all():
        return ["non-finite output"], float("nan"), float("nan")
    max_abs, row_rel = errors(got, ref)
    if dtype == "fp16" and max_abs > FP16_ATOL:
        bad.append(f"max-abs {max_abs:.3e} > {FP16_ATOL}")
    if dtype == "fp8" and row_rel > FP8_RTOL_STATED:
        bad.append(f"row-relative {row_rel:.3e} > {FP8_RTOL_STATED}")
    if row_rel > ROW_RTOL:
        bad.append(f"row-relative {row_rel:.3e} > {ROW_RTOL}")
    return bad, max_abs, row_rel


def record(what, dtype, max_abs, row_rel, **extra):
    """Append one case's observed errors to the margins file (one JSON line)."""
    rec = {"test": os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], "case": what,
           "dtype": dtype, "max_abs": max_abs, "max_row_rel": row_rel,
           "atol": FP16_ATOL if dtype == "fp16" else None, "row_rtol": ROW_RTOL, **extra}
    try:
        os.makedirs(os.path.dirname(MARGINS_PATH), exist_ok=True)
        with open(MARGINS_PATH, "a") as f:
            f.write(json.dumps(rec) + "\n")
    except OSError:
        pass  # the margins file is a record, not part of the check
