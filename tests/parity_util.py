"""Helpers shared by the GPU parity tests (test infrastructure only)."""

from __future__ import annotations

import sys

import numpy as np
import torch

# Tolerances on the per-row infinity-norm relative error
#   max_rows ||y - y_ref||_inf / ||y_ref||_inf   (one row = one d_v vector):
# fp32 inputs: 1e-5; bf16 inputs with fp32 accumulation: 2e-3.  The
# denominator state z of a head is compared as one row (its 273 entries): its
# linear entries are sums of k that can sit near zero, so an entry-wise
# relative error is not meaningful there.
TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-3}


def rowinf_rel(y, ref) -> float:
    y = y.detach().to("cpu", torch.float64).numpy() if hasattr(y, "detach") else np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    if y.size == 0:
        return 0.0
    assert np.all(np.isfinite(y)), "non-finite output"
    num = np.abs(y - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return float((num / np.maximum(den, 1e-30)).max())


def report(name: str, err: float, tol: float) -> None:
    print(f"[parity] {name}: rowinf_rel={err:.3e} tol={tol:.0e}", flush=True)
    sys.stdout.flush()


def say(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
