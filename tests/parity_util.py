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


def z_block_rel(z, ref) -> float:
    """A denominator state [..., 273] (or compact [..., 153]) compared block by
    block: the constant entry (the token count), the 16 linear entries (sums
    of k) and the quadratic entries, each block as one row of rowinf_rel.
    One row over all entries would measure the linear sums against the token
    count, which dwarfs them."""
    z = z.detach().to("cpu", torch.float64).numpy() if hasattr(z, "detach") else np.asarray(z, np.float64)
    ref = np.asarray(ref, np.float64)
    assert z.shape == ref.shape, (z.shape, ref.shape)
    return max(rowinf_rel(z[..., a:b], ref[..., a:b]) for a, b in ((0, 1), (1, 17), (17, z.shape[-1])))


def row_rel_floor(g, ref, frac: float) -> float:
    """Per-row infinity-norm relative error of a gradient [..., L, d]: each
    row (one position's gradient vector) against max(its own largest
    magnitude, frac x the largest magnitude of its head's [L, d] block)."""
    g = g.detach().to("cpu", torch.float64).numpy() if hasattr(g, "detach") else np.asarray(g, np.float64)
    ref = np.asarray(ref, np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    if g.size == 0:
        return 0.0
    assert np.all(np.isfinite(g)), "non-finite gradient"
    err = np.abs(g - ref).max(axis=-1)
    own = np.abs(ref).max(axis=-1)
    head = np.abs(ref).max(axis=(-1, -2), keepdims=False)[..., None]
    return float((err / np.maximum(np.maximum(own, frac * head), 1e-30)).max())
