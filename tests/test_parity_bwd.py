"""GPU parity of the backward entry points (based_linattn_bwd and
based_swa_bwd) against the oracle's gradients, on the same seeded inputs and
upstream gradients.

Metric: per head, max |g - g_ref| / max |g_ref| over the head's [L, d] block,
with the forward tolerances (fp32 1e-5, bf16 2e-3).  A gradient row can
vanish exactly (dq of the first position always; dq and dk of a length-1
sequence entirely), so the row-wise metric of the forward tests does not
apply, and each head's scale is at least 0.1 of its largest dv reference
(dv ~ dy sets the natural size of the gradients; a gradient that is zero in
exact arithmetic, such as dq at L = 1 where y_0 = v_0, comes out as rounding
noise of a cancellation)."""

import numpy as np
import pytest
import torch

import synth
from oracle import based_oracle as O
from parity_util import TOL, report, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
SMALL = synth.FwdConfig("small", B=2, H=3, L=300, dv=64)


def head_max(ref) -> np.ndarray:
    ref = np.asarray(ref, np.float64)
    return np.abs(ref).reshape(-1, ref.shape[-2] * ref.shape[-1]).max(axis=-1)


def head_rel(g, ref, floor=None) -> float:
    g = g.detach().to("cpu", torch.float64).numpy() if hasattr(g, "detach") else np.asarray(g, np.float64)
    ref = np.asarray(ref, np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    if g.size == 0:
        return 0.0
    assert np.all(np.isfinite(g)), "non-finite gradient"
    err = np.abs(g - ref).reshape(-1, g.shape[-2] * g.shape[-1]).max(axis=-1)
    scale = head_max(ref)
    if floor is not None:
        scale = np.maximum(scale, 0.1 * floor)
    return float((err / np.maximum(scale, 1e-30)).max())


def run_case(based, cfg, which, heads=None, window=64, scale=1.0, seed=0):
    q, k, v = synth.fwd_inputs(cfg, seed)
    dy = synth.upstream_grad(cfg, seed)
    say(f"{which} bwd {cfg.name} B{cfg.B} H{cfg.H} L{cfg.L} dv{cfg.dv} {cfg.dtype} window{window}")
    qd, kd, vd, dyd = q.to(DEV), k.to(DEV), v.to(DEV), dy.to(DEV)
    if which == "lin":
        y = based.linattn_fwd(qd, kd, vd)
        grads = based.linattn_bwd(qd, kd, vd, y, dyd)
    else:
        y = based.swa_fwd(qd, kd, vd, window, scale)
        grads = based.swa_bwd(qd, kd, vd, y, dyd, window, scale)
    torch.cuda.synchronize()
    sel = [(b, h) for b in range(cfg.B) for h in range(cfg.H)] if heads is None else heads
    bi, hi = [b for b, _ in sel], [h for _, h in sel]
    args = (q[bi, hi], k[bi, hi], v[bi, hi], dy[bi, hi])
    refs = O.linattn_bwd(*args) if which == "lin" else O.swa_bwd(*args, window, scale)
    tol = TOL[q.dtype]
    floor = head_max(refs[2]) if refs[2].size else None
    for name, g, r in zip(("dq", "dk", "dv"), grads, refs):
        if cfg.L == 1 and name != "dv":
            # zero in exact arithmetic (y_0 = v_0 whatever q, k are): only the
            # rounding noise of dy.v_0 - dy.y_0 remains
            err = float(g[bi, hi].abs().max().cpu()) / float(floor.max())
            report(f"{which} {name} {cfg.name} (zero gradient, noise / max|dv|)", err, 100 * tol)
            assert err <= 100 * tol, (name, err)
            continue
        err = head_rel(g[bi, hi], r, floor)
        report(f"{which} {name} {cfg.name}", err, tol)
        assert err <= tol, (name, err)
    return grads


@pytest.mark.parametrize("which", ["lin", "swa"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("L", [1, 2, 63, 64, 65, 130, 300])
def test_bwd_lengths(based, which, dtype, L):
    run_case(based, SMALL.replace(L=L, dtype=dtype, name=f"L{L}"), which)


@pytest.mark.parametrize("which", ["lin", "swa"])
@pytest.mark.parametrize("dv", [16, 32, 48, 96, 128])
def test_bwd_value_dims(based, which, dv):
    run_case(based, SMALL.replace(L=200, dv=dv, name=f"dv{dv}"), which)


@pytest.mark.parametrize("window", [1, 2, 17, 63])
def test_swa_bwd_windows(based, window):
    run_case(based, SMALL.replace(L=200, name=f"w{window}"), "swa", window=window, scale=0.37)


def test_bwd_heavy_rows(based):
    cfg = SMALL.replace(L=700, heavy_frac=0.01, name="heavy")
    run_case(based, cfg, "lin")
    run_case(based, cfg, "swa", scale=0.5)


@pytest.mark.parametrize("name,heads", [
    ("based360m", [(0, 0), (7, 15)]),
    ("based1p3b", [(0, 0), (3, 15)]),
])
def test_bwd_full_size_sampled_heads(based, name, heads):
    cfg = synth.FWD_CONFIGS[name]
    run_case(based, cfg, "lin", heads)
    run_case(based, cfg, "swa", heads)


def test_bwd_long_sampled_rows(based):
    """32k positions: the window backward on whole sampled heads; the linear
    attention backward at sampled positions (row-wise oracle)."""
    cfg = synth.FWD_CONFIGS["long32k"]
    q, k, v = synth.fwd_inputs(cfg, 0)
    dy = synth.upstream_grad(cfg, 0)
    say(f"lin bwd long32k L{cfg.L}")
    qd, kd, vd, dyd = q.to(DEV), k.to(DEV), v.to(DEV), dy.to(DEV)
    y = based.linattn_fwd(qd, kd, vd)
    grads = based.linattn_bwd(qd, kd, vd, y, dyd)
    torch.cuda.synchronize()
    rows = [0, 1, 63, 64, 4095, 4096, 20000, cfg.L - 65, cfg.L - 1]
    for h in (0, 11):
        refs = O.linattn_bwd_rows(q[0, h], k[0, h], v[0, h], dy[0, h], rows)
        for name, g, r in zip(("dq", "dk", "dv"), grads, refs):
            got = g[0, h, rows].double().cpu().numpy()
            err = np.abs(got - r).max() / np.abs(r).max()
            report(f"lin {name} long32k head {h} sampled rows", err, TOL[q.dtype])
            assert err <= TOL[q.dtype], (name, err)
    # the value-shift identity over the whole sequence, sum_j dv_j = sum_i dy_i,
    # per head in the same infinity-norm relative measure
    s = grads[2].double().sum(dim=2).cpu().numpy()
    want = dy.double().sum(dim=2).numpy()
    err = float((np.abs(s - want).max(axis=-1) / np.abs(want).max(axis=-1)).max())
    report("lin sum of dv vs sum of dy, long32k (every head)", err, TOL[q.dtype])
    assert err <= TOL[q.dtype], err
    y = based.swa_fwd(qd, kd, vd)
    grads = based.swa_bwd(qd, kd, vd, y, dyd)
    torch.cuda.synchronize()
    refs = O.swa_bwd(q[0, 11], k[0, 11], v[0, 11], dy[0, 11])
    for name, g, r in zip(("dq", "dk", "dv"), grads, refs):
        err = head_rel(g[0, 11], r)
        report(f"swa {name} long32k head 11", err, TOL[q.dtype])
        assert err <= TOL[q.dtype], (name, err)


def test_bwd_empty(based):
    q = torch.zeros(1, 2, 0, 16, device=DEV, dtype=torch.bfloat16)
    v = torch.zeros(1, 2, 0, 64, device=DEV, dtype=torch.bfloat16)
    y = torch.zeros(1, 2, 0, 64, device=DEV)
    for fn in (based.linattn_bwd, based.swa_bwd):
        dq, dk, dv = fn(q, q, v, y, y)
        assert dq.shape == (1, 2, 0, 16) and dv.shape == (1, 2, 0, 64)
