"""GPU parity of the backward entry points (based_linattn_bwd and
based_swa_bwd) against the oracle's gradients, on the same seeded inputs and
upstream gradients.

Metric: per row (one position's gradient vector), max |g - g_ref| over the
row divided by max(the row's own largest |g_ref|, FLOOR x the largest |g_ref|
of its head's [L, d] block), with the forward tolerances (fp32 1e-5, bf16
2e-3).  FLOOR is 0.02 for bf16 inputs and 0.1 for fp32: a gradient row is a
sum of terms of the head's size that may cancel to far less, and then only
rounding noise of the head's size remains (dq of position 0 is zero in
exact arithmetic, since y_0 = v_0 whatever q_0 is; dq and dk vanish at
L = 1).  Those identically vanishing rows (and gradients that vanish everywhere, as dq and dk of
a window of 1, where y = v) are checked as noise against the head's largest
dv: at most 100x the tolerance."""

import numpy as np
import pytest
import torch

import synth
from oracle import based_oracle as O
from parity_util import TOL, report, row_rel_floor, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
SMALL = synth.FwdConfig("small", B=2, H=3, L=300, dv=64)
FLOOR = {torch.bfloat16: 0.02, torch.float32: 0.1}


def head_max(ref) -> np.ndarray:
    ref = np.asarray(ref, np.float64)
    return np.abs(ref).reshape(-1, ref.shape[-2] * ref.shape[-1]).max(axis=-1)


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
        g = g[bi, hi]
        # rows that vanish in exact arithmetic (y_0 = v_0 whatever q, k are):
        # dq of position 0, and dk too at L = 1
        zero_rows = cfg.L if (cfg.L == 1 and name != "dv") else (1 if name == "dq" else 0)
        if np.abs(r).max() == 0:  # vanishes everywhere (window 1: y = v)
            zero_rows = cfg.L
        if zero_rows:
            err = float(g[..., :zero_rows, :].abs().max().cpu()) / float(floor.max())
            report(f"{which} {name} {cfg.name} (zero rows, noise / max|dv|)", err, 100 * tol)
            assert err <= 100 * tol, (name, err)
        if zero_rows == cfg.L:
            continue
        err = row_rel_floor(g[..., zero_rows:, :], r[..., zero_rows:, :], FLOOR[q.dtype])
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


def test_bwd_split_records_ragged_end(based):
    """B 8, H 16, L 2000: two segments whose forward record is split over two
    half-width workgroups and whose suffix-state increment is split into two
    sub-records, the second ending inside a chunk (L is not a multiple of 64);
    the oracle on two heads."""
    cfg = synth.FWD_CONFIGS["based360m"].replace(L=2000, name="split2000")
    run_case(based, cfg, "lin", [(0, 0), (7, 15)])


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
            keep = slice(1, None) if name == "dq" else slice(None)  # dq of position 0 vanishes
            err = row_rel_floor(got[keep], r[keep], FLOOR[q.dtype])
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
        keep = slice(1, None) if name == "dq" else slice(None)  # dq of position 0 vanishes
        err = row_rel_floor(g[0, 11, keep], r[keep], FLOOR[q.dtype])
        report(f"swa {name} long32k head 11", err, TOL[q.dtype])
        assert err <= TOL[q.dtype], (name, err)


def test_bwd_empty(based):
    q = torch.zeros(1, 2, 0, 16, device=DEV, dtype=torch.bfloat16)
    v = torch.zeros(1, 2, 0, 64, device=DEV, dtype=torch.bfloat16)
    y = torch.zeros(1, 2, 0, 64, device=DEV)
    for fn in (based.linattn_bwd, based.swa_bwd):
        dq, dk, dv = fn(q, q, v, y, y)
        assert dq.shape == (1, 2, 0, 16) and dv.shape == (1, 2, 0, 64)


@pytest.mark.parametrize("which", ["lin", "swa"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_deterministic(based, which, dtype):
    """Repeated calls give the same bits.  The fp32 window backward adds each
    query's two dq shares (its own chunk's keys, the previous chunk's) onto a
    zeroed dq with atomics: two addends onto an exact zero sum to the same
    value in either order."""
    cfg = SMALL.replace(B=2, H=4, L=1000, dtype=dtype)
    q, k, v = (t.to(DEV) for t in synth.fwd_inputs(cfg, 0))
    dy = synth.upstream_grad(cfg, 0).to(DEV)
    say(f"{which} bwd determinism {dtype}")
    if which == "lin":
        y = based.linattn_fwd(q, k, v)
        runs = [based.linattn_bwd(q, k, v, y, dy) for _ in range(5)]
    else:
        y = based.swa_fwd(q, k, v, 64)
        runs = [based.swa_bwd(q, k, v, y, dy, 64) for _ in range(5)]
    torch.cuda.synchronize()
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert torch.equal(a, b)


@pytest.mark.parametrize("dtype,dv", [("f32", 64), ("f32", 128), ("bf16", 48)])
def test_vector_bwd_long_sequence(based, dtype, dv):
    """The vector backward (fp32, and widths the matrix cores do not take)
    over 4000 positions -- 125 chunks per pass and a ragged tail -- on whole
    heads against the oracle's gradients, per row with the floor."""
    cfg = synth.FwdConfig(f"vector bwd long {dtype} dv{dv}", B=1, H=2, L=4000, dv=dv, dtype=dtype)
    run_case(based, cfg, "lin")
