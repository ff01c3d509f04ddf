"""GPU parity of the decayed linear attention (based_linattn_decay_fwd)
against the oracle's decayed forms on the same seeded inputs: per-row
infinity-norm relative error at the bf16 tolerance.  Heads cycle through
decays 1, 0.75, 0.875, ..., so an undecayed head also ties the variant to
based_linattn_fwd's output."""

import numpy as np
import pytest
import torch

import synth
from oracle import based_oracle as O
from parity_util import TOL, report, rowinf_rel, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
SMALL = synth.FwdConfig("small", B=2, H=8, L=1000, dv=64)


def run(based, cfg, heads=None):
    q, k, v = synth.fwd_inputs(cfg, 0)
    g = synth.decay_rates(cfg.H)
    say(f"decay {cfg.name} B{cfg.B} H{cfg.H} L{cfg.L} dv{cfg.dv}")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    y, S, z = based.linattn_decay_fwd(qd, kd, vd, g.to(DEV), return_state=True)
    torch.cuda.synchronize()
    sel = [(b, h) for b in range(cfg.B) for h in range(cfg.H)] if heads is None else heads
    for b, h in sel:
        ref = O.linattn_decay_quadratic(q[b, h][None], k[b, h][None], v[b, h][None], g[h:h + 1].numpy())[0][0]
        err = rowinf_rel(y[b, h], ref)
        assert err <= TOL[q.dtype], (b, h, err)
    report(f"decay {cfg.name} (sampled heads)", err, TOL[q.dtype])
    return q, k, v, g, y, S, z


@pytest.mark.parametrize("L", [1, 63, 64, 65, 1000])
def test_decay_lengths(based, L):
    run(based, SMALL.replace(L=L, name=f"L{L}"))


@pytest.mark.parametrize("dv", [32, 96, 128])
def test_decay_value_dims(based, dv):
    run(based, SMALL.replace(L=300, dv=dv, name=f"dv{dv}"))


def test_decay_undecayed_head_matches_plain(based):
    """gamma = 1 (head 0 of each group of eight) is the plain linear attention."""
    cfg = SMALL.replace(L=2000, name="gamma1")
    q, k, v, g, y, _, _ = run(based, cfg, heads=[(0, 0), (1, 5)])
    y_plain = based.linattn_fwd(q.to(DEV), k.to(DEV), v.to(DEV))
    gap = rowinf_rel(y[:, 0], y_plain[:, 0].double().cpu().numpy())
    report("decay gamma=1 vs based_linattn_fwd", gap, 1e-5)
    assert gap <= 1e-5


def test_decay_full_size_segments(based):
    """360M-shaped (four segments per head, summed with decay weights)."""
    run(based, synth.FWD_CONFIGS["based360m"].replace(H=16), heads=[(0, 1), (3, 7), (7, 12)])


def test_decay_long_scan(based):
    """32k positions (a scan over 32 segment records with the decay), rows
    sampled across the sequence."""
    cfg = synth.FWD_CONFIGS["long32k"]
    q, k, v = synth.fwd_inputs(cfg, 0)
    g = synth.decay_rates(cfg.H)
    say(f"decay long32k L{cfg.L}")
    y = based.linattn_decay_fwd(q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV))
    torch.cuda.synchronize()
    rows = [0, 1, 2047, 2048, 10000, 20001, cfg.L - 1]
    for h in (0, 3, 7, 9):
        ref = O.linattn_decay_rows(q[0, h], k[0, h], v[0, h], float(g[h]), rows)
        err = rowinf_rel(y[0, h, rows], ref)
        report(f"decay long32k head {h} sampled rows", err, TOL[q.dtype])
        assert err <= TOL[q.dtype]


def test_decay_resume_state(based):
    """Two calls, the second from the first's S_out / z_out, equal one call."""
    cfg = SMALL.replace(L=700, name="resume")
    q, k, v = (t.to(DEV) for t in synth.fwd_inputs(cfg, 0))
    g = synth.decay_rates(cfg.H).to(DEV)
    n = 320
    y_full = based.linattn_decay_fwd(q, k, v, g)
    _, S1, z1 = based.linattn_decay_fwd(q[:, :, :n].contiguous(), k[:, :, :n].contiguous(), v[:, :, :n].contiguous(),
                                        g, return_state=True)
    y2 = based.linattn_decay_fwd(q[:, :, n:].contiguous(), k[:, :, n:].contiguous(), v[:, :, n:].contiguous(), g,
                                 S1, z1)
    gap = rowinf_rel(y2, y_full[:, :, n:].double().cpu().numpy())
    report("decay resume vs one call", gap, TOL[torch.bfloat16])
    assert gap <= TOL[torch.bfloat16]


@pytest.mark.parametrize("L", [768, 2560])
def test_decay_initial_state_across_segments(based, L):
    """S_in with the decay and several segments: the state-only pass adds
    gamma^n S_in to segment 0's record (three segments), and the scan
    carries it on (ten)."""
    cfg = SMALL.replace(L=L, name=f"S_in L{L}")
    q, k, v = synth.fwd_inputs(cfg, 0)
    g = synth.decay_rates(cfg.H)
    _, kp, vp = synth.fwd_inputs(cfg.replace(L=500), 1)  # S_in: a seeded prefix's exported state
    S0, z0 = (torch.from_numpy(x).float() for x in O.linattn_state(kp, vp))
    say(f"decay {cfg.name} B{cfg.B} H{cfg.H} with S_in")
    y = based.linattn_decay_fwd(q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV), S0.to(DEV), z0.to(DEV))
    torch.cuda.synchronize()
    for b, h in [(0, 0), (0, 3), (1, 6), (1, 7)]:
        ref = O.linattn_decay_quadratic(q[b, h][None], k[b, h][None], v[b, h][None], g[h:h + 1].numpy(),
                                        S0[b, h][None], z0[b, h][None])[0][0]
        err = rowinf_rel(y[b, h], ref)
        report(f"decay {cfg.name} head ({b}, {h})", err, TOL[q.dtype])
        assert err <= TOL[q.dtype], (b, h, err)


# ------------------------------------------- the vector path (fp32, other d_v)
@pytest.mark.parametrize("dtype,dv,L", [("f32", 64, 256), ("f32", 48, 130), ("f32", 128, 1), ("bf16", 48, 300),
                                        ("bf16", 80, 65)])
def test_decay_vector_path(based, dtype, dv, L):
    """fp32 inputs (the tiny config's dtype, tolerance 1e-5) and widths the
    matrix-core pass does not take run the decayed chunked pass on the vector
    ALUs."""
    run(based, SMALL.replace(L=L, dv=dv, dtype=dtype, name=f"vector {dtype} dv{dv} L{L}"))


def test_decay_tiny_config_fp32(based):
    """The tiny layer configuration (B1 H2 L256 d_v 64, fp32) with decays 1 and
    0.75: y and the exported state against the recurrence at 1e-5."""
    cfg = synth.FWD_CONFIGS["tiny"]
    q, k, v = synth.fwd_inputs(cfg, 0)
    g = synth.decay_rates(cfg.H)
    y, S, z = based.linattn_decay_fwd(q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV), return_state=True)
    torch.cuda.synchronize()
    y_ref, _, S_ref, z_ref = O.linattn_decay_recurrent(q, k, v, g.numpy())
    err = max(rowinf_rel(y, y_ref), rowinf_rel(S, S_ref))
    report("decay tiny fp32 y / S_out", err, 1e-5)
    assert err <= 1e-5


def test_decay_vector_path_initial_state(based):
    """fp32 with an initial state: it decays as gamma^(i+1) at position i."""
    cfg = SMALL.replace(B=1, H=3, L=200, dtype="f32")
    q, k, v = synth.fwd_inputs(cfg, 0)
    _, kp, vp = synth.fwd_inputs(cfg.replace(L=100), 1)
    S0, z0 = (torch.from_numpy(t).float() for t in O.linattn_state(kp, vp))
    g = synth.decay_rates(cfg.H)
    y = based.linattn_decay_fwd(q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV), S0.to(DEV), z0.to(DEV))
    torch.cuda.synchronize()
    y_ref = O.linattn_decay_recurrent(q, k, v, g.numpy(), S0, z0)[0]
    err = rowinf_rel(y, y_ref)
    report("decay fp32 with S_in", err, 1e-5)
    assert err <= 1e-5


# ------------------------------------------------------------ decayed layer
@pytest.mark.parametrize("case", ["360m", "window17", "f32", "bf16_dv48"])
def test_layer_decay(based, case):
    """based_layer_decay_fwd: y_lin against the decayed oracle and equal to
    based_linattn_decay_fwd's output (1e-6: the same arithmetic in another
    kernel), y_swa against the window softmax (no decay).  The 360M shape runs
    the fused matrix-core pass over four segments; a window of 17 its general
    window path; fp32 and d_v 48 the separate vector kernels."""
    cfg, window, heads = {
        "360m": (synth.FWD_CONFIGS["based360m"], 64, [(0, 1), (7, 14)]),
        "window17": (SMALL.replace(B=1, H=8, L=700), 17, None),
        "f32": (SMALL.replace(B=1, H=4, L=300, dtype="f32"), 64, None),
        "bf16_dv48": (SMALL.replace(B=1, H=4, L=300, dv=48), 64, None),
    }[case]
    q, k, v = synth.fwd_inputs(cfg, 0)
    g = synth.decay_rates(cfg.H)
    say(f"layer decay {case} B{cfg.B} H{cfg.H} L{cfg.L} dv{cfg.dv} {cfg.dtype} window{window}")
    qd, kd, vd, gd = q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV)
    y_lin, y_swa = based.layer_decay_fwd(qd, kd, vd, gd, window)
    y_sep = based.linattn_decay_fwd(qd, kd, vd, gd)
    torch.cuda.synchronize()
    gap = rowinf_rel(y_lin, y_sep.double().cpu().numpy())
    report(f"layer decay {case}: y_lin vs based_linattn_decay_fwd", gap, 1e-6)
    assert gap <= 1e-6
    tol = TOL[q.dtype]
    sel = [(b, h) for b in range(cfg.B) for h in range(cfg.H)] if heads is None else heads
    for b, h in sel:
        ref = O.linattn_decay_quadratic(q[b, h][None], k[b, h][None], v[b, h][None], g[h:h + 1].numpy())[0][0]
        assert rowinf_rel(y_lin[b, h], ref) <= tol, (b, h)
        assert rowinf_rel(y_swa[b, h], O.swa(q[b, h], k[b, h], v[b, h], window)) <= tol, (b, h)
    report(f"layer decay {case} (oracle, sampled heads)", 0.0, tol)


# ---------------------------------------------------------- decayed backward
FLOOR = {torch.bfloat16: 0.02, torch.float32: 0.1}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("L,dv", [(1, 64), (2, 64), (65, 64), (300, 64), (130, 48), (200, 128)])
def test_decay_bwd(based, dtype, L, dv):
    """based_linattn_decay_bwd against the oracle's decayed gradients, per
    row with a floor (as the plain backward's tests), decays 1, 0.75, ...
    over eight heads; rows that vanish identically (dq of position 0; dq and
    dk at L = 1) are checked as noise against the head's largest dv."""
    from parity_util import row_rel_floor
    cfg = SMALL.replace(B=1, L=L, dv=dv, dtype=dtype, name=f"decay bwd L{L} dv{dv} {dtype}")
    q, k, v = synth.fwd_inputs(cfg, 0)
    dy = synth.upstream_grad(cfg, 0)
    g = synth.decay_rates(cfg.H)
    say(cfg.name)
    qd, kd, vd, gd, dyd = q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV), dy.to(DEV)
    y = based.linattn_decay_fwd(qd, kd, vd, gd)
    grads = based.linattn_decay_bwd(qd, kd, vd, gd, y, dyd)
    torch.cuda.synchronize()
    refs = O.linattn_decay_bwd(q, k, v, g.numpy(), dy)
    tol = TOL[q.dtype]
    dvmax = float(np.abs(refs[2]).max())
    for name, gr, r in zip(("dq", "dk", "dv"), grads, refs):
        zero = L if (L == 1 and name != "dv") else (1 if name == "dq" else 0)
        if zero:
            noise = float(gr[..., :zero, :].abs().max().cpu()) / dvmax
            assert noise <= 100 * tol, (name, noise)
        if zero == L:
            continue
        err = row_rel_floor(gr[..., zero:, :], r[..., zero:, :], FLOOR[q.dtype])
        report(f"{cfg.name} {name}", err, tol)
        assert err <= tol, (name, err)


def test_decay_bwd_360m_sampled_heads(based):
    """The 360M shape (B 8, H 16, L 2048) through the decayed backward; the
    oracle on two heads."""
    from parity_util import row_rel_floor
    cfg = synth.FWD_CONFIGS["based360m"]
    q, k, v = synth.fwd_inputs(cfg, 0)
    dy = synth.upstream_grad(cfg, 0)
    g = synth.decay_rates(cfg.H)
    say("decay bwd 360m")
    qd, kd, vd, gd = q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV)
    y = based.linattn_decay_fwd(qd, kd, vd, gd)
    grads = based.linattn_decay_bwd(qd, kd, vd, gd, y, dy.to(DEV))
    torch.cuda.synchronize()
    for b, h in ((0, 1), (5, 14)):
        refs = O.linattn_decay_bwd(q[b, h][None], k[b, h][None], v[b, h][None], g[h:h + 1].numpy(), dy[b, h][None])
        for name, gr, r in zip(("dq", "dk", "dv"), grads, refs):
            zero = 1 if name == "dq" else 0
            err = row_rel_floor(gr[b, h, zero:][None], r[:, zero:], FLOOR[q.dtype])
            report(f"decay bwd 360m head ({b},{h}) {name}", err, TOL[q.dtype])
            assert err <= TOL[q.dtype], (name, err)


def test_decay_bwd_split_records_ragged_end(based):
    """The decayed backward at B 8, H 16, L 2000: split forward records and
    suffix-state sub-records weighted by their distance, the last one ending
    inside a chunk; the oracle on two heads."""
    from parity_util import row_rel_floor
    cfg = synth.FWD_CONFIGS["based360m"].replace(L=2000, name="split2000")
    q, k, v = synth.fwd_inputs(cfg, 0)
    dy = synth.upstream_grad(cfg, 0)
    g = synth.decay_rates(cfg.H)
    say("decay bwd split2000")
    qd, kd, vd, gd = q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV)
    y = based.linattn_decay_fwd(qd, kd, vd, gd)
    grads = based.linattn_decay_bwd(qd, kd, vd, gd, y, dy.to(DEV))
    torch.cuda.synchronize()
    for b, h in ((0, 1), (6, 13)):
        refs = O.linattn_decay_bwd(q[b, h][None], k[b, h][None], v[b, h][None], g[h:h + 1].numpy(), dy[b, h][None])
        for name, gr, r in zip(("dq", "dk", "dv"), grads, refs):
            zero = 1 if name == "dq" else 0
            err = row_rel_floor(gr[b, h, zero:][None], r[:, zero:], FLOOR[q.dtype])
            report(f"decay bwd split2000 head ({b},{h}) {name}", err, TOL[q.dtype])
            assert err <= TOL[q.dtype], (name, err)


# ------------------------------------------------ the range of gamma
# Out-of-range decays read as their clamped values: NaN and negatives as 0,
# values above 1 as 1.  gamma = 0 leaves each position its own term (y = v).
RAW = [0.0, -0.5, float("nan"), 1.5, 0.75, 0.0, 1.0, 0.5]
CLAMPED = [0.0, 0.0, 0.0, 1.0, 0.75, 0.0, 1.0, 0.5]


@pytest.mark.parametrize("dtype,dv,L", [("bf16", 64, 1000), ("f32", 48, 130)])
def test_decay_gamma_clamped(based, dtype, dv, L):
    """The decayed forward (matrix-core pass over several segments with a
    ragged last chunk; the vector pass in fp32) and the decayed layer: raw
    and clamped gammas give the same bits; the gamma = 0 heads equal v."""
    cfg = SMALL.replace(L=L, dv=dv, dtype=dtype, name=f"gamma range {dtype} dv{dv} L{L}")
    q, k, v = synth.fwd_inputs(cfg, 0)
    say(cfg.name)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    raw, cl = torch.tensor(RAW, device=DEV), torch.tensor(CLAMPED, device=DEV)
    ya, Sa, za = based.linattn_decay_fwd(qd, kd, vd, raw, return_state=True)
    yb, Sb, zb = based.linattn_decay_fwd(qd, kd, vd, cl, return_state=True)
    la = based.layer_decay_fwd(qd, kd, vd, raw, 64)[0]
    lb = based.layer_decay_fwd(qd, kd, vd, cl, 64)[0]
    torch.cuda.synchronize()
    assert torch.equal(ya, yb) and torch.equal(Sa, Sb) and torch.equal(za, zb) and torch.equal(la, lb)
    assert torch.isfinite(ya).all()
    tol = TOL[q.dtype]
    for h in (0, 1, 2, 5):
        err = rowinf_rel(ya[:, h], v[:, h].double().numpy())
        assert err <= tol, (h, err)
    for b, h in [(0, 3), (1, 4), (0, 7)]:
        ref = O.linattn_decay_quadratic(q[b, h][None], k[b, h][None], v[b, h][None], np.array([CLAMPED[h]]))[0][0]
        assert rowinf_rel(ya[b, h], ref) <= tol, (b, h)
    report(f"{cfg.name}: raw = clamped bit for bit, gamma 0 heads = v", 0.0, tol)


def test_decay_bwd_and_decode_gamma_clamped(based):
    """The decayed backward and decode step: raw and clamped gammas give the
    same bits; at gamma = 0 dv = dy and dq, dk vanish (y = v)."""
    cfg = SMALL.replace(B=1, L=200, name="gamma range bwd")
    q, k, v = synth.fwd_inputs(cfg, 0)
    dy = synth.upstream_grad(cfg, 0)
    say(cfg.name)
    qd, kd, vd, dyd = q.to(DEV), k.to(DEV), v.to(DEV), dy.to(DEV)
    raw, cl = torch.tensor(RAW, device=DEV), torch.tensor(CLAMPED, device=DEV)
    y = based.linattn_decay_fwd(qd, kd, vd, cl)
    ga = based.linattn_decay_bwd(qd, kd, vd, raw, y, dyd)
    gb = based.linattn_decay_bwd(qd, kd, vd, cl, y, dyd)
    torch.cuda.synchronize()
    for a, b in zip(ga, gb):
        assert torch.equal(a, b)
    tol = TOL[q.dtype]
    dvmax = float(dy.abs().max())
    for h in (0, 1, 2, 5):
        assert rowinf_rel(ga[2][:, h], dy[:, h].double().numpy()) <= tol, h
        assert float(ga[0][:, h].abs().max().cpu()) <= tol * dvmax and float(ga[1][:, h].abs().max().cpu()) <= tol * dvmax
    dcfg = synth.DecodeConfig("gamma range decode", B=2, H=8, ctx=70, steps=4)
    (qc, kc, vc), (qs, ks, vs) = synth.decode_inputs(dcfg)
    _, _, sa = based.decode_init(qc.to(DEV), kc.to(DEV), vc.to(DEV), gamma=cl)
    _, _, sb = based.decode_init(qc.to(DEV), kc.to(DEV), vc.to(DEV), gamma=cl)
    for s in range(dcfg.steps):
        ya = based.decode_step(sa, qs[s].to(DEV), ks[s].to(DEV), vs[s].to(DEV), gamma=raw)
        yb = based.decode_step(sb, qs[s].to(DEV), ks[s].to(DEV), vs[s].to(DEV), gamma=cl)
        assert torch.equal(ya[0], yb[0]) and torch.equal(ya[1], yb[1])
        assert rowinf_rel(ya[0][:, 0], vs[s][:, 0].double().numpy()) <= tol
    assert torch.equal(sa.S, sb.S) and torch.equal(sa.z, sb.z)
    report("gamma range: backward and decode, raw = clamped bit for bit", 0.0, tol)


@pytest.mark.parametrize("L,dv", [(2500, 64), (1500, 96), (700, 128)])
def test_decay_bwd_matrix_core_segments(based, L, dv):
    """bf16 decayed backward on the matrix-core passes over several segments
    per head (decayed forward records, decayed suffix records) with a ragged
    last chunk, d_v 64 / 96 / 128: heads with decays 1, 0.75, 0.5 and 0.875
    against the oracle, per row with the floor."""
    from parity_util import row_rel_floor
    cfg = SMALL.replace(B=1, L=L, dv=dv, name=f"decay bwd segments L{L} dv{dv}")
    q, k, v = synth.fwd_inputs(cfg, 0)
    dy = synth.upstream_grad(cfg, 0)
    g = synth.decay_rates(cfg.H)
    say(cfg.name)
    qd, kd, vd, gd = q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV)
    y = based.linattn_decay_fwd(qd, kd, vd, gd)
    grads = based.linattn_decay_bwd(qd, kd, vd, gd, y, dy.to(DEV))
    torch.cuda.synchronize()
    for h in (0, 1, 2, 7):
        refs = O.linattn_decay_bwd(q[0, h][None], k[0, h][None], v[0, h][None], g[h:h + 1].numpy(), dy[0, h][None])
        for name, gr, r in zip(("dq", "dk", "dv"), grads, refs):
            zero = 1 if name == "dq" else 0
            err = row_rel_floor(gr[0, h, zero:][None], r[:, zero:], FLOOR[q.dtype])
            report(f"{cfg.name} head {h} (gamma {float(g[h])}) {name}", err, TOL[q.dtype])
            assert err <= TOL[q.dtype], (h, name, err)


def test_decay_bwd_vector_form_with_small_workspace(based):
    """A workspace of 2 B H L 4 bytes selects the fp32 vector form for bf16
    as well; both forms match the oracle."""
    from parity_util import row_rel_floor
    cfg = SMALL.replace(B=1, L=300, name="decay bwd vector form vs matrix core")
    q, k, v = synth.fwd_inputs(cfg, 0)
    dy = synth.upstream_grad(cfg, 0)
    g = synth.decay_rates(cfg.H)
    say(cfg.name)
    qd, kd, vd, gd, dyd = q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV), dy.to(DEV)
    y = based.linattn_decay_fwd(qd, kd, vd, gd)
    small = torch.empty(2 * cfg.B * cfg.H * cfg.L * 4, dtype=torch.uint8, device=DEV)
    vec = based.linattn_decay_bwd(qd, kd, vd, gd, y, dyd, workspace=small)
    mfma = based.linattn_decay_bwd(qd, kd, vd, gd, y, dyd)
    torch.cuda.synchronize()
    refs = O.linattn_decay_bwd(q, k, v, g.numpy(), dy)
    for name, a, b, r in zip(("dq", "dk", "dv"), vec, mfma, refs):
        zero = 1 if name == "dq" else 0
        for label, gr in (("vector form", a), ("matrix core", b)):
            err = row_rel_floor(gr[..., zero:, :], r[..., zero:, :], FLOOR[q.dtype])
            report(f"{cfg.name}: {label} {name}", err, TOL[q.dtype])
            assert err <= TOL[q.dtype], (label, name, err)


def test_decay_bwd_vector_form_long(based):
    """The fp32 decayed backward over 3000 positions (94 chunks per pass):
    heads with decays 1, 0.75, 0.5 and 0.875 against the oracle."""
    from parity_util import row_rel_floor
    cfg = SMALL.replace(B=1, L=3000, dtype="f32", name="decay bwd fp32 long")
    q, k, v = synth.fwd_inputs(cfg, 0)
    dy = synth.upstream_grad(cfg, 0)
    g = synth.decay_rates(cfg.H)
    say(cfg.name)
    qd, kd, vd, gd = q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV)
    y = based.linattn_decay_fwd(qd, kd, vd, gd)
    grads = based.linattn_decay_bwd(qd, kd, vd, gd, y, dy.to(DEV))
    torch.cuda.synchronize()
    for h in (0, 1, 2, 7):
        refs = O.linattn_decay_bwd(q[0, h][None], k[0, h][None], v[0, h][None], g[h:h + 1].numpy(), dy[0, h][None])
        for name, gr, r in zip(("dq", "dk", "dv"), grads, refs):
            zero = 1 if name == "dq" else 0
            err = row_rel_floor(gr[0, h, zero:][None], r[:, zero:], FLOOR[q.dtype])
            report(f"{cfg.name} head {h} {name}", err, TOL[q.dtype])
            assert err <= TOL[q.dtype], (h, name, err)
