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
