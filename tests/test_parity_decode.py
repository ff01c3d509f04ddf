"""GPU parity of recurrent decode (based_decode_prefill + based_decode_step)
against the oracle's DecodeState, on the same seeded inputs."""

import numpy as np
import pytest
import torch

import synth
from oracle import based_oracle as O
from parity_util import TOL, report, rowinf_rel, say, z_block_rel

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_decode(based, cfg, seqs=None, check_steps=None, seed=0, compact=False):
    """Prefill on the GPU (linear attention state export + ring fill), then
    cfg.steps decode steps; compare the sampled sequences with the oracle
    (compact: the state in the compact layout, compared with the oracle's
    state compacted)."""
    (qc, kc, vc), (qs, ks, vs) = synth.decode_inputs(cfg, seed)
    say(f"decode B{cfg.B} H{cfg.H} ctx{cfg.ctx} steps{cfg.steps} dv{cfg.dv} {cfg.dtype}"
        + (" compact" if compact else ""))
    seqs = list(range(cfg.B)) if seqs is None else seqs
    check_steps = set(range(cfg.steps)) if check_steps is None else set(check_steps)
    tol = TOL[qc.dtype]
    _, _, st = based.decode_init(qc.to(DEV), kc.to(DEV), vc.to(DEV), cfg.window, compact=compact)
    ref = O.DecodeState.prefill(kc[seqs], vc[seqs], cfg.window)
    errs = []
    qd, kd, vd = qs.to(DEV), ks.to(DEV), vs.to(DEV)
    for s in range(cfg.steps):
        yl, ys = based.decode_step(st, qd[s], kd[s], vd[s])
        rl, rs = ref.step(qs[s, seqs], ks[s, seqs], vs[s, seqs])
        if s in check_steps:
            el, es = rowinf_rel(yl[seqs], rl), rowinf_rel(ys[seqs], rs)
            errs.append((el, es))
            assert el <= tol and es <= tol, (s, el, es)
    torch.cuda.synchronize()
    report(f"decode y_lin B{cfg.B} ctx{cfg.ctx}", max(e[0] for e in errs), tol)
    report(f"decode y_swa B{cfg.B} ctx{cfg.ctx}", max(e[1] for e in errs), tol)
    S_ref, z_ref = O.state_compact(ref.S, ref.z) if compact else (ref.S, ref.z)
    assert rowinf_rel(st.S[seqs], S_ref) <= tol
    assert z_block_rel(st.z[seqs], z_ref) <= tol
    assert torch.all(st.pos.cpu() == cfg.ctx + cfg.steps)
    return st


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_small_wraps_ring(based, dtype):
    cfg = synth.DecodeConfig("small", B=3, H=4, ctx=100, steps=70, dtype=dtype)
    run_decode(based, cfg)


def test_decode_from_empty_context(based):
    """No prefill tokens: the first steps see fewer than 64 keys."""
    cfg = synth.DecodeConfig("empty", B=2, H=2, ctx=0, steps=80)
    run_decode(based, cfg)


@pytest.mark.parametrize("dv,window", [(128, 64), (32, 17), (48, 1)])
def test_decode_shapes(based, dv, window):
    cfg = synth.DecodeConfig("shape", B=2, H=20, ctx=37, steps=30, dv=dv, window=window)
    run_decode(based, cfg)


def test_decode_sequences_at_different_positions(based):
    """Sequence 0 resumes after 10 context tokens, sequence 1 after 30."""
    cfg = synth.DecodeConfig("mixed", B=2, H=3, ctx=30, steps=70)
    (qc, kc, vc), (qs, ks, vs) = synth.decode_inputs(cfg)
    dev = lambda *ts: [t.contiguous().to(DEV) for t in ts]
    _, _, sa = based.decode_init(*dev(qc[:, :, :10], kc[:, :, :10], vc[:, :, :10]))
    _, _, sb = based.decode_init(*dev(qc, kc, vc))
    st = based.DecodeState(*[torch.cat([a[:1], b[1:]]).contiguous()
                             for a, b in zip((sa.S, sa.z, sa.ring_k, sa.ring_v, sa.pos),
                                             (sb.S, sb.z, sb.ring_k, sb.ring_v, sb.pos))])
    ra = O.DecodeState.prefill(kc[:, :, :10], vc[:, :, :10])
    rb = O.DecodeState.prefill(kc, vc)
    ref = O.DecodeState(np.concatenate([ra.S[:1], rb.S[1:]]), np.concatenate([ra.z[:1], rb.z[1:]]),
                        np.concatenate([ra.ring_k[:1], rb.ring_k[1:]]),
                        np.concatenate([ra.ring_v[:1], rb.ring_v[1:]]), [10, 30])
    for s in range(cfg.steps):
        yl, ys = based.decode_step(st, *dev(qs[s], ks[s], vs[s]))
        rl, rs = ref.step(qs[s], ks[s], vs[s])
        assert rowinf_rel(yl, rl) <= 2e-3 and rowinf_rel(ys, rs) <= 2e-3, s
    assert st.pos.cpu().tolist() == [10 + cfg.steps, 30 + cfg.steps]


FULL_DECODE_CHECKS = [0, 1, 2, 62, 63, 64, 65, 500, 999]


def test_decode_full_workload_sampled(based):
    """The decode workload as benchmarked: 256 sequences x 16 heads, a
    2048-token context, d_v 64, bf16 ring, all 1000 steps; the oracle follows
    sampled sequences, outputs checked around the ring turns and at the end,
    and the final S, z and positions."""
    cfg = synth.DECODE_CONFIG
    assert cfg.steps == 1000
    run_decode(based, cfg, seqs=[0, 101, 255], check_steps=FULL_DECODE_CHECKS)


def test_decode_snapshot_restore(based):
    """Copying the state out and back in resumes bit-identically."""
    cfg = synth.DecodeConfig("snap", B=2, H=4, ctx=50, steps=20)
    (qc, kc, vc), (qs, ks, vs) = synth.decode_inputs(cfg)
    _, _, st = based.decode_init(qc.to(DEV), kc.to(DEV), vc.to(DEV))
    qd, kd, vd = qs.to(DEV), ks.to(DEV), vs.to(DEV)
    for s in range(10):
        based.decode_step(st, qd[s], kd[s], vd[s])
    snap = [t.cpu().clone() for t in (st.S, st.z, st.ring_k, st.ring_v, st.pos)]
    outs_a = [based.decode_step(st, qd[s], kd[s], vd[s]) for s in range(10, 20)]
    outs_a = [(a.cpu(), b.cpu()) for a, b in outs_a]
    st2 = based.DecodeState(*[t.to(DEV) for t in snap])
    outs_b = [based.decode_step(st2, qd[s], kd[s], vd[s]) for s in range(10, 20)]
    torch.cuda.synchronize()
    for (a1, b1), (a2, b2) in zip(outs_a, outs_b):
        assert torch.equal(a1, a2.cpu()) and torch.equal(b1, b2.cpu())


def run_decay_decode(based, cfg, compact=False):
    """Decode with a per-head state decay (heads cycle through 1, 0.75,
    0.875, ...): the context's state from based_linattn_decay_fwd (bf16) or an
    empty one (ctx = 0), then steps through based_decode_step_decay, against
    the oracle's decayed recurrence and its DecodeState with gamma."""
    (qc, kc, vc), (qs, ks, vs) = synth.decode_inputs(cfg, 0)
    g = synth.decay_rates(cfg.H)
    gd = g.to(DEV)
    say(f"decay decode B{cfg.B} H{cfg.H} ctx{cfg.ctx} steps{cfg.steps} dv{cfg.dv} {cfg.dtype}")
    tol = TOL[qc.dtype]
    ref = O.DecodeState.prefill(kc, vc, cfg.window)
    if cfg.ctx > 0:
        _, _, S, z = O.linattn_decay_recurrent(qc, kc, vc, g.numpy())
        ref.S, ref.z = S, z
        _, _, st = based.decode_init(qc.to(DEV), kc.to(DEV), vc.to(DEV), cfg.window, gamma=gd, compact=compact)
    else:
        ref.S[:], ref.z[:] = 0.0, 0.0
        B, H = cfg.B, cfg.H
        rows = O.D_CMP if compact else O.D_PHI
        st = based.DecodeState(torch.zeros(B, H, rows, cfg.dv, device=DEV), torch.zeros(B, H, rows, device=DEV),
                               torch.zeros(B, H, cfg.window, 16, device=DEV, dtype=qc.dtype),
                               torch.zeros(B, H, cfg.window, cfg.dv, device=DEV, dtype=qc.dtype),
                               torch.zeros(B, device=DEV, dtype=torch.int32), compact)
    qd, kd, vd = qs.to(DEV), ks.to(DEV), vs.to(DEV)
    el = es = 0.0
    for s in range(cfg.steps):
        yl, ys = based.decode_step(st, qd[s], kd[s], vd[s], gamma=gd)
        rl, rs = ref.step(qs[s], ks[s], vs[s], gamma=g.numpy())
        el, es = max(el, rowinf_rel(yl, rl)), max(es, rowinf_rel(ys, rs))
        assert el <= tol and es <= tol, (s, el, es)
    torch.cuda.synchronize()
    report(f"decay decode y_lin ctx{cfg.ctx} {cfg.dtype}", el, tol)
    report(f"decay decode y_swa ctx{cfg.ctx} {cfg.dtype}", es, tol)
    S_ref, z_ref = O.state_compact(ref.S, ref.z) if compact else (ref.S, ref.z)
    assert rowinf_rel(st.S, S_ref) <= tol and z_block_rel(st.z, z_ref) <= tol
    assert torch.all(st.pos.cpu() == cfg.ctx + cfg.steps)
    return st


def test_decay_decode_after_context(based):
    run_decay_decode(based, synth.DecodeConfig("decay", B=2, H=8, ctx=150, steps=70, dtype="bf16"))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decay_decode_from_empty_context(based, dtype):
    run_decay_decode(based, synth.DecodeConfig("decay0", B=2, H=9, ctx=0, steps=40, dv=48, dtype=dtype))


def test_decay_decode_gamma_one_is_plain_decode(based):
    """gamma = 1 on every head: the decayed step is the plain step, bit for bit."""
    cfg = synth.DecodeConfig("g1", B=2, H=3, ctx=70, steps=5)
    (qc, kc, vc), (qs, ks, vs) = synth.decode_inputs(cfg)
    ones = torch.ones(cfg.H, device=DEV)
    _, _, a = based.decode_init(qc.to(DEV), kc.to(DEV), vc.to(DEV))
    _, _, b = based.decode_init(qc.to(DEV), kc.to(DEV), vc.to(DEV))
    for s in range(cfg.steps):
        ya = based.decode_step(a, qs[s].to(DEV), ks[s].to(DEV), vs[s].to(DEV))
        yb = based.decode_step(b, qs[s].to(DEV), ks[s].to(DEV), vs[s].to(DEV), gamma=ones)
        assert torch.equal(ya[0], yb[0]) and torch.equal(ya[1], yb[1])
    assert torch.equal(a.S, b.S) and torch.equal(a.z, b.z)


# ------------------------------------------------------------- compact state
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_compact_decode_small_wraps_ring(based, dtype):
    cfg = synth.DecodeConfig("small", B=3, H=4, ctx=100, steps=70, dtype=dtype)
    run_decode(based, cfg, compact=True)


@pytest.mark.parametrize("dv,window", [(128, 64), (16, 9), (80, 64)])
def test_compact_decode_shapes(based, dv, window):
    cfg = synth.DecodeConfig("shape", B=2, H=20, ctx=37, steps=30, dv=dv, window=window)
    run_decode(based, cfg, compact=True)


def test_compact_decode_full_workload_sampled(based):
    cfg = synth.DECODE_CONFIG
    run_decode(based, cfg, seqs=[0, 101, 255], check_steps=FULL_DECODE_CHECKS, compact=True)


def test_compact_decay_decode_after_context(based):
    run_decay_decode(based, synth.DecodeConfig("decay", B=2, H=8, ctx=150, steps=70, dtype="bf16"), compact=True)


def test_compact_decay_decode_from_empty_context(based):
    run_decay_decode(based, synth.DecodeConfig("decay0", B=2, H=9, ctx=0, steps=40, dv=48, dtype="f32"),
                     compact=True)


def test_state_conversions_match_oracle(based):
    """based_state_compact / based_state_expand against the oracle's
    definitions: a random (non-symmetric) state compacted (pair rows summed
    in fp32), and a random compact state expanded (exact halves)."""
    g = torch.Generator().manual_seed(31)
    B, H, dv = 2, 5, 48
    S, z = torch.randn(B, H, 273, dv, generator=g), torch.randn(B, H, 273, generator=g)
    Sc, zc = based.state_compact(S.to(DEV), z.to(DEV))
    rS, rz = O.state_compact(S, z)
    err = max(rowinf_rel(Sc, rS), rowinf_rel(zc, rz))
    report("state_compact vs oracle", err, 1e-6)
    assert err <= 1e-6
    C, cz = torch.randn(B, H, 153, dv, generator=g), torch.randn(B, H, 153, generator=g)
    S2, z2 = based.state_expand(C.to(DEV), cz.to(DEV))
    eS, ez = O.state_expand(C, cz)
    assert np.array_equal(S2.double().cpu().numpy(), eS) and np.array_equal(z2.double().cpu().numpy(), ez)
    C2, cz2 = based.state_compact(S2, z2)
    assert torch.equal(C2.cpu(), C) and torch.equal(cz2.cpu(), cz)


def test_compact_and_full_decode_agree(based):
    """The same context and tokens through both layouts: outputs within fp32
    rounding of each other, and the expanded compact state equals the full
    one to the same order."""
    cfg = synth.DecodeConfig("both", B=2, H=6, ctx=90, steps=40, dtype="f32")
    (qc, kc, vc), (qs, ks, vs) = synth.decode_inputs(cfg)
    _, _, full = based.decode_init(qc.to(DEV), kc.to(DEV), vc.to(DEV))
    _, _, comp = based.decode_init(qc.to(DEV), kc.to(DEV), vc.to(DEV), compact=True)
    worst = 0.0
    for s in range(cfg.steps):
        a = based.decode_step(full, qs[s].to(DEV), ks[s].to(DEV), vs[s].to(DEV))
        b = based.decode_step(comp, qs[s].to(DEV), ks[s].to(DEV), vs[s].to(DEV))
        worst = max(worst, rowinf_rel(b[0], a[0].double().cpu().numpy()))
        assert torch.equal(a[1], b[1])  # the window attention does not touch the state
    report("compact vs full decode y_lin", worst, 1e-5)
    assert worst <= 1e-5
    S, z = based.state_expand(comp.S, comp.z)
    assert rowinf_rel(S, full.S.double().cpu().numpy()) <= 1e-5
    assert torch.all(comp.pos == full.pos)


def test_compact_state_hands_over_to_full_decode(based):
    """Steps on the compact state, then the state expanded and the rest on the
    273-row step: the outputs follow an all-full run within fp32 rounding."""
    cfg = synth.DecodeConfig("handover", B=2, H=5, ctx=40, steps=30, dv=32, dtype="f32")
    (qc, kc, vc), (qs, ks, vs) = synth.decode_inputs(cfg)
    _, _, full = based.decode_init(qc.to(DEV), kc.to(DEV), vc.to(DEV))
    _, _, comp = based.decode_init(qc.to(DEV), kc.to(DEV), vc.to(DEV), compact=True)
    worst = 0.0
    for s in range(cfg.steps):
        a = based.decode_step(full, qs[s].to(DEV), ks[s].to(DEV), vs[s].to(DEV))
        if s == 12:  # hand the compact generation over to the full layout
            S, z = based.state_expand(comp.S, comp.z)
            comp = based.DecodeState(S, z, comp.ring_k, comp.ring_v, comp.pos)
        b = based.decode_step(comp, qs[s].to(DEV), ks[s].to(DEV), vs[s].to(DEV))
        worst = max(worst, rowinf_rel(b[0], a[0].double().cpu().numpy()))
        assert torch.equal(a[1], b[1])
    report("compact -> full handover y_lin", worst, 1e-5)
    assert worst <= 1e-5
    assert not comp.compact and comp.S.shape[2] == 273
