"""GPU parity of the forward entry points (based_linattn_fwd, based_swa_fwd)
against the fp64 oracle, on the same seeded inputs."""

import numpy as np
import pytest
import torch

import synth
from oracle import based_oracle as O
from parity_util import TOL, report, rowinf_rel, say, z_block_rel

pytestmark = pytest.mark.gpu
DEV = "cuda"


def inputs(cfg, seed=0):
    return synth.fwd_inputs(cfg, seed)


def check_linattn(based, cfg, heads=None, seed=0, chunk=64):
    """Full-size GPU call; oracle on all heads, or on the sampled (b, h) heads."""
    q, k, v = inputs(cfg, seed)
    say(f"linattn {cfg.name} B{cfg.B} H{cfg.H} L{cfg.L} dv{cfg.dv} {cfg.dtype}")
    y, S, z = based.linattn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), return_state=True)
    torch.cuda.synchronize()
    tol = TOL[q.dtype]
    sel = [(b, h) for b in range(cfg.B) for h in range(cfg.H)] if heads is None else heads
    bi = [b for b, _ in sel]
    hi = [h for _, h in sel]
    qs, ks, vs = q[bi, hi], k[bi, hi], v[bi, hi]
    y_ref, _, S_ref, z_ref = O.linattn_chunked(qs, ks, vs, chunk)
    err = rowinf_rel(y[bi, hi], y_ref)
    report(f"linattn y {cfg.name}", err, tol)
    assert err <= tol
    errS = rowinf_rel(S[bi, hi], S_ref)
    errz = z_block_rel(z[bi, hi], z_ref)
    report(f"linattn S_out {cfg.name}", errS, tol)
    assert errS <= tol and errz <= tol
    return y


def check_swa(based, cfg, heads=None, seed=0, window=64):
    q, k, v = inputs(cfg, seed)
    say(f"swa {cfg.name} B{cfg.B} H{cfg.H} L{cfg.L} dv{cfg.dv} {cfg.dtype} window{window}")
    y = based.swa_fwd(q.to(DEV), k.to(DEV), v.to(DEV), window)
    torch.cuda.synchronize()
    sel = [(b, h) for b in range(cfg.B) for h in range(cfg.H)] if heads is None else heads
    bi = [b for b, _ in sel]
    hi = [h for _, h in sel]
    y_ref = O.swa(q[bi, hi], k[bi, hi], v[bi, hi], window)
    err = rowinf_rel(y[bi, hi], y_ref)
    report(f"swa y {cfg.name} w{window}", err, TOL[q.dtype])
    assert err <= TOL[q.dtype]


# ---------------------------------------------------------------- the workloads
def test_tiny_fp32(based):
    cfg = synth.FWD_CONFIGS["tiny"]
    check_linattn(based, cfg)
    check_swa(based, cfg)


@pytest.mark.parametrize("name,heads", [
    ("based360m", [(0, 0), (3, 7), (7, 15)]),
    ("based1p3b", [(0, 0), (2, 9), (3, 15)]),
    ("long32k", [(0, 0), (0, 11)]),
])
def test_full_size_sampled_heads(based, name, heads):
    cfg = synth.FWD_CONFIGS[name]
    check_linattn(based, cfg, heads)
    check_swa(based, cfg, heads)


# ------------------------------------------------------ shapes, tails and edges
SMALL = synth.FwdConfig("small", B=2, H=3, L=1000, dv=64)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("L", [1, 2, 63, 64, 65, 130, 1000])
def test_lengths(based, dtype, L):
    cfg = SMALL.replace(L=L, dtype=dtype, name=f"L{L}")
    check_linattn(based, cfg)
    check_swa(based, cfg)


@pytest.mark.parametrize("dv", [16, 32, 48, 80, 96, 112, 128])
def test_value_dims(based, dv):
    cfg = SMALL.replace(L=300, dv=dv, name=f"dv{dv}")
    check_linattn(based, cfg)
    check_swa(based, cfg)


@pytest.mark.parametrize("window", [1, 2, 17, 63, 64])
def test_windows(based, window):
    check_swa(based, SMALL.replace(L=200, name=f"w{window}"), window=window)


@pytest.mark.parametrize("dqk", [32, 128])
def test_swa_wider_qk(based, dqk):
    cfg = SMALL.replace(L=150, dk=dqk, name=f"dqk{dqk}")
    check_swa(based, cfg)


def test_swa_scale(based):
    cfg = SMALL.replace(L=150)
    q, k, v = inputs(cfg)
    y = based.swa_fwd(q.to(DEV), k.to(DEV), v.to(DEV), 64, scale=0.37)
    err = rowinf_rel(y, O.swa(q, k, v, 64, 0.37))
    report("swa scale 0.37", err, 2e-3)
    assert err <= 2e-3


def test_heavy_tailed_small(based):
    cfg = SMALL.replace(L=2000, heavy_frac=0.01, name="heavy")
    check_linattn(based, cfg)
    check_swa(based, cfg)


def test_empty_sequence(based):
    q = torch.zeros(1, 2, 0, 16, device=DEV, dtype=torch.bfloat16)
    v = torch.zeros(1, 2, 0, 64, device=DEV, dtype=torch.bfloat16)
    y, S, z = based.linattn_fwd(q, q, v, return_state=True)
    assert y.shape == (1, 2, 0, 64)
    torch.cuda.synchronize()
    assert torch.all(S == 0) and torch.all(z == 0)
    assert based.swa_fwd(q, q, v).shape == (1, 2, 0, 64)


# --------------------------------------------------------- state and resume
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_resume_from_exported_state(based, dtype):
    """fwd(x[:n]) -> (S, z) -> fwd(x[n:], S_in, z_in) equals fwd(x)."""
    cfg = SMALL.replace(L=700, dtype=dtype)
    q, k, v = [t.to(DEV) for t in inputs(cfg)]
    y = based.linattn_fwd(q, k, v)
    n = 333
    _, S1, z1 = based.linattn_fwd(q[:, :, :n].contiguous(), k[:, :, :n].contiguous(), v[:, :, :n].contiguous(),
                                  return_state=True)
    y2, S2, z2 = based.linattn_fwd(q[:, :, n:].contiguous(), k[:, :, n:].contiguous(), v[:, :, n:].contiguous(),
                                   S1, z1, return_state=True)
    yq, _, S_ref, z_ref = O.linattn_chunked(*inputs(cfg), 64)
    tol = TOL[q.dtype]
    err = rowinf_rel(y2, yq[:, :, n:])
    report(f"resume {dtype}", err, tol)
    assert err <= tol
    assert rowinf_rel(y[:, :, n:], yq[:, :, n:]) <= tol
    assert rowinf_rel(S2, S_ref) <= tol


def test_state_in_place_update(based):
    """S_out may alias S_in: the state advances in place."""
    cfg = SMALL.replace(L=200)
    q, k, v = [t.to(DEV) for t in inputs(cfg)]
    _, S, z = based.linattn_fwd(q[:, :, :90].contiguous(), k[:, :, :90].contiguous(), v[:, :, :90].contiguous(),
                                return_state=True)
    based.linattn_fwd(q[:, :, 90:].contiguous(), k[:, :, 90:].contiguous(), v[:, :, 90:].contiguous(), S, z,
                      S_out=S, z_out=z)
    S_ref, z_ref = O.linattn_state(*inputs(cfg)[1:])
    assert rowinf_rel(S, S_ref) <= 2e-3
    assert z_block_rel(z, z_ref) <= 2e-3


def test_nonsymmetric_initial_state(based):
    """A state enters only through S[ab] + S[ba] (documented): an arbitrary
    S_in gives the oracle's result for that S_in."""
    cfg = SMALL.replace(L=150, dtype="f32")
    q, k, v = inputs(cfg)
    g = torch.Generator().manual_seed(5)
    S0 = torch.randn(cfg.B, cfg.H, 273, cfg.dv, generator=g)
    z0 = torch.rand(cfg.B, cfg.H, 273, generator=g) + 50.0
    y = based.linattn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), S0.to(DEV), z0.to(DEV))
    y_ref = O.linattn_recurrent(q, k, v, S0, z0)[0]
    err = rowinf_rel(y, y_ref)
    report("non-symmetric S_in", err, 1e-5)
    assert err <= 1e-5


def prefix_state(cfg, n=500, seed=1):
    """The state a seeded prefix of n positions leaves (what a resumed call
    receives as S_in), from the oracle."""
    _, k, v = inputs(cfg.replace(L=n), seed)
    S0, z0 = O.linattn_state(k, v)
    return torch.from_numpy(S0).float(), torch.from_numpy(z0).float()


@pytest.mark.parametrize("B,H,L", [(2, 3, 768), (2, 3, 2560), (1, 12, 768)])
def test_initial_state_across_segments(based, B, H, L):
    """S_in with the sequence split into segments: segment 0 reads S_in,
    the later ones receive it through the state-only pass's records (three
    segments) or through the scan (ten); B*H = 12 puts heads on both sides of
    the XCD-grouped block mapping (eight grouped, four in plain order).  S_in
    is a prefix's exported state (an arbitrary one is covered in fp32 above:
    the bf16 path reads the state through an fp16 copy)."""
    cfg = SMALL.replace(B=B, H=H, L=L, name=f"S_in B{B}H{H}L{L}")
    q, k, v = inputs(cfg)
    S0, z0 = prefix_state(cfg)
    say(f"linattn {cfg.name} with S_in")
    y, S, z = based.linattn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), S0.to(DEV), z0.to(DEV), return_state=True)
    torch.cuda.synchronize()
    y_ref, _, S_ref, z_ref = O.linattn_chunked(q, k, v, 64, S0, z0)
    tol = TOL[q.dtype]
    err = rowinf_rel(y, y_ref)
    report(f"linattn y {cfg.name}", err, tol)
    assert err <= tol
    errS, errz = rowinf_rel(S, S_ref), z_block_rel(z, z_ref)
    report(f"linattn S_out {cfg.name}", max(errS, errz), tol)
    assert errS <= tol and errz <= tol


# ------------------------------------------------------------------ robustness
def test_no_writes_outside_outputs(based):
    """Guard bands around y and the state stay untouched."""
    cfg = SMALL.replace(L=333)
    q, k, v = [t.to(DEV) for t in inputs(cfg)]
    G = 4096
    n = cfg.B * cfg.H * cfg.L * cfg.dv
    buf = torch.full((n + 2 * G,), 7.5, device=DEV)
    y = buf[G:G + n].view(cfg.B, cfg.H, cfg.L, cfg.dv)
    ns = cfg.B * cfg.H * 273 * cfg.dv
    sbuf = torch.full((ns + 2 * G,), -3.0, device=DEV)
    zbuf = torch.full((cfg.B * cfg.H * 273 + 2 * G,), -3.0, device=DEV)
    based.linattn_fwd(q, k, v, y=y, S_out=sbuf[G:G + ns].view(cfg.B, cfg.H, 273, cfg.dv),
                      z_out=zbuf[G:G + cfg.B * cfg.H * 273].view(cfg.B, cfg.H, 273))
    ys = torch.full((n + 2 * G,), 7.5, device=DEV)
    based.swa_fwd(q, k, v, y=ys[G:G + n].view(cfg.B, cfg.H, cfg.L, cfg.dv))
    torch.cuda.synchronize()
    for b, val in ((buf, 7.5), (sbuf, -3.0), (zbuf, -3.0), (ys, 7.5)):
        assert torch.all(b[:G] == val) and torch.all(b[-G:] == val)


def test_repeat_runs_bitwise_identical(based):
    cfg = synth.FWD_CONFIGS["based360m"]
    q, k, v = [t.to(DEV) for t in inputs(cfg)]
    a = based.linattn_fwd(q, k, v)
    b = based.linattn_fwd(q, k, v)
    sa = based.swa_fwd(q, k, v)
    sb = based.swa_fwd(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(sa, sb)


def test_nan_stays_near_its_rows(based):
    """A NaN in v at position p = 150 reaches linear-attention rows >= p and
    window rows p..p+63.  Matrix-core tiles of 64 positions may also carry it
    to other rows of the tiles that hold position p (0 x NaN = NaN), never
    further: rows before 128 stay finite, and window rows from 256 on."""
    cfg = SMALL.replace(L=300, B=1, H=1)
    q, k, v = inputs(cfg)
    v[0, 0, 150, 3] = float("nan")
    y = based.linattn_fwd(q.to(DEV), k.to(DEV), v.to(DEV)).cpu()
    s = based.swa_fwd(q.to(DEV), k.to(DEV), v.to(DEV)).cpu()
    assert torch.isfinite(y[0, 0, :128]).all() and torch.isnan(y[0, 0, 150:, 3]).all()
    assert torch.isfinite(y[0, 0, :, [0, 1, 2, 4]]).all()
    assert torch.isfinite(s[0, 0, :128]).all() and torch.isfinite(s[0, 0, 256:]).all()
    assert torch.isnan(s[0, 0, 150:214, 3]).all()


# ---------------------------------------------- in-place state, arbitrary S_in
SEGMENT_SHAPES = [(2, 3, 150), (2, 3, 768), (2, 3, 2560)]  # 1, 3 and 10 segments per head


@pytest.mark.parametrize("B,H,L", SEGMENT_SHAPES)
@pytest.mark.parametrize("op", ["linattn", "layer", "decay"])
def test_state_in_place_several_segments(based, B, H, L, op):
    """S_out = S_in, z_out = z_in (the in-place update the header allows) with
    the sequence split into 1, 3 and 10 segments: the state-only pass copies
    S_in into the workspace before the main pass writes S_out, so the result
    is the oracle's state after prefix + sequence."""
    cfg = SMALL.replace(B=B, H=H, L=L, name=f"in-place {op} B{B}H{H}L{L}")
    q, k, v = inputs(cfg)
    S0, z0 = prefix_state(cfg)
    say(f"{cfg.name}")
    S, z = S0.clone().to(DEV), z0.clone().to(DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    if op == "linattn":
        y = based.linattn_fwd(qd, kd, vd, S, z, S_out=S, z_out=z)[0]
        y_ref, _, S_ref, z_ref = O.linattn_chunked(q, k, v, 64, S0, z0)
    elif op == "layer":
        y = based.layer_fwd(qd, kd, vd, 64, 1.0, S, z, S_out=S, z_out=z)[0]
        y_ref, _, S_ref, z_ref = O.linattn_chunked(q, k, v, 64, S0, z0)
    else:
        g = synth.decay_rates(H)
        y = based.linattn_decay_fwd(qd, kd, vd, g.to(DEV), S, z, S_out=S, z_out=z)[0]
        y_ref, _, S_ref, z_ref = O.linattn_decay_recurrent(q, k, v, g.numpy(), S0, z0)
    torch.cuda.synchronize()
    tol = TOL[q.dtype]
    err, errS, errz = rowinf_rel(y, y_ref), rowinf_rel(S, S_ref), z_block_rel(z, z_ref)
    report(f"{cfg.name} y / S / z", max(err, errS, errz), tol)
    assert err <= tol and errS <= tol and errz <= tol


def symmetrized(S, z):
    """The state the library exports for an initial state S, z: each pair of
    quadratic rows (a, b), (b, a) replaced by their mean (a state enters only
    through S[ab] + S[ba], and exported states are symmetric)."""
    S, z = np.array(S, np.float64), np.array(z, np.float64)
    Q = S[..., 17:, :].reshape(S.shape[:-2] + (16, 16, S.shape[-1]))
    S[..., 17:, :] = (0.5 * (Q + np.swapaxes(Q, -2, -3))).reshape(S.shape[:-2] + (256, S.shape[-1]))
    qz = z[..., 17:].reshape(z.shape[:-1] + (16, 16))
    z[..., 17:] = (0.5 * (qz + np.swapaxes(qz, -1, -2))).reshape(z.shape[:-1] + (256,))
    return S, z


def random_state(cfg, seed=5):
    """A unit-scale random initial state in every one of the 273 rows (not one
    the recurrence could build: not symmetric in (a, b)), with a denominator
    state near 50 so that every denominator stays positive."""
    g = torch.Generator().manual_seed(seed)
    S0 = torch.randn(cfg.B, cfg.H, 273, cfg.dv, generator=g)
    z0 = torch.rand(cfg.B, cfg.H, 273, generator=g) + 50.0
    return S0, z0


@pytest.mark.parametrize("B,H,L", SEGMENT_SHAPES)
@pytest.mark.parametrize("op", ["linattn", "layer", "decay"])
def test_bf16_arbitrary_initial_state(based, B, H, L, op):
    """bf16 inputs with an arbitrary S_in, z_in: the readout of such a state
    cancels over its feature rows, and the kernels read it out with hi + lo
    query features and state (1, 3 and 10 segments per head).  Bound on y:
    1e-3, half the bf16 tolerance."""
    cfg = SMALL.replace(B=B, H=H, L=L, name=f"arbitrary S_in {op} B{B}H{H}L{L}")
    q, k, v = inputs(cfg)
    S0, z0 = random_state(cfg)
    say(cfg.name)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    if op == "linattn":
        y, S, z = based.linattn_fwd(qd, kd, vd, S0.to(DEV), z0.to(DEV), return_state=True)
        y_ref, _, S_ref, z_ref = O.linattn_chunked(q, k, v, 64, S0, z0)
    elif op == "layer":
        y, ys, S, z = based.layer_fwd(qd, kd, vd, 64, 1.0, S0.to(DEV), z0.to(DEV), return_state=True)
        y_ref, _, S_ref, z_ref = O.linattn_chunked(q, k, v, 64, S0, z0)
        assert rowinf_rel(ys, O.swa(q, k, v, 64)) <= TOL[q.dtype]
    else:
        g = synth.decay_rates(H)
        y, S, z = based.linattn_decay_fwd(qd, kd, vd, g.to(DEV), S0.to(DEV), z0.to(DEV), return_state=True)
        y_ref, _, S_ref, z_ref = O.linattn_decay_recurrent(q, k, v, g.numpy(), S0, z0)
    torch.cuda.synchronize()
    err = rowinf_rel(y, y_ref)
    report(f"{cfg.name} y", err, 1e-3)
    assert err <= 1e-3
    # the exported state: the forward's bf16 tolerance (the decayed update
    # rounds key features and their decay weights to fp16)
    S_ref, z_ref = symmetrized(S_ref, z_ref)
    errS, errz = rowinf_rel(S, S_ref), z_block_rel(z, z_ref)
    report(f"{cfg.name} S_out / z_out", max(errS, errz), TOL[q.dtype])
    assert errS <= TOL[q.dtype] and errz <= TOL[q.dtype]


@pytest.mark.parametrize("dv", [32, 96, 128])
@pytest.mark.parametrize("op", ["linattn", "layer", "decay"])
def test_value_dims_across_segments(based, dv, op):
    """The other matrix-core widths with the sequence split into segments (L =
    1000 on six heads: four per head) and an arbitrary bf16 S_in: the
    state-only pass with its initial-state record (at d_v = 128 split over
    two workgroups by value columns), the record sums of the later segments,
    plain, fused with the window and decayed.  Same bounds as the d_v = 64
    case."""
    cfg = SMALL.replace(L=1000, dv=dv, name=f"segments {op} dv{dv}")
    q, k, v = inputs(cfg)
    S0, z0 = random_state(cfg)
    say(cfg.name)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    if op == "linattn":
        y, S, z = based.linattn_fwd(qd, kd, vd, S0.to(DEV), z0.to(DEV), return_state=True)
        y_ref, _, S_ref, z_ref = O.linattn_chunked(q, k, v, 64, S0, z0)
    elif op == "layer":
        y, ys, S, z = based.layer_fwd(qd, kd, vd, 64, 1.0, S0.to(DEV), z0.to(DEV), return_state=True)
        y_ref, _, S_ref, z_ref = O.linattn_chunked(q, k, v, 64, S0, z0)
        assert rowinf_rel(ys, O.swa(q, k, v, 64)) <= TOL[q.dtype]
    else:
        g = synth.decay_rates(cfg.H)
        y, S, z = based.linattn_decay_fwd(qd, kd, vd, g.to(DEV), S0.to(DEV), z0.to(DEV), return_state=True)
        y_ref, _, S_ref, z_ref = O.linattn_decay_recurrent(q, k, v, g.numpy(), S0, z0)
    torch.cuda.synchronize()
    err = rowinf_rel(y, y_ref)
    report(f"{cfg.name} y", err, 1e-3)
    assert err <= 1e-3
    S_ref, z_ref = symmetrized(S_ref, z_ref)
    errS, errz = rowinf_rel(S, S_ref), z_block_rel(z, z_ref)
    report(f"{cfg.name} S_out / z_out", max(errS, errz), TOL[q.dtype])
    assert errS <= TOL[q.dtype] and errz <= TOL[q.dtype]


@pytest.mark.parametrize("mode", ["separate", "S in place", "S and z in place", "decayed"])
def test_fp32_column_slices(based, mode):
    """fp32 inputs on few heads: the vector pass splits each head's value
    columns over 16-column workgroups (each reads its columns of S_in and
    writes them to S_out, slice 0 writes z_out), except for an in-place z
    (z_out = z_in: one workgroup per head).  An arbitrary S_in, z_in; y and
    the exported state against the oracle."""
    cfg = SMALL.replace(L=150, dtype="f32", name=f"fp32 slices {mode}")
    q, k, v = inputs(cfg)
    S0, z0 = random_state(cfg)
    say(cfg.name)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    S, z = S0.clone().to(DEV), z0.clone().to(DEV)
    if mode == "decayed":
        g = synth.decay_rates(cfg.H)
        y, S, z = based.linattn_decay_fwd(qd, kd, vd, g.to(DEV), S, z, return_state=True)
        y_ref, _, S_ref, z_ref = O.linattn_decay_recurrent(q, k, v, g.numpy(), S0, z0)
    else:
        if mode == "separate":
            y, S, z = based.linattn_fwd(qd, kd, vd, S, z, return_state=True)
        elif mode == "S in place":
            z_out = torch.empty_like(z)
            y = based.linattn_fwd(qd, kd, vd, S, z, S_out=S, z_out=z_out)[0]
            z = z_out
        else:
            y = based.linattn_fwd(qd, kd, vd, S, z, S_out=S, z_out=z)[0]
        y_ref, _, S_ref, z_ref = O.linattn_recurrent(q, k, v, S0, z0)
    torch.cuda.synchronize()
    S_ref, z_ref = symmetrized(S_ref, z_ref)
    err, errS, errz = rowinf_rel(y, y_ref), rowinf_rel(S, S_ref), z_block_rel(z, z_ref)
    report(f"{cfg.name} y / S / z", max(err, errS, errz), 1e-5)
    assert err <= 1e-5 and errS <= 1e-5 and errz <= 1e-5


@pytest.mark.parametrize("dtype,dv", [("f32", 64), ("bf16", 48), ("f32", 128)])
@pytest.mark.parametrize("L", [1, 31, 33, 256, 512])
@pytest.mark.parametrize("decayed", [False, True])
def test_quadratic_form_short(based, dtype, dv, L, decayed):
    """The vector path's quadratic form (no state argument, L <= 512): one
    workgroup per 32 queries against every earlier key block, plain and
    decayed, against the oracle's recurrent form; and, with a state argument
    (the chunked vector pass), the same y within fp32 rounding."""
    cfg = SMALL.replace(L=L, dv=dv, dtype=dtype, name=f"quadratic {dtype} dv{dv} L{L} decayed={decayed}")
    q, k, v = inputs(cfg)
    say(cfg.name)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    if decayed:
        g = synth.decay_rates(cfg.H)
        y = based.linattn_decay_fwd(qd, kd, vd, g.to(DEV))
        y_chunked = based.linattn_decay_fwd(qd, kd, vd, g.to(DEV), return_state=True)[0]
        y_ref = O.linattn_decay_recurrent(q, k, v, g.numpy())[0]
    else:
        y = based.linattn_fwd(qd, kd, vd)
        y_chunked = based.linattn_fwd(qd, kd, vd, return_state=True)[0]
        y_ref = O.linattn_recurrent(q, k, v)[0]
    torch.cuda.synchronize()
    err = rowinf_rel(y, y_ref)
    report(cfg.name, err, TOL[q.dtype])
    assert err <= TOL[q.dtype]
    gap = rowinf_rel(y, y_chunked.double().cpu().numpy())
    report(f"{cfg.name} vs the chunked pass", gap, 1e-5)
    assert gap <= 1e-5


def test_bf16_near_fp16_range(based):
    """Inputs near the bound the header states for the bf16 path (|q.k| < 256,
    |v| < 32768): every coordinate of k is +-3.5 and q_i = k_{i-5}, so that
    q_i.k_{i-5} = 196 (kernel weight ~1.9e4) and other scores reach about
    +-150; v ~ 1e4 N(0,1) clipped to +-3e4.  Both attentions of the layer,
    over 3 segments."""
    B, H, L, dv = 1, 4, 768, 64
    g = torch.Generator().manual_seed(11)
    k = 3.5 * torch.sign(torch.randn(B, H, L, 16, generator=g))
    q = torch.roll(k, 5, dims=2)
    v = (1e4 * torch.randn(B, H, L, dv, generator=g)).clamp(-3e4, 3e4)
    q, k, v = q.bfloat16(), k.bfloat16(), v.bfloat16()
    s = (q.double() @ k.double().transpose(-1, -2)).abs()
    assert s.max() < 256 and float(v.abs().max()) < 32768
    y_lin, y_swa, S, z = based.layer_fwd(q.to(DEV), k.to(DEV), v.to(DEV), 64, 1.0, return_state=True)
    torch.cuda.synchronize()
    y_ref, _, S_ref, z_ref = O.linattn_chunked(q, k, v, 64)
    e1, e2 = rowinf_rel(y_lin, y_ref), rowinf_rel(y_swa, O.swa(q, k, v, 64))
    e3 = max(rowinf_rel(S, S_ref), z_block_rel(z, z_ref))
    report("near fp16 range: y_lin / y_swa / state", max(e1, e2, e3), 2e-3)
    assert e1 <= 2e-3 and e2 <= 2e-3 and e3 <= 2e-3


@pytest.mark.parametrize("dtype,dv", [("f32", 64), ("f32", 128), ("bf16", 48)])
def test_vector_pass_long_sequence(based, dtype, dv):
    """The vector pass (fp32, and widths the matrix cores do not take) over
    6000 positions -- 188 chunks in sequence and a ragged tail -- on whole
    heads: y and the exported state against the chunked oracle."""
    check_linattn(based, synth.FwdConfig(f"vector long {dtype} dv{dv}", B=1, H=2, L=6000, dv=dv, dtype=dtype))
