"""GPU parity of the fused layer entry point (based_layer_fwd): one pass that
returns both attentions of the layer over the same q, k, v.  y_lin is checked
against the oracle's chunked linear attention and against based_linattn_fwd's
output (the same arithmetic; only the compiler's fusing of multiply-adds may
differ between the two kernels, so they agree to 1e-6, not bit for bit);
y_swa is checked against the oracle's sliding-window softmax with
d_qk = d_k = 16."""

import pytest
import torch

import synth
from oracle import based_oracle as O
from parity_util import TOL, report, rowinf_rel, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
SMALL = synth.FwdConfig("small", B=2, H=3, L=1000, dv=64)


def check_layer(based, cfg, heads=None, window=64, scale=1.0, seed=0):
    q, k, v = synth.fwd_inputs(cfg, seed)
    say(f"layer {cfg.name} B{cfg.B} H{cfg.H} L{cfg.L} dv{cfg.dv} {cfg.dtype} window{window} scale{scale}")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    y_lin, y_swa, S, z = based.layer_fwd(qd, kd, vd, window, scale, return_state=True)
    # the same arguments (the final state asked for): the same evaluation
    y_sep = based.linattn_fwd(qd, kd, vd, return_state=True)[0]
    torch.cuda.synchronize()
    gap = rowinf_rel(y_lin, y_sep.double().cpu().numpy())
    report(f"layer y_lin vs based_linattn_fwd {cfg.name}", gap, 1e-6)
    assert gap <= 1e-6
    tol = TOL[q.dtype]
    sel = [(b, h) for b in range(cfg.B) for h in range(cfg.H)] if heads is None else heads
    bi = [b for b, _ in sel]
    hi = [h for _, h in sel]
    qs, ks, vs = q[bi, hi], k[bi, hi], v[bi, hi]
    y_ref, _, S_ref, _ = O.linattn_chunked(qs, ks, vs, 64)
    err = rowinf_rel(y_lin[bi, hi], y_ref)
    report(f"layer y_lin {cfg.name}", err, tol)
    assert err <= tol
    assert rowinf_rel(S[bi, hi], S_ref) <= tol
    s_ref = O.swa(qs, ks, vs, window, scale)
    err = rowinf_rel(y_swa[bi, hi], s_ref)
    report(f"layer y_swa {cfg.name} w{window}", err, tol)
    assert err <= tol


@pytest.mark.parametrize("name,heads", [
    ("based360m", [(0, 0), (3, 7), (7, 15)]),
    ("based1p3b", [(0, 0), (2, 9), (3, 15)]),
    ("long32k", [(0, 0), (0, 11)]),
])
def test_layer_full_size_sampled_heads(based, name, heads):
    """The workloads at full size; the window crosses every segment boundary."""
    check_layer(based, synth.FWD_CONFIGS[name], heads)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("L", [1, 2, 63, 64, 65, 130, 1000])
def test_layer_lengths(based, dtype, L):
    check_layer(based, SMALL.replace(L=L, dtype=dtype, name=f"L{L}"))


@pytest.mark.parametrize("dv", [32, 48, 96, 128])
def test_layer_value_dims(based, dv):
    check_layer(based, SMALL.replace(L=300, dv=dv, name=f"dv{dv}"))


@pytest.mark.parametrize("window", [1, 2, 17, 63, 64])
def test_layer_windows(based, window):
    check_layer(based, SMALL.replace(L=300, name=f"w{window}"), window=window)


def test_layer_scale_and_heavy_rows(based):
    check_layer(based, SMALL.replace(L=2000, heavy_frac=0.01, name="heavy"), scale=0.37)


def test_layer_segments_and_window(based):
    """Many segments per head (B = H = 1, long L): each segment's first chunk
    takes its window from the previous segment."""
    check_layer(based, synth.FwdConfig("seg", B=1, H=1, L=8192 + 37, dv=64), window=64)
    check_layer(based, synth.FwdConfig("seg", B=1, H=1, L=8192 + 37, dv=64), window=5)


def check_layer_vector_fused(based, cfg, window=64, scale=1.0, decay=False, seed=0):
    """The vector path's one-pass layer (short sequences, no state argument):
    y_lin and y_swa against the oracle and against the separate calls."""
    q, k, v = synth.fwd_inputs(cfg, seed)
    say(f"vector layer {cfg.name} B{cfg.B} H{cfg.H} L{cfg.L} dv{cfg.dv} {cfg.dtype} window{window} scale{scale}"
        f" decay{int(decay)}")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    if decay:
        g = synth.decay_rates(cfg.H)
        y_lin, y_swa = based.layer_decay_fwd(qd, kd, vd, g.to(DEV), window, scale)
        y_sep = based.linattn_decay_fwd(qd, kd, vd, g.to(DEV))
    else:
        y_lin, y_swa = based.layer_fwd(qd, kd, vd, window, scale)
        y_sep = based.linattn_fwd(qd, kd, vd)
    s_sep = based.swa_fwd(qd, kd, vd, window, scale)
    torch.cuda.synchronize()
    tol = TOL[q.dtype]
    # y_lin: the separate call takes the same one-pass form (1e-6); y_swa: the
    # separate window kernel sums and exponentiates differently (fp32), or
    # runs on the matrix cores (bf16), so the oracle's tolerance
    for name, got, sep, bound in (("y_lin", y_lin, y_sep, 1e-6), ("y_swa", y_swa, s_sep, tol)):
        gap = rowinf_rel(got, sep.double().cpu().numpy())
        report(f"vector layer {name} vs the separate call {cfg.name}", gap, bound)
        assert gap <= bound
    if decay:
        y_ref = O.linattn_decay_quadratic(q, k, v, g.numpy())[0]
    else:
        y_ref = O.linattn_chunked(q, k, v, 64)[0]
    err = rowinf_rel(y_lin, y_ref)
    report(f"vector layer y_lin {cfg.name}", err, tol)
    assert err <= tol
    err = rowinf_rel(y_swa, O.swa(q, k, v, window, scale))
    report(f"vector layer y_swa {cfg.name} w{window}", err, tol)
    assert err <= tol


@pytest.mark.parametrize("L", [1, 2, 31, 32, 33, 63, 64, 65, 130, 256, 300, 512])
def test_layer_vector_fused_lengths(based, L):
    """fp32, lengths around the 32-query blocks up to the longest one-pass
    length (512)."""
    check_layer_vector_fused(based, SMALL.replace(L=L, dtype="f32", name=f"L{L}"))


@pytest.mark.parametrize("window,scale", [(1, 1.0), (17, 0.37), (33, 2.0), (63, 1.0), (64, 0.25)])
def test_layer_vector_fused_windows(based, window, scale):
    check_layer_vector_fused(based, SMALL.replace(L=300, dtype="f32", name=f"w{window}"), window, scale)


@pytest.mark.parametrize("dtype,dv", [("f32", 16), ("f32", 128), ("bf16", 48), ("bf16", 112)])
def test_layer_vector_fused_value_dims(based, dtype, dv):
    """Other widths; bf16 inputs at the widths the matrix-core pass does not take."""
    check_layer_vector_fused(based, SMALL.replace(L=200, dtype=dtype, dv=dv, name=f"dv{dv}"))


@pytest.mark.parametrize("L", [45, 512])
def test_layer_vector_fused_decay(based, L):
    check_layer_vector_fused(based, SMALL.replace(L=L, dtype="f32", name=f"decay{L}"), 64, 1.0, decay=True)


def test_layer_vector_fused_tiny_config(based):
    """The tiny fp32 workload (B 1, H 2, L 256) as the bench times it."""
    check_layer_vector_fused(based, synth.FWD_CONFIGS["tiny"])


def test_layer_resume_state(based):
    """The linear-attention state threads through layer calls like through
    based_linattn_fwd (the window restarts with each call)."""
    cfg = SMALL.replace(L=700)
    q, k, v = [t.to(DEV) for t in synth.fwd_inputs(cfg)]
    n = 320
    _, _, S1, z1 = based.layer_fwd(q[:, :, :n].contiguous(), k[:, :, :n].contiguous(), v[:, :, :n].contiguous(),
                                   return_state=True)
    y2, s2 = based.layer_fwd(q[:, :, n:].contiguous(), k[:, :, n:].contiguous(), v[:, :, n:].contiguous(), 64, 1.0,
                             S1, z1)
    y_ref = O.linattn_chunked(*synth.fwd_inputs(cfg), 64)[0]
    err = rowinf_rel(y2, y_ref[:, :, n:])
    report("layer resume y_lin", err, 2e-3)
    assert err <= 2e-3
    qc, kc, vc = (t[:, :, n:] for t in synth.fwd_inputs(cfg))
    assert rowinf_rel(s2, O.swa(qc, kc, vc, 64)) <= 2e-3


def test_layer_empty(based):
    q = torch.zeros(1, 2, 0, 16, device=DEV, dtype=torch.bfloat16)
    v = torch.zeros(1, 2, 0, 64, device=DEV, dtype=torch.bfloat16)
    y_lin, y_swa, S, z = based.layer_fwd(q, q, v, return_state=True)
    torch.cuda.synchronize()
    assert y_lin.shape == y_swa.shape == (1, 2, 0, 64)
    assert torch.all(S == 0) and torch.all(z == 0)


@pytest.mark.parametrize("name", ["based360m", "based1p3b"])
def test_layer_reused_workspace(based, name):
    """One workspace, with arbitrary contents on entry, serves two calls on
    different inputs (the workload shapes, four segments per head): the
    second call's outputs equal a call on a fresh workspace bit for bit (no
    record of the first call is read) and match the oracle on sampled
    heads."""
    cfg = synth.FWD_CONFIGS[name]
    B, H, L, dv = cfg.B, cfg.H, cfg.L, cfg.dv
    need = based.linattn_workspace_bytes(B, H, L, dv)
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device=DEV)  # arbitrary contents on entry
    outs = []
    for seed in (0, 1):
        q, k, v = [t.to(DEV) for t in synth.fwd_inputs(cfg, seed)]
        say(f"layer {name} seed {seed}, shared workspace")
        outs.append(based.layer_fwd(q, k, v, 64, 1.0, return_state=True, workspace=ws))
        torch.cuda.synchronize()
    q, k, v = [t.to(DEV) for t in synth.fwd_inputs(cfg, 1)]
    fresh = based.layer_fwd(q, k, v, 64, 1.0, return_state=True)
    torch.cuda.synchronize()
    for a, b in zip(outs[1], fresh):
        assert torch.equal(a, b)
    q, k, v = synth.fwd_inputs(cfg, 1)
    heads = [(0, 0), (B - 1, H - 1)]
    bi, hi = [b for b, _ in heads], [h for _, h in heads]
    y_ref = O.linattn_chunked(q[bi, hi], k[bi, hi], v[bi, hi], 64)[0]
    err = max(rowinf_rel(outs[1][0][bi, hi], y_ref), rowinf_rel(outs[1][1][bi, hi], O.swa(q[bi, hi], k[bi, hi],
                                                                                           v[bi, hi], 64)))
    report(f"layer {name} second call on a shared workspace", err, TOL[q.dtype])
    assert err <= TOL[q.dtype]
