"""based_layer_fwd_noalloc (the allocation-free form of based_layer_fwd,
segment records in the library's static device array) against
based_layer_fwd with a caller workspace: the same kernels, so the outputs
must agree bit for bit.  Two calls in a row, the second on a smaller input
(the array keeps the first call's records, which the second must not
depend on), each also against the fp64 oracle on sampled heads."""

import ctypes

import numpy as np
import pytest
import torch

import synth
from oracle import based_oracle as O
from parity_util import TOL, report, rowinf_rel, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_pair(based, cfg, state):
    q, k, v = synth.fwd_inputs(cfg, 0)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    B, H, L, dv = cfg.B, cfg.H, cfg.L, cfg.dv
    say(f"no-alloc layer B{B} H{H} L{L} dv{dv} state={state}")
    S0 = z0 = None
    if state:
        _, kp, vp = synth.fwd_inputs(cfg.replace(L=300), 1)
        S0, z0 = [torch.from_numpy(t).float().to(DEV) for t in O.linattn_state(kp, vp)]
    y_lin, y_swa = torch.empty(B, H, L, dv, device=DEV), torch.empty(B, H, L, dv, device=DEV)
    S_out, z_out = torch.empty(B, H, 273, dv, device=DEV), torch.empty(B, H, 273, device=DEV)
    # straight through the C ABI
    so = based.load_library()
    st = so.based_layer_fwd_noalloc(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), y_lin.data_ptr(), y_swa.data_ptr(),
                                    S0.data_ptr() if state else None, z0.data_ptr() if state else None,
                                    S_out.data_ptr(), z_out.data_ptr(), B, H, L, 16, dv, 64, ctypes.c_float(1.0), 1,
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, so.based_status_string(st)
    ref = based.layer_fwd(qd, kd, vd, 64, 1.0, S0, z0, return_state=True)
    torch.cuda.synchronize()
    for a, b in zip((y_lin, y_swa, S_out, z_out), ref):
        assert torch.equal(a, b)
    heads = [(0, 0), (B - 1, H - 1)]
    bi, hi = [b for b, _ in heads], [h for _, h in heads]
    y_ref = O.linattn_chunked(q[bi, hi], k[bi, hi], v[bi, hi], 64,
                              None if not state else S0.cpu()[bi, hi], None if not state else z0.cpu()[bi, hi])[0]
    err = max(rowinf_rel(y_lin[bi, hi], y_ref), rowinf_rel(y_swa[bi, hi], O.swa(q[bi, hi], k[bi, hi], v[bi, hi], 64)))
    report(f"no-alloc layer B{B} H{H} L{L} vs oracle", err, TOL[q.dtype])
    assert err <= TOL[q.dtype]


def test_noalloc_matches_workspace_entry_point(based):
    """The 360M-shaped step (4 segments per head), then a smaller call with
    an initial state (3 segments), then one small enough for one segment."""
    run_pair(based, synth.FWD_CONFIGS["based360m"], state=False)
    run_pair(based, synth.FwdConfig("smaller", B=2, H=3, L=768), state=True)
    run_pair(based, synth.FwdConfig("smallest", B=1, H=2, L=200), state=False)


def test_noalloc_rejects_without_touching_memory(based):
    """Validation errors are those of based_layer_fwd (no launch)."""
    so = based.load_library()
    assert so.based_layer_fwd_noalloc(None, None, None, None, None, None, None, None, None, 1, 1, 100, 16, 64, 64,
                                      ctypes.c_float(1.0), 1, None) == -1  # BASED_ERR_NULL
    assert so.based_layer_fwd_noalloc(None, None, None, None, None, None, None, None, None, 1, 1, 100, 16, 64, 99,
                                      ctypes.c_float(1.0), 1, None) == -7  # BASED_ERR_WINDOW
