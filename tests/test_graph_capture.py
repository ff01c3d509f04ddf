"""Forward calls captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.

The chunked linear attention keeps segment records in its workspace (or, for
based_layer_fwd_noalloc, in the library's static array) between its state-only
pass and its main pass; a replayed graph reuses the same workspace with new
inputs.  Each replay (new inputs copied in, eager work and a synchronisation
between replays) must give exactly what an eager call gives on the same
inputs, and the first replay's sampled heads must match the oracle."""

import pytest
import torch

import synth
from oracle import based_oracle as O
from parity_util import TOL, report, rowinf_rel, say

pytestmark = pytest.mark.gpu
DEV = "cuda"

# 128 heads of 1024 positions: four segments per head (three records summed
# by the main pass)
CFG = synth.FwdConfig("graph", B=4, H=32, L=1024, dv=64)


def _call(based, op, q, k, v, gam, y1, y2, ws):
    if op == "layer":
        based.layer_fwd(q, k, v, 64, y_lin=y1, y_swa=y2, workspace=ws)
    elif op == "layer_noalloc":
        based.layer_fwd_noalloc(q, k, v, 64, y_lin=y1, y_swa=y2)
    elif op == "linattn":
        based.linattn_fwd(q, k, v, y=y1, workspace=ws)
    else:
        based.linattn_decay_fwd(q, k, v, gam, y=y1, workspace=ws)


@pytest.mark.parametrize("op", ["layer", "layer_noalloc", "linattn", "decay"])
def test_graph_replay_matches_eager(based, op):
    cfg = CFG
    B, H, L, dv = cfg.B, cfg.H, cfg.L, cfg.dv
    say(f"graph capture {op} B{B} H{H} L{L} dv{dv}")
    sets = [[t.to(DEV) for t in synth.fwd_inputs(cfg, seed)] for seed in (1, 2, 3)]
    q, k, v = (torch.empty_like(t) for t in sets[0])
    gam = synth.decay_rates(H).to(DEV)
    y1 = torch.empty(B, H, L, dv, device=DEV)
    y2 = torch.empty(B, H, L, dv, device=DEV)
    ws = torch.empty(max(1, based.linattn_workspace_bytes(B, H, L, dv)), dtype=torch.uint8, device=DEV)
    run = lambda: _call(based, op, q, k, v, gam, y1, y2, ws)

    # eager results (one launch) for each input set
    refs = []
    for s in sets:
        for dst, src in zip((q, k, v), s):
            dst.copy_(src)
        run()
        refs.append((y1.clone(), y2.clone()))
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()

    first = None
    for rep in range(2):
        for i, s in enumerate(sets):
            for dst, src in zip((q, k, v), s):
                dst.copy_(src)
            y1.fill_(float("nan"))
            y2.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            got = (y1.clone(), y2.clone())
            if first is None:
                first = got[0]
            # the same kernels on the same inputs: bitwise the eager result
            assert torch.equal(got[0], refs[i][0])
            if op.startswith("layer"):
                assert torch.equal(got[1], refs[i][1])
            # eager work between replays, on other buffers
            e1, e2 = torch.empty_like(y1), torch.empty_like(y2)
            based.layer_fwd(*sets[(i + 1) % 3], 64, y_lin=e1, y_swa=e2)
            torch.cuda.synchronize()

    # the captured form against the oracle on two sampled heads of input set 1
    qc, kc, vc = synth.fwd_inputs(cfg, 1)
    heads = [(0, 0), (B - 1, H - 1)]
    bi, hi = [b for b, _ in heads], [h for _, h in heads]
    if op == "decay":
        y_ref = O.linattn_decay_recurrent(qc[bi, hi], kc[bi, hi], vc[bi, hi],
                                          synth.decay_rates(H).numpy()[hi])[0]
    else:
        y_ref = O.linattn_chunked(qc[bi, hi], kc[bi, hi], vc[bi, hi], 64)[0]
    err = rowinf_rel(first[bi, hi], y_ref)
    report(f"graph {op} first replay vs oracle", err, TOL[qc.dtype])
    assert err <= TOL[qc.dtype]
