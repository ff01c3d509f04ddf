"""GPU parity of the BaseConv gate (based_baseconv_fwd) against the oracle's
baseconv on the same seeded inputs: per-row (one D-vector per position)
infinity-norm relative error, fp32 1e-5 / bf16 2e-3 (the arithmetic is fp32
on exactly converted inputs either way)."""

import pytest
import torch

import synth
from oracle import based_oracle as O
from parity_util import TOL, report, rowinf_rel, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
SMALL = synth.ConvConfig("small", B=2, L=300, D=64, K=3)


def check(based, cfg, bias=True, batches=None):
    x, u, h, b = synth.baseconv_inputs(cfg, 0)
    say(f"baseconv {cfg.name} B{cfg.B} L{cfg.L} D{cfg.D} K{cfg.K} {cfg.dtype} bias={bias}")
    y = based.baseconv_fwd(x.to(DEV), u.to(DEV), h.to(DEV), b.to(DEV) if bias else None)
    torch.cuda.synchronize()
    sel = list(range(cfg.B)) if batches is None else batches
    ref = O.baseconv(x[sel], u[sel], h, b if bias else None)
    err = rowinf_rel(y[sel], ref)
    report(f"baseconv {cfg.name}", err, TOL[x.dtype])
    assert err <= TOL[x.dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("L", [1, 2, 15, 16, 17, 300])
def test_baseconv_lengths(based, dtype, L):
    check(based, SMALL.replace(L=L, dtype=dtype, name=f"L{L}"))


@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("D", [4, 60, 1028])
def test_baseconv_taps_and_widths(based, K, D):
    """Widths that leave part of a 1024-channel block empty, and every filter length."""
    check(based, SMALL.replace(L=70, D=D, K=K, name=f"D{D}K{K}"))


def test_baseconv_no_bias(based):
    check(based, SMALL.replace(name="nobias"), bias=False)


def test_baseconv_full_size(based):
    check(based, synth.CONV_CONFIGS["baseconv360m"], batches=[0, 7])


def test_baseconv_empty(based):
    x = torch.zeros(2, 0, 8, device=DEV, dtype=torch.bfloat16)
    y = based.baseconv_fwd(x, x, torch.zeros(8, 3, device=DEV))
    assert y.shape == (2, 0, 8)
