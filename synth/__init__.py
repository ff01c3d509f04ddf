"""Seeded synthetic inputs for the Based layer workloads.

This module draws random numbers and nothing else: it holds none of the
layer's arithmetic.  Both the oracle-side tests and the GPU-side tests and
benchmark take their inputs from here, so the two sides see bit-identical
q, k, v.

Recipe (the same for every workload):

* ``torch.Generator("cpu").manual_seed(seed)``; fp32 ``randn`` drawn in the
  order q, k, v (then the heavy-row selections, then decode steps);
* q and k are multiplied by ``qk_std``, v by ``v_std``;
* heavy tails: ``round(frac * rows)`` token rows of q, and independently of k,
  picked without replacement by ``randperm``, are multiplied by ``mult``;
* finally everything is cast to the workload dtype with round-to-nearest-even;
* upstream gradients dy for the backward: fp32 ``randn`` [B,H,L,dv] from a
  generator seeded with ``seed + 1_000_003`` (independent of q, k, v);
* BaseConv: x, u [B,L,D] ~ N(0,1) cast to the dtype, filter h [D,K] ~
  N(0,1)/sqrt(K) and bias [D] ~ N(0,1)/10 in fp32, drawn in that order.

The workloads stand in for the activations of the 360M / 1.3B Based models
that the pages train on the Pile (d_k = 16 feature dim, 16 heads, d_v 64/128),
which are not available here.
"""

from __future__ import annotations

import dataclasses

import torch

__all__ = ["FwdConfig", "DecodeConfig", "FWD_CONFIGS", "DECODE_CONFIG", "fwd_inputs", "decode_inputs",
           "upstream_grad", "ConvConfig", "CONV_CONFIGS", "baseconv_inputs", "decay_rates"]


@dataclasses.dataclass(frozen=True)
class FwdConfig:
    name: str
    B: int
    H: int
    L: int
    dk: int = 16
    dv: int = 64
    dtype: str = "bf16"  # "f32" or "bf16"
    qk_std: float = 0.25
    v_std: float = 1.0
    heavy_frac: float = 0.0
    heavy_mult: float = 3.0
    window: int = 64

    def replace(self, **kw) -> "FwdConfig":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    B: int
    H: int
    ctx: int
    steps: int
    dk: int = 16
    dv: int = 64
    window: int = 64
    dtype: str = "bf16"
    std: float = 1.0

    def replace(self, **kw) -> "DecodeConfig":
        return dataclasses.replace(self, **kw)


FWD_CONFIGS = {
    # tiny layer forward, fp32, q,k ~ N(0,1)/4
    "tiny": FwdConfig("tiny", B=1, H=2, L=256, dv=64, dtype="f32"),
    # 360M-shaped layer forward (d_k 16, d_v 64, 16 heads, 2k tokens)
    "based360m": FwdConfig("based360m", B=8, H=16, L=2048, dv=64),
    # 1.3B-shaped layer forward (d_v 128, 4k tokens)
    "based1p3b": FwdConfig("based1p3b", B=4, H=16, L=4096, dv=128),
    # long context with heavy-tailed scores: 1% of q rows and of k rows x3
    "long32k": FwdConfig("long32k", B=1, H=16, L=32768, dv=64, heavy_frac=0.01),
}

# 256 sequences x 16 heads, prefilled from 2048 random tokens, 1000 steps,
# q, k, v ~ N(0, 1) unscaled
DECODE_CONFIG = DecodeConfig("decode", B=256, H=16, ctx=2048, steps=1000)

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    return _DT[name]


def _heavy(x: torch.Tensor, frac: float, mult: float, g: torch.Generator) -> None:
    rows = x.view(-1, x.shape[-1])
    n = int(round(frac * rows.shape[0]))
    if n > 0:
        idx = torch.randperm(rows.shape[0], generator=g)[:n]
        rows[idx] *= mult


def fwd_inputs(cfg: FwdConfig, seed: int = 0):
    """q, k [B,H,L,dk] and v [B,H,L,dv] as contiguous CPU tensors of cfg.dtype."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(cfg.B, cfg.H, cfg.L, cfg.dk, generator=g)
    k = torch.randn(cfg.B, cfg.H, cfg.L, cfg.dk, generator=g)
    v = torch.randn(cfg.B, cfg.H, cfg.L, cfg.dv, generator=g)
    q.mul_(cfg.qk_std)
    k.mul_(cfg.qk_std)
    v.mul_(cfg.v_std)
    if cfg.heavy_frac > 0:
        _heavy(q, cfg.heavy_frac, cfg.heavy_mult, g)
        _heavy(k, cfg.heavy_frac, cfg.heavy_mult, g)
    dt = _DT[cfg.dtype]
    return q.to(dt).contiguous(), k.to(dt).contiguous(), v.to(dt).contiguous()


def decode_inputs(cfg: DecodeConfig, seed: int = 0):
    """Context (q, k, v) [B,H,ctx,.] then per-step (q, k, v) [steps,B,H,.].

    Steps are drawn after the context from the same generator, step-major,
    so a shorter ``steps`` yields a prefix of the longer run's tokens.
    """
    g = torch.Generator("cpu").manual_seed(seed)
    dt = _DT[cfg.dtype]
    ctx = []
    for d in (cfg.dk, cfg.dk, cfg.dv):
        ctx.append((torch.randn(cfg.B, cfg.H, cfg.ctx, d, generator=g) * cfg.std).to(dt).contiguous())
    qs, ks, vs = [], [], []
    for _ in range(cfg.steps):
        for out, d in ((qs, cfg.dk), (ks, cfg.dk), (vs, cfg.dv)):
            out.append(torch.randn(cfg.B, cfg.H, d, generator=g) * cfg.std)
    steps = tuple(torch.stack(s).to(dt).contiguous() for s in (qs, ks, vs))
    return tuple(ctx), steps


def upstream_grad(cfg: FwdConfig, seed: int = 0) -> torch.Tensor:
    """dy [B,H,L,dv], fp32 N(0,1): the loss gradient fed to the backward."""
    g = torch.Generator("cpu").manual_seed(seed + 1_000_003)
    return torch.randn(cfg.B, cfg.H, cfg.L, cfg.dv, generator=g).contiguous()


@dataclasses.dataclass(frozen=True)
class ConvConfig:
    name: str
    B: int
    L: int
    D: int
    K: int = 3
    dtype: str = "bf16"

    def replace(self, **kw) -> "ConvConfig":
        return dataclasses.replace(self, **kw)


CONV_CONFIGS = {
    # the 360M model's hidden states (width 1024) over the step's 8 x 2048 tokens, 3-tap filter
    "baseconv360m": ConvConfig("baseconv360m", B=8, L=2048, D=1024, K=3),
}


def baseconv_inputs(cfg: ConvConfig, seed: int = 0):
    """x, u [B,L,D] (cfg.dtype), h [D,K] and bias [D] (fp32), CPU tensors."""
    g = torch.Generator("cpu").manual_seed(seed)
    x = torch.randn(cfg.B, cfg.L, cfg.D, generator=g)
    u = torch.randn(cfg.B, cfg.L, cfg.D, generator=g)
    h = torch.randn(cfg.D, cfg.K, generator=g) / cfg.K ** 0.5
    bias = torch.randn(cfg.D, generator=g) / 10
    dt = _DT[cfg.dtype]
    return x.to(dt).contiguous(), u.to(dt).contiguous(), h.contiguous(), bias.contiguous()


def decay_rates(H: int) -> torch.Tensor:
    """Per-head state decay for the decayed variant (no draw): gamma_h =
    1 - 2^-(h + 1) cycling over h mod 8, with head 0 undecayed (gamma = 1):
    1, 0.75, 0.875, ..., 0.9921875, then again."""
    g = [1.0 if h % 8 == 0 else 1.0 - 2.0 ** -((h % 8) + 1) for h in range(H)]
    return torch.tensor(g, dtype=torch.float32)
