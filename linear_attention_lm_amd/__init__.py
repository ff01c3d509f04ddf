"""Based sequence-mixing layer on AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI in ``include/based.h`` (``libbased.so``,
built in-tree by ``python -m linear_attention_lm_amd.build``).  The wrappers
only check and marshal arguments; every step of the computation runs in the
library's HIP kernels on the caller's current HIP stream.  PyTorch provides
device memory and streams.

The library is loaded on first use (so that the build script in this package
can run before it exists); if it is missing, that first call fails loudly --
there is no CPU fallback.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

__all__ = [
    "LIB_PATH", "lib", "abi_version", "linattn_fwd", "linattn_workspace_bytes", "swa_fwd", "layer_fwd",
    "layer_decay_fwd", "linattn_decay_bwd",
    "linattn_bwd", "linattn_bwd_workspace_bytes", "swa_bwd", "baseconv_fwd", "linattn_decay_fwd",
    "DecodeState", "decode_init", "decode_prefill", "decode_step", "BasedError", "DPHI", "DK",
]

# The in-tree build; BASED_LIB_PATH names another build of the same ABI (the
# tests load the sanitized host-only build of the argument checks this way).
LIB_PATH = os.environ.get("BASED_LIB_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbased.so")
DK = 16
DPHI = 273
DCMP = 153  # compact decode state rows: constant, 16 linear, 136 unordered pairs
F32, BF16 = 0, 1

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_SIGNATURES = {
    "based_abi_version": (_i, []),
    "based_status_string": (ctypes.c_char_p, [_i]),
    "based_linattn_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "based_linattn_fwd": (_i, [_vp] * 8 + [_i] * 6 + [_vp, _sz, _vp]),
    "based_swa_fwd": (_i, [_vp] * 4 + [_i] * 6 + [_f, _i, _vp]),
    "based_layer_fwd": (_i, [_vp] * 9 + [_i] * 6 + [_f, _i, _vp, _sz, _vp]),
    "based_layer_fwd_noalloc": (_i, [_vp] * 9 + [_i] * 6 + [_f, _i, _vp]),
    "based_decode_prefill": (_i, [_vp] * 5 + [_i] * 7 + [_vp]),
    "based_decode_step": (_i, [_vp] * 10 + [_i] * 5 + [_f, _i, _vp]),
    "based_linattn_bwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "based_linattn_bwd": (_i, [_vp] * 8 + [_i] * 6 + [_vp, _sz, _vp]),
    "based_swa_bwd": (_i, [_vp] * 8 + [_i] * 6 + [_f, _i, _vp]),
    "based_baseconv_fwd": (_i, [_vp] * 5 + [_i] * 5 + [_vp]),
    "based_linattn_decay_fwd": (_i, [_vp] * 9 + [_i] * 6 + [_vp, _sz, _vp]),
    "based_linattn_decay_bwd": (_i, [_vp] * 9 + [_i] * 6 + [_vp, _sz, _vp]),
    "based_layer_decay_fwd": (_i, [_vp] * 10 + [_i] * 6 + [_f, _i, _vp, _sz, _vp]),
    "based_decode_step_decay": (_i, [_vp] * 11 + [_i] * 5 + [_f, _i, _vp]),
    "based_decode_step_compact": (_i, [_vp] * 11 + [_i] * 5 + [_f, _i, _vp]),
    "based_state_compact": (_i, [_vp] * 4 + [_i] * 3 + [_vp]),
    "based_state_expand": (_i, [_vp] * 4 + [_i] * 3 + [_vp]),
}


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build the HIP library first (python -m linear_attention_lm_amd.build)")
    so = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        if hasattr(so, name):  # a host-only build lacks the entry points with device code
            fn = getattr(so, name)
            fn.restype, fn.argtypes = res, args
    return so


_LIB = None


def _lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        _LIB = load_library()
    return _LIB


def __getattr__(name):
    if name == "lib":
        return _lib()
    raise AttributeError(name)


class BasedError(RuntimeError):
    def __init__(self, code: int):
        self.code = code
        super().__init__(f"based: {_lib().based_status_string(code).decode()} (status {code})")


def _check(code: int) -> None:
    if code != 0:
        raise BasedError(code)


def abi_version() -> int:
    return _lib().based_abi_version()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"q/k/v must be float32 or bfloat16, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors must be on one device")
    return dev


def linattn_workspace_bytes(B, H, L, dv, dtype=torch.bfloat16) -> int:
    return _lib().based_linattn_workspace_bytes(B, H, L, DK, dv, BF16 if dtype == torch.bfloat16 else F32)


def linattn_fwd(q, k, v, S_in=None, z_in=None, *, return_state=False, y=None, S_out=None, z_out=None,
                workspace=None):
    """Causal Taylor linear attention.  q, k [B,H,L,16], v [B,H,L,dv] (fp32 or
    bf16, same dtype).  Returns y [B,H,L,dv] fp32, or (y, S, z) with the final
    state [B,H,273,dv], [B,H,273] when ``return_state``."""
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k must be [B,H,L,16] and v [B,H,L,dv] of one dtype")
    _dev(q, k, v, S_in, z_in, y, S_out, z_out, workspace)
    if y is None:
        y = torch.empty(B, H, L, dv, device=q.device, dtype=torch.float32)
    if return_state and S_out is None:
        S_out = torch.empty(B, H, DPHI, dv, device=q.device, dtype=torch.float32)
        z_out = torch.empty(B, H, DPHI, device=q.device, dtype=torch.float32)
    dt = _dtype_code(q)
    need = _lib().based_linattn_workspace_bytes(B, H, L, dk, dv, dt)
    if need and workspace is None:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib().based_linattn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(y), _ptr(S_in), _ptr(z_in), _ptr(S_out),
                                 _ptr(z_out), B, H, L, dk, dv, dt, _ptr(workspace), wbytes, _stream()))
    return (y, S_out, z_out) if (return_state or S_out is not None) else y


def linattn_decay_fwd(q, k, v, gamma, S_in=None, z_in=None, *, return_state=False, y=None, S_out=None,
                      z_out=None, workspace=None):
    """Causal Taylor linear attention with a per-head state decay gamma [H]
    (fp32, taken clamped to [0, 1]): S_i = gamma S_{i-1} + phi(k_i) v_i^T, likewise z.
    Either dtype, d_v in {16, ..., 128}.  Returns y, or (y, S, z)."""
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k must be [B,H,L,16] and v [B,H,L,dv] of one dtype")
    if gamma.shape != (H,) or gamma.dtype != torch.float32:
        raise ValueError("gamma must be fp32 [H]")
    _dev(q, k, v, gamma, S_in, z_in, y, S_out, z_out, workspace)
    if y is None:
        y = torch.empty(B, H, L, dv, device=q.device, dtype=torch.float32)
    if return_state and S_out is None:
        S_out = torch.empty(B, H, DPHI, dv, device=q.device, dtype=torch.float32)
        z_out = torch.empty(B, H, DPHI, device=q.device, dtype=torch.float32)
    dt = _dtype_code(q)
    need = _lib().based_linattn_workspace_bytes(B, H, L, dk, dv, dt)
    if need and workspace is None:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib().based_linattn_decay_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(y), _ptr(S_in), _ptr(z_in),
                                       _ptr(S_out), _ptr(z_out), B, H, L, dk, dv, dt, _ptr(workspace), wbytes,
                                       _stream()))
    return (y, S_out, z_out) if (return_state or S_out is not None) else y


def swa_fwd(q, k, v, window: int = 64, scale: float = 1.0, *, y=None):
    """Causal sliding-window softmax attention over ``window`` positions."""
    B, H, L, dqk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k must be [B,H,L,d] and v [B,H,L,dv] of one dtype")
    _dev(q, k, v, y)
    if y is None:
        y = torch.empty(B, H, L, dv, device=q.device, dtype=torch.float32)
    _check(_lib().based_swa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(y), B, H, L, dqk, dv, window, float(scale),
                             _dtype_code(q), _stream()))
    return y


def layer_decay_fwd(q, k, v, gamma, window: int = 64, scale: float = 1.0, S_in=None, z_in=None, *,
                    return_state=False, y_lin=None, y_swa=None, S_out=None, z_out=None, workspace=None):
    """:func:`layer_fwd` with the linear attention's state decayed per head
    by gamma [H] (fp32), as in :func:`linattn_decay_fwd`; the window
    attention has no decay.  Returns (y_lin, y_swa), plus (S, z) when
    ``return_state``."""
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k must be [B,H,L,16] and v [B,H,L,dv] of one dtype")
    if gamma.shape != (H,) or gamma.dtype != torch.float32:
        raise ValueError("gamma must be fp32 [H]")
    _dev(q, k, v, gamma, S_in, z_in, y_lin, y_swa, S_out, z_out, workspace)
    if y_lin is None:
        y_lin = torch.empty(B, H, L, dv, device=q.device, dtype=torch.float32)
    if y_swa is None:
        y_swa = torch.empty(B, H, L, dv, device=q.device, dtype=torch.float32)
    if return_state and S_out is None:
        S_out = torch.empty(B, H, DPHI, dv, device=q.device, dtype=torch.float32)
        z_out = torch.empty(B, H, DPHI, device=q.device, dtype=torch.float32)
    dt = _dtype_code(q)
    need = _lib().based_linattn_workspace_bytes(B, H, L, dk, dv, dt)
    if need and workspace is None:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib().based_layer_decay_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(y_lin), _ptr(y_swa),
                                        _ptr(S_in), _ptr(z_in), _ptr(S_out), _ptr(z_out), B, H, L, dk, dv, window,
                                        float(scale), dt, _ptr(workspace), wbytes, _stream()))
    if return_state or S_out is not None:
        return y_lin, y_swa, S_out, z_out
    return y_lin, y_swa


def layer_fwd(q, k, v, window: int = 64, scale: float = 1.0, S_in=None, z_in=None, *, return_state=False,
              y_lin=None, y_swa=None, S_out=None, z_out=None, workspace=None):
    """Both attentions of the layer over the same q, k [B,H,L,16], v [B,H,L,dv]
    in one pass: returns (y_lin, y_swa), plus the final linear-attention state
    (S, z) when ``return_state`` -- the outputs of :func:`linattn_fwd` and of
    :func:`swa_fwd` with the same arguments."""
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k must be [B,H,L,16] and v [B,H,L,dv] of one dtype")
    _dev(q, k, v, S_in, z_in, y_lin, y_swa, S_out, z_out, workspace)
    if y_lin is None:
        y_lin = torch.empty(B, H, L, dv, device=q.device, dtype=torch.float32)
    if y_swa is None:
        y_swa = torch.empty(B, H, L, dv, device=q.device, dtype=torch.float32)
    if return_state and S_out is None:
        S_out = torch.empty(B, H, DPHI, dv, device=q.device, dtype=torch.float32)
        z_out = torch.empty(B, H, DPHI, device=q.device, dtype=torch.float32)
    dt = _dtype_code(q)
    need = _lib().based_linattn_workspace_bytes(B, H, L, dk, dv, dt)
    if need and workspace is None:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib().based_layer_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(y_lin), _ptr(y_swa), _ptr(S_in), _ptr(z_in),
                                  _ptr(S_out), _ptr(z_out), B, H, L, dk, dv, window, float(scale), dt,
                                  _ptr(workspace), wbytes, _stream()))
    if return_state or S_out is not None:
        return y_lin, y_swa, S_out, z_out
    return y_lin, y_swa


def layer_fwd_noalloc(q, k, v, window: int = 64, scale: float = 1.0, S_in=None, z_in=None, *, y_lin, y_swa,
                      S_out=None, z_out=None):
    """:func:`layer_fwd` through based_layer_fwd_noalloc: no workspace and no
    allocation -- the caller passes every output (y_lin, y_swa and, to get
    the final state, S_out / z_out); the segment records live in the
    library's static device array (calls overlapping on one GPU race)."""
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k must be [B,H,L,16] and v [B,H,L,dv] of one dtype")
    _dev(q, k, v, S_in, z_in, y_lin, y_swa, S_out, z_out)
    _check(_lib().based_layer_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(y_lin), _ptr(y_swa), _ptr(S_in),
                                          _ptr(z_in), _ptr(S_out), _ptr(z_out), B, H, L, dk, dv, window,
                                          float(scale), _dtype_code(q), _stream()))
    return y_lin, y_swa


def _grads_out(q, k, v, dq, dk, dv):
    mk = lambda t, like: torch.empty(like.shape, device=like.device, dtype=torch.float32) if t is None else t
    return mk(dq, q), mk(dk, k), mk(dv, v)


def _check_bwd_args(q, k, v, y, dy):
    if k.shape != q.shape or v.shape[:3] != q.shape[:3] or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k must be [B,H,L,16] and v [B,H,L,dv] of one dtype")
    if y.shape != v.shape or dy.shape != v.shape or y.dtype != torch.float32 or dy.dtype != torch.float32:
        raise ValueError("y and dy must be fp32 shaped like v")


def linattn_bwd_workspace_bytes(B, H, L, dv, dtype=torch.bfloat16) -> int:
    return _lib().based_linattn_bwd_workspace_bytes(B, H, L, DK, dv, BF16 if dtype == torch.bfloat16 else F32)


def linattn_bwd(q, k, v, y, dy, *, dq=None, dk=None, dv=None, workspace=None):
    """Gradients (dq, dk, dv), fp32, of :func:`linattn_fwd`'s output y (zero
    initial state) for the upstream gradient dy (fp32, shaped like y)."""
    _check_bwd_args(q, k, v, y, dy)
    B, H, L, dk_ = q.shape
    dvw = v.shape[-1]
    _dev(q, k, v, y, dy, dq, dk, dv, workspace)
    dq, dk, dv = _grads_out(q, k, v, dq, dk, dv)
    dt = _dtype_code(q)
    need = _lib().based_linattn_bwd_workspace_bytes(B, H, L, dk_, dvw, dt)
    if need and workspace is None:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib().based_linattn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(y), _ptr(dy), _ptr(dq), _ptr(dk), _ptr(dv),
                                 B, H, L, dk_, dvw, dt, _ptr(workspace), wbytes, _stream()))
    return dq, dk, dv


def linattn_decay_bwd(q, k, v, gamma, y, dy, *, dq=None, dk=None, dv=None, workspace=None):
    """Gradients (dq, dk, dv), fp32, of :func:`linattn_decay_fwd`'s output y
    (zero initial state, per-head decay gamma [H] fp32) for the upstream
    gradient dy.  The default workspace is
    :func:`linattn_bwd_workspace_bytes` (bf16 with d_v in {32, 64, 96, 128}
    then takes the matrix-core passes); one of 2*B*H*L*4 bytes selects the
    fp32 vector form."""
    _check_bwd_args(q, k, v, y, dy)
    B, H, L, dk_ = q.shape
    dvw = v.shape[-1]
    if gamma.shape != (H,) or gamma.dtype != torch.float32:
        raise ValueError("gamma must be fp32 [H]")
    _dev(q, k, v, gamma, y, dy, dq, dk, dv, workspace)
    dq, dk, dv = _grads_out(q, k, v, dq, dk, dv)
    if workspace is None:
        need = max(2 * B * H * L * 4, linattn_bwd_workspace_bytes(B, H, L, dvw, q.dtype), 1)
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    wbytes = workspace.numel() * workspace.element_size()
    _check(_lib().based_linattn_decay_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(y), _ptr(dy), _ptr(dq),
                                       _ptr(dk), _ptr(dv), B, H, L, dk_, dvw, _dtype_code(q), _ptr(workspace), wbytes,
                                       _stream()))
    return dq, dk, dv


def swa_bwd(q, k, v, y, dy, window: int = 64, scale: float = 1.0, *, dq=None, dk=None, dv=None):
    """Gradients (dq, dk, dv), fp32, of :func:`swa_fwd`'s output y (d_qk = 16)
    for the upstream gradient dy."""
    _check_bwd_args(q, k, v, y, dy)
    B, H, L, dqk = q.shape
    _dev(q, k, v, y, dy, dq, dk, dv)
    dq, dk, dv = _grads_out(q, k, v, dq, dk, dv)
    _check(_lib().based_swa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(y), _ptr(dy), _ptr(dq), _ptr(dk), _ptr(dv), B, H,
                             L, dqk, v.shape[-1], window, float(scale), _dtype_code(q), _stream()))
    return dq, dk, dv


def baseconv_fwd(x, u, h, bias=None, *, y=None):
    """BaseConv gate y = u * (bias + causal depthwise conv of x with h):
    x, u [B,L,D] (fp32 or bf16, same dtype; u = linear(x) from the caller),
    h [D,K] fp32 (tap s on x_{t-s}), bias [D] fp32 or None.  Returns y
    [B,L,D] fp32."""
    if x.dim() != 3 or u.shape != x.shape or u.dtype != x.dtype:
        raise ValueError("x and u must be [B,L,D] of one dtype")
    B, L, D = x.shape
    if h.dim() != 2 or h.shape[0] != D or h.dtype != torch.float32:
        raise ValueError("h must be fp32 [D,K]")
    if bias is not None and (bias.shape != (D,) or bias.dtype != torch.float32):
        raise ValueError("bias must be fp32 [D]")
    _dev(x, u, h, bias, y)
    if y is None:
        y = torch.empty(B, L, D, device=x.device, dtype=torch.float32)
    _check(_lib().based_baseconv_fwd(_ptr(x), _ptr(u), _ptr(h), _ptr(bias), _ptr(y), B, L, D, h.shape[1],
                                  _dtype_code(x), _stream()))
    return y


@dataclass
class DecodeState:
    """Caller-owned generation state: S [B,H,273,dv] fp32, z [B,H,273] fp32,
    ring_k [B,H,W,16], ring_v [B,H,W,dv] (input dtype), pos [B] int32.  With
    ``compact`` the state has one row per unordered feature pair: S
    [B,H,153,dv], z [B,H,153] (see :func:`state_compact`)."""

    S: torch.Tensor
    z: torch.Tensor
    ring_k: torch.Tensor
    ring_v: torch.Tensor
    pos: torch.Tensor
    compact: bool = False

    @property
    def window(self) -> int:
        return self.ring_k.shape[2]


def decode_prefill(k, v, state: DecodeState) -> None:
    """Fill the ring buffers of ``state`` from a context k, v [B,H,L,.] and set pos = L."""
    B, H, L, dk = k.shape
    _dev(k, v, state.ring_k, state.ring_v, state.pos)
    _check(_lib().based_decode_prefill(_ptr(k), _ptr(v), _ptr(state.ring_k), _ptr(state.ring_v), _ptr(state.pos),
                                    B, H, L, dk, v.shape[-1], state.window, _dtype_code(k), _stream()))


def decode_init(q, k, v, window: int = 64, gamma=None, compact: bool = False):
    """Consume a context (q, k, v [B,H,L,.]): returns (y_lin, y_swa, state)
    where the outputs are the context's own layer outputs and ``state`` is
    ready for :func:`decode_step` at position L.  With a per-head decay gamma
    [H] the linear attention is the decayed one (then continue with
    decode_step(..., gamma=gamma)).  ``compact``: the state in the compact
    layout (one row per unordered feature pair)."""
    B, H, L, _ = k.shape
    dv = v.shape[-1]
    if gamma is None:
        y_lin, y_swa, S, z = layer_fwd(q, k, v, window, return_state=True)
    else:
        y_lin, S, z = linattn_decay_fwd(q, k, v, gamma, return_state=True)
        y_swa = swa_fwd(q, k, v, window)
    if compact:
        S, z = state_compact(S, z)
    st = DecodeState(S, z, torch.zeros(B, H, window, DK, device=k.device, dtype=k.dtype),
                     torch.zeros(B, H, window, dv, device=k.device, dtype=k.dtype),
                     torch.zeros(B, device=k.device, dtype=torch.int32), compact)
    decode_prefill(k, v, st)
    return y_lin, y_swa, st


def decode_step(state: DecodeState, q, k, v, scale: float = 1.0, *, y_lin=None, y_swa=None, gamma=None):
    """One token per sequence: q, k [B,H,16], v [B,H,dv].  Updates ``state`` in
    place (including pos += 1) and returns (y_lin, y_swa) [B,H,dv] fp32.  With
    gamma (fp32 [H]) the state decays: S <- gamma S + phi(k) v^T, likewise z."""
    B, H, dk = q.shape
    dv = v.shape[-1]
    if gamma is not None and (gamma.shape != (H,) or gamma.dtype != torch.float32):
        raise ValueError("gamma must be fp32 [H]")
    _dev(q, k, v, state.S, state.z, state.ring_k, state.ring_v, state.pos, y_lin, y_swa, gamma)
    if y_lin is None:
        y_lin = torch.empty(B, H, dv, device=q.device, dtype=torch.float32)
    if y_swa is None:
        y_swa = torch.empty(B, H, dv, device=q.device, dtype=torch.float32)
    common = (_ptr(state.S), _ptr(state.z), _ptr(state.ring_k), _ptr(state.ring_v), _ptr(state.pos), _ptr(y_lin),
              _ptr(y_swa), B, H, dk, dv, state.window, float(scale), _dtype_code(q), _stream())
    if state.compact:
        _check(_lib().based_decode_step_compact(_ptr(q), _ptr(k), _ptr(v), _ptr(gamma), *common))
    elif gamma is None:
        _check(_lib().based_decode_step(_ptr(q), _ptr(k), _ptr(v), *common))
    else:
        _check(_lib().based_decode_step_decay(_ptr(q), _ptr(k), _ptr(v), _ptr(gamma), *common))
    return y_lin, y_swa


def state_compact(S, z, *, Sc=None, zc=None):
    """A state S [B,H,273,dv], z [B,H,273] (fp32) in the compact layout:
    Sc [B,H,153,dv], zc [B,H,153] -- rows 0..16 as in S, then for a <= b the
    pair row S[(a,b)] + S[(b,a)] (S[(a,a)] on the diagonal)."""
    B, H, _, dv = S.shape
    _dev(S, z, Sc, zc)
    Sc = torch.empty(B, H, DCMP, dv, device=S.device, dtype=torch.float32) if Sc is None else Sc
    zc = torch.empty(B, H, DCMP, device=S.device, dtype=torch.float32) if zc is None else zc
    _check(_lib().based_state_compact(_ptr(S), _ptr(z), _ptr(Sc), _ptr(zc), B, H, dv, _stream()))
    return Sc, zc


def state_expand(Sc, zc, *, S=None, z=None):
    """The 273-row state of a compact one: each ordered pair row gets half its
    pair row (the diagonal as is)."""
    B, H, _, dv = Sc.shape
    _dev(Sc, zc, S, z)
    S = torch.empty(B, H, DPHI, dv, device=Sc.device, dtype=torch.float32) if S is None else S
    z = torch.empty(B, H, DPHI, device=Sc.device, dtype=torch.float32) if z is None else z
    _check(_lib().based_state_expand(_ptr(Sc), _ptr(zc), _ptr(S), _ptr(z), B, H, dv, _stream()))
    return S, z
