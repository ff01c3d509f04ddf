"""CPU-side checks of the C ABI: the library loads, exports every function
include/based.h declares, and rejects bad arguments on the host with the
documented status codes before anything reaches the GPU (no compute here)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "based.h")

import linear_attention_lm_amd as lal  # noqa: E402

ERR = dict(NULL=-1, SHAPE=-2, UNSUPPORTED=-3, DTYPE=-4, ALIGN=-5, WORKSPACE=-6, WINDOW=-7, HIP=-8, ALIAS=-9)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(based_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def so():
    return lal.load_library()


def test_every_declared_symbol_is_exported(so):
    names = declared_functions()
    assert len(names) == 20, names
    for n in names:
        assert hasattr(so, n), n


def test_header_status_codes_match():
    text = open(HEADER).read()
    for name, code in ERR.items():
        assert re.search(rf"BASED_ERR_{name}\s*=\s*{code}\b", text), name


def test_version_and_strings(so):
    assert so.based_abi_version() == 9
    for code in [0, *ERR.values(), 12345]:
        s = so.based_status_string(code)
        assert isinstance(s, bytes) and len(s) > 0


P = 0x10000  # fake, 16-byte aligned device addresses: validation never dereferences them


def fwd(so, q=P, k=2 * P, v=3 * P, y=4 * P, S_in=None, z_in=None, S_out=None, z_out=None, B=1, H=2, L=256,
        dk=16, dv=64, dt=1, ws=None, wsb=0):
    return so.based_linattn_fwd(q, k, v, y, S_in, z_in, S_out, z_out, B, H, L, dk, dv, dt, ws, wsb, None)


def test_linattn_validation(so):
    assert fwd(so, dt=2) == ERR["DTYPE"]
    assert fwd(so, B=0) == ERR["SHAPE"]
    assert fwd(so, H=-1) == ERR["SHAPE"]
    assert fwd(so, L=-5) == ERR["SHAPE"]
    assert fwd(so, dk=8) == ERR["UNSUPPORTED"]
    for dv in (0, 8, 24, 144, 256):
        assert fwd(so, dv=dv) == ERR["UNSUPPORTED"], dv
    assert fwd(so, q=None) == ERR["NULL"]
    assert fwd(so, y=None) == ERR["NULL"]
    assert fwd(so, S_in=5 * P) == ERR["NULL"]  # S_in without z_in
    assert fwd(so, z_out=5 * P) == ERR["NULL"]  # z_out without S_out
    assert fwd(so, v=3 * P + 8) == ERR["ALIGN"]
    assert fwd(so, y=1 * P) == ERR["ALIAS"]  # y overlaps q
    assert fwd(so, y=2 * P + 64) == ERR["ALIAS"]  # y overlaps k


def test_swa_validation(so):
    f = lambda **kw: so.based_swa_fwd(kw.get("q", P), kw.get("k", 2 * P), kw.get("v", 3 * P), kw.get("y", 4 * P),
                                      kw.get("B", 1), kw.get("H", 1), kw.get("L", 100), kw.get("dqk", 16),
                                      kw.get("dv", 64), kw.get("window", 64), 1.0, kw.get("dt", 1), None)
    assert f(dt=-1) == ERR["DTYPE"]
    assert f(window=0) == ERR["WINDOW"]
    assert f(window=65) == ERR["WINDOW"]
    assert f(dqk=20) == ERR["UNSUPPORTED"]
    assert f(dv=256) == ERR["UNSUPPORTED"]
    assert f(k=None) == ERR["NULL"]
    assert f(q=P + 4) == ERR["ALIGN"]
    assert f(y=3 * P) == ERR["ALIAS"]
    assert f(L=0, q=None, k=None, v=None, y=None) == 0  # nothing to do, nothing touched


def test_decode_validation(so):
    def f(**kw):
        a = dict(q=P, k=2 * P, v=3 * P, S=4 * P, z=40 * P, rk=50 * P, rv=60 * P, pos=70 * P, yl=80 * P, ys=90 * P,
                 B=2, H=2, dk=16, dv=64, window=64, dt=1)
        a.update(kw)
        return so.based_decode_step(a["q"], a["k"], a["v"], a["S"], a["z"], a["rk"], a["rv"], a["pos"], a["yl"],
                                    a["ys"], a["B"], a["H"], a["dk"], a["dv"], a["window"], 1.0, a["dt"], None)

    assert f(dt=7) == ERR["DTYPE"]
    assert f(B=0) == ERR["SHAPE"]
    assert f(dk=32) == ERR["UNSUPPORTED"]
    assert f(window=100) == ERR["WINDOW"]
    assert f(pos=None) == ERR["NULL"]
    assert f(ys=90 * P + 2) == ERR["ALIGN"]
    assert f(ys=80 * P) == ERR["ALIAS"]  # both outputs in one buffer
    assert f(S=P) == ERR["ALIAS"]  # state overlaps an input


def test_prefill_validation(so):
    f = lambda **kw: so.based_decode_prefill(kw.get("k", P), kw.get("v", 2 * P), kw.get("rk", 3 * P),
                                             kw.get("rv", 4 * P), kw.get("pos", 5 * P), 1, 1, kw.get("L", 10), 16,
                                             64, kw.get("window", 64), kw.get("dt", 0), None)
    assert f(dt=3) == ERR["DTYPE"]
    assert f(L=-1) == ERR["SHAPE"]
    assert f(window=0) == ERR["WINDOW"]
    assert f(rk=None) == ERR["NULL"]
    assert f(pos=5 * P + 1) == ERR["ALIGN"]


def test_workspace_query_is_pure(so):
    a = so.based_linattn_workspace_bytes(8, 16, 2048, 16, 64, 1)
    assert a == so.based_linattn_workspace_bytes(8, 16, 2048, 16, 64, 1)
    assert so.based_linattn_workspace_bytes(0, 16, 2048, 16, 64, 1) == 0


def test_product_path_has_no_oracle_or_fallback():
    """The package never imports the oracle and has no CPU code path."""
    pkg = os.path.join(ROOT, "linear_attention_lm_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "oracle" not in text.lower(), fn


def test_layer_validation(so):
    def f(**kw):
        a = dict(q=P, k=2 * P, v=3 * P, y_lin=4 * P, y_swa=6 * P, S_in=None, z_in=None, S_out=None, z_out=None,
                 B=1, H=1, L=100, dk=16, dv=64, window=64, scale=1.0, dt=1, ws=None, wsb=0)
        a.update(kw)
        return so.based_layer_fwd(a["q"], a["k"], a["v"], a["y_lin"], a["y_swa"], a["S_in"], a["z_in"], a["S_out"],
                                  a["z_out"], a["B"], a["H"], a["L"], a["dk"], a["dv"], a["window"], a["scale"],
                                  a["dt"], a["ws"], a["wsb"], None)
    assert f(dt=3) == ERR["DTYPE"]
    assert f(B=0) == ERR["SHAPE"]
    assert f(dk=32) == ERR["UNSUPPORTED"]
    assert f(dv=72) == ERR["UNSUPPORTED"]
    assert f(window=0) == ERR["WINDOW"] and f(window=65) == ERR["WINDOW"]
    assert f(y_swa=None) == ERR["NULL"]
    assert f(S_in=8 * P) == ERR["NULL"]
    assert f(y_swa=6 * P + 4) == ERR["ALIGN"]
    assert f(y_swa=4 * P + 256) == ERR["ALIAS"]  # the two outputs overlap
    assert f(y_lin=3 * P) == ERR["ALIAS"]        # output over v
    assert f(L=4096, B=8, H=16) == ERR["WORKSPACE"]  # segmented sizes need a workspace


def bwd_args(q=P, k=2 * P, v=3 * P, y=4 * P, dy=5 * P, dq=6 * P, dk=7 * P, dv=8 * P):
    return [q, k, v, y, dy, dq, dk, dv]


def test_linattn_bwd_validation(so):
    B, H, L = 1, 2, 100
    ws = 0x200000
    need = so.based_linattn_bwd_workspace_bytes(B, H, L, 16, 64, 1)
    assert need > 0
    call = lambda args, dk=16, dv=64, dt=1, w=ws, wb=need, L=L: so.based_linattn_bwd(
        *args, B, H, L, dk, dv, dt, w, wb, None)
    big = 0x100000  # spacing so that the fake buffers do not overlap
    ok = bwd_args(*(big * (i + 1) for i in range(8)))
    assert call(ok, dt=2) == ERR["DTYPE"]
    assert call(ok, dk=32) == ERR["UNSUPPORTED"]
    assert call(ok, dv=40) == ERR["UNSUPPORTED"]
    assert call(ok, L=0) == 0  # nothing to do
    assert call(bwd_args(*(big * (i + 1) for i in range(7)), None)) == ERR["NULL"]
    bad = list(ok)
    bad[5] = big + 8
    assert call(bad) == ERR["ALIGN"]
    alias = list(ok)
    alias[6] = alias[0]  # dk on top of q
    assert call(alias) == ERR["ALIAS"]
    assert call(ok, w=None) == ERR["WORKSPACE"]
    assert call(ok, wb=need - 1) == ERR["WORKSPACE"]
    assert call(ok, w=ok[3]) == ERR["ALIAS"]  # workspace on top of y
    assert so.based_linattn_bwd_workspace_bytes(B, H, L, 16, 64, 7) == 0


def test_swa_bwd_validation(so):
    big = 0x100000
    ok = bwd_args(*(big * (i + 1) for i in range(8)))
    call = lambda args, dqk=16, dv=64, window=64, dt=1: so.based_swa_bwd(*args, 1, 2, 100, dqk, dv, window, 1.0,
                                                                          dt, None)
    assert call(ok, dt=5) == ERR["DTYPE"]
    assert call(ok, dqk=32) == ERR["UNSUPPORTED"]
    assert call(ok, window=0) == ERR["WINDOW"]
    assert call(ok, window=65) == ERR["WINDOW"]
    out_overlap = list(ok)
    out_overlap[7] = out_overlap[5]  # dv on top of dq
    assert call(out_overlap) == ERR["ALIAS"]
    assert call(bwd_args(*(big * (i + 1) for i in range(4)), None, *(big * (i + 6) for i in range(3)))) == ERR["NULL"]


def test_baseconv_validation(so):
    big = 0x100000
    x, u, h, b, y = (big * (i + 1) for i in range(5))
    call = lambda x=x, u=u, h=h, b=b, y=y, B=2, L=100, D=64, K=3, dt=1: so.based_baseconv_fwd(
        x, u, h, b, y, B, L, D, K, dt, None)
    assert call(dt=3) == ERR["DTYPE"]
    assert call(B=0) == ERR["SHAPE"]
    assert call(D=66) == ERR["UNSUPPORTED"]
    assert call(K=0) == ERR["UNSUPPORTED"]
    assert call(K=5) == ERR["UNSUPPORTED"]
    assert call(L=0) == 0
    assert call(h=None) == ERR["NULL"]
    assert call(y=x) == ERR["ALIAS"]
    assert call(u=big + 4) == ERR["ALIGN"]


def test_decay_validation(so):
    big = 0x100000
    q, k, v, gam, y = (big * (i + 1) for i in range(5))
    need = so.based_linattn_workspace_bytes(1, 2, 5000, 16, 64, 1)
    call = lambda gam=gam, y=y, dv=64, dt=1, ws=big * 10, wsb=need: so.based_linattn_decay_fwd(
        q, k, v, gam, y, None, None, None, None, 1, 2, 5000, 16, dv, dt, ws, wsb, None)
    # fp32 and widths the matrix cores do not take are offered (the vector
    # path): such calls get as far as the later checks
    assert call(dt=0, gam=None) == ERR["NULL"]
    assert call(dv=48, y=q) == ERR["ALIAS"]
    assert call(dv=24) == ERR["UNSUPPORTED"]
    assert call(gam=None) == ERR["NULL"]
    assert call(y=q) == ERR["ALIAS"]
    assert call(y=gam) == ERR["ALIAS"]
    if need:
        assert call(ws=None) == ERR["WORKSPACE"]


def test_decode_decay_validation(so):
    big = 0x100000
    q, k, v, gam, S, z, rk, rv, pos, yl, ys = (big * (i + 1) for i in range(11))
    call = lambda gam=gam, S=S, dt=1, dv=64, win=64: so.based_decode_step_decay(
        q, k, v, gam, S, z, rk, rv, pos, yl, ys, 2, 3, 16, dv, win, 1.0, dt, None)
    assert call(gam=None) == ERR["NULL"]
    assert call(dt=5) == ERR["DTYPE"]
    assert call(dv=20) == ERR["UNSUPPORTED"]
    assert call(win=65) == ERR["WINDOW"]
    assert call(gam=S) == ERR["ALIAS"]          # gamma inside the state S


def test_decode_compact_validation(so):
    """The compact step checks the 153-row state's extent (a z just past a
    153-row S does not overlap it, one inside it does) and takes a null gamma."""
    big = 0x100000
    B, H, dv = 2, 3, 64
    S = big
    z_after = S + B * H * 153 * dv * 4
    q, k, v, rk, rv, pos, yl, ys = (big * (i + 2) * 16 for i in range(8))
    call = lambda gam=None, z=z_after, dt=1, d=dv: so.based_decode_step_compact(
        q, k, v, gam, S, z, rk, rv, pos, yl, ys, B, H, 16, d, 64, 1.0, dt, None)
    assert call(dt=3) == ERR["DTYPE"]
    assert call(d=24) == ERR["UNSUPPORTED"]
    assert call(z=z_after - 16) == ERR["ALIAS"]
    assert call(gam=S + 64) == ERR["ALIAS"]     # gamma inside the state


def test_state_conversion_validation(so):
    big = 0x1000000
    B, H, dv = 2, 3, 32
    S, z, Sc, zc = big, 2 * big, 3 * big, 4 * big
    assert so.based_state_compact(S, z, Sc, zc, 0, H, dv, None) == ERR["SHAPE"]
    assert so.based_state_compact(S, z, Sc, zc, B, H, 20, None) == ERR["UNSUPPORTED"]
    assert so.based_state_compact(S, None, Sc, zc, B, H, dv, None) == ERR["NULL"]
    assert so.based_state_compact(S + 4, z, Sc, zc, B, H, dv, None) == ERR["ALIGN"]
    assert so.based_state_compact(S, z, S + 16, zc, B, H, dv, None) == ERR["ALIAS"]
    assert so.based_state_expand(Sc, zc, S, Sc, B, H, dv, None) == ERR["ALIAS"]
    assert so.based_state_expand(Sc, zc, S, S + B * H * 273 * dv * 4 - 16, B, H, dv, None) == ERR["ALIAS"]


def test_head_extent_limit(so):
    """Each head's [L, d] block must stay under 2^31 bytes in fp32 (the
    kernels address it through 32-bit buffer offsets): a longer L is
    rejected on the host, for every entry point that takes [B,H,L,d]."""
    big = (1 << 31) // (4 * 128)  # first L whose fp32 block at d = 128 reaches 2^31 bytes
    assert fwd(so, L=big, dv=128) == ERR["SHAPE"]
    assert fwd(so, L=big - 1, dv=128, q=None) == ERR["NULL"]  # one less passes the size check
    assert fwd(so, L=2 * big, dv=64) == ERR["SHAPE"]
    assert so.based_linattn_decay_fwd(P, 2 * P, 3 * P, 5 * P, 4 * P, None, None, None, None, 1, 1, big, 16, 128, 1,
                                      None, 0, None) == ERR["SHAPE"]
    assert so.based_layer_fwd(P, 2 * P, 3 * P, 4 * P, 6 * P, None, None, None, None, 1, 1, big, 16, 128, 64,
                              ctypes.c_float(1.0), 1, None, 0, None) == ERR["SHAPE"]
    assert so.based_swa_fwd(P, 2 * P, 3 * P, 4 * P, 1, 1, big, 128, 64, 64, ctypes.c_float(1.0), 1,
                            None) == ERR["SHAPE"]
    for fn in (so.based_linattn_bwd, so.based_swa_bwd):
        if fn is so.based_linattn_bwd:
            st = fn(P, 2 * P, 3 * P, 4 * P, 5 * P, 6 * P, 7 * P, 8 * P, 1, 1, big, 16, 128, 1, None, 0, None)
        else:
            st = fn(P, 2 * P, 3 * P, 4 * P, 5 * P, 6 * P, 7 * P, 8 * P, 1, 1, big, 16, 128, 64,
                    ctypes.c_float(1.0), 1, None)
        assert st == ERR["SHAPE"]


def test_state_alias_rules(so):
    """S_out may be S_in itself (in-place update) but may not overlap it
    otherwise; z_out likewise; S_out may not overlap z_in, the inputs or
    the workspace.  (Exact aliasing is exercised on the GPU.)"""
    B, H, dv = 1, 2, 64
    nS = B * H * 273 * dv * 4
    S0, z0 = 100 * P, 200 * P
    ws_need = so.based_linattn_workspace_bytes(B, H, 256, 16, dv, 1)
    assert ws_need == 0  # L = 256 on 2 heads: one segment, no workspace
    assert fwd(so, S_in=S0, z_in=z0, S_out=S0 + 16 * 64, z_out=300 * P) == ERR["ALIAS"]  # shifted S_out
    assert fwd(so, S_in=S0, z_in=z0, S_out=300 * P, z_out=z0 + 16) == ERR["ALIAS"]  # shifted z_out
    assert fwd(so, S_in=S0, z_in=z0, S_out=z0, z_out=300 * P) == ERR["ALIAS"]  # S_out over z_in
    assert fwd(so, S_in=S0, z_in=z0, S_out=300 * P, z_out=S0 + nS - 64) == ERR["ALIAS"]  # z_out over S_in
    assert fwd(so, S_out=2 * P, z_out=300 * P) == ERR["ALIAS"]  # S_out over k
    assert fwd(so, S_out=300 * P, z_out=4 * P) == ERR["ALIAS"]  # z_out over y
    # a workspace that overlaps a state or an input (L = 4096 on 2 heads
    # needs one); buffers 1 GiB apart so that only the named pair overlaps
    G = 1 << 30
    need = so.based_linattn_workspace_bytes(B, H, 4096, 16, dv, 1)
    assert need > 0
    far = dict(q=G, k=2 * G, v=3 * G, y=4 * G, L=4096, wsb=need)
    assert fwd(so, S_in=5 * G, z_in=6 * G, ws=5 * G + 64, **far) == ERR["ALIAS"]
    assert fwd(so, S_out=5 * G, z_out=6 * G, ws=6 * G - 64, **far) == ERR["ALIAS"]
    assert fwd(so, ws=2 * G + 128, **far) == ERR["ALIAS"]  # workspace over k


def test_decay_layer_and_backward_validation(so):
    """based_layer_decay_fwd and based_linattn_decay_bwd: a null gamma, gamma
    under an output, a short workspace, an unsupported width."""
    G = 1 << 28
    q, k, v, gam, y1, y2 = (G * (i + 1) for i in range(6))
    lay = lambda gam=gam, y1=y1, dv=64, win=64: so.based_layer_decay_fwd(
        q, k, v, gam, y1, y2, None, None, None, None, 1, 2, 300, 16, dv, win, ctypes.c_float(1.0), 1, None, 0, None)
    assert lay(gam=None) == ERR["NULL"]
    assert lay(y1=gam) == ERR["ALIAS"]
    assert lay(win=0) == ERR["WINDOW"]
    assert lay(dv=40) == ERR["UNSUPPORTED"]
    y, dy, dq, dk, dv_ = (G * (i + 7) for i in range(5))
    bwd = lambda gam=gam, dq=dq, ws=G * 13, wsb=2 * 2 * 300 * 4, dt=1: so.based_linattn_decay_bwd(
        q, k, v, gam, y, dy, dq, dk, dv_, 1, 2, 300, 16, 64, dt, ws, wsb, None)
    assert bwd(gam=None) == ERR["NULL"]
    assert bwd(dq=gam) == ERR["ALIAS"]
    assert bwd(wsb=100) == ERR["WORKSPACE"]
    assert bwd(ws=None) == ERR["WORKSPACE"]
    assert bwd(ws=gam) == ERR["ALIAS"]
    assert bwd(dt=5) == ERR["DTYPE"]
