"""Pins for the fp64 oracle: closed forms, invariants, textbook special cases,
SciPy's softmax, brute force and hand-worked fixtures.  None of these re-types
the oracle's own formulas; each is chosen so that a plausible slip (a dropped
term, a wrong sign, an off-by-one in the causal mask or the window, a wrong
feature scale, a transposed operand) fails at least one of them."""

import json
import os

import numpy as np
import pytest
import scipy.special

from oracle import based_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


def rand(*shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def e(axis, d=16):
    x = np.zeros(d)
    x[axis] = 1.0
    return x


# ---------------------------------------------------------------- feature map
def test_phi_shape_and_layout():
    x = rand(16)
    p = O.phi(x)
    assert p.shape == (273,)
    assert p[0] == 1.0
    np.testing.assert_array_equal(p[1:17], x)
    # quadratic block: index 17 + 16 a + b holds x_a x_b / sqrt 2
    for a, b in [(0, 0), (0, 15), (15, 0), (3, 7), (7, 3), (15, 15)]:
        assert p[17 + 16 * a + b] == pytest.approx(x[a] * x[b] / np.sqrt(2), rel=1e-15)


def test_phi_dot_is_taylor_closed_form():
    """phi(q).phi(k) = 1 + s + s^2/2 with s = q.k (blog pseudocode, last line)."""
    for _ in range(50):
        q, k = rand(16, scale=0.7), rand(16, scale=0.7)
        s = float(q @ k)
        got = float(O.phi(q) @ O.phi(k))
        assert got == pytest.approx(1 + s + s * s / 2, rel=1e-14)


@pytest.mark.parametrize(
    "q,k,want",
    [
        (np.zeros(16), rand(16), 1.0),  # q = 0 -> only the constant feature
        (e(0), e(0), 2.5),  # s = 1
        (e(0), -e(0), 0.5),  # s = -1: the minimum of 1 + s + s^2/2
        (e(0) + e(5), e(0) + e(5), 5.0),  # s = 2
        (e(2), e(9), 1.0),  # orthogonal
    ],
)
def test_phi_special_values(q, k, want):
    assert float(O.phi(q) @ O.phi(k)) == pytest.approx(want, rel=1e-15)


def test_taylor_kernel_lower_bound():
    s = np.linspace(-10, 10, 2001)
    w = O.taylor_kernel(s)
    assert w.min() == pytest.approx(0.5)
    assert s[np.argmin(w)] == pytest.approx(-1.0)
    np.testing.assert_allclose(w, ((1 + s) ** 2 + 1) / 2, rtol=1e-14)


# ------------------------------------------------------- linear attention forms
def _tiny(B=2, H=3, L=37, dv=5, s=0.4):
    return rand(B, H, L, 16, scale=s), rand(B, H, L, 16, scale=s), rand(B, H, L, dv)


def test_golden_hand_example():
    g = json.load(open(os.path.join(GOLD, "linattn_hand.json")))
    q = np.array([e(0) * a for a in g["q_axis0"]])[None, None]
    k = np.array([e(0) * a for a in g["k_axis0"]])[None, None]
    v = np.array(g["v"])[None, None]
    for kern in ("features", "taylor"):
        y, den = O.linattn_quadratic(q, k, v, kernel=kern)
        np.testing.assert_allclose(y[0, 0], g["y"], rtol=1e-15, atol=1e-15)
        np.testing.assert_allclose(den[0, 0], g["den"], rtol=1e-15)
    y, den, S, z = O.linattn_recurrent(q, k, v)
    np.testing.assert_allclose(y[0, 0], g["y"], rtol=1e-15, atol=1e-15)
    for row, val in g["S_rows"].items():
        np.testing.assert_allclose(S[0, 0, int(row)], val, rtol=1e-15)
    for row, val in g["z_rows"].items():
        assert z[0, 0, int(row)] == pytest.approx(val, abs=1e-15)
    others = [r for r in range(273) if str(r) not in g["S_rows"]]
    assert np.all(S[0, 0, others] == 0)
    assert np.all(z[0, 0, [r for r in range(273) if str(r) not in g["z_rows"]]] == 0)


def test_forms_agree():
    q, k, v = _tiny()
    yf, denf = O.linattn_quadratic(q, k, v, kernel="features")
    yt, dent = O.linattn_quadratic(q, k, v, kernel="taylor")
    yr, denr, S, z = O.linattn_recurrent(q, k, v)
    np.testing.assert_allclose(yt, yf, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(yr, yf, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(denr, denf, rtol=1e-12)
    L = q.shape[-2]
    for C in (1, 7, 16, 64, L):
        yc, denc, Sc, zc = O.linattn_chunked(q, k, v, C)
        np.testing.assert_allclose(yc, yf, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(Sc, S, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(zc, z, rtol=1e-12, atol=1e-12)


def test_state_matches_recurrence():
    q, k, v = _tiny(L=23)
    _, _, S, z = O.linattn_recurrent(q, k, v)
    S2, z2 = O.linattn_state(k, v)
    np.testing.assert_allclose(S2, S, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z2, z, rtol=1e-12, atol=1e-12)
    # z's constant row counts tokens exactly; its linear rows are sums of k
    assert np.all(z2[..., 0] == 23)
    np.testing.assert_allclose(z2[..., 1:17], k.sum(axis=-2), rtol=1e-12, atol=1e-12)


def test_resume_from_state():
    """Running on a prefix, then continuing from its state, equals one run."""
    q, k, v = _tiny(L=40)
    y, _, S, z = O.linattn_chunked(q, k, v, 8)
    _, _, S1, z1 = O.linattn_chunked(q[..., :17, :], k[..., :17, :], v[..., :17, :], 5)
    y2, _, S2, z2 = O.linattn_chunked(q[..., 17:, :], k[..., 17:, :], v[..., 17:, :], 6, S1, z1)
    np.testing.assert_allclose(y2, y[..., 17:, :], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S2, S, rtol=1e-12, atol=1e-12)


def test_denominator_lower_bound():
    """Each kernel value is >= 1/2, so den_i >= (i+1)/2 > 0; no epsilon needed."""
    q, k, v = _tiny(L=64, s=1.5)
    _, den = O.linattn_quadratic(q, k, v, kernel="taylor")
    i = np.arange(64)
    assert np.all(den >= (i + 1) / 2 - 1e-12)
    # adversarial: q.k = -1 for every pair gives exactly (i+1)/2
    qa = np.broadcast_to(e(0), (1, 1, 8, 16))
    ka = np.broadcast_to(-e(0), (1, 1, 8, 16))
    _, den = O.linattn_quadratic(qa, ka, rand(1, 1, 8, 3), kernel="features")
    np.testing.assert_allclose(den[0, 0], (np.arange(8) + 1) / 2, rtol=1e-15)


def test_zero_query_gives_cumulative_mean():
    """q = 0: every kernel value is 1, so y_i is the mean of v_0..v_i."""
    _, k, v = _tiny(L=30)
    q = np.zeros_like(k)
    want = np.cumsum(v, axis=-2) / np.arange(1, 31)[:, None]
    for fn in (lambda: O.linattn_quadratic(q, k, v)[0], lambda: O.linattn_chunked(q, k, v, 7)[0]):
        np.testing.assert_allclose(fn(), want, rtol=1e-12, atol=1e-13)
    # and likewise for k = 0
    np.testing.assert_allclose(O.linattn_recurrent(k, q, v)[0], want, rtol=1e-12, atol=1e-13)


def test_normalisation_properties():
    q, k, v = _tiny()
    y, _ = O.linattn_quadratic(q, k, v)
    # constant values pass through, weights sum to one
    c = np.full_like(v, 3.25)
    np.testing.assert_allclose(O.linattn_quadratic(q, k, c)[0], c, rtol=1e-13)
    # affine equivariance in v
    y2, _ = O.linattn_quadratic(q, k, -2.0 * v + 0.5)
    np.testing.assert_allclose(y2, -2.0 * y + 0.5, rtol=1e-12, atol=1e-12)
    # L = 1: y_0 = v_0
    np.testing.assert_allclose(O.linattn_quadratic(q[..., :1, :], k[..., :1, :], v[..., :1, :])[0], v[..., :1, :], rtol=1e-14)
    # permuting batch/head permutes outputs
    perm = [2, 0, 1]
    np.testing.assert_allclose(O.linattn_quadratic(q[:, perm], k[:, perm], v[:, perm])[0], y[:, perm], rtol=1e-14)


def test_causality():
    """Changing token t changes no output before t (and does change row t)."""
    q, k, v = _tiny(L=20)
    y, _ = O.linattn_quadratic(q, k, v)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[..., 11, :] += 1.0
    k2[..., 11, :] -= 1.0
    v2[..., 11, :] += 5.0
    ya, _ = O.linattn_quadratic(q2, k2, v2)
    np.testing.assert_array_equal(ya[..., :11, :], y[..., :11, :])
    assert np.all(np.abs(ya[..., 11, :] - y[..., 11, :]).max(axis=-1) > 1e-3)


# --------------------------------------------------------- sliding window attn
def _swa_bruteforce(q, k, v, window, scale):
    """Full L x L score matrix, -inf outside the band, SciPy softmax rows."""
    L = q.shape[-2]
    s = scale * q @ np.swapaxes(k, -1, -2)
    i, j = np.arange(L)[:, None], np.arange(L)[None, :]
    band = (j <= i) & (j > i - window)
    s = np.where(band, s, -np.inf)
    return scipy.special.softmax(s, axis=-1) @ v


@pytest.mark.parametrize("L,window,scale", [(1, 64, 1.0), (50, 64, 1.0), (130, 64, 1.0), (130, 17, 0.7), (70, 1, 1.0), (9, 200, 2.0)])
def test_swa_matches_scipy_softmax(L, window, scale):
    q, k, v = rand(2, 2, L, 16), rand(2, 2, L, 16), rand(2, 2, L, 7)
    np.testing.assert_allclose(O.swa(q, k, v, window, scale), _swa_bruteforce(q, k, v, window, scale), rtol=1e-12, atol=1e-13)


def test_swa_golden_hand_example():
    g = json.load(open(os.path.join(GOLD, "swa_hand.json")))
    q = np.array([e(0)] * 3)[None, None]
    k = np.array([e(0) * c for c in g["k_axis0"]])[None, None]
    v = np.array(g["v"])[None, None]
    np.testing.assert_allclose(O.swa(q, k, v, g["window"])[0, 0], g["y"], rtol=1e-14, atol=1e-15)


def test_swa_special_cases():
    q, k, v = rand(1, 2, 90, 16), rand(1, 2, 90, 16), rand(1, 2, 90, 4)
    # window 1: each row sees only itself
    np.testing.assert_allclose(O.swa(q, k, v, 1), v, rtol=1e-14)
    # q = 0: uniform weights over the last min(i+1, W) rows -> sliding mean
    W = 64
    cs = np.concatenate([np.zeros((1, 2, 1, 4)), np.cumsum(v, axis=-2)], axis=-2)
    i = np.arange(90)
    lo = np.maximum(0, i - W + 1)
    want = (cs[..., i + 1, :] - cs[..., lo, :]) / (i + 1 - lo)[:, None]
    np.testing.assert_allclose(O.swa(np.zeros_like(q), k, v, W), want, rtol=1e-11, atol=1e-12)
    # huge scores stay finite (max-shifted softmax)
    y = O.swa(q * 40, k * 40, v, W)
    assert np.all(np.isfinite(y))


def test_swa_taylor_weights_tie_to_linear_attention():
    """With weights 1 + s + s^2/2 and a window covering the sequence, the window
    attention is the causal Taylor linear attention."""
    q, k, v = _tiny(L=45)
    np.testing.assert_allclose(O.swa(q, k, v, window=45, weight="taylor"), O.linattn_quadratic(q, k, v)[0], rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------- decode
def test_decode_matches_forward():
    B, H, n, steps, dv, W = 2, 3, 70, 75, 6, 64
    q, k, v = rand(B, H, n + steps, 16, scale=0.5), rand(B, H, n + steps, 16, scale=0.5), rand(B, H, n + steps, dv)
    st = O.DecodeState.prefill(k[..., :n, :], v[..., :n, :], W)
    assert np.all(st.t == n)
    assert np.all(st.z[..., 0] == n)
    y_lin_ref, _ = O.linattn_quadratic(q, k, v, kernel="taylor")
    y_swa_ref = _swa_bruteforce(q, k, v, W, 1.0)
    for s in range(steps):
        yl, ys = st.step(q[..., n + s, :], k[..., n + s, :], v[..., n + s, :])
        np.testing.assert_allclose(yl, y_lin_ref[..., n + s, :], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(ys, y_swa_ref[..., n + s, :], rtol=1e-11, atol=1e-12)
    S, z = O.linattn_state(k, v)
    np.testing.assert_allclose(st.S, S, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(st.z, z, rtol=1e-11, atol=1e-11)
    assert np.all(st.t == n + steps)


def test_decode_from_empty_context():
    """Prefill of zero tokens; the first steps see fewer than W keys."""
    B, H, steps, dv = 1, 2, 5, 3
    q, k, v = rand(B, H, steps, 16), rand(B, H, steps, 16), rand(B, H, steps, dv)
    st = O.DecodeState.prefill(k[..., :0, :], v[..., :0, :], 64)
    yq, _ = O.linattn_quadratic(q, k, v)
    for s in range(steps):
        yl, ys = st.step(q[..., s, :], k[..., s, :], v[..., s, :])
        np.testing.assert_allclose(yl, yq[..., s, :], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(ys, _swa_bruteforce(q, k, v, 64, 1.0)[..., s, :], rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------ gradients
def _fd_grads(loss, arrays, eps=1e-6):
    """Central finite differences of a scalar loss, element by element."""
    out = []
    for arr in arrays:
        g = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            old = arr[i]
            arr[i] = old + eps
            lp = loss()
            arr[i] = old - eps
            lm = loss()
            arr[i] = old
            g[i] = (lp - lm) / (2 * eps)
        out.append(g)
    return out


@pytest.mark.parametrize("L,dv", [(1, 3), (6, 4), (9, 2)])
def test_linattn_bwd_finite_differences(L, dv):
    """Gradients against central differences of the Taylor-kernel forward
    (the taylor form of the quadratic definition, itself pinned above)."""
    q, k, v, dy = rand(2, L, 16, scale=0.3), rand(2, L, 16, scale=0.3), rand(2, L, dv), rand(2, L, dv)
    loss = lambda: float((O.linattn_quadratic(q, k, v, "taylor")[0] * dy).sum())
    fd = _fd_grads(loss, [q, k, v])
    for got, want in zip(O.linattn_bwd(q, k, v, dy), fd):
        np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("L,window,scale", [(7, 3, 0.7), (5, 1, 1.0), (6, 64, 1.3)])
def test_swa_bwd_finite_differences(L, window, scale):
    q, k, v, dy = rand(2, L, 16, scale=0.5), rand(2, L, 16, scale=0.5), rand(2, L, 5), rand(2, L, 5)
    loss = lambda: float((O.swa(q, k, v, window, scale) * dy).sum())
    fd = _fd_grads(loss, [q, k, v])
    for got, want in zip(O.swa_bwd(q, k, v, dy, window, scale), fd):
        np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-8)


def test_bwd_against_torch_autograd():
    """torch fp64 autograd through plain torch forwards (the masked Taylor
    kernel with a row normalisation; torch's own softmax under a band mask)."""
    torch = pytest.importorskip("torch")
    L, dv, W, scale = 40, 8, 9, 0.8
    q, k, v, dy = rand(L, 16, scale=0.3), rand(L, 16, scale=0.3), rand(L, dv), rand(L, dv)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    x = tq @ tk.T
    w = torch.tril(1 + x + x * x / 2)
    y = (w @ tv) / w.sum(-1, keepdim=True)
    (y * torch.tensor(dy)).sum().backward()
    for got, want in zip(O.linattn_bwd(q, k, v, dy), (tq.grad, tk.grad, tv.grad)):
        np.testing.assert_allclose(got, want.numpy(), rtol=1e-10, atol=1e-12)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    i, j = torch.arange(L)[:, None], torch.arange(L)[None, :]
    band = (j <= i) & (j > i - W)
    s = (scale * tq @ tk.T).masked_fill(~band, float("-inf"))
    y = torch.softmax(s, dim=-1) @ tv
    (y * torch.tensor(dy)).sum().backward()
    for got, want in zip(O.swa_bwd(q, k, v, dy, W, scale), (tq.grad, tk.grad, tv.grad)):
        np.testing.assert_allclose(got, want.numpy(), rtol=1e-10, atol=1e-12)


def test_bwd_shift_identity():
    """Both outputs are convex combinations of the values, so shifting every
    v_j by c shifts every y_i by c: sum_j dv_j = sum_i dy_i exactly."""
    L, dv = 50, 6
    q, k, v, dy = rand(L, 16, scale=0.3), rand(L, 16, scale=0.3), rand(L, dv), rand(L, dv)
    _, _, dv_lin = O.linattn_bwd(q, k, v, dy)
    np.testing.assert_allclose(dv_lin.sum(0), dy.sum(0), rtol=1e-12, atol=1e-12)
    _, _, dv_swa = O.swa_bwd(q, k, v, dy, 7, 1.1)
    np.testing.assert_allclose(dv_swa.sum(0), dy.sum(0), rtol=1e-12, atol=1e-12)


def test_swa_bwd_special_cases():
    """Window 1: y = v, so dv = dy and q, k get nothing.  A zero upstream
    gradient gives zero everywhere."""
    L = 12
    q, k, v, dy = rand(L, 16), rand(L, 16), rand(L, 4), rand(L, 4)
    dq, dk, dv = O.swa_bwd(q, k, v, dy, 1, 1.0)
    np.testing.assert_array_equal(dv, dy)
    assert not dq.any() and not dk.any()
    for g in O.swa_bwd(q, k, v, np.zeros_like(dy), 5, 1.0) + O.linattn_bwd(q * 0.2, k * 0.2, v, np.zeros_like(dy)):
        assert not g.any()


def test_linattn_bwd_first_position():
    """Row 0 sees only itself: y_0 = v_0 whatever q_0, k_0 are, so the first
    row's upstream gradient reaches only dv_0 (with L = 1, dq = dk = 0)."""
    q, k, v, dy = rand(1, 16), rand(1, 16), rand(1, 5), rand(1, 5)
    dq, dk, dv = O.linattn_bwd(q, k, v, dy)
    np.testing.assert_allclose(dv, dy, rtol=1e-15)
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15


def test_linattn_bwd_rows_matches_full():
    """The row-sampled gradient (for long sequences) against the full one."""
    L, dv = 300, 8
    q, k, v, dy = rand(L, 16, scale=0.25), rand(L, 16, scale=0.25), rand(L, dv), rand(L, dv)
    full = O.linattn_bwd(q, k, v, dy)
    rows = [0, 5, 63, 64, 299]
    for got, want in zip(O.linattn_bwd_rows(q, k, v, dy, rows, 64), full):
        np.testing.assert_allclose(got, want[rows], rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------ BaseConv
def test_baseconv_matches_numpy_convolve():
    """Per channel, the causal depthwise convolution is the first L terms of
    the full linear convolution (numpy.convolve); the gate multiplies."""
    L, D, K = 37, 5, 4
    x, u, h, b = rand(2, L, D), rand(2, L, D), rand(D, K), rand(D)
    y = O.baseconv(x, u, h, b)
    for bi in range(2):
        for c in range(D):
            want = u[bi, :, c] * (np.convolve(x[bi, :, c], h[c])[:L] + b[c])
            np.testing.assert_allclose(y[bi, :, c], want, rtol=1e-13, atol=1e-13)


def test_baseconv_special_cases():
    L, D = 9, 3
    x, u = rand(L, D), rand(L, D)
    # one tap: y = u * (h0 x + b)
    h, b = rand(D, 1), rand(D)
    np.testing.assert_allclose(O.baseconv(x, u, h, b), u * (h[:, 0] * x + b), rtol=1e-15)
    # an impulse at t0 returns the filter, shifted, times the gate
    h = rand(D, 3)
    imp = np.zeros((L, D))
    imp[4] = 1.0
    y = O.baseconv(imp, np.ones((L, D)), h)
    assert not y[:4].any() and not y[7:].any()
    np.testing.assert_allclose(y[4:7], h.T, rtol=1e-15)
    # filter longer than the sequence: only the taps that reach back exist
    y = O.baseconv(x[:2], u[:2], rand(D, 4))
    assert y.shape == (2, D)


def test_baseconv_causal_and_linear():
    L, D, K = 20, 4, 3
    x, u, h = rand(L, D), rand(L, D), rand(D, K)
    y = O.baseconv(x, u, h)
    x2 = x.copy()
    x2[12:] = rand(L - 12, D)
    np.testing.assert_array_equal(O.baseconv(x2, u, h)[:12], y[:12])  # no look-ahead
    z = rand(L, D)
    np.testing.assert_allclose(O.baseconv(2.0 * x - z, u, h), 2.0 * y - O.baseconv(z, u, h), rtol=1e-12,
                               atol=1e-12)


# ------------------------------------------------------------ decay variant
def test_decay_forms_agree_and_reduce():
    """Quadratic and recurrent decayed forms agree (with an initial state);
    gamma = 1 is the undecayed layer."""
    B, H, L, dv = 2, 3, 13, 4
    q, k, v = rand(B, H, L, 16, scale=0.3), rand(B, H, L, 16, scale=0.3), rand(B, H, L, dv)
    g = np.array([1.0, 0.93, 0.5])
    S0, z0 = rand(B, H, 273, dv), np.abs(rand(B, H, 273)) + 5
    a = O.linattn_decay_quadratic(q, k, v, g, S0, z0)[0]
    b = O.linattn_decay_recurrent(q, k, v, g, S0, z0)[0]
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O.linattn_decay_quadratic(q, k, v, np.ones(H))[0], O.linattn_quadratic(q, k, v)[0],
                               rtol=1e-13, atol=1e-13)


def test_decay_closed_forms():
    """L = 2: y_1 = (g K10 v0 + K11 v1) / (g K10 + K11).  A vanishing decay
    leaves each row its own value."""
    q, k, v = rand(2, 16, scale=0.4), rand(2, 16, scale=0.4), rand(2, 3)
    g = 0.7
    K = lambda a, b: 1 + a @ b + (a @ b) ** 2 / 2
    k10, k11 = K(q[1], k[0]), K(q[1], k[1])
    want = (g * k10 * v[0] + k11 * v[1]) / (g * k10 + k11)
    y = O.linattn_decay_quadratic(q[None], k[None], v[None], np.array([g]))[0][0]
    np.testing.assert_allclose(y[1], want, rtol=1e-14)
    np.testing.assert_allclose(y[0], v[0], rtol=1e-14)
    y = O.linattn_decay_quadratic(q[None], k[None], v[None], np.array([1e-30]))[0][0]
    np.testing.assert_allclose(y, v, rtol=1e-12)
    # gamma = 0 exactly: gamma^0 = 1 keeps each row's own term and nothing else
    for form in (O.linattn_decay_quadratic, O.linattn_decay_recurrent):
        y = form(q[None], k[None], v[None], np.array([0.0]))[0][0]
        np.testing.assert_allclose(y, v, rtol=1e-14)


def test_decay_resume_from_state():
    """Running [0, n) then [n, L) from the exported state equals one run."""
    H, L, n, dv = 2, 20, 7, 3
    q, k, v = rand(H, L, 16, scale=0.3), rand(H, L, 16, scale=0.3), rand(H, L, dv)
    g = np.array([0.8, 0.99])
    full = O.linattn_decay_recurrent(q, k, v, g)[0]
    _, _, S, z = O.linattn_decay_recurrent(q[:, :n], k[:, :n], v[:, :n], g)
    rest = O.linattn_decay_quadratic(q[:, n:], k[:, n:], v[:, n:], g, S, z)[0]
    np.testing.assert_allclose(rest, full[:, n:], rtol=1e-12, atol=1e-12)


def test_decay_rows_match_quadratic():
    L, dv = 90, 5
    q, k, v = rand(1, L, 16, scale=0.3), rand(1, L, 16, scale=0.3), rand(1, L, dv)
    g = 0.93
    full = O.linattn_decay_quadratic(q, k, v, np.array([g]))[0][0]
    rows = [0, 1, 44, 89]
    np.testing.assert_allclose(O.linattn_decay_rows(q[0], k[0], v[0], g, rows), full[rows], rtol=1e-13)


def test_decay_decode_matches_decayed_forward():
    """Decode steps with a decay, from the decayed recurrence's state after a
    context, equal the decayed quadratic form over context + steps; gamma = 1
    is the plain decode."""
    B, H, n, steps, dv = 2, 3, 20, 9, 5
    q, k, v = rand(B, H, n + steps, 16, scale=0.4), rand(B, H, n + steps, 16, scale=0.4), rand(B, H, n + steps, dv)
    g = np.array([1.0, 0.9, 0.6])
    _, _, S, z = O.linattn_decay_recurrent(q[..., :n, :], k[..., :n, :], v[..., :n, :], g)
    st = O.DecodeState.prefill(k[..., :n, :], v[..., :n, :], 64)
    st.S, st.z = S.copy(), z.copy()
    plain = O.DecodeState.prefill(k[..., :n, :], v[..., :n, :], 64)
    y_ref = O.linattn_decay_quadratic(q, k, v, g)[0]
    for s in range(steps):
        t = n + s
        yl, ys = st.step(q[..., t, :], k[..., t, :], v[..., t, :], gamma=g)
        np.testing.assert_allclose(yl, y_ref[..., t, :], rtol=1e-11, atol=1e-12)
        yp, ysp = plain.step(q[..., t, :], k[..., t, :], v[..., t, :], gamma=np.ones(H))
        yp0 = O.linattn_quadratic(q, k, v)[0][..., t, :]
        np.testing.assert_allclose(yp, yp0, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(ys, ysp, rtol=0, atol=0)  # the window part does not decay


# ------------------------------------------------------------ compact state
def test_compact_layout():
    """153 rows: constant, 16 linear, then the 136 unordered pairs a <= b with
    a outermost (the order the header states for the compact decode state)."""
    assert O.D_CMP == 153 == 1 + 16 + 136
    P = O.pairs()
    assert len(P) == 136 and P[0] == (0, 0) and P[1] == (0, 1) and P[15] == (0, 15) and P[16] == (1, 1)
    assert P[-1] == (15, 15) and len(set(P)) == 136 and all(a <= b for a, b in P)


def test_compact_readout_identity_for_any_state():
    """phi(q)^T S depends on rows (a, b), (b, a) only through their sum, so the
    compact state read with the compact query weights gives the pages' readout
    for any S, symmetric or not (numerator and denominator)."""
    g = np.random.default_rng(21)
    S = g.normal(size=(3, 273, 8))
    z = g.normal(size=(3, 273))
    q = g.normal(size=(3, 16))
    Sc, zc = O.state_compact(S, z)
    pq, pqc = O.phi(q), O.phi_compact_query(q)
    np.testing.assert_allclose(np.einsum("hf,hfd->hd", pqc, Sc), np.einsum("hf,hfd->hd", pq, S), rtol=1e-12,
                               atol=1e-12)
    np.testing.assert_allclose((pqc * zc).sum(-1), (pq * z).sum(-1), rtol=1e-12, atol=1e-12)


def test_compact_update_identity():
    """What a key adds to the 273-row state, compacted, is what the compact key
    feature adds: compact(phi(k) v^T) = phi_c(k) v^T, compact(phi(k)) = phi_c(k)."""
    g = np.random.default_rng(22)
    k, v = g.normal(size=(4, 16)), g.normal(size=(4, 8))
    Sc, zc = O.state_compact(O.phi(k)[:, :, None] * v[:, None, :], O.phi(k))
    np.testing.assert_allclose(Sc, O.phi_compact_key(k)[:, :, None] * v[:, None, :], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(zc, O.phi_compact_key(k), rtol=1e-13, atol=1e-15)
    # a diagonal pair row takes k_a^2 / sqrt2 once, an off-diagonal one sqrt2 k_a k_b
    x = np.zeros(16)
    x[2], x[5] = 3.0, 7.0
    f = O.phi_compact_key(x)
    row = {p: 17 + i for i, p in enumerate(O.pairs())}
    assert f[row[(2, 2)]] == pytest.approx(9.0 / np.sqrt(2.0))
    assert f[row[(2, 5)]] == pytest.approx(21.0 * np.sqrt(2.0))
    assert f[row[(5, 5)]] == pytest.approx(49.0 / np.sqrt(2.0))
    assert np.count_nonzero(f[17:]) == 3


def test_compact_round_trips():
    """expand(compact(S)) = S for a state the recurrence builds (its ordered
    pair rows are equal), and compact(expand(Sc)) = Sc for any compact state,
    both exactly."""
    g = np.random.default_rng(23)
    k, v = g.normal(size=(2, 40, 16)) * 0.25, g.normal(size=(2, 40, 8))
    S, z = O.linattn_state(k, v)
    S2, z2 = O.state_expand(*O.state_compact(S, z))
    assert np.array_equal(S2, S) and np.array_equal(z2, z)
    Sc, zc = g.normal(size=(2, 153, 8)), g.normal(size=(2, 153))
    Sc2, zc2 = O.state_compact(*O.state_expand(Sc, zc))
    assert np.array_equal(Sc2, Sc) and np.array_equal(zc2, zc)


# ------------------------------------------------------------ decayed gradients
@pytest.mark.parametrize("L,dv,gam", [(1, 3, 0.5), (6, 4, 0.7), (9, 2, 0.95)])
def test_linattn_decay_bwd_finite_differences(L, dv, gam):
    """Decayed gradients against central differences of the decayed
    quadratic forward (itself pinned against the recurrence above); two heads
    with different decays."""
    q, k, v, dy = rand(2, L, 16, scale=0.3), rand(2, L, 16, scale=0.3), rand(2, L, dv), rand(2, L, dv)
    g = np.array([gam, 1.0 - 0.5 * (1.0 - gam)])
    loss = lambda: float((O.linattn_decay_quadratic(q, k, v, g)[0] * dy).sum())
    fd = _fd_grads(loss, [q, k, v])
    for got, want in zip(O.linattn_decay_bwd(q, k, v, g, dy), fd):
        np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-8)


def test_linattn_decay_bwd_gamma_one_and_autograd():
    """gamma = 1 gives the undecayed gradients; and torch fp64 autograd
    through a plain torch decayed forward (the masked Taylor kernel times
    gamma^(i-j), row-normalised) agrees."""
    torch = pytest.importorskip("torch")
    L, dv = 30, 5
    q, k, v, dy = rand(2, L, 16, scale=0.3), rand(2, L, 16, scale=0.3), rand(2, L, dv), rand(2, L, dv)
    for got, want in zip(O.linattn_decay_bwd(q, k, v, np.ones(2), dy), O.linattn_bwd(q, k, v, dy)):
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)
    g = np.array([0.8, 0.97])
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    i, j = torch.arange(L)[:, None], torch.arange(L)[None, :]
    dec = torch.tensor(g)[:, None, None] ** (i - j).clamp(min=0).double() * (j <= i)
    x = tq @ tk.transpose(-1, -2)
    w = (1 + x + x * x / 2) * dec
    y = (w @ tv) / w.sum(-1, keepdim=True)
    (y * torch.tensor(dy)).sum().backward()
    for got, want in zip(O.linattn_decay_bwd(q, k, v, g, dy), (tq.grad, tk.grad, tv.grad)):
        np.testing.assert_allclose(got, want.numpy(), rtol=1e-10, atol=1e-12)


def test_linattn_decay_bwd_shift_and_vanishing_decay():
    """The decayed output is still a convex combination of the values:
    sum_j dv_j = sum_i dy_i.  A vanishing decay leaves each row its own value
    (y_i -> v_i): dv -> dy and dq, dk -> 0."""
    L, dv = 40, 6
    q, k, v, dy = rand(L, 16, scale=0.3), rand(L, 16, scale=0.3), rand(L, dv), rand(L, dv)
    _, _, dvg = O.linattn_decay_bwd(q[None], k[None], v[None], np.array([0.6]), dy[None])
    np.testing.assert_allclose(dvg[0].sum(0), dy.sum(0), rtol=1e-12, atol=1e-12)
    dq, dk, dvs = O.linattn_decay_bwd(q[None], k[None], v[None], np.array([1e-12]), dy[None])
    np.testing.assert_allclose(dvs[0], dy, rtol=1e-9, atol=1e-9)
    assert np.abs(dq).max() < 1e-9 and np.abs(dk).max() < 1e-9
    # gamma = 0 exactly: y = v whatever q and k are
    dq, dk, dvs = O.linattn_decay_bwd(q[None], k[None], v[None], np.array([0.0]), dy[None])
    np.testing.assert_allclose(dvs[0], dy, rtol=1e-14, atol=1e-14)
    assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14
