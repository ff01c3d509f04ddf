"""fp64 CPU oracle for the Based sequence-mixing layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the smoke check in ``__graft_entry__`` and
the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP kernels and imports nothing from the GPU package; it takes plain arrays
and returns plain fp64 NumPy arrays.

Sources (the web pages that describe the method):

* [README]  "based" -- HazyResearch/based project README (Chinese translation
  on dongaigc.com), introduction: Based combines a short sliding-window
  softmax attention (window 64, exact softmax locally) with a dense, global
  linear attention that approximates softmax for all other tokens.
* [BLOG]    "Базированная модель, часть 2" (Telegram channel botka_chronics),
  the paragraph on linear attention and the feature-map pseudocode after it:
  exp(q.k) is replaced by its 2nd-order Taylor expansion 1 + qk + (qk)^2/2,
  realised as a dot product of feature vectors [1, x, x x^T / sqrt(2)], where
  the quadratic block lists every ordered pair (x_a x_b for a, then b).
  The paragraph on the state: the recurrent form keeps a KV-state for the
  numerator and a K-state for the denominator of the softmax simulation.
* [BLOG1]   "Базированная модель, часть 1" (same channel), the list of what
  the paper proves: the BaseConv block y = linear(x) * conv(h, x), an
  elementwise product of a linear map of the input with a learned filter
  h convolved over the sequence; the README's acknowledgements name the
  short causal conv1d kernel of Mamba as the convolution used.
* [TRAIN]   HazyResearch/based ``train/`` README, "training views": the
  quadratic PyTorch view, the flash-linear-attention kernel and the
  fast-transformers kernel are interchangeable implementations of one
  computation (here: the quadratic, recurrent and chunked forms below).

Readings where the pages are silent (all listed in the design doc as well):

* no temperature inside phi; the inputs carry whatever scale they have;
* causal means inclusive (j <= i), for both attentions;
* the window holds ``window`` keys including the query's own position;
* linear attention is normalised (numerator / denominator) with no epsilon:
  every kernel value 1 + x + x^2/2 = ((1 + x)^2 + 1)/2 is at least 1/2, so the
  denominator of row i is at least (i + 1)/2;
* the window softmax uses scale * q.k with a caller-given scale (1.0 in the
  workloads), the exact exponential that the Taylor map approximates;
* linear attention and window attention are two separate outputs;
* the backward is the exact derivative of these forwards with respect to
  q, k and v (no initial state), as the training views imply;
* decay (the train README points to an optional decay strategy with no
  formula on the pages): a per-head factor 0 <= gamma <= 1 on the state,
  S_i = gamma S_{i-1} + phi(k_i) v_i^T and z likewise, so the kernel weight of
  key j in row i is K_ij gamma^(i-j); gamma = 1 is the layer without decay;
* BaseConv's convolution is causal and depthwise (one short filter per
  channel, zero history before the first position, tap s on x_{t-s}), with
  an optional per-channel bias; linear(x) is computed by the caller (a plain
  matrix product) and enters as u.

Every function here is pinned by ``tests/test_oracle_pins.py`` against
closed forms, invariants, textbook special cases, SciPy's softmax and
hand-derived fixtures in ``tests/golden/``; the gradients against central
finite differences of the forwards, torch fp64 autograd through plain torch
forwards, and the value-shift identity.
"""

from __future__ import annotations

import numpy as np

D_K = 16
D_PHI = 1 + D_K + D_K * D_K  # 273 Taylor features for d_k = 16

_INV_SQRT2 = 1.0 / np.sqrt(2.0)


def _f64(x) -> np.ndarray:
    """Exact widening of whatever the caller holds (fp32, bf16 via torch, fp64)."""
    if hasattr(x, "detach"):  # torch tensor: widen on the torch side, exactly
        import torch

        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# Feature map  [BLOG, feature-map pseudocode]
# --------------------------------------------------------------------------
def phi(x) -> np.ndarray:
    """Second-order Taylor feature map, applied along the last axis.

    phi(x) = [1, x_1..x_d, (x_a * x_b / sqrt(2) for a in 1..d for b in 1..d)],
    i.e. the constant, the linear block, then every ordered pair with the
    first index outermost.  Length 1 + d + d^2 (273 for d = 16).  Feature
    index of x_a x_b / sqrt(2) is 1 + d + d*a + b (0-based a, b).
    """
    x = _f64(x)
    d = x.shape[-1]
    lead = x.shape[:-1]
    quad = (x[..., :, None] * x[..., None, :]).reshape(lead + (d * d,)) * _INV_SQRT2
    return np.concatenate([np.ones(lead + (1,)), x, quad], axis=-1)


# --------------------------------------------------------------------------
# Compact state  [BLOG, feature-map pseudocode and the paragraph on the state]
# --------------------------------------------------------------------------
D_CMP = 1 + D_K + D_K * (D_K + 1) // 2  # 153: constant, linear, unordered pairs


def pairs(d: int = D_K):
    """The unordered index pairs (a, b), a <= b, a outermost."""
    return [(a, b) for a in range(d) for b in range(a, d)]


def _pair_rows():
    """For each unordered pair: its row (a, b) and row (b, a) in phi's layout,
    and whether the pair is off the diagonal."""
    a = np.array([p[0] for p in pairs()])
    b = np.array([p[1] for p in pairs()])
    return 1 + D_K + D_K * a + b, 1 + D_K + D_K * b + a, a != b


def state_compact(S, z):
    """A state with one row per unordered pair of the quadratic features.

    phi lists x_a x_b / sqrt(2) under both orders of a pair, so every state the
    recurrence builds has equal rows (a, b) and (b, a), and phi(q)^T S only uses
    their sum.  Compact rows: the constant and linear rows as they are, then
    for each pair of pairs(): S[(a,b)] + S[(b,a)] for a < b, S[(a,a)] for
    a = b.  S [..., 273, d_v], z [..., 273] -> [..., 153, d_v], [..., 153].
    """
    S, z = _f64(S), _f64(z)
    rab, rba, off = _pair_rows()
    Sq = S[..., rab, :] + np.where(off[:, None], S[..., rba, :], 0.0)
    zq = z[..., rab] + np.where(off, z[..., rba], 0.0)
    return (np.concatenate([S[..., : 1 + D_K, :], Sq], axis=-2),
            np.concatenate([z[..., : 1 + D_K], zq], axis=-1))


def state_expand(Sc, zc):
    """The 273-row state of a compact one: both ordered rows of an off-diagonal
    pair get half of the pair row, the diagonal rows the pair row itself."""
    Sc, zc = _f64(Sc), _f64(zc)
    rab, rba, off = _pair_rows()
    lead = Sc.shape[:-2]
    S = np.zeros(lead + (D_PHI, Sc.shape[-1]))
    z = np.zeros(zc.shape[:-1] + (D_PHI,))
    S[..., : 1 + D_K, :] = Sc[..., : 1 + D_K, :]
    z[..., : 1 + D_K] = zc[..., : 1 + D_K]
    half = np.where(off, 0.5, 1.0)
    S[..., rab, :] = Sc[..., 1 + D_K:, :] * half[:, None]
    S[..., rba, :] = Sc[..., 1 + D_K:, :] * half[:, None]
    z[..., rab] = zc[..., 1 + D_K:] * half
    z[..., rba] = zc[..., 1 + D_K:] * half
    return S, z


def phi_compact_key(x) -> np.ndarray:
    """What a key adds to the compact state's rows: 1, x_a, then per pair
    sqrt(2) x_a x_b off the diagonal (both ordered rows' x_a x_b / sqrt(2))
    and x_a^2 / sqrt(2) on it."""
    x = _f64(x)
    a = np.array([p[0] for p in pairs()])
    b = np.array([p[1] for p in pairs()])
    quad = x[..., a] * x[..., b] * np.where(a != b, np.sqrt(2.0), _INV_SQRT2)
    return np.concatenate([np.ones(x.shape[:-1] + (1,)), x, quad], axis=-1)


def phi_compact_query(x) -> np.ndarray:
    """Readout weights of the compact state's rows: 1, x_a, then
    x_a x_b / sqrt(2) per pair (the weight of either ordered row)."""
    x = _f64(x)
    a = np.array([p[0] for p in pairs()])
    b = np.array([p[1] for p in pairs()])
    return np.concatenate([np.ones(x.shape[:-1] + (1,)), x, x[..., a] * x[..., b] * _INV_SQRT2], axis=-1)


def taylor_kernel(s) -> np.ndarray:
    """1 + s + s^2/2: the 2nd-order Taylor expansion of exp(s) [BLOG]."""
    s = _f64(s)
    return 1.0 + s + 0.5 * s * s


# --------------------------------------------------------------------------
# Causal linear attention  [README intro; BLOG linear-attention paragraph]
# --------------------------------------------------------------------------
def linattn_quadratic(q, k, v, kernel: str = "features"):
    """Quadratic masked form, the definition of record.

    y_i = sum_{j<=i} K(q_i, k_j) v_j / sum_{j<=i} K(q_i, k_j), computed per
    (batch, head) from the full L x L kernel matrix with the upper triangle
    zeroed.  ``kernel="features"`` forms K as the 273-dim dot product
    phi(q_i).phi(k_j); ``kernel="taylor"`` forms it as 1 + x + x^2/2 with
    x = q_i.k_j.  Returns (y, den) with den[..., i] the denominator.
    Shapes: q, k [..., L, d_k]; v [..., L, d_v].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    if kernel == "features":
        A = phi(q) @ np.swapaxes(phi(k), -1, -2)
    elif kernel == "taylor":
        A = taylor_kernel(q @ np.swapaxes(k, -1, -2))
    else:
        raise ValueError(kernel)
    L = q.shape[-2]
    A = A * np.tril(np.ones((L, L)))
    den = A.sum(axis=-1)
    y = (A @ v) / den[..., None]
    return y, den


def linattn_recurrent(q, k, v, S0=None, z0=None):
    """Recurrent (constant-state) form [BLOG, paragraph on the state].

    Start from S = S0 (273 x d_v, zero if None) and z = z0 (273, zero if
    None).  For i = 0..L-1: S += phi(k_i) v_i^T; z += phi(k_i);
    y_i = phi(q_i)^T S / phi(q_i)^T z.  Returns (y, den, S, z).
    A pure Python loop over positions: meant for short L.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    lead = q.shape[:-2]
    L, dv = q.shape[-2], v.shape[-1]
    S = np.zeros(lead + (D_PHI, dv)) if S0 is None else _f64(S0).copy()
    z = np.zeros(lead + (D_PHI,)) if z0 is None else _f64(z0).copy()
    pq, pk = phi(q), phi(k)
    y = np.empty(lead + (L, dv))
    den = np.empty(lead + (L,))
    for i in range(L):
        S += pk[..., i, :, None] * v[..., i, None, :]
        z += pk[..., i, :]
        num = np.einsum("...f,...fd->...d", pq[..., i, :], S)
        den[..., i] = np.einsum("...f,...f->...", pq[..., i, :], z)
        y[..., i, :] = num / den[..., i, None]
    return y, den, S, z


def linattn_chunked(q, k, v, chunk: int, S0=None, z0=None):
    """Chunked form: per chunk, the in-chunk masked quadratic term plus a
    readout of the state accumulated over all earlier chunks, then the
    state update [TRAIN, training views: the chunked kernels compute the
    same result as the quadratic view].

    For a chunk c of positions P: num_i = phi(q_i)^T S + sum_{j in P, j<=i}
    (phi(q_i).phi(k_j)) v_j, den_i likewise with z and 1, and then
    S += phi(K_P)^T V_P, z += sum_{j in P} phi(k_j).  Returns (y, den, S, z).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    lead = q.shape[:-2]
    L, dv = q.shape[-2], v.shape[-1]
    S = np.zeros(lead + (D_PHI, dv)) if S0 is None else _f64(S0).copy()
    z = np.zeros(lead + (D_PHI,)) if z0 is None else _f64(z0).copy()
    y = np.empty(lead + (L, dv))
    den = np.empty(lead + (L,))
    for c0 in range(0, L, chunk):
        c1 = min(L, c0 + chunk)
        pq, pk, vc = phi(q[..., c0:c1, :]), phi(k[..., c0:c1, :]), v[..., c0:c1, :]
        n = c1 - c0
        A = (pq @ np.swapaxes(pk, -1, -2)) * np.tril(np.ones((n, n)))
        num = pq @ S + A @ vc
        dn = pq @ z[..., :, None]
        dn = dn[..., 0] + A.sum(axis=-1)
        y[..., c0:c1, :] = num / dn[..., None]
        den[..., c0:c1] = dn
        S = S + np.swapaxes(pk, -1, -2) @ vc
        z = z + pk.sum(axis=-2)
    return y, den, S, z


def linattn_state(k, v):
    """Final state after a sequence: S = sum_j phi(k_j) v_j^T, z = sum_j phi(k_j)
    [BLOG, paragraph on the state].  Shapes [..., 273, d_v] and [..., 273]."""
    pk, v = phi(k), _f64(v)
    return np.swapaxes(pk, -1, -2) @ v, pk.sum(axis=-2)


# --------------------------------------------------------------------------
# Sliding-window softmax attention  [README intro]
# --------------------------------------------------------------------------
def swa(q, k, v, window: int = 64, scale: float = 1.0, weight: str = "exp"):
    """Causal sliding-window attention.

    Row i attends to keys j with max(0, i - window + 1) <= j <= i (``window``
    keys including itself).  With s_j = scale * q_i.k_j:
    ``weight="exp"``: p_j = exp(s_j - max_j s_j) and y_i = sum p_j v_j / sum p_j,
    the exact softmax; ``weight="taylor"``: p_j = 1 + s_j + s_j^2/2 (no max
    shift: the Taylor weights are not shift-invariant), which ties this
    function to the linear attention when the window covers the sequence.
    Vectorised over rows with a (L, window) band of key indices.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    L = q.shape[-2]
    if window < 1:
        raise ValueError("window must be >= 1")
    idx = np.arange(L)[:, None] - (window - 1) + np.arange(window)[None, :]  # (L, W)
    valid = idx >= 0
    idxc = np.where(valid, idx, 0)
    kb = k[..., idxc, :]  # [..., L, W, d]
    vb = v[..., idxc, :]
    s = scale * np.einsum("...ld,...lwd->...lw", q, kb)
    if weight == "exp":
        s = np.where(valid, s, -np.inf)
        m = s.max(axis=-1, keepdims=True)
        p = np.exp(s - m)
    elif weight == "taylor":
        p = np.where(valid, taylor_kernel(s), 0.0)
    else:
        raise ValueError(weight)
    return np.einsum("...lw,...lwd->...ld", p, vb) / p.sum(axis=-1)[..., None]


# --------------------------------------------------------------------------
# Gradients of the two attentions  [TRAIN, training views: the layer is
# trained through these forwards, so the backward is their exact derivative]
# --------------------------------------------------------------------------
def linattn_decay_quadratic(q, k, v, gamma, S0=None, z0=None):
    """Decayed linear attention, quadratic form [TRAIN, decay strategy; the
    reading: a per-head factor gamma on the state].  Per (batch, head) with
    decay g = gamma[head] (gamma has one entry per head, the axis before L):
      y_i = (sum_{j<=i} g^(i-j) K_ij v_j + g^(i+1) phi(q_i)^T S0)
            / (sum_{j<=i} g^(i-j) K_ij + g^(i+1) phi(q_i)^T z0),
    K_ij = 1 + x + x^2/2.  Returns (y, den)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    g = _f64(gamma)
    L, dv = q.shape[-2], v.shape[-1]
    i = np.arange(L)
    d = (i[:, None] - i[None, :]).astype(np.float64)
    lead = q.shape[:-2]
    gb = g.reshape(g.shape + (1,) * 2)  # [H, 1, 1], broadcast over leading batch dims
    W = np.where(d >= 0, gb ** np.maximum(d, 0), 0.0)
    A = taylor_kernel(q @ np.swapaxes(k, -1, -2)) * W
    num = A @ v
    den = A.sum(axis=-1)
    if S0 is not None:
        pq = phi(q)
        w0 = g.reshape(g.shape + (1,)) ** (i + 1.0)  # [H, L]
        num = num + w0[..., None] * (pq @ _f64(S0))
        den = den + w0 * np.einsum("...lf,...f->...l", pq, _f64(z0))
    return num / den[..., None], den


def linattn_decay_recurrent(q, k, v, gamma, S0=None, z0=None):
    """Decayed linear attention, recurrent form: for i = 0..L-1,
    S = g S + phi(k_i) v_i^T, z = g z + phi(k_i), y_i = phi(q_i)^T S / phi(q_i)^T z
    with g = gamma[head].  Returns (y, den, S, z).  Loop over positions."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    g = _f64(gamma)
    lead = q.shape[:-2]
    L, dv = q.shape[-2], v.shape[-1]
    S = np.zeros(lead + (D_PHI, dv)) if S0 is None else _f64(S0).copy()
    z = np.zeros(lead + (D_PHI,)) if z0 is None else _f64(z0).copy()
    pq, pk = phi(q), phi(k)
    gS = g.reshape(g.shape + (1, 1))
    gz = g.reshape(g.shape + (1,))
    y = np.empty(lead + (L, dv))
    den = np.empty(lead + (L,))
    for t in range(L):
        S = gS * S + pk[..., t, :, None] * v[..., t, None, :]
        z = gz * z + pk[..., t, :]
        den[..., t] = np.einsum("...f,...f->...", pq[..., t, :], z)
        y[..., t, :] = np.einsum("...f,...fd->...d", pq[..., t, :], S) / den[..., t, None]
    return y, den, S, z


def linattn_decay_rows(q, k, v, g, rows):
    """The decayed output of ``linattn_decay_quadratic`` (no initial state) at
    selected positions of one head, for sequences too long for L x L
    matrices: y_i = sum_{j<=i} g^(i-j) K_ij v_j / sum_{j<=i} g^(i-j) K_ij.
    q, k [L, d_k], v [L, d_v], scalar decay g.  Returns [len(rows), d_v]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    out = []
    for i in rows:
        w = taylor_kernel(k[: i + 1] @ q[i]) * float(g) ** (i - np.arange(i + 1, dtype=np.float64))
        out.append(w @ v[: i + 1] / w.sum())
    return np.array(out)


def linattn_bwd(q, k, v, dy):
    """Gradients of the normalised causal linear attention (no initial state)
    with respect to q, k and v, for an upstream gradient dy of y.

    Written from the quadratic definition (``linattn_quadratic``): with the
    kernel matrix A_ij = 1 + x_ij + x_ij^2/2 (x = q_i.k_j, j <= i, else 0),
    num = A V, den = A 1 and y = num / den, the chain rule gives, per row i,
      g_i = dy_i / den_i             (through the numerator)
      h_i = -(dy_i . y_i) / den_i    (through the denominator)
      dA_ij = g_i . v_j + h_i        (j <= i)
      dV = A^T G,  dX = dA * (1 + X)  (the kernel's derivative in x),
      dQ = dX K,   dK = dX^T Q.
    Returns (dq, dk, dv) as fp64 arrays shaped like q, k, v.
    """
    q, k, v, dy = _f64(q), _f64(k), _f64(v), _f64(dy)
    L = q.shape[-2]
    mask = np.tril(np.ones((L, L)))
    X = q @ np.swapaxes(k, -1, -2)
    A = taylor_kernel(X) * mask
    den = A.sum(axis=-1)
    y = (A @ v) / den[..., None]
    g = dy / den[..., None]
    h = -(dy * y).sum(axis=-1) / den
    dA = (g @ np.swapaxes(v, -1, -2) + h[..., None]) * mask
    dX = dA * (1.0 + X)
    dq = dX @ k
    dk = np.swapaxes(dX, -1, -2) @ q
    dv = np.swapaxes(A, -1, -2) @ g
    return dq, dk, dv


def linattn_decay_bwd(q, k, v, gamma, dy):
    """Gradients of the decayed linear attention (``linattn_decay_quadratic``,
    no initial state) with respect to q, k and v, for an upstream gradient dy.

    The decayed kernel matrix is A = K * W with W_ij = g^(i-j) for j <= i (0
    otherwise), g = gamma[head]; W does not depend on q, k, v.  With
    num = A V, den = A 1 and y = num / den, as in ``linattn_bwd``:
      g_i = dy_i / den_i,  h_i = -(dy_i . y_i) / den_i,
      dA_ij = g_i . v_j + h_i  (j <= i),  dV = A^T G,
      dK = dA * W  (A's derivative in the kernel entries),
      dX = dK * (1 + X),  dQ = dX K,  dK_keys = dX^T Q.
    gamma has one entry per head (the axis before L).  Returns (dq, dk, dv).
    """
    q, k, v, dy = _f64(q), _f64(k), _f64(v), _f64(dy)
    g = _f64(gamma)
    L = q.shape[-2]
    i = np.arange(L)
    d = (i[:, None] - i[None, :]).astype(np.float64)
    gb = g.reshape(g.shape + (1,) * 2)
    W = np.where(d >= 0, gb ** np.maximum(d, 0), 0.0)
    X = q @ np.swapaxes(k, -1, -2)
    A = taylor_kernel(X) * W
    den = A.sum(axis=-1)
    y = (A @ v) / den[..., None]
    gg = dy / den[..., None]
    h = -(dy * y).sum(axis=-1) / den
    dA = (gg @ np.swapaxes(v, -1, -2) + h[..., None]) * (d >= 0)
    dX = dA * W * (1.0 + X)
    dq = dX @ k
    dk = np.swapaxes(dX, -1, -2) @ q
    dv = np.swapaxes(A, -1, -2) @ gg
    return dq, dk, dv


def linattn_bwd_rows(q, k, v, dy, rows, chunk: int = 256):
    """The gradients of ``linattn_bwd`` at selected positions only, for
    sequences too long for the L x L matrices: dq_i, dk_i and dv_i for each
    position i in ``rows``.  Same definition, evaluated by rows: the row
    denominators and outputs come from the chunked forward (``linattn_chunked``,
    equal to the quadratic form), then g and h for every row, then
      dq_i = sum_{j<=i} (g_i.v_j + h_i)(1 + x_ij) k_j,
      dk_j = sum_{i>=j} (g_i.v_j + h_i)(1 + x_ij) q_i,
      dv_j = sum_{i>=j} K_ij g_i.
    Shapes: q, k [L, d_k], v, dy [L, d_v] (one head).  Returns three arrays
    [len(rows), d] in the order of ``rows``."""
    q, k, v, dy = _f64(q), _f64(k), _f64(v), _f64(dy)
    y, den, _, _ = linattn_chunked(q, k, v, chunk)
    g = dy / den[:, None]
    h = -(dy * y).sum(axis=-1) / den
    dq, dk, dv = [], [], []
    for i in rows:
        x = k[: i + 1] @ q[i]  # x_ij, j <= i
        c = (v[: i + 1] @ g[i] + h[i]) * (1.0 + x)
        dq.append(c @ k[: i + 1])
        xs = q[i:] @ k[i]  # x_si, s >= i (key i)
        cs = (g[i:] @ v[i] + h[i:]) * (1.0 + xs)
        dk.append(cs @ q[i:])
        dv.append(taylor_kernel(xs) @ g[i:])
    return np.array(dq), np.array(dk), np.array(dv)


def swa_bwd(q, k, v, dy, window: int = 64, scale: float = 1.0):
    """Gradients of the sliding-window softmax attention (``swa``, exact
    exponential weights) with respect to q, k and v.

    Per row i over its band of keys j (max(0, i - window + 1) <= j <= i):
    p_ij = softmax_j(s_ij) with s_ij = scale * q_i.k_j, y_i = sum_j p_ij v_j;
      dP_ij = dy_i . v_j,  D_i = sum_j p_ij dP_ij (= dy_i . y_i),
      dS_ij = p_ij (dP_ij - D_i)   (softmax Jacobian),
      dq_i = scale * sum_j dS_ij k_j,
      dk_j = scale * sum_i dS_ij q_i,  dv_j = sum_i p_ij dy_i  (sums over the
      rows whose band holds j).
    Returns (dq, dk, dv) as fp64 arrays shaped like q, k, v.
    """
    q, k, v, dy = _f64(q), _f64(k), _f64(v), _f64(dy)
    L = q.shape[-2]
    if window < 1:
        raise ValueError("window must be >= 1")
    idx = np.arange(L)[:, None] - (window - 1) + np.arange(window)[None, :]  # (L, W)
    valid = idx >= 0
    idxc = np.where(valid, idx, 0)
    kb = k[..., idxc, :]
    vb = v[..., idxc, :]
    s = scale * np.einsum("...ld,...lwd->...lw", q, kb)
    s = np.where(valid, s, -np.inf)
    p = np.exp(s - s.max(axis=-1, keepdims=True))
    p = p / p.sum(axis=-1, keepdims=True)
    dP = np.einsum("...ld,...lwd->...lw", dy, vb)
    D = (p * dP).sum(axis=-1, keepdims=True)
    dS = np.where(valid, p * (dP - D), 0.0)
    dq = scale * np.einsum("...lw,...lwd->...ld", dS, kb)
    # scatter the band back onto key positions
    lead = q.shape[:-2]
    dk = np.zeros(lead + k.shape[-2:])
    dv = np.zeros(lead + v.shape[-2:])
    for w in range(window):
        rows = np.nonzero(valid[:, w])[0]
        if rows.size == 0:
            continue
        # key idx[rows, w] receives row i's term of band slot w
        dk[..., idx[rows, w], :] += scale * dS[..., rows, w, None] * q[..., rows, :]
        dv[..., idx[rows, w], :] += p[..., rows, w, None] * dy[..., rows, :]
    return dq, dk, dv


# --------------------------------------------------------------------------
# BaseConv gating  [BLOG1, BaseConv block; README acknowledgements: short
# causal conv1d]
# --------------------------------------------------------------------------
def baseconv(x, u, h, bias=None):
    """y = u * conv(h, x): the gated short convolution of the BaseConv block.

    x, u [..., L, D] (u = linear(x), computed by the caller); h [D, K] the
    per-channel filter, tap s applied to x_{t-s}; bias [D] or None.
    conv(h, x)[t, c] = bias[c] + sum_{s=0}^{K-1} h[c, s] x[t-s, c], with
    x[t] = 0 before the first position.  Returns y [..., L, D] (fp64).
    """
    x, u, h = _f64(x), _f64(u), _f64(h)
    L = x.shape[-2]
    conv = np.zeros_like(x) + (0.0 if bias is None else _f64(bias))
    for s in range(h.shape[1]):
        if s < L:
            conv[..., s:, :] += h[:, s] * x[..., : L - s, :]
    return u * conv


# --------------------------------------------------------------------------
# Recurrent decode  [BLOG, paragraph on the state; README intro]
# --------------------------------------------------------------------------
class DecodeState:
    """Generation state of one Based layer for B sequences x H heads.

    S [B,H,273,d_v] and z [B,H,273] (the KV-state and K-state), a ring of the
    last ``window`` keys/values [B,H,window,d] where position t lives in slot
    t mod window, and t [B], the index of the next token of each sequence.
    """

    def __init__(self, S, z, ring_k, ring_v, t):
        self.S = _f64(S).copy()
        self.z = _f64(z).copy()
        self.ring_k = _f64(ring_k).copy()
        self.ring_v = _f64(ring_v).copy()
        self.t = np.asarray(t, dtype=np.int64).copy()
        self.window = self.ring_k.shape[-2]

    @classmethod
    def prefill(cls, k, v, window: int = 64):
        """State after consuming a context k, v [B,H,n,.] (all sequences n long)."""
        k, v = _f64(k), _f64(v)
        B, H, n, _ = k.shape
        S, z = linattn_state(k, v)
        rk = np.zeros((B, H, window, k.shape[-1]))
        rv = np.zeros((B, H, window, v.shape[-1]))
        for t in range(max(0, n - window), n):
            rk[:, :, t % window] = k[:, :, t]
            rv[:, :, t % window] = v[:, :, t]
        return cls(S, z, rk, rv, np.full(B, n))

    def step(self, q, k, v, scale: float = 1.0, gamma=None):
        """Consume one token per sequence: q, k [B,H,d_k], v [B,H,d_v].

        The state is updated with (k, v) first, so the token attends to
        itself; y_lin = phi(q)^T S / phi(q)^T z; (k, v) goes to ring slot
        t mod window; y_swa is the exact softmax over positions
        max(0, t - window + 1) .. t held in the ring.  With a per-head decay
        gamma [H] (the decayed variant) the state is S <- gamma S + phi(k) v^T,
        z <- gamma z + phi(k).  Returns (y_lin, y_swa).
        """
        q, k, v = _f64(q), _f64(k), _f64(v)
        pk, pq = phi(k), phi(q)
        if gamma is not None:
            g = _f64(gamma)
            self.S *= g[:, None, None]
            self.z *= g[:, None]
        self.S += pk[..., :, None] * v[..., None, :]
        self.z += pk
        num = np.einsum("bhf,bhfd->bhd", pq, self.S)
        den = np.einsum("bhf,bhf->bh", pq, self.z)
        y_lin = num / den[..., None]
        W = self.window
        B = q.shape[0]
        y_swa = np.empty_like(y_lin)
        for b in range(B):
            t = int(self.t[b])
            self.ring_k[b, :, t % W] = k[b]
            self.ring_v[b, :, t % W] = v[b]
            slots = [p % W for p in range(max(0, t - W + 1), t + 1)]
            kb = self.ring_k[b][:, slots]  # [H, n, d_k]
            vb = self.ring_v[b][:, slots]
            s = scale * np.einsum("hd,hnd->hn", q[b], kb)
            p = np.exp(s - s.max(axis=-1, keepdims=True))
            y_swa[b] = np.einsum("hn,hnd->hd", p, vb) / p.sum(axis=-1)[:, None]
        self.t += 1
        return y_lin, y_swa
