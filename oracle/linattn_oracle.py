"""Float64 CPU oracle for causal linear attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the package smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library
and imports nothing from it.

Sources (page titles as printed; section in brackets):
  [TR]  "Transformers are RNNs: Fast Autoregressive Transformers with Linear
        Attention" -- abstract: attention as a dot product of kernel feature
        maps, associativity turns O(N^2) into O(N), iterative (RNN) form.
  [SLA] "Simple linear attention language models balance the
        recall-throughput tradeoff" -- Knowl 3 (the causal output equation,
        the recurrent state equations, the Taylor kernel identity) and Knowl 5
        (prefill writes final states; generation updates the state, then reads
        it).
        Knowl 4 (sliding-window exact attention: query i sees keys
        max(1, i-w+1) .. i, a w-token key-value cache in generation).
  [HN]  the discussion page of "Transformers are RNNs" (hackerpapers),
        section "In the conversation": one comment writes the gated linear
        recurrences as a state decayed by a forget factor plus a gated outer
        product k v^T, read as C^T q; another describes the state-space layer
        whose transition is a scalar times the identity as causal linear
        attention with the coefficients a_1 ... a_t compounded.

Everything here is plain float64 numpy.  The functions follow the
definitions as written; there is no chunking, blocking or fusion.

Readings taken where the pages are silent:
  * elu(x)+1 is named by the [TR] abstract's source paper but not defined on
    the pages: ELU with alpha = 1, so phi(x) = x + 1 for x > 0 and exp(x) for
    x <= 0 (both branches give 1 at 0).
  * The Taylor map is [1, x, vec(x outer x)/sqrt(2)] with vec in row-major
    order, feature index 1 + d + i*d + j for x_i*x_j; [SLA] Knowl 3 gives only
    the identity phi(q).phi(k) = 1 + q.k + (q.k)^2/2 and "constant,
    first-order, second-order pairwise products".
  * The unordered-pair Taylor map ("taylor2sym") is [1, x, q_ab] with q_ab
    = x_a x_b for a < b and x_a^2 / sqrt(2) for a = b, pairs in row-major
    upper-triangular order; [SLA] Knowl 7 gives only its size.
  * The causal sum includes the diagonal (sum over j = 1..i, [SLA] Knowl 3).
  * No epsilon in the denominator; it is positive for both maps.
  * Generation updates the state first and then reads it ([SLA] Knowl 3
    recurrent equations; Knowl 5 second paragraph).
  * Scalar decay ([HN]): one coefficient a_t per sequence, head and position
    multiplies the whole state (S and z) before token t is added:
    S_t = a_t S_{t-1} + phi(k_t)^T v_t, z_t = a_t z_{t-1} + phi(k_t)^T.  The
    forget factor of the comment is a_t times the identity; its input gate is
    left to the caller (it can be folded into k_t or v_t).  Unrolled, token j
    enters the state at position i >= j with weight a_{j+1} ... a_i (1 for
    j = i).  The output is either the [SLA] Knowl 3 ratio of the decayed sums
    (normalize=True) or the comment's unnormalised read phi(q_t) S_t
    (normalize=False).
  * Sliding-window attention ([SLA] Knowl 4) is softmax attention with the
    score scale * q.k; the pages name it exact softmax attention and the
    page on the Taylor approximation calls the target "standard scaled
    dot-product attention", so the default scale is 1/sqrt(d) (the kernels
    take it as an argument).  The window counts the query's own key, so
    w = 1 returns v_i.  The generation cache is a ring of w slots: token t
    lives in slot t mod w.

Parity pins (all in tests/test_oracle_pins.py): exact rational brute force,
quadratic == recurrent, Taylor identity and its exp limit, torch's elu,
closed-form special cases (first token, constant key, zero Taylor query,
constant value), convex-hull and positivity invariants, final-state closed
form, decode continuation, and a hand-worked golden example.  Every function
below is pinned; none is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

ELU1 = "elu1"
TAYLOR2 = "taylor2"
TAYLOR2_SYM = "taylor2sym"
MAPS = (ELU1, TAYLOR2, TAYLOR2_SYM)


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# Feature maps
# --------------------------------------------------------------------------
def phi_elu1(x) -> np.ndarray:
    """elu(x) + 1 elementwise, ELU with alpha = 1 (reading; see header)."""
    x = _f64(x)
    return np.where(x > 0.0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def phi_taylor2(x) -> np.ndarray:
    """Second-order Taylor map [1, x, vec(x (x) x)/sqrt(2)] over the last axis.

    [SLA] Knowl 3: the map is the concatenation of a constant term, the
    first-order coordinates and the second-order pairwise products, chosen so
    that phi(q).phi(k) = 1 + q.k + (q.k)^2/2.  Output width 1 + d + d*d.
    """
    x = _f64(x)
    d = x.shape[-1]
    ones = np.ones(x.shape[:-1] + (1,), dtype=np.float64)
    outer = x[..., :, None] * x[..., None, :]             # [..., d, d], (i, j)
    quad = outer.reshape(x.shape[:-1] + (d * d,)) / math.sqrt(2.0)
    return np.concatenate([ones, x, quad], axis=-1)


def sym_pairs(d: int):
    """Unordered pairs (a, b), a <= b, in row-major upper-triangular order:
    (0,0), (0,1), ..., (0,d-1), (1,1), ..., (d-1,d-1)."""
    return [(a, b) for a in range(d) for b in range(a, d)]


def phi_taylor2_sym(x) -> np.ndarray:
    """Second-order Taylor map on unordered pairs (reading; see header).

    [SLA] Knowl 7 counts the generation state of the Taylor map as
    (d + 1)(1 + 3d'/2 + d'^2/2) per head: constant, d' first-order and
    d'(d' + 1)/2 second-order features, i.e. each unordered pair once.
    Keeping phi(q).phi(k) = 1 + q.k + (q.k)^2/2 (Knowl 3) fixes the weights:
    (q.k)^2/2 = sum_a q_a^2 k_a^2 / 2 + sum_{a<b} q_a q_b k_a k_b, so the
    square x_a^2 carries 1/sqrt(2) and the product x_a x_b (a < b) weight 1.
    Layout [1, x, pairs in sym_pairs order]; width 1 + d + d(d+1)/2.
    """
    x = _f64(x)
    d = x.shape[-1]
    ones = np.ones(x.shape[:-1] + (1,), dtype=np.float64)
    quad = np.stack([x[..., a] * x[..., b] * (1.0 / math.sqrt(2.0) if a == b else 1.0)
                     for a, b in sym_pairs(d)], axis=-1)
    return np.concatenate([ones, x, quad], axis=-1)


def feature_dim(fmap: str, d_k: int) -> int:
    if fmap == ELU1:
        return d_k
    if fmap == TAYLOR2:
        return 1 + d_k + d_k * d_k
    if fmap == TAYLOR2_SYM:
        return 1 + d_k + d_k * (d_k + 1) // 2
    raise ValueError(f"unknown feature map {fmap!r}")


def feature_map(x, fmap: str) -> np.ndarray:
    if fmap == ELU1:
        return phi_elu1(x)
    if fmap == TAYLOR2:
        return phi_taylor2(x)
    if fmap == TAYLOR2_SYM:
        return phi_taylor2_sym(x)
    raise ValueError(f"unknown feature map {fmap!r}")


# --------------------------------------------------------------------------
# The causal output: definition (quadratic masked form)
# --------------------------------------------------------------------------
def attention_quadratic(q, k, v, fmap: str) -> np.ndarray:
    """y_i = phi(q_i) sum_{j<=i} phi(k_j)^T v_j / phi(q_i) sum_{j<=i} phi(k_j)^T.

    [SLA] Knowl 3, first equation, written as ((phi(Q) phi(K)^T) * M) V divided
    row by row by ((phi(Q) phi(K)^T) * M) 1, with M lower-triangular including
    the diagonal.  q, k: [..., N, d_k]; v: [..., N, d_v].  O(N^2) memory: for
    small N only (see attention_rows for single rows at any N).
    """
    fq = feature_map(q, fmap)
    fk = feature_map(k, fmap)
    v = _f64(v)
    n = fq.shape[-2]
    scores = fq @ np.swapaxes(fk, -1, -2)                   # [..., N, N]
    mask = np.tril(np.ones((n, n), dtype=np.float64))
    w = scores * mask
    num = w @ v
    den = w.sum(axis=-1)
    return num / den[..., None]


def attention_rows(q, k, v, fmap: str, rows) -> np.ndarray:
    """The same definition evaluated only at the (0-based) positions `rows`.

    q, k: [N, d_k], v: [N, d_v] for ONE sequence and head.  Each output row
    t needs phi(q_t) and phi(k_1..k_t): O(t * (D + d_v)) work, so it can be
    used at any sequence length.  Returns [len(rows), d_v].
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    out = np.empty((len(rows), v.shape[-1]), dtype=np.float64)
    for r, t in enumerate(rows):
        fq = feature_map(q[t], fmap)                        # [D]
        fk = feature_map(k[: t + 1], fmap)                  # [t+1, D]
        w = fk @ fq                                         # [t+1]
        out[r] = (w @ v[: t + 1]) / w.sum()
    return out


# --------------------------------------------------------------------------
# Recurrent form
# --------------------------------------------------------------------------
def decode_step(q, k, v, S, z, fmap: str):
    """One recurrent step from the state (S, z); returns (y, S_new, z_new).

    [SLA] Knowl 3 second equation: s_i = s_{i-1} + phi(k_i)^T v_i,
    z_i = z_{i-1} + phi(k_i)^T, y_i = phi(q_i) s_i / phi(q_i) z_i -- the state
    is updated before it is read (Knowl 5, generation paragraph).
    q, k: [..., d_k]; v: [..., d_v]; S: [..., D, d_v]; z: [..., D].
    The inputs are not modified.
    """
    fq = feature_map(q, fmap)
    fk = feature_map(k, fmap)
    v = _f64(v)
    S_new = _f64(S) + fk[..., :, None] * v[..., None, :]
    z_new = _f64(z) + fk
    num = np.einsum("...r,...rc->...c", fq, S_new)
    den = np.einsum("...r,...r->...", fq, z_new)
    return num / den[..., None], S_new, z_new


def attention_recurrent(q, k, v, fmap: str, S0=None, z0=None):
    """Run the recurrence over all N positions; returns (y, S_N, z_N).

    q, k: [..., N, d_k]; v: [..., N, d_v].  The state starts at zero (the sums
    of the definition start at j = 1) unless (S0, z0) is given, in which case
    the sequence continues from that state.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    batch = q.shape[:-2]
    n = q.shape[-2]
    D = feature_dim(fmap, q.shape[-1])
    dv = v.shape[-1]
    S = np.zeros(batch + (D, dv)) if S0 is None else _f64(S0).copy()
    z = np.zeros(batch + (D,)) if z0 is None else _f64(z0).copy()
    y = np.empty(batch + (n, dv), dtype=np.float64)
    for t in range(n):
        y[..., t, :], S, z = decode_step(q[..., t, :], k[..., t, :],
                                         v[..., t, :], S, z, fmap)
    return y, S, z


def final_state(k, v, fmap: str):
    """Closed form of the state after N tokens: S_N = phi(K)^T V, z_N = phi(K)^T 1.

    [SLA] Knowl 3 (the recurrence summed) and Knowl 5 (prefill optionally
    writes the final states for later generation).
    """
    fk = feature_map(k, fmap)
    v = _f64(v)
    S = np.swapaxes(fk, -1, -2) @ v
    z = fk.sum(axis=-2)
    return S, z


# --------------------------------------------------------------------------
# Scalar-decay (gated) form
# --------------------------------------------------------------------------
def decay_matrix(a) -> np.ndarray:
    """W[..., i, j] = a_{j+1} a_{j+2} ... a_i for j <= i (an empty product, 1,
    on the diagonal) and 0 for j > i: the compounded coefficients of the
    scalar-transition state-space form ([HN] comment on the duality).

    a: [..., N].  Built column by column from explicit products (no
    logarithms), so a_t = 0 gives exact zeros.  O(N^2): small N only.
    """
    a = _f64(a)
    n = a.shape[-1]
    W = np.zeros(a.shape[:-1] + (n, n), dtype=np.float64)
    for i in range(n):
        W[..., i, i] = 1.0
        for j in range(i - 1, -1, -1):
            W[..., i, j] = W[..., i, j + 1] * a[..., j + 1]
    return W


def attention_gated_quadratic(q, k, v, a, fmap: str, normalize=True) -> np.ndarray:
    """Gated causal output, definition form.

    y_i = sum_{j<=i} W_ij phi(q_i).phi(k_j) v_j  [/ sum_{j<=i} W_ij phi(q_i).phi(k_j)]
    with W = decay_matrix(a): the [SLA] Knowl 3 masked form with the causal
    mask replaced by the compounded decays ([HN]).  q, k: [..., N, d_k];
    v: [..., N, d_v]; a: [..., N].
    """
    fq = feature_map(q, fmap)
    fk = feature_map(k, fmap)
    v = _f64(v)
    w = (fq @ np.swapaxes(fk, -1, -2)) * decay_matrix(a)
    num = w @ v
    if not normalize:
        return num
    return num / w.sum(axis=-1)[..., None]


def gated_decode_step(q, k, v, a, S, z, fmap: str, normalize=True):
    """One gated step: S' = a S + phi(k)^T v, z' = a z + phi(k)^T, then the read
    phi(q) S' [/ phi(q) z'].  Returns (y, S', z'); the inputs are not modified.

    q, k: [..., d_k]; v: [..., d_v]; a: [...]; S: [..., D, d_v]; z: [..., D].
    """
    fq = feature_map(q, fmap)
    fk = feature_map(k, fmap)
    v = _f64(v)
    a = _f64(a)
    S_new = a[..., None, None] * _f64(S) + fk[..., :, None] * v[..., None, :]
    z_new = a[..., None] * _f64(z) + fk
    num = np.einsum("...r,...rc->...c", fq, S_new)
    if not normalize:
        return num, S_new, z_new
    den = np.einsum("...r,...r->...", fq, z_new)
    return num / den[..., None], S_new, z_new


def attention_gated_recurrent(q, k, v, a, fmap: str, S0=None, z0=None,
                              normalize=True):
    """The gated recurrence over all N positions; returns (y, S_N, z_N).

    The state starts at zero unless (S0, z0) is given (it is then decayed by
    a_1 before token 1 is added, like any earlier state).
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    a = _f64(a)
    batch = q.shape[:-2]
    n = q.shape[-2]
    D = feature_dim(fmap, q.shape[-1])
    dv = v.shape[-1]
    S = np.zeros(batch + (D, dv)) if S0 is None else _f64(S0).copy()
    z = np.zeros(batch + (D,)) if z0 is None else _f64(z0).copy()
    y = np.empty(batch + (n, dv), dtype=np.float64)
    for t in range(n):
        y[..., t, :], S, z = gated_decode_step(q[..., t, :], k[..., t, :],
                                               v[..., t, :], a[..., t], S, z,
                                               fmap, normalize)
    return y, S, z


def _suffix_products(a) -> np.ndarray:
    """P[..., j] = a_{j+1} ... a_N (1 for j = N): the weight of token j in the
    state after the last token.  Explicit running products, last to first."""
    a = _f64(a)
    n = a.shape[-1]
    P = np.empty(a.shape, dtype=np.float64)
    run = np.ones(a.shape[:-1], dtype=np.float64)
    for j in range(n - 1, -1, -1):
        P[..., j] = run
        run = run * a[..., j]
    return P


def gated_final_state(k, v, a, fmap: str, S0=None, z0=None):
    """State after N gated tokens, summed in closed form:
    S_N = sum_j (a_{j+1} ... a_N) phi(k_j)^T v_j + (a_1 ... a_N) S0, and the same
    for z with v replaced by 1."""
    fk = feature_map(k, fmap)
    v = _f64(v)
    P = _suffix_products(a)                                  # [..., N]
    S = np.swapaxes(fk * P[..., None], -1, -2) @ v
    z = (fk * P[..., None]).sum(axis=-2)
    if S0 is not None:
        total = np.prod(_f64(a), axis=-1)
        S = S + total[..., None, None] * _f64(S0)
        z = z + total[..., None] * _f64(z0)
    return S, z


def attention_gated_rows(q, k, v, a, fmap: str, rows, normalize=True) -> np.ndarray:
    """The gated definition at the (0-based) positions `rows` of ONE sequence
    and head (q, k: [N, d_k], v: [N, d_v], a: [N]); any N.  Row t weighs
    token j <= t by a_{j+1} ... a_t."""
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    a = _f64(a)
    out = np.empty((len(rows), v.shape[-1]), dtype=np.float64)
    for r, t in enumerate(rows):
        fq = feature_map(q[t], fmap)
        fk = feature_map(k[: t + 1], fmap)
        w = (fk @ fq) * _suffix_products(a[: t + 1])
        out[r] = w @ v[: t + 1]
        if normalize:
            out[r] /= w.sum()
    return out


# --------------------------------------------------------------------------
# Sliding-window softmax attention ([SLA] Knowl 4)
# --------------------------------------------------------------------------
def swa_attention(q, k, v, window: int, scale: float) -> np.ndarray:
    """y_i = sum_j p_ij v_j, p_i = softmax over j in [i - w + 1, i] (0-based,
    clipped at 0) of scale * q_i . k_j.

    q, k: [..., N, d_k]; v: [..., N, d_v].  Dense band mask: small N only
    (swa_rows evaluates single rows at any N).
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    n = q.shape[-2]
    s = scale * (q @ np.swapaxes(k, -1, -2))
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    band = (j <= i) & (j > i - window)
    s = np.where(band, s, -np.inf)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    return p @ v


def swa_rows(q, k, v, window: int, scale: float, rows) -> np.ndarray:
    """The same definition at the (0-based) positions `rows` of ONE sequence
    and head (q, k: [N, d_k], v: [N, d_v]); O(w d) per row, any N."""
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    out = np.empty((len(rows), v.shape[-1]), dtype=np.float64)
    for r, t in enumerate(rows):
        lo = max(0, t - window + 1)
        s = scale * (k[lo:t + 1] @ q[t])
        p = np.exp(s - s.max())
        out[r] = (p / p.sum()) @ v[lo:t + 1]
    return out


def swa_cache_after_prefill(k, v, window: int):
    """The w-slot key/value cache after N tokens: token t in slot t mod w for
    the last min(N, w) tokens; slots never written hold zeros.
    k: [..., N, d_k]; v: [..., N, d_v] -> ([..., w, d_k], [..., w, d_v])."""
    k = _f64(k)
    v = _f64(v)
    n = k.shape[-2]
    kc = np.zeros(k.shape[:-2] + (window, k.shape[-1]))
    vc = np.zeros(v.shape[:-2] + (window, v.shape[-1]))
    for t in range(max(0, n - window), n):
        kc[..., t % window, :] = k[..., t, :]
        vc[..., t % window, :] = v[..., t, :]
    return kc, vc


def swa_decode_step(q, k, v, k_cache, v_cache, pos: int, window: int, scale: float):
    """One generation step at 0-based position `pos`: write (k, v) into slot
    pos mod w, then attend over the min(pos + 1, w) most recent tokens.
    q, k: [..., d_k]; v: [..., d_v]; caches [..., w, d].  Returns
    (y, k_cache', v_cache'); the inputs are not modified."""
    kc = _f64(k_cache).copy()
    vc = _f64(v_cache).copy()
    kc[..., pos % window, :] = _f64(k)
    vc[..., pos % window, :] = _f64(v)
    valid = [t % window for t in range(max(0, pos - window + 1), pos + 1)]
    s = scale * np.einsum("...d,...jd->...j", _f64(q), kc[..., valid, :])
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    y = np.einsum("...j,...jd->...d", p, vc[..., valid, :])
    return y, kc, vc


def kernel_value(q, k, fmap: str) -> np.ndarray:
    """phi(q) . phi(k) over the last axis, through the explicit features."""
    return np.sum(feature_map(q, fmap) * feature_map(k, fmap), axis=-1)
