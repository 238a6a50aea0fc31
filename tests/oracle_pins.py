"""Pins for the float64 oracle: checks against things other than itself.

Each pin is a function pin(o) that raises AssertionError when the oracle
namespace `o` is wrong.  The real oracle must pass all of them
(test_oracle_pins.py); copies of it with a planted mistake must fail at least
one (test_oracle_mutants.py).

What pins what (sources: "Simple linear attention language models balance the
recall-throughput tradeoff" = SLA; "Transformers are RNNs ..." = TR):
  exact_*          exact rational brute force of SLA Knowl 3's causal output
                   equation, written with Python fractions from scratch
  quad_vs_rec      the definition (SLA Knowl 3 eq. 1) equals the recurrence
                   (eq. 2) -- the TR abstract's "iterative implementation"
  taylor_identity  SLA Knowl 3: phi(q).phi(k) = 1 + q.k + (q.k)^2 / 2
  taylor_exp       the same kernel is exp's second-order Taylor polynomial:
                   |kernel - exp(s)| <= |s|^3 / 6 * exp(|s|)
  taylor_layout    hand-written feature vector for x = (1, 2, -3)
  taylor_sym_*     the unordered-pair map: SLA Knowl 7's state size (153 at
                   d' = 16), the Knowl 3 identity, hand-written features,
                   and the fold relation to the ordered-pair state
  elu_torch        torch.nn.functional.elu(x) + 1 (a library routine)
  gated_*          the scalar-decay form (the gated recurrence and the
                   scalar-transition duality in the Hacker News comments on
                   "Transformers are RNNs" = HN): exact rational brute force
                   with the decay products multiplied out, scipy's IIR filter
                   for a constant decay, a reset (a_t = 0) cutting the past
                   off, a = 0 and a = 1 as closed forms, continuation through
                   a state, and the final state summed three ways
  swa_*            sliding-window softmax attention (SLA Knowl 4): torch's
                   scaled_dot_product_attention with a causal or band mask
                   (a library routine), w = 1, a two-key closed form through
                   the logistic function, constant keys as a moving average
                   (numpy's convolve), locality, rows, and the ring cache
                   with decode steps continuing a prefill
  closed forms     first token, constant key, zero Taylor query, constant v,
                   linearity in v, convex hull, positivity, final state,
                   decode continuation, sampled rows, hand-worked golden file
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------- exact ----
def _exact_kernel(fmap, qi, kj):
    """phi(q).phi(k) from the explicit features, exactly (Fractions).

    ELU1 for non-negative inputs only (there phi(x) = x + 1 is rational).
    TAYLOR2 multiplies the feature vectors term by term: 1*1, q_a*k_a, and
    (q_a q_b / sqrt2)(k_a k_b / sqrt2) = q_a q_b k_a k_b / 2.
    """
    if fmap == "elu1":
        assert all(x >= 0 for x in qi) and all(x >= 0 for x in kj)
        return sum((a + 1) * (b + 1) for a, b in zip(qi, kj))
    d = len(qi)
    tot = Fraction(1)
    tot += sum(qi[a] * kj[a] for a in range(d))
    tot += sum(qi[a] * qi[b] * kj[a] * kj[b] for a in range(d)
               for b in range(d)) / 2
    return tot


def _exact_kernel_sym(qi, kj):
    """phi(q).phi(k) through the unordered-pair features, exactly: 1*1,
    q_a*k_a, (q_a^2/sqrt2)(k_a^2/sqrt2) = q_a^2 k_a^2 / 2, and
    (q_a q_b)(k_a k_b) for a < b (SLA Knowl 7 counts each pair once)."""
    d = len(qi)
    tot = Fraction(1)
    tot += sum(qi[a] * kj[a] for a in range(d))
    tot += sum(qi[a] * qi[a] * kj[a] * kj[a] for a in range(d)) / 2
    tot += sum(qi[a] * qi[b] * kj[a] * kj[b] for a in range(d) for b in range(a + 1, d))
    return tot


def _exact_outputs(fmap, q, k, v):
    n = len(q)
    out = []
    for i in range(n):
        w = [_exact_kernel_sym(q[i], k[j]) if fmap == "taylor2sym"
             else _exact_kernel(fmap, q[i], k[j]) for j in range(i + 1)]
        den = sum(w)
        out.append([sum(w[j] * v[j][c] for j in range(i + 1)) / den
                    for c in range(len(v[0]))])
    return out


def _rational_inputs(seed, n, dk, dv, nonneg):
    r = _rng(seed)
    lo = 0 if nonneg else -3
    q = [[Fraction(int(r.integers(lo, 4)), int(r.integers(1, 4)))
          for _ in range(dk)] for _ in range(n)]
    k = [[Fraction(int(r.integers(lo, 4)), int(r.integers(1, 4)))
          for _ in range(dk)] for _ in range(n)]
    v = [[Fraction(int(r.integers(-5, 6)), int(r.integers(1, 5)))
          for _ in range(dv)] for _ in range(n)]
    return q, k, v


def _as_f64(rows):
    return np.array([[float(x) for x in row] for row in rows])


def _check_exact(o, fmap, nonneg):
    for seed, (n, dk, dv) in enumerate([(1, 1, 1), (5, 2, 3), (9, 3, 2),
                                        (12, 4, 4)]):
        q, k, v = _rational_inputs(100 + seed, n, dk, dv, nonneg)
        want = _as_f64(_exact_outputs(fmap, q, k, v))
        qf, kf, vf = _as_f64(q), _as_f64(k), _as_f64(v)
        got_q = o.attention_quadratic(qf, kf, vf, fmap)
        got_r, _, _ = o.attention_recurrent(qf, kf, vf, fmap)
        got_rows = o.attention_rows(qf, kf, vf, fmap, list(range(n)))
        for got in (got_q, got_r, got_rows):
            assert _rel(got, want) < 1e-13, (fmap, n, dk, dv)


def pin_exact_elu1(o):
    _check_exact(o, "elu1", nonneg=True)


def pin_exact_taylor2(o):
    _check_exact(o, "taylor2", nonneg=False)


def pin_exact_taylor2_sym(o):
    _check_exact(o, "taylor2sym", nonneg=False)


def pin_taylor_sym_size_and_identity(o):
    """SLA Knowl 7: the unordered-pair map has 1 + 3d/2 + d^2/2 features
    (153 at d = 16); SLA Knowl 3: its kernel is still 1 + q.k + (q.k)^2/2."""
    for d in (1, 2, 3, 16):
        assert 2 * o.feature_dim("taylor2sym", d) == 2 + 3 * d + d * d
    assert o.feature_dim("taylor2sym", 16) == 153
    r = _rng(21)
    q = r.standard_normal((40, 16)) * 0.6
    k = r.standard_normal((40, 16)) * 0.6
    s = np.sum(q * k, axis=-1)
    got = o.kernel_value(q, k, "taylor2sym")
    assert _rel(got, 1.0 + s + 0.5 * s * s) < 1e-13
    assert o.feature_map(q, "taylor2sym").shape == (40, 153)


def pin_taylor_sym_layout(o):
    """Hand-written unordered-pair features of x = (1, 2, -3)."""
    r2 = math.sqrt(2.0)
    want = np.array([1.0, 1.0, 2.0, -3.0,
                     1.0 / r2, 2.0, -3.0, 4.0 / r2, -6.0, 9.0 / r2])
    got = o.feature_map(np.array([1.0, 2.0, -3.0]), "taylor2sym")
    assert np.allclose(got, want, rtol=0, atol=1e-15)


def pin_taylor_sym_fold(o):
    """The unordered-pair state is the ordered-pair state folded: a square
    row is kept, and the pair (a, b), a < b, is (S_ab + S_ba) / sqrt(2)."""
    r = _rng(22)
    d, dv = 4, 5
    k = r.standard_normal((3, 30, d))
    v = r.standard_normal((3, 30, dv))
    S, z = o.final_state(k, v, "taylor2")
    Ss, zs = o.final_state(k, v, "taylor2sym")
    base = 1 + d
    rows, zrows = [], []
    for a in range(d):
        for b in range(a, d):
            ab, ba = base + a * d + b, base + b * d + a
            if a == b:
                rows.append(S[:, ab]); zrows.append(z[:, ab])
            else:
                rows.append((S[:, ab] + S[:, ba]) / math.sqrt(2.0))
                zrows.append((z[:, ab] + z[:, ba]) / math.sqrt(2.0))
    want_S = np.concatenate([S[:, :base], np.stack(rows, axis=1)], axis=1)
    want_z = np.concatenate([z[:, :base], np.stack(zrows, axis=1)], axis=1)
    assert _rel(Ss, want_S) < 1e-12 and _rel(zs, want_z) < 1e-12


# ---------------------------------------------------------- equivalences ----
def pin_quad_vs_rec(o):
    for fmap in ("elu1", "taylor2", "taylor2sym"):
        for seed, (b, n, dk, dv) in enumerate([(1, 1, 3, 2), (2, 2, 1, 1),
                                               (2, 17, 4, 3), (1, 64, 16, 8),
                                               (1, 256, 16, 16)]):
            r = _rng(seed)
            q = r.standard_normal((b, 2, n, dk)) * 0.5
            k = r.standard_normal((b, 2, n, dk)) * 0.5
            v = r.standard_normal((b, 2, n, dv))
            yq = o.attention_quadratic(q, k, v, fmap)
            yr, S, z = o.attention_recurrent(q, k, v, fmap)
            assert _rel(yr, yq) < 1e-12, (fmap, n, dk)


def pin_rows_match_definition(o):
    for fmap in ("elu1", "taylor2", "taylor2sym"):
        r = _rng(7)
        q = r.standard_normal((40, 5))
        k = r.standard_normal((40, 5))
        v = r.standard_normal((40, 3))
        rows = [0, 1, 13, 39]
        full = o.attention_quadratic(q, k, v, fmap)[rows]
        part = o.attention_rows(q, k, v, fmap, rows)
        assert _rel(part, full) < 1e-13


# -------------------------------------------------------------- features ----
def pin_taylor_identity(o):
    r = _rng(3)
    for d in (1, 2, 16):
        q = r.standard_normal((50, d))
        k = r.standard_normal((50, d))
        s = np.einsum("nd,nd->n", q, k)
        want = 1.0 + s + 0.5 * s * s
        got = o.kernel_value(q, k, "taylor2")
        assert np.max(np.abs(got - want)) < 1e-12 * np.max(np.abs(want))
        assert o.feature_map(q, "taylor2").shape == (50, 1 + d + d * d)
        assert o.feature_dim("taylor2", d) == 1 + d + d * d


def pin_taylor_exp(o):
    r = _rng(4)
    q = r.standard_normal((200, 16)) * 0.15
    k = r.standard_normal((200, 16)) * 0.15
    s = np.einsum("nd,nd->n", q, k)
    got = o.kernel_value(q, k, "taylor2")
    bound = np.abs(s) ** 3 / 6.0 * np.exp(np.abs(s)) + 1e-15
    assert np.all(np.abs(got - np.exp(s)) <= bound)


def pin_taylor_layout(o):
    r2 = 1.0 / math.sqrt(2.0)
    x = np.array([1.0, 2.0, -3.0])
    want = [1.0, 1.0, 2.0, -3.0,
            1 * r2, 2 * r2, -3 * r2,
            2 * r2, 4 * r2, -6 * r2,
            -3 * r2, -6 * r2, 9 * r2]
    assert np.allclose(o.phi_taylor2(x), want, rtol=0, atol=1e-15)


def pin_elu_torch(o):
    import torch

    x = np.concatenate([np.linspace(-30, 30, 2001), [0.0, -0.0, 1e-30,
                                                     -1e-30]])
    want = (torch.nn.functional.elu(torch.from_numpy(x), alpha=1.0)
            + 1.0).numpy()
    got = o.phi_elu1(x)
    assert np.max(np.abs(got - want)) <= 1e-15 * np.max(np.abs(want))
    assert o.phi_elu1(np.array([0.0]))[0] == 1.0
    assert o.feature_dim("elu1", 64) == 64


# ---------------------------------------------------- closed-form cases ----
def pin_first_token(o):
    for fmap in ("elu1", "taylor2", "taylor2sym"):
        r = _rng(5)
        q = r.standard_normal((3, 1, 4))
        k = r.standard_normal((3, 1, 4))
        v = r.standard_normal((3, 1, 6))
        for y in (o.attention_quadratic(q, k, v, fmap),
                  o.attention_recurrent(q, k, v, fmap)[0]):
            assert _rel(y, v) < 1e-15


def _cummean(v):
    n = v.shape[-2]
    return np.cumsum(v, axis=-2) / np.arange(1, n + 1)[:, None]


def pin_constant_key(o):
    for fmap in ("elu1", "taylor2", "taylor2sym"):
        r = _rng(6)
        q = r.standard_normal((30, 4))
        k = np.tile(r.standard_normal((1, 4)), (30, 1))
        v = r.standard_normal((30, 3))
        for y in (o.attention_quadratic(q, k, v, fmap),
                  o.attention_recurrent(q, k, v, fmap)[0]):
            assert _rel(y, _cummean(v)) < 1e-12


def pin_zero_taylor_query(o):
    r = _rng(8)
    q = np.zeros((25, 4))
    k = r.standard_normal((25, 4)) * 2.0
    v = r.standard_normal((25, 5))
    for y in (o.attention_quadratic(q, k, v, "taylor2"),
              o.attention_recurrent(q, k, v, "taylor2")[0]):
        assert _rel(y, _cummean(v)) < 1e-12


def pin_constant_and_linear_v(o):
    for fmap in ("elu1", "taylor2", "taylor2sym"):
        r = _rng(9)
        q = r.standard_normal((20, 3))
        k = r.standard_normal((20, 3))
        c = r.standard_normal(4)
        v1 = r.standard_normal((20, 4))
        v2 = r.standard_normal((20, 4))
        y_c = o.attention_recurrent(q, k, np.tile(c, (20, 1)), fmap)[0]
        assert _rel(y_c, np.tile(c, (20, 1))) < 1e-13
        y1 = o.attention_quadratic(q, k, v1, fmap)
        y2 = o.attention_quadratic(q, k, v2, fmap)
        y12 = o.attention_quadratic(q, k, 2.0 * v1 - 3.0 * v2, fmap)
        assert _rel(y12, 2.0 * y1 - 3.0 * y2) < 1e-12


def pin_convex_hull_and_positive(o):
    for fmap in ("elu1", "taylor2", "taylor2sym"):
        r = _rng(10)
        q = r.standard_normal((2, 300, 8))
        k = r.standard_normal((2, 300, 8))
        v = r.standard_normal((2, 300, 5))
        y = o.attention_recurrent(q, k, v, fmap)[0]
        lo = np.minimum.accumulate(v, axis=-2)
        hi = np.maximum.accumulate(v, axis=-2)
        assert np.all(y >= lo - 1e-12) and np.all(y <= hi + 1e-12)
        fk = o.feature_map(k, fmap)
        fq = o.feature_map(q, fmap)
        den = np.einsum("...ir,...jr->...ij", fq, fk)
        if fmap == "elu1":
            assert np.all(fk > 0)
            assert np.all(den > 0)
        else:
            # 1 + s + s^2/2 >= 1/2 for every real s
            assert np.all(den >= 0.5 - 1e-12)


def pin_final_state(o):
    for fmap, dk, dv in (("elu1", 6, 6), ("taylor2", 3, 13), ("taylor2sym", 3, 13)):
        r = _rng(11)
        q = r.standard_normal((2, 3, 33, dk))
        k = r.standard_normal((2, 3, 33, dk))
        v = r.standard_normal((2, 3, 33, dv))
        _, S, z = o.attention_recurrent(q, k, v, fmap)
        S2, z2 = o.final_state(k, v, fmap)
        D = o.feature_dim(fmap, dk)
        assert S.shape == (2, 3, D, dv) and z.shape == (2, 3, D)
        assert S2.shape == S.shape and z2.shape == z.shape
        assert _rel(S, S2) < 1e-12 and _rel(z, z2) < 1e-12
        # independent construction: outer products summed by a plain loop
        fk = o.feature_map(k, fmap)
        S3 = np.zeros_like(S)
        for t in range(33):
            S3 += np.einsum("bhr,bhc->bhrc", fk[:, :, t], v[:, :, t])
        assert _rel(S, S3) < 1e-12


def pin_decode_continuation(o):
    for fmap in ("elu1", "taylor2", "taylor2sym"):
        r = _rng(12)
        q = r.standard_normal((2, 40, 4))
        k = r.standard_normal((2, 40, 4))
        v = r.standard_normal((2, 40, 3))
        y_all, S_all, z_all = o.attention_recurrent(q, k, v, fmap)
        y_a, S_a, z_a = o.attention_recurrent(q[:, :25], k[:, :25],
                                              v[:, :25], fmap)
        y_b, S_b, z_b = o.attention_recurrent(q[:, 25:], k[:, 25:],
                                              v[:, 25:], fmap, S_a, z_a)
        assert _rel(np.concatenate([y_a, y_b], axis=1), y_all) < 1e-12
        assert _rel(S_b, S_all) < 1e-12 and _rel(z_b, z_all) < 1e-12
        S0 = S_a.copy()
        _ = o.decode_step(q[:, 25], k[:, 25], v[:, 25], S_a, z_a, fmap)
        assert np.array_equal(S0, S_a), "decode_step must not modify inputs"


# --------------------------------------------------------------- golden ----
def _parse(s):
    """'a/b' or 'a/b*sqrt2' -> float."""
    s = str(s).strip()
    mult = 1.0
    if s.endswith("*sqrt2"):
        mult = math.sqrt(2.0)
        s = s[: -len("*sqrt2")]
    elif s.endswith("/sqrt2"):
        mult = 1.0 / math.sqrt(2.0)
        s = s[: -len("/sqrt2")]
    return float(Fraction(s)) * mult


def pin_golden_handworked(o):
    with open(os.path.join(GOLDEN, "handworked.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        fmap = case["map"]
        q = np.array(case["q"], dtype=np.float64)
        k = np.array(case["k"], dtype=np.float64)
        v = np.array(case["v"], dtype=np.float64)
        y_want = np.array([[_parse(x) for x in row] for row in case["y"]])
        S_want = np.array([[_parse(x) for x in row] for row in case["S"]])
        z_want = np.array([_parse(x) for x in case["z"]])
        y, S, z = o.attention_recurrent(q, k, v, fmap)
        assert _rel(y, y_want) < 1e-14, case["name"]
        assert _rel(o.attention_quadratic(q, k, v, fmap), y_want) < 1e-14
        assert _rel(S, S_want) < 1e-14 and _rel(z, z_want) < 1e-14


# ----------------------------------------------------------- gated form ----
def _exact_gated(fmap, q, k, v, a, normalize):
    """HN gated recurrence unrolled, exactly: token j's weight at position i
    is the product a_{j+1} ... a_i, multiplied out factor by factor."""
    n, dv = len(q), len(v[0])
    out = []
    for i in range(n):
        w = []
        for j in range(i + 1):
            c = Fraction(1)
            for t in range(j + 1, i + 1):
                c *= a[t]
            kv = (_exact_kernel_sym(q[i], k[j]) if fmap == "taylor2sym"
                  else _exact_kernel(fmap, q[i], k[j]))
            w.append(c * kv)
        num = [sum(w[j] * v[j][col] for j in range(i + 1)) for col in range(dv)]
        if normalize:
            den = sum(w)
            num = [x / den for x in num]
        out.append(num)
    return out


_GATES = [Fraction(0), Fraction(1, 4), Fraction(1, 2), Fraction(2, 3), Fraction(1)]


def _check_exact_gated(o, fmap, nonneg):
    for seed, (n, dk, dv) in enumerate([(1, 1, 1), (6, 2, 3), (11, 3, 2)]):
        q, k, v = _rational_inputs(200 + seed, n, dk, dv, nonneg)
        r = _rng(300 + seed)
        a = [_GATES[int(r.integers(0, len(_GATES)))] for _ in range(n)]
        if n > 4:
            a[4] = Fraction(0)       # at least one reset
            a[2] = Fraction(2, 3)    # and one partial decay
        qf, kf, vf = _as_f64(q), _as_f64(k), _as_f64(v)
        af = np.array([float(x) for x in a])
        for normalize in (True, False):
            want = _as_f64(_exact_gated(fmap, q, k, v, a, normalize))
            got_q = o.attention_gated_quadratic(qf, kf, vf, af, fmap, normalize)
            got_r = o.attention_gated_recurrent(qf, kf, vf, af, fmap,
                                                normalize=normalize)[0]
            got_rows = o.attention_gated_rows(qf, kf, vf, af, fmap, list(range(n)),
                                              normalize)
            for got in (got_q, got_r, got_rows):
                assert _rel(got, want) < 1e-13, (fmap, n, normalize)
        if fmap == "elu1":
            # ELU1 on non-negative rationals: phi(k) = k + 1, so the final
            # state is exact too
            S_want = [[sum(_prod(a[j + 1:]) * (k[j][r_] + 1) * v[j][c]
                           for j in range(n)) for c in range(dv)] for r_ in range(dk)]
            z_want = [sum(_prod(a[j + 1:]) * (k[j][r_] + 1) for j in range(n))
                      for r_ in range(dk)]
            _, S, z = o.attention_gated_recurrent(qf, kf, vf, af, fmap)
            S2, z2 = o.gated_final_state(kf, vf, af, fmap)
            for SS, zz in ((S, z), (S2, z2)):
                assert _rel(SS, _as_f64(S_want)) < 1e-13
                assert _rel(zz, np.array([float(x) for x in z_want])) < 1e-13


def _prod(xs):
    p = Fraction(1)
    for x in xs:
        p *= x
    return p


def pin_gated_exact_elu1(o):
    _check_exact_gated(o, "elu1", nonneg=True)


def pin_gated_exact_taylor(o):
    _check_exact_gated(o, "taylor2", nonneg=False)
    _check_exact_gated(o, "taylor2sym", nonneg=False)


def pin_gated_iir_filter(o):
    """Constant decay alpha and a constant key: the decayed sums are the
    first-order recursive filter y_n = alpha y_{n-1} + x_n, which scipy's
    lfilter([1], [1, -alpha]) computes; the normalised output is the
    filtered v over the filtered ones."""
    from scipy.signal import lfilter
    r = _rng(21)
    for fmap in ("elu1", "taylor2", "taylor2sym"):
        for alpha in (0.0, 0.37, 0.9, 1.0):
            n = 50
            q = r.standard_normal((n, 3))
            k = np.tile(r.standard_normal((1, 3)), (n, 1))
            v = r.standard_normal((n, 4))
            a = np.full(n, alpha)
            fv = lfilter([1.0], [1.0, -alpha], v, axis=0)
            f1 = lfilter([1.0], [1.0, -alpha], np.ones(n))
            y = o.attention_gated_recurrent(q, k, v, a, fmap)[0]
            assert _rel(y, fv / f1[:, None]) < 1e-12, (fmap, alpha)
            y = o.attention_gated_quadratic(q, k, v, a, fmap)
            assert _rel(y, fv / f1[:, None]) < 1e-12, (fmap, alpha)
            kq = o.kernel_value(q, k, fmap)
            y_un = o.attention_gated_recurrent(q, k, v, a, fmap, normalize=False)[0]
            assert _rel(y_un, kq[:, None] * fv) < 1e-12, (fmap, alpha)
            _, S, z = o.attention_gated_recurrent(q, k, v, a, fmap)
            fk = o.feature_map(k[0], fmap)
            assert _rel(S, np.outer(fk, fv[-1])) < 1e-12
            assert _rel(z, fk * f1[-1]) < 1e-12


def pin_gated_zero_and_one(o):
    """a = 0 keeps only the current token: the normalised output is v_t and
    the unnormalised one (phi(q_t).phi(k_t)) v_t, with the kernel value
    computed without features (torch's elu, or 1 + s + s^2/2).  a = 1 is the
    ungated recurrence."""
    import torch
    r = _rng(22)
    q = r.standard_normal((2, 30, 4))
    k = r.standard_normal((2, 30, 4))
    v = r.standard_normal((2, 30, 5))
    zero = np.zeros((2, 30))
    one = np.ones((2, 30))
    for fmap in ("elu1", "taylor2", "taylor2sym"):
        if fmap == "elu1":
            e = lambda x: torch.nn.functional.elu(torch.from_numpy(x)).numpy() + 1.0
            kq = np.sum(e(q) * e(k), axis=-1)
        else:
            s_ = np.sum(q * k, axis=-1)
            kq = 1.0 + s_ + 0.5 * s_ * s_
        for f in (o.attention_gated_quadratic,
                  lambda *x, **kw: o.attention_gated_recurrent(*x, **kw)[0]):
            assert _rel(f(q, k, v, zero, fmap), v) < 1e-14
            assert _rel(f(q, k, v, zero, fmap, normalize=False), kq[..., None] * v) < 1e-13
            assert _rel(f(q, k, v, one, fmap), o.attention_quadratic(q, k, v, fmap)) < 1e-12


def pin_gated_reset_cuts_the_past(o):
    """A reset a_r = 0 removes every token before r: from r on, outputs and
    state equal a fresh run over the tail."""
    r = _rng(23)
    for fmap in ("elu1", "taylor2sym"):
        q = r.standard_normal((3, 40, 4))
        k = r.standard_normal((3, 40, 4))
        v = r.standard_normal((3, 40, 2))
        a = r.uniform(0.5, 1.0, (3, 40))
        a[:, 17] = 0.0
        for normalize in (True, False):
            y, S, z = o.attention_gated_recurrent(q, k, v, a, fmap, normalize=normalize)
            y2, S2, z2 = o.attention_gated_recurrent(q[:, 17:], k[:, 17:], v[:, 17:],
                                                     a[:, 17:], fmap, normalize=normalize)
            assert _rel(y[:, 17:], y2) < 1e-12
            assert _rel(S, S2) < 1e-12 and _rel(z, z2) < 1e-12
            yq = o.attention_gated_quadratic(q, k, v, a, fmap, normalize)
            assert _rel(yq[:, 17:], y2) < 1e-12


def pin_gated_continuation_and_state(o):
    """Two runs joined through the state equal one run; the final state from
    the recurrence, the closed form and a plain loop of decayed outer
    products agree (with a start state)."""
    r = _rng(24)
    for fmap, dk, dv in (("elu1", 5, 3), ("taylor2", 3, 4), ("taylor2sym", 3, 4)):
        q = r.standard_normal((2, 45, dk))
        k = r.standard_normal((2, 45, dk))
        v = r.standard_normal((2, 45, dv))
        a = r.uniform(0.0, 1.0, (2, 45))
        D = o.feature_dim(fmap, dk)
        S0 = r.standard_normal((2, D, dv))
        z0 = np.abs(r.standard_normal((2, D))) + 1.0
        y_all, S_all, z_all = o.attention_gated_recurrent(q, k, v, a, fmap, S0, z0)
        y_a, S_a, z_a = o.attention_gated_recurrent(q[:, :19], k[:, :19], v[:, :19],
                                                    a[:, :19], fmap, S0, z0)
        y_b, S_b, z_b = o.attention_gated_recurrent(q[:, 19:], k[:, 19:], v[:, 19:],
                                                    a[:, 19:], fmap, S_a, z_a)
        assert _rel(np.concatenate([y_a, y_b], axis=1), y_all) < 1e-12
        assert _rel(S_b, S_all) < 1e-12 and _rel(z_b, z_all) < 1e-12
        S2, z2 = o.gated_final_state(k, v, a, fmap, S0, z0)
        assert _rel(S2, S_all) < 1e-12 and _rel(z2, z_all) < 1e-12
        fk = o.feature_map(k, fmap)
        S3, z3 = S0.copy(), z0.copy()
        for t in range(45):
            S3 = S3 * a[:, t, None, None] + np.einsum("br,bc->brc", fk[:, t], v[:, t])
            z3 = z3 * a[:, t, None] + fk[:, t]
        assert _rel(S3, S_all) < 1e-12 and _rel(z3, z_all) < 1e-12
        rows = [0, 7, 44]
        for b in range(2):
            got = o.attention_gated_rows(q[b], k[b], v[b], a[b], fmap, rows)
            want = o.attention_gated_recurrent(q[b], k[b], v[b], a[b], fmap)[0][rows]
            assert _rel(got, want) < 1e-12


# ------------------------------------------------------ sliding window ----
def pin_swa_matches_torch_sdpa(o):
    """Band-masked softmax attention equals torch's scaled_dot_product_attention
    with the same boolean band mask; w >= N is its causal mode."""
    import torch
    r = _rng(31)
    q = r.standard_normal((2, 3, 70, 8))
    k = r.standard_normal((2, 3, 70, 8))
    v = r.standard_normal((2, 3, 70, 5))
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    for w in (1, 3, 16, 40, 70, 100):
        i = torch.arange(70)[:, None]
        j = torch.arange(70)[None, :]
        band = (j <= i) & (j > i - w)
        for scale in (8 ** -0.5, 0.3):
            want = torch.nn.functional.scaled_dot_product_attention(
                tq, tk, tv, attn_mask=band, scale=scale).numpy()
            assert _rel(o.swa_attention(q, k, v, w, scale), want) < 1e-12, (w, scale)
    want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True).numpy()
    assert _rel(o.swa_attention(q, k, v, 70, 8 ** -0.5), want) < 1e-12


def pin_swa_closed_forms(o):
    """w = 1 returns v.  w = 2: y_i = v_i + sigma(a - b) (v_{i-1} - v_i) with
    a, b the scaled scores of keys i-1 and i (logistic written with math.exp).
    Constant keys: equal weights, so y_i is the mean of the last
    min(i + 1, w) values (numpy's convolve)."""
    r = _rng(32)
    q = r.standard_normal((30, 4))
    k = r.standard_normal((30, 4))
    v = r.standard_normal((30, 3))
    assert _rel(o.swa_attention(q, k, v, 1, 0.5), v) < 1e-15
    y2 = o.swa_attention(q, k, v, 2, 0.5)
    for i in range(1, 30):
        a = 0.5 * float(q[i] @ k[i - 1])
        b = 0.5 * float(q[i] @ k[i])
        sig = 1.0 / (1.0 + math.exp(-(a - b)))
        assert _rel(y2[i], v[i] + sig * (v[i - 1] - v[i])) < 1e-13
    assert _rel(y2[0], v[0]) < 1e-15
    kc = np.tile(r.standard_normal((1, 4)), (30, 1))
    for w in (1, 4, 7, 30):
        y = o.swa_attention(q, kc, v, w, 0.5)
        counts = np.convolve(np.ones(30), np.ones(w))[:30]
        means = np.stack([np.convolve(v[:, c], np.ones(w))[:30] for c in range(3)], -1)
        assert _rel(y, means / counts[:, None]) < 1e-12, w


def pin_swa_locality_and_rows(o):
    """Changing tokens outside row i's window leaves y_i unchanged; single
    rows agree with the dense form."""
    r = _rng(33)
    q = r.standard_normal((60, 6))
    k = r.standard_normal((60, 6))
    v = r.standard_normal((60, 4))
    w = 9
    y = o.swa_attention(q, k, v, w, 0.4)
    k2, v2 = k.copy(), v.copy()
    k2[:30] = r.standard_normal((30, 6))   # before row 40's window [32, 40]
    v2[:30] = r.standard_normal((30, 4))
    k2[41:] = r.standard_normal((19, 6))   # after row 40
    v2[41:] = r.standard_normal((19, 4))
    y2 = o.swa_attention(q, k2, v2, w, 0.4)
    assert _rel(y2[38:41], y[38:41]) < 1e-14
    assert _rel(y2[:30], y[:30]) > 1e-3    # and the change is visible elsewhere
    rows = [0, 1, 8, 9, 10, 59]
    assert _rel(o.swa_rows(q, k, v, w, 0.4, rows), y[rows]) < 1e-13


def pin_swa_decode_continues_prefill(o):
    """Cache from a prefill of P tokens, then T decode steps, equals the dense
    form over all P + T tokens; the cache built step by step equals the one
    from the prefill."""
    r = _rng(34)
    for w, P in ((5, 12), (16, 3), (7, 7)):
        T = 11
        q = r.standard_normal((2, P + T, 4))
        k = r.standard_normal((2, P + T, 4))
        v = r.standard_normal((2, P + T, 3))
        want = o.swa_attention(q, k, v, w, 0.7)
        kc, vc = o.swa_cache_after_prefill(k[:, :P], v[:, :P], w)
        for t in range(P, P + T):
            kc0 = kc.copy()
            y, kc, vc = o.swa_decode_step(q[:, t], k[:, t], v[:, t], kc, vc, t, w, 0.7)
            assert _rel(y, want[:, t]) < 1e-12, (w, P, t)
        kc2, vc2 = o.swa_cache_after_prefill(k, v, w)
        assert _rel(kc, kc2) < 1e-15 and _rel(vc, vc2) < 1e-15
        # from an empty cache, step by step from token 0
        kc = np.zeros((2, w, 4))
        vc = np.zeros((2, w, 3))
        for t in range(P + T):
            y, kc, vc = o.swa_decode_step(q[:, t], k[:, t], v[:, t], kc, vc, t, w, 0.7)
            assert _rel(y, want[:, t]) < 1e-12
        assert np.array_equal(kc0.shape, kc.shape)


PINS = [
    pin_exact_elu1,
    pin_exact_taylor2,
    pin_exact_taylor2_sym,
    pin_taylor_sym_size_and_identity,
    pin_taylor_sym_layout,
    pin_taylor_sym_fold,
    pin_quad_vs_rec,
    pin_rows_match_definition,
    pin_taylor_identity,
    pin_taylor_exp,
    pin_taylor_layout,
    pin_elu_torch,
    pin_first_token,
    pin_constant_key,
    pin_zero_taylor_query,
    pin_constant_and_linear_v,
    pin_convex_hull_and_positive,
    pin_final_state,
    pin_decode_continuation,
    pin_golden_handworked,
    pin_gated_exact_elu1,
    pin_gated_exact_taylor,
    pin_gated_iir_filter,
    pin_gated_zero_and_one,
    pin_gated_reset_cuts_the_past,
    pin_gated_continuation_and_state,
    pin_swa_matches_torch_sdpa,
    pin_swa_closed_forms,
    pin_swa_locality_and_rows,
    pin_swa_decode_continues_prefill,
]
