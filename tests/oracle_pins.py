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
]
