"""Plant plausible mistakes in copies of the oracle; the pins must catch each.

Every mutant is a fresh copy of oracle/linattn_oracle.py with one function
replaced.  The real oracle is never modified.
"""
import importlib.util
import math
import os

import numpy as np
import pytest

from oracle_pins import PINS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "linattn_oracle.py")


def _fresh_copy(tag):
    spec = importlib.util.spec_from_file_location(f"oracle_mutant_{tag}", SRC)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _m_elu_no_exp(o):
    o.phi_elu1 = lambda x: np.asarray(x, dtype=np.float64) + 1.0


def _m_elu_plain_exp(o):
    o.phi_elu1 = lambda x: np.exp(np.asarray(x, dtype=np.float64))


def _m_elu_missing_plus_one(o):
    def phi(x):
        x = np.asarray(x, dtype=np.float64)
        return np.where(x > 0, x, np.exp(np.minimum(x, 0.0)) - 1.0) + 0.5
    o.phi_elu1 = phi


def _m_taylor_no_sqrt2(o):
    def phi(x):
        x = np.asarray(x, dtype=np.float64)
        d = x.shape[-1]
        ones = np.ones(x.shape[:-1] + (1,))
        quad = (x[..., :, None] * x[..., None, :]).reshape(x.shape[:-1] + (d * d,))
        return np.concatenate([ones, x, quad], axis=-1)
    o.phi_taylor2 = phi


def _m_taylor_no_constant(o):
    real = o.phi_taylor2

    def phi(x):
        f = real(x).copy()
        f[..., 0] = 0.0
        return f
    o.phi_taylor2 = phi


def _m_taylor_wrong_layout(o):
    # pairs ordered (i, j) with the linear block after the quadratic one
    def phi(x):
        x = np.asarray(x, dtype=np.float64)
        d = x.shape[-1]
        ones = np.ones(x.shape[:-1] + (1,))
        quad = (x[..., :, None] * x[..., None, :]).reshape(x.shape[:-1] + (d * d,))
        return np.concatenate([ones, quad / math.sqrt(2.0), x], axis=-1)
    o.phi_taylor2 = phi


def _m_mask_strict(o):
    def quad(q, k, v, fmap):
        fq, fk = o.feature_map(q, fmap), o.feature_map(k, fmap)
        n = fq.shape[-2]
        w = (fq @ np.swapaxes(fk, -1, -2)) * np.tril(np.ones((n, n)), -1)
        with np.errstate(all="ignore"):
            return (w @ np.asarray(v, float)) / w.sum(-1)[..., None]
    o.attention_quadratic = quad


def _m_no_mask(o):
    def quad(q, k, v, fmap):
        fq, fk = o.feature_map(q, fmap), o.feature_map(k, fmap)
        w = fq @ np.swapaxes(fk, -1, -2)
        return (w @ np.asarray(v, float)) / w.sum(-1)[..., None]
    o.attention_quadratic = quad


def _m_read_before_update(o):
    def step(q, k, v, S, z, fmap):
        fq, fk = o.feature_map(q, fmap), o.feature_map(k, fmap)
        v = np.asarray(v, float)
        num = np.einsum("...r,...rc->...c", fq, S)
        den = np.einsum("...r,...r->...", fq, z)
        S_new = S + fk[..., :, None] * v[..., None, :]
        z_new = z + fk
        with np.errstate(all="ignore"):
            y = num / den[..., None]
        return np.where(np.isfinite(y), y, 0.0), S_new, z_new
    o.decode_step = step


def _m_den_uses_key(o):
    def step(q, k, v, S, z, fmap):
        fq, fk = o.feature_map(q, fmap), o.feature_map(k, fmap)
        v = np.asarray(v, float)
        S_new = S + fk[..., :, None] * v[..., None, :]
        z_new = z + fk
        num = np.einsum("...r,...rc->...c", fq, S_new)
        den = np.einsum("...r,...r->...", fk, z_new)
        return num / den[..., None], S_new, z_new
    o.decode_step = step


def _m_state_transposed(o):
    # V^T phi(K) instead of phi(K)^T V: the same shape when D == d_v
    def fin(k, v, fmap):
        fk = o.feature_map(k, fmap)
        return np.swapaxes(np.asarray(v, float), -1, -2) @ fk, fk.sum(-2)
    o.final_state = fin


def _m_rows_off_by_one(o):
    def rows_fn(q, k, v, fmap, rows):
        q, k, v = (np.asarray(a, float) for a in (q, k, v))
        out = np.empty((len(rows), v.shape[-1]))
        for r, t in enumerate(rows):
            fq = o.feature_map(q[t], fmap)
            hi = max(t, 1)
            fk = o.feature_map(k[:hi], fmap)
            w = fk @ fq
            out[r] = (w @ v[:hi]) / w.sum()
        return out
    o.attention_rows = rows_fn


def _m_value_sign(o):
    def step(q, k, v, S, z, fmap):
        fq, fk = o.feature_map(q, fmap), o.feature_map(k, fmap)
        v = np.asarray(v, float)
        S_new = S - fk[..., :, None] * v[..., None, :]
        z_new = z + fk
        num = np.einsum("...r,...rc->...c", fq, S_new)
        den = np.einsum("...r,...r->...", fq, z_new)
        return num / den[..., None], S_new, z_new
    o.decode_step = step


def _sym_map(weight_sq, weight_off):
    def phi(x):
        x = np.asarray(x, dtype=np.float64)
        d = x.shape[-1]
        ones = np.ones(x.shape[:-1] + (1,))
        pairs = [(a, b) for a in range(d) for b in range(a, d)]
        quad = np.stack([x[..., a] * x[..., b] * (weight_sq if a == b else weight_off)
                         for a, b in pairs], axis=-1)
        return np.concatenate([ones, x, quad], axis=-1)
    return phi


def _m_sym_square_unscaled(o):
    o.phi_taylor2_sym = _sym_map(1.0, 1.0)


def _m_sym_pair_scaled(o):
    o.phi_taylor2_sym = _sym_map(1.0 / math.sqrt(2.0), 1.0 / math.sqrt(2.0))


def _m_sym_pair_doubled(o):
    o.phi_taylor2_sym = _sym_map(1.0 / math.sqrt(2.0), math.sqrt(2.0))


def _m_sym_lower_order(o):
    # pairs listed column by column (lower triangle order): same values,
    # different layout
    def phi(x):
        x = np.asarray(x, dtype=np.float64)
        d = x.shape[-1]
        ones = np.ones(x.shape[:-1] + (1,))
        pairs = [(a, b) for b in range(d) for a in range(b + 1)]
        quad = np.stack([x[..., a] * x[..., b] * (1.0 / math.sqrt(2.0) if a == b else 1.0)
                         for a, b in pairs], axis=-1)
        return np.concatenate([ones, x, quad], axis=-1)
    o.phi_taylor2_sym = phi


def _m_gated_decay_after_add(o):
    # the new token decayed together with the old state
    def step(q, k, v, a, S, z, fmap, normalize=True):
        fq, fk = o.feature_map(q, fmap), o.feature_map(k, fmap)
        a = np.asarray(a, dtype=np.float64)
        S_new = a[..., None, None] * (S + fk[..., :, None] * np.asarray(v)[..., None, :])
        z_new = a[..., None] * (z + fk)
        num = np.einsum("...r,...rc->...c", fq, S_new)
        if not normalize:
            return num, S_new, z_new
        return num / np.einsum("...r,...r->...", fq, z_new)[..., None], S_new, z_new
    o.gated_decode_step = step


def _m_gated_z_not_decayed(o):
    def step(q, k, v, a, S, z, fmap, normalize=True):
        fq, fk = o.feature_map(q, fmap), o.feature_map(k, fmap)
        a = np.asarray(a, dtype=np.float64)
        S_new = a[..., None, None] * S + fk[..., :, None] * np.asarray(v)[..., None, :]
        z_new = z + fk
        num = np.einsum("...r,...rc->...c", fq, S_new)
        if not normalize:
            return num, S_new, z_new
        return num / np.einsum("...r,...r->...", fq, z_new)[..., None], S_new, z_new
    o.gated_decode_step = step


def _m_gated_matrix_own_factor(o):
    # W_ij = a_j ... a_i: token j's own coefficient included
    def W(a):
        a = np.asarray(a, dtype=np.float64)
        n = a.shape[-1]
        out = np.zeros(a.shape[:-1] + (n, n))
        for i in range(n):
            for j in range(i + 1):
                out[..., i, j] = np.prod(a[..., j:i + 1], axis=-1)
        return out
    o.decay_matrix = W


def _m_gated_suffix_own_factor(o):
    def P(a):
        a = np.asarray(a, dtype=np.float64)
        return np.flip(np.cumprod(np.flip(a, -1), axis=-1), -1)
    o._suffix_products = P


def _m_gated_normalize_ignored(o):
    f = o.attention_gated_quadratic
    o.attention_gated_quadratic = lambda q, k, v, a, fmap, normalize=True: f(q, k, v, a, fmap, True)


def _swa_band(lo_fn):
    def swa(q, k, v, window, scale):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        n = q.shape[-2]
        s = scale * (q @ np.swapaxes(k, -1, -2))
        i = np.arange(n)[:, None]
        j = np.arange(n)[None, :]
        s = np.where(lo_fn(i, j, window), s, -np.inf)
        p = np.exp(s - s.max(axis=-1, keepdims=True))
        return (p / p.sum(axis=-1, keepdims=True)) @ v
    return swa


def _m_swa_window_one_wider(o):
    o.swa_attention = _swa_band(lambda i, j, w: (j <= i) & (j >= i - w))


def _m_swa_not_causal(o):
    o.swa_attention = _swa_band(lambda i, j, w: np.abs(i - j) < w)


def _m_swa_no_scale(o):
    f = o.swa_attention
    o.swa_attention = lambda q, k, v, window, scale: f(q, k, v, window, 1.0)


def _m_swa_decode_wrong_slot(o):
    f = o.swa_decode_step
    o.swa_decode_step = lambda q, k, v, kc, vc, pos, w, s: f(q, k, v, kc, vc, pos + 1, w, s)


def _m_swa_rows_window_short(o):
    f = o.swa_rows
    o.swa_rows = lambda q, k, v, window, scale, rows: f(q, k, v, max(1, window - 1), scale, rows)


MUTANTS = [
    _m_elu_no_exp, _m_elu_plain_exp, _m_elu_missing_plus_one,
    _m_taylor_no_sqrt2, _m_taylor_no_constant, _m_taylor_wrong_layout,
    _m_mask_strict, _m_no_mask, _m_read_before_update, _m_den_uses_key,
    _m_state_transposed, _m_rows_off_by_one, _m_value_sign,
    _m_sym_square_unscaled, _m_sym_pair_scaled, _m_sym_pair_doubled, _m_sym_lower_order,
    _m_gated_decay_after_add, _m_gated_z_not_decayed, _m_gated_matrix_own_factor,
    _m_gated_suffix_own_factor, _m_gated_normalize_ignored,
    _m_swa_window_one_wider, _m_swa_not_causal, _m_swa_no_scale, _m_swa_decode_wrong_slot,
    _m_swa_rows_window_short,
]


@pytest.mark.parametrize("mutate", MUTANTS, ids=[m.__name__ for m in MUTANTS])
def test_pins_catch_planted_mistake(mutate):
    o = _fresh_copy(mutate.__name__)
    mutate(o)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(o)
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught {mutate.__name__}"
