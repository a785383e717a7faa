"""The CPU oracle against its pins (exact arithmetic, closed forms, golden
examples, finite differences, autograd), and the pins against planted mistakes."""
import types

import numpy as np
import pytest

import oracle_pins as P
from oracle import dora_oracle as O


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(O)


def _mutant(**overrides):
    ns = types.SimpleNamespace(weight_norm=O.weight_norm, row_sqnorm=O.row_sqnorm,
                               weight_norm_cached=O.weight_norm_cached, compose_fwd=O.compose_fwd,
                               lora_compose_fwd=O.lora_compose_fwd, lora_compose_bwd=O.lora_compose_bwd,
                               compose_bwd=O.compose_bwd, weight_norm_bwd=O.weight_norm_bwd)
    for k, v in overrides.items():
        setattr(ns, k, v)
    return ns


def _f(x):
    return O.as_f64(x)


def _norm_dense(W0, A, B, s, *, sign=1.0, s_pow=1, axis=1, root=True):
    W0, A, B = _f(W0), _f(A), _f(B)
    V = W0 + sign * (float(s) ** s_pow) * (B @ A)
    sq = np.sum(V * V, axis=axis)
    return np.sqrt(sq) if root else sq


def _cached(c, W0, A, B, s, *, use_cache=True, cross=True, double_base=False, s_pow=2, clamp=True):
    c, W0, A, B = _f(c), _f(W0), _f(A), _f(B)
    s = float(s)
    V = B @ A
    base = np.sum(W0 * W0, axis=1)
    n2 = (c if use_cache else base) + (base if double_base else 0.0)
    n2 = n2 + (2.0 * s * np.sum(W0 * V, axis=1) if cross else 0.0) + s ** s_pow * np.sum(V * V, axis=1)
    return np.sqrt(np.maximum(n2, 0.0) if clamp else np.abs(n2))


def _fwd(base, lora, m, n, s, add_base=False, *, corr_one=True, s_on_lora=True, invert=False, honour_add=True):
    base, lora, m, n = _f(base), _f(lora), _f(m), _f(n)
    g = n / m if invert else m / n
    y = ((g - 1.0) if corr_one else g) * base + g * (float(s) if s_on_lora else 1.0) * lora
    if add_base and honour_add:
        y = y + base
    return y


def _bwd(dy, base, lora, m, n, s, add_base=False, *, div_n=True, lora_sign=1.0, dbase_g=False,
         dlora_s=True, extra_g=False):
    dy, base, lora, m, n = _f(dy), _f(base), _f(lora), _f(m), _f(n)
    g = m / n
    s = float(s)
    d_lora = g * (s if dlora_s else 1.0) * dy
    d_base = (g if (add_base or dbase_g) else (g - 1.0)) * dy
    d_mag = np.sum(dy * (base + lora_sign * s * lora), axis=0)
    if div_n:
        d_mag = d_mag / n
    if extra_g:
        d_mag = d_mag * g
    return d_lora, d_base, d_mag


def _nbwd(d, n, W0, A, B, s, *, s_on_dB=True, use_adapter=True, n_pow=1, sign=1.0, dA_rows_reversed=False,
          dA_gram=True):
    d, n, W0, A, B = _f(d), _f(n), _f(W0), _f(A), _f(B)
    s = float(s)
    c = d / n ** n_pow
    dV = c[:, None] * (W0 + (sign * s * (B @ A) if use_adapter else 0.0))
    dVa = c[:, None] * (W0 + (s * (B @ A) if dA_gram else 0.0))
    dA = s * (B.T @ (dVa[::-1] if dA_rows_reversed else dVa))
    dB = (s if s_on_dB else 1.0) * (dV @ A.T)
    return dA, dB


MUTANTS = {
    "nbwd_dB_drops_s": _mutant(weight_norm_bwd=lambda *a: _nbwd(*a, s_on_dB=False)),
    "nbwd_W0_for_V": _mutant(weight_norm_bwd=lambda *a: _nbwd(*a, use_adapter=False)),
    "nbwd_divides_by_n_squared": _mutant(weight_norm_bwd=lambda *a: _nbwd(*a, n_pow=2)),
    "nbwd_minus_adapter": _mutant(weight_norm_bwd=lambda *a: _nbwd(*a, sign=-1.0)),
    "nbwd_dA_rows_misaligned": _mutant(weight_norm_bwd=lambda *a: _nbwd(*a, dA_rows_reversed=True)),
    "nbwd_dA_drops_gram": _mutant(weight_norm_bwd=lambda *a: _nbwd(*a, dA_gram=False)),
    "norm_drops_s": _mutant(weight_norm=lambda W0, A, B, s: _norm_dense(W0, A, B, 1.0)),
    "norm_minus_adapter": _mutant(weight_norm=lambda W0, A, B, s: _norm_dense(W0, A, B, s, sign=-1.0)),
    "norm_s_squared": _mutant(weight_norm=lambda W0, A, B, s: _norm_dense(W0, A, B, s, s_pow=2)),
    "norm_no_sqrt": _mutant(weight_norm=lambda W0, A, B, s: _norm_dense(W0, A, B, s, root=False)),
    "norm_column_axis": _mutant(weight_norm=lambda W0, A, B, s: _norm_dense(W0, A, B, s, axis=0)),
    "norm_base_only": _mutant(weight_norm=lambda W0, A, B, s: np.linalg.norm(_f(W0), axis=1)),
    "norm_drops_cross": _mutant(weight_norm=lambda W0, A, B, s: np.sqrt(
        np.sum(_f(W0) ** 2, axis=1) + float(s) ** 2 * np.sum((_f(B) @ _f(A)) ** 2, axis=1))),
    "norm_drops_gram": _mutant(weight_norm=lambda W0, A, B, s: np.sqrt(np.maximum(
        np.sum(_f(W0) ** 2, axis=1) + 2 * float(s) * np.sum(_f(B) * (_f(W0) @ _f(A).T), axis=1), 0))),
    "norm_transposed_gram": _mutant(weight_norm=lambda W0, A, B, s: np.sqrt(np.maximum(
        np.sum(_f(W0) ** 2, axis=1) + 2 * float(s) * np.sum(_f(B) * (_f(W0) @ _f(A).T), axis=1)
        + float(s) ** 2 * np.sum((_f(B) @ (_f(A) @ _f(A).T)[::-1, ::-1]) * _f(B), axis=1), 0))),
    "sqnorm_not_squared": _mutant(row_sqnorm=lambda W0: np.linalg.norm(_f(W0), axis=1)),
    "sqnorm_column_axis": _mutant(row_sqnorm=lambda W0: np.sum(_f(W0) ** 2, axis=0)),
    "cached_ignores_cache": _mutant(weight_norm_cached=lambda c, W0, A, B, s: _cached(c, W0, A, B, s, use_cache=False)),
    "cached_double_base": _mutant(weight_norm_cached=lambda c, W0, A, B, s: _cached(c, W0, A, B, s, double_base=True)),
    "cached_drops_cross": _mutant(weight_norm_cached=lambda c, W0, A, B, s: _cached(c, W0, A, B, s, cross=False)),
    "cached_gram_s_linear": _mutant(weight_norm_cached=lambda c, W0, A, B, s: _cached(c, W0, A, B, s, s_pow=1)),
    "cached_abs_not_clamp": _mutant(weight_norm_cached=lambda c, W0, A, B, s: _cached(c, W0, A, B, s, clamp=False)),
    "lora_transposed_B": _mutant(lora_compose_fwd=lambda base, h, B, m, n, s, add_base=False: O.compose_fwd(
        base, _f(h) @ _f(B), m, n, s, add_base)),
    "lora_drops_s": _mutant(lora_compose_fwd=lambda base, h, B, m, n, s, add_base=False: O.compose_fwd(
        base, _f(h) @ _f(B).T, m, n, 1.0, add_base)),
    "lora_ignores_add_base": _mutant(lora_compose_fwd=lambda base, h, B, m, n, s, add_base=False: O.compose_fwd(
        base, _f(h) @ _f(B).T, m, n, s, False)),
    "lora_first_column_only": _mutant(lora_compose_fwd=lambda base, h, B, m, n, s, add_base=False: O.compose_fwd(
        base, np.outer(_f(h)[:, 0], _f(B)[:, 0]), m, n, s, add_base)),
    "lora_bwd_dB_no_g": _mutant(lora_compose_bwd=lambda dy, base, h, B, m, n, s, add_base=False: (
        O.lora_compose_bwd(dy, base, h, B, m, n, s, add_base)[0],
        float(s) * _f(dy).T @ _f(h), O.lora_compose_bwd(dy, base, h, B, m, n, s, add_base)[2])),
    "lora_bwd_dB_transposed_h": _mutant(lora_compose_bwd=lambda dy, base, h, B, m, n, s, add_base=False: (
        O.lora_compose_bwd(dy, base, h, B, m, n, s, add_base)[0],
        (O.scale_factor(m, n) * float(s) * _f(dy)).T @ _f(h)[::-1], O.lora_compose_bwd(dy, base, h, B, m, n, s, add_base)[2])),
    "lora_bwd_dmag_drops_lora": _mutant(lora_compose_bwd=lambda dy, base, h, B, m, n, s, add_base=False: (
        O.lora_compose_bwd(dy, base, h, B, m, n, s, add_base)[0], O.lora_compose_bwd(dy, base, h, B, m, n, s, add_base)[1],
        np.sum(_f(dy) * _f(base), axis=0) / _f(n))),
    "lora_bwd_dbase_g": _mutant(lora_compose_bwd=lambda dy, base, h, B, m, n, s, add_base=False: (
        O.scale_factor(m, n) * _f(dy), O.lora_compose_bwd(dy, base, h, B, m, n, s, add_base)[1],
        O.lora_compose_bwd(dy, base, h, B, m, n, s, add_base)[2])),
    "fwd_no_minus_one": _mutant(compose_fwd=lambda *a, add_base=False: _fwd(*a, add_base=add_base, corr_one=False)),
    "fwd_drops_s": _mutant(compose_fwd=lambda *a, add_base=False: _fwd(*a, add_base=add_base, s_on_lora=False)),
    "fwd_inverted_g": _mutant(compose_fwd=lambda *a, add_base=False: _fwd(*a, add_base=add_base, invert=True)),
    "fwd_ignores_add_base": _mutant(compose_fwd=lambda *a, add_base=False: _fwd(*a, add_base=add_base, honour_add=False)),
    "bwd_no_div_n": _mutant(compose_bwd=lambda *a, add_base=False: _bwd(*a, add_base=add_base, div_n=False)),
    "bwd_lora_sign": _mutant(compose_bwd=lambda *a, add_base=False: _bwd(*a, add_base=add_base, lora_sign=-1.0)),
    "bwd_dbase_g": _mutant(compose_bwd=lambda *a, add_base=False: _bwd(*a, add_base=add_base, dbase_g=True)),
    "bwd_dlora_no_s": _mutant(compose_bwd=lambda *a, add_base=False: _bwd(*a, add_base=add_base, dlora_s=False)),
    "bwd_extra_g": _mutant(compose_bwd=lambda *a, add_base=False: _bwd(*a, add_base=add_base, extra_g=True)),
}


def test_mutant_helpers_match_oracle_when_unmutated():
    # the helpers above reproduce the oracle when no mistake is planted, so a
    # caught mutant is caught because of its mistake
    rng = np.random.default_rng(0)
    W0, A, B = rng.standard_normal((5, 7)), rng.standard_normal((3, 7)), rng.standard_normal((5, 3))
    np.testing.assert_allclose(_norm_dense(W0, A, B, 1.3), O.weight_norm(W0, A, B, 1.3), rtol=1e-15)
    c = rng.uniform(1, 3, 5)
    np.testing.assert_allclose(_cached(c, W0, A, B, 1.3), O.weight_norm_cached(c, W0, A, B, 1.3), rtol=1e-15)
    d, n5 = rng.standard_normal(5), rng.uniform(1, 2, 5)
    for x, y in zip(_nbwd(d, n5, W0, A, B, 1.3), O.weight_norm_bwd(d, n5, W0, A, B, 1.3)):
        np.testing.assert_allclose(x, y, rtol=1e-14)
    base, lora, dy = rng.standard_normal((3, (4))), rng.standard_normal((3, 4)), rng.standard_normal((3, 4))
    m, n = rng.uniform(1, 2, 4), rng.uniform(1, 2, 4)
    for ab in (False, True):
        np.testing.assert_allclose(_fwd(base, lora, m, n, 0.7, ab), O.compose_fwd(base, lora, m, n, 0.7, ab), rtol=1e-15)
        for x, y in zip(_bwd(dy, base, lora, m, n, 0.7, ab), O.compose_bwd(dy, base, lora, m, n, 0.7, ab)):
            np.testing.assert_allclose(x, y, rtol=1e-15)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    caught = []
    for pin in P.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(MUTANTS[name])
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
