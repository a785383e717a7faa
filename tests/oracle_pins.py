"""Pins of the CPU oracle to facts other than itself.

Each ``pin_*`` takes an object with the oracle's functions (``weight_norm``,
``row_sqnorm``, ``weight_norm_cached``, ``compose_fwd``, ``compose_bwd``,
``lora_compose_fwd``, ``lora_compose_bwd``, ``weight_norm_bwd``) and
raises AssertionError
when the oracle disagrees with:

* exact rational arithmetic on tiny inputs (brute force, using the factored
  base + cross + Gram expansion, a different formula from the oracle's dense one),
* special cases that reduce to a library routine (``numpy.linalg.norm``),
* closed forms (rank one, orthonormal A, exact cancellation, g = 1, m = 0),
* hand-worked examples stored under ``golden/`` with their derivation,
* central finite differences and fp64 autograd for the backward.

The mutation tests run every pin against planted mistakes to show that each
plausible error (a dropped term, a wrong sign, a transposed operand, a missing
division) fails at least one of them.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bf16_exact(rng, shape, sigma):
    """Random values exactly representable in bf16 (so fp64 and Fraction agree)."""
    a = (rng.standard_normal(shape) * sigma).astype(np.float32)
    return torch.from_numpy(a).to(torch.bfloat16).double().numpy()


# --------------------------------------------------------------------------- norm


def _norm_sq_fraction_factored(W0, A, B, s):
    """n_i^2 = ||W_i||^2 + 2 s B_i (A W_i^T) + s^2 B_i (A A^T) B_i^T, exactly."""
    out, inn = W0.shape
    r = A.shape[0]
    W = [[Fraction(float(v)) for v in row] for row in W0]
    Af = [[Fraction(float(v)) for v in row] for row in A]
    Bf = [[Fraction(float(v)) for v in row] for row in B]
    sf = Fraction(float(s))
    G = [[sum(Af[j][k] * Af[l][k] for k in range(inn)) for l in range(r)] for j in range(r)]
    res = []
    for i in range(out):
        base = sum(w * w for w in W[i])
        U = [sum(W[i][k] * Af[j][k] for k in range(inn)) for j in range(r)]
        cross = 2 * sf * sum(Bf[i][j] * U[j] for j in range(r))
        gram = sf * sf * sum(Bf[i][j] * G[j][l] * Bf[i][l] for j in range(r) for l in range(r))
        res.append(base + cross + gram)
    return res


def pin_norm_exact_bruteforce(o, seed=0, trials=6):
    rng = np.random.default_rng(seed)
    for t in range(trials):
        out, inn, r = int(rng.integers(1, 7)), int(rng.integers(1, 11)), int(rng.integers(1, 5))
        W0 = _bf16_exact(rng, (out, inn), 0.5)
        A = _bf16_exact(rng, (r, inn), 1.0)
        B = _bf16_exact(rng, (out, r), 0.5)
        s = float(np.float32(rng.uniform(0.3, 3.0)))
        exact = _norm_sq_fraction_factored(W0, A, B, s)
        got = np.asarray(o.weight_norm(W0, A, B, s), dtype=np.float64)
        assert got.shape == (out,), got.shape
        for i in range(out):
            want = math.sqrt(float(exact[i]))
            assert abs(got[i] - want) <= 1e-12 * max(want, 1e-300) + 1e-300, (t, i, got[i], want)


def pin_norm_special_cases(o, seed=1):
    rng = np.random.default_rng(seed)
    out, inn, r = 9, 13, 3
    W0 = _bf16_exact(rng, (out, inn), 0.02)
    A = _bf16_exact(rng, (r, inn), 0.3)
    B = _bf16_exact(rng, (out, r), 0.01)
    ref = np.linalg.norm(W0, axis=1)
    # B = 0 and A = 0 reduce to plain row norms of W0
    np.testing.assert_allclose(o.weight_norm(W0, A, np.zeros_like(B), 1.7), ref, rtol=1e-14)
    np.testing.assert_allclose(o.weight_norm(W0, np.zeros_like(A), B, 1.7), ref, rtol=1e-14)
    # s = 0 also drops the adapter
    np.testing.assert_allclose(o.weight_norm(W0, A, B, 0.0), ref, rtol=1e-14)
    # W0 = 0, rank one: n_i = |s b_i| ||a||
    a = A[:1]
    b = B[:, :1]
    got = o.weight_norm(np.zeros_like(W0), a, b, 2.5)
    np.testing.assert_allclose(got, np.abs(2.5 * b[:, 0]) * np.linalg.norm(a[0]), rtol=1e-14)
    # orthonormal rows of A (unit basis vectors) and W0 orthogonal to them:
    # n_i^2 = ||W0_i||^2 + s^2 ||B_i||^2 (Pythagoras)
    Aon = np.zeros((r, inn))
    for j in range(r):
        Aon[j, 2 * j + 1] = 1.0
    W0p = W0.copy()
    W0p[:, [2 * j + 1 for j in range(r)]] = 0.0
    s = 1.25
    want = np.sqrt(np.sum(W0p**2, axis=1) + s * s * np.sum(B**2, axis=1))
    np.testing.assert_allclose(o.weight_norm(W0p, Aon, B, s), want, rtol=1e-14)
    # orthonormal A with W0 along A: n_i = || W0_i A^T + s B_i || (the coefficients add)
    W0a = (B[:, ::-1].copy() * 3.0) @ Aon
    want = np.linalg.norm(B[:, ::-1] * 3.0 + s * B, axis=1)
    np.testing.assert_allclose(o.weight_norm(W0a, Aon, B, s), want, rtol=1e-14)
    # exact cancellation W0 = -s B A: the norm is exactly zero
    Bi = np.array([[1.0, -2.0], [0.5, 0.0], [0.0, 0.25]])
    Ai = np.array([[1.0, 2.0, 0.0, -1.0], [0.0, 1.0, 4.0, 0.5]])
    s = 2.0
    W0c = -s * (Bi @ Ai)
    assert np.all(o.weight_norm(W0c, Ai, Bi, s) == 0.0)
    # non-negativity and per-row independence (rows can be evaluated alone)
    full = o.weight_norm(W0, A, B, 1.3)
    assert np.all(full >= 0)
    rows = [7, 0, 4]
    np.testing.assert_allclose(o.weight_norm(W0[rows], A, B[rows], 1.3), full[rows], rtol=0, atol=0)


def pin_norm_golden(o):
    for ex in _golden("worked_examples.json")["norm"]:
        got = np.asarray(o.weight_norm(np.array(ex["W0"], float), np.array(ex["A"], float),
                                       np.array(ex["B"], float), ex["s"]))
        want = np.sqrt(np.array(ex["expected_norm_sq"], float))
        np.testing.assert_allclose(got, want, rtol=1e-15, atol=0, err_msg=ex["name"])


def pin_norm_invariances(o, seed=2):
    """Invariances fixed by the mathematics: sign flips, scaling, permutations."""
    rng = np.random.default_rng(seed)
    out, inn, r = 6, 10, 4
    W0 = _bf16_exact(rng, (out, inn), 0.1)
    A = _bf16_exact(rng, (r, inn), 0.5)
    B = _bf16_exact(rng, (out, r), 0.2)
    s = 1.5
    ref = o.weight_norm(W0, A, B, s)
    # (B, s) -> (-B, -s) leaves s*B*A unchanged; (B, A) -> (2B, A/2) as well
    np.testing.assert_allclose(o.weight_norm(W0, A, -B, -s), ref, rtol=1e-14)
    np.testing.assert_allclose(o.weight_norm(W0, A / 2, 2 * B, s), ref, rtol=1e-14)
    # scaling W0 and B together scales the norm
    np.testing.assert_allclose(o.weight_norm(4 * W0, A, 4 * B, s), 4 * ref, rtol=1e-14)
    # permuting the input axis of W0 and A, or the rank axis of A and B, changes nothing
    p = rng.permutation(inn)
    np.testing.assert_allclose(o.weight_norm(W0[:, p], A[:, p], B, s), ref, rtol=1e-13)
    q = rng.permutation(r)
    np.testing.assert_allclose(o.weight_norm(W0, A[q], B[:, q], s), ref, rtol=1e-13)
    # the norm changes when the adapter changes sign relative to W0 (detects a
    # dropped cross term, which is the only term odd in s)
    flipped = o.weight_norm(W0, A, B, -s)
    assert np.max(np.abs(flipped - ref)) > 1e-6


# ----------------------------------------------------------------------- compose


def pin_row_sqnorm(o, seed=6):
    """||W0_i||^2: exact rational sums on tiny inputs, numpy.linalg.norm squared
    on larger ones, and zero rows / an empty input axis."""
    rng = np.random.default_rng(seed)
    for t in range(4):
        out, inn = int(rng.integers(1, 6)), int(rng.integers(1, 13))
        W0 = _bf16_exact(rng, (out, inn), 0.7)
        got = np.asarray(o.row_sqnorm(W0), dtype=np.float64)
        assert got.shape == (out,), got.shape
        for i in range(out):
            want = float(sum(Fraction(float(v)) ** 2 for v in W0[i]))
            assert abs(got[i] - want) <= 1e-14 * want + 1e-300, (t, i, got[i], want)
    W0 = rng.standard_normal((37, 300))
    np.testing.assert_allclose(o.row_sqnorm(W0), np.linalg.norm(W0, axis=1) ** 2, rtol=1e-13)
    W0[3] = 0.0
    assert o.row_sqnorm(W0)[3] == 0.0
    assert np.all(np.asarray(o.row_sqnorm(np.zeros((4, 0)))) == 0.0)


def pin_norm_cached(o, seed=7):
    """The cached-base norm against exact rational arithmetic with the factored
    expansion and an arbitrary cache value, against the plain norm when the
    cache holds ||W0_i||^2, and at the clamp."""
    rng = np.random.default_rng(seed)
    for t in range(5):
        out, inn, r = int(rng.integers(1, 6)), int(rng.integers(1, 10)), int(rng.integers(1, 5))
        W0 = _bf16_exact(rng, (out, inn), 0.5)
        A = _bf16_exact(rng, (r, inn), 1.0)
        B = _bf16_exact(rng, (out, r), 0.5)
        s = float(np.float32(rng.uniform(0.3, 3.0)))
        c = (rng.uniform(0.5, 4.0, out) * (1.0 + np.sum(W0 * W0, axis=1))).astype(np.float32)
        full = _norm_sq_fraction_factored(W0, A, B, s)
        got = np.asarray(o.weight_norm_cached(c, W0, A, B, s), dtype=np.float64)
        assert got.shape == (out,), got.shape
        for i in range(out):
            base = sum(Fraction(float(v)) ** 2 for v in W0[i])
            n2 = full[i] - base + Fraction(float(c[i]))
            want = math.sqrt(max(float(n2), 0.0))
            assert abs(got[i] - want) <= 1e-12 * max(want, 1e-300) + 1e-300, (t, i, got[i], want)
    # a cache holding the true base term gives the plain norm
    W0, A, B = rng.standard_normal((9, 23)), rng.standard_normal((4, 23)), rng.standard_normal((9, 4))
    c = np.sum(W0 * W0, axis=1)
    np.testing.assert_allclose(o.weight_norm_cached(c, W0, A, B, 0.9),
                               np.linalg.norm(W0 + 0.9 * (B @ A), axis=1), rtol=1e-12)
    # B = 0 leaves sqrt(c); a cache far below the true base term clamps at 0
    np.testing.assert_allclose(o.weight_norm_cached(c, W0, A, np.zeros_like(B), 0.9), np.sqrt(c), rtol=1e-15)
    # c = 0, W0 = (1,1,1), BA = -(1,1,1), s = 1: n^2 = 0 - 6 + 3 = -3, clamped to 0
    r1 = np.ones((1, 3))
    assert o.weight_norm_cached(np.zeros(1), r1, -r1, np.ones((1, 1)), 1.0)[0] == 0.0


def pin_compose_golden(o):
    for ex in _golden("worked_examples.json")["compose"]:
        args = [np.array(ex[k], float) for k in ("base", "lora", "m", "n")]
        s = ex["s"]
        np.testing.assert_allclose(o.compose_fwd(*args, s, add_base=False), ex["expected_delta"], rtol=0, atol=1e-15)
        np.testing.assert_allclose(o.compose_fwd(*args, s, add_base=True), ex["expected_full"], rtol=0, atol=1e-15)
        dy = np.array(ex["dy"], float)
        dl, db, dm = o.compose_bwd(dy, *args, s, add_base=False)
        np.testing.assert_allclose(dl, ex["expected_d_lora"], rtol=0, atol=1e-15)
        np.testing.assert_allclose(db, ex["expected_d_base_delta"], rtol=0, atol=1e-15)
        np.testing.assert_allclose(dm, ex["expected_d_mag"], rtol=0, atol=1e-15)
        dl, db, dm = o.compose_bwd(dy, *args, s, add_base=True)
        np.testing.assert_allclose(db, ex["expected_d_base_full"], rtol=0, atol=1e-15)
        np.testing.assert_allclose(dm, ex["expected_d_mag"], rtol=0, atol=1e-15)


def _compose_inputs(seed, T=7, out=5):
    rng = np.random.default_rng(seed)
    base = _bf16_exact(rng, (T, out), 1.0)
    lora = _bf16_exact(rng, (T, out), 0.3)
    n = rng.uniform(0.5, 2.0, out).astype(np.float32).astype(np.float64)
    m = (n * (1 + rng.standard_normal(out) * 0.05)).astype(np.float32).astype(np.float64)
    return base, lora, m, n


def pin_compose_closed_forms(o, seed=3):
    base, lora, m, n = _compose_inputs(seed)
    s = 1.75
    # m == n: g = 1, the delta is exactly s * lora and the full output base + s * lora
    np.testing.assert_array_equal(o.compose_fwd(base, lora, n, n, s), s * lora)
    np.testing.assert_array_equal(o.compose_fwd(base, np.zeros_like(lora), n, n, s, add_base=True), base)
    # m == 0: the layer output vanishes, the delta is -base
    np.testing.assert_allclose(o.compose_fwd(base, lora, np.zeros_like(m), n, s, add_base=True), 0.0, atol=1e-15)
    np.testing.assert_allclose(o.compose_fwd(base, lora, np.zeros_like(m), n, s), -base, atol=1e-15)
    # the stable form equals the direct DoRA output g * (base + s * lora) (and minus base for the delta)
    g = m / n
    full = g * (base + s * lora)
    np.testing.assert_allclose(o.compose_fwd(base, lora, m, n, s, add_base=True), full, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(o.compose_fwd(base, lora, m, n, s), full - base, rtol=1e-12, atol=1e-14)
    # the correction term alone: with lora = 0 the delta is (g - 1) * base, nonzero where m != n
    corr = o.compose_fwd(base, np.zeros_like(lora), m, n, s)
    assert np.all((corr != 0) == ((m != n)[None, :] & (base != 0)))
    # column scaling: doubling m doubles the full output
    np.testing.assert_allclose(o.compose_fwd(base, lora, 2 * m, n, s, add_base=True), 2 * full, rtol=1e-13)


def pin_lora_compose_exact(o, seed=8):
    """The fused compose against exact rational arithmetic on tiny inputs
    (square and non-square B, so a transposed operand shows), the unfused
    compose with B = identity, and h = 0."""
    rng = np.random.default_rng(seed)
    for t in range(6):
        T, out, r = int(rng.integers(1, 5)), int(rng.integers(1, 6)), int(rng.integers(1, 5))
        if t % 2 == 0:
            r = out
        base = _bf16_exact(rng, (T, out), 1.0)
        h = _bf16_exact(rng, (T, r), 1.0)
        B = _bf16_exact(rng, (out, r), 0.5)
        n = rng.uniform(0.5, 2.0, out).astype(np.float32)
        m = (n * (1 + rng.uniform(-0.01, 0.01, out))).astype(np.float32)
        s = float(np.float32(rng.uniform(0.5, 3.0)))
        for add_base in (False, True):
            got = np.asarray(o.lora_compose_fwd(base, h, B, m, n, s, add_base=add_base), dtype=np.float64)
            assert got.shape == (T, out), got.shape
            for i in range(T):
                for j in range(out):
                    g = Fraction(float(m[j])) / Fraction(float(n[j]))
                    lora = sum(Fraction(float(h[i, k])) * Fraction(float(B[j, k])) for k in range(r))
                    bb = Fraction(float(base[i, j]))
                    want = (g - 1) * bb + g * Fraction(s) * lora + (bb if add_base else 0)
                    tol = 1e-13 * (abs(float((g - 1) * bb)) + abs(float(g * Fraction(s) * lora)) + abs(float(bb)))
                    assert abs(got[i, j] - float(want)) <= tol + 1e-300, (t, i, j, got[i, j], float(want))
    base, lora, m, n = _compose_inputs(seed, T=6, out=5)
    eye = np.eye(5)
    np.testing.assert_array_equal(o.lora_compose_fwd(base, lora, eye, m, n, 1.25),
                                  o.compose_fwd(base, lora, m, n, 1.25))
    y0 = o.lora_compose_fwd(base, np.zeros((6, 3)), np.ones((5, 3)), m, n, 1.25)
    g = m.astype(np.float64) / n.astype(np.float64)
    np.testing.assert_allclose(y0, (g - 1.0) * base, rtol=1e-15, atol=0)


def pin_lora_compose_bwd(o, seed=9):
    """The fused backward against central finite differences of the fp64 loss
    L = sum(dy * y) through lora_compose_fwd (with respect to base, B and m),
    torch.autograd in fp64 through the dense formula, and the identity
    sum_t dy lora = sum_k B (dy^T h) on the magnitude gradient."""
    rng = np.random.default_rng(seed)
    T, out, r = 7, 5, 3
    base = rng.standard_normal((T, out))
    h = rng.standard_normal((T, r))
    B = rng.standard_normal((out, r)) * 0.5
    n = rng.uniform(0.5, 2.0, out)
    m = n * (1 + rng.uniform(-0.05, 0.05, out))
    dy = rng.standard_normal((T, out))
    s = 1.375
    for add_base in (False, True):
        db, dB, dm = (np.asarray(a, np.float64) for a in o.lora_compose_bwd(dy, base, h, B, m, n, s, add_base=add_base))
        assert db.shape == (T, out) and dB.shape == (out, r) and dm.shape == (out,)
        L = lambda b_, B_, m_: float(np.sum(dy * o.lora_compose_fwd(b_, h, B_, m_, n, s, add_base=add_base)))
        eps = 1e-6
        for (i, j) in [(0, 0), (3, 2), (6, 4)]:
            e = np.zeros_like(base); e[i, j] = eps
            fd = (L(base + e, B, m) - L(base - e, B, m)) / (2 * eps)
            assert abs(db[i, j] - fd) <= 1e-6 * max(1.0, abs(fd)), (add_base, i, j, db[i, j], fd)
        for (j, k) in [(0, 0), (2, 1), (4, 2)]:
            e = np.zeros_like(B); e[j, k] = eps
            fd = (L(base, B + e, m) - L(base, B - e, m)) / (2 * eps)
            assert abs(dB[j, k] - fd) <= 1e-6 * max(1.0, abs(fd)), (add_base, j, k, dB[j, k], fd)
        for j in range(out):
            e = np.zeros_like(m); e[j] = eps
            fd = (L(base, B, m + e) - L(base, B, m - e)) / (2 * eps)
            assert abs(dm[j] - fd) <= 1e-6 * max(1.0, abs(fd)), (add_base, j, dm[j], fd)
        tb = torch.tensor(base, requires_grad=True)
        tB = torch.tensor(B, requires_grad=True)
        tm = torch.tensor(m, requires_grad=True)
        y = (tm / torch.tensor(n)) * (tb + s * (torch.tensor(h) @ tB.T))
        if not add_base:
            y = y - tb
        (y * torch.tensor(dy)).sum().backward()
        np.testing.assert_allclose(db, tb.grad.numpy(), rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(dB, tB.grad.numpy(), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(dm, tm.grad.numpy(), rtol=1e-12, atol=1e-13)
    E = dy.T @ h
    alt = (np.sum(dy * base, axis=0) + s * np.sum(B * E, axis=1)) / n
    np.testing.assert_allclose(o.lora_compose_bwd(dy, base, h, B, m, n, s)[2], alt, rtol=1e-12)


def pin_compose_bwd_finite_differences(o, seed=4):
    """Central differences of L = sum(dy * y); y is affine in m, base and lora, so
    the differences are exact up to rounding."""
    base, lora, m, n = _compose_inputs(seed)
    s = 1.25
    rng = np.random.default_rng(seed + 100)
    dy = _bf16_exact(rng, base.shape, 1.0)
    for add_base in (False, True):
        dl, db, dm = o.compose_bwd(dy, base, lora, m, n, s, add_base=add_base)

        def L(mm=m, bb=base, ll=lora):
            return float(np.sum(dy * o.compose_fwd(bb, ll, mm, n, s, add_base=add_base)))

        h = 1e-3
        for j in range(len(m)):
            e = np.zeros_like(m)
            e[j] = h
            fd = (L(mm=m + e) - L(mm=m - e)) / (2 * h)
            assert abs(fd - dm[j]) <= 1e-9 * (1 + abs(fd)), (add_base, j, fd, dm[j])
        for (t, j) in [(0, 0), (3, 2), (6, 4), (2, 1)]:
            e = np.zeros_like(base)
            e[t, j] = h
            fd_b = (L(bb=base + e) - L(bb=base - e)) / (2 * h)
            fd_l = (L(ll=lora + e) - L(ll=lora - e)) / (2 * h)
            assert abs(fd_b - db[t, j]) <= 1e-9 * (1 + abs(fd_b)), (add_base, t, j, fd_b, db[t, j])
            assert abs(fd_l - dl[t, j]) <= 1e-9 * (1 + abs(fd_l)), (add_base, t, j, fd_l, dl[t, j])


def pin_compose_bwd_autograd(o, seed=5):
    """torch.autograd in fp64 through g * (base + s * lora) (n detached)."""
    base, lora, m, n = _compose_inputs(seed, T=11, out=6)
    s = 0.875
    rng = np.random.default_rng(seed + 7)
    dy = _bf16_exact(rng, base.shape, 1.0)
    for add_base in (False, True):
        tb = torch.tensor(base, requires_grad=True)
        tl = torch.tensor(lora, requires_grad=True)
        tm = torch.tensor(m, requires_grad=True)
        tn = torch.tensor(n)
        y = (tm / tn) * (tb + s * tl)
        if not add_base:
            y = y - tb
        (y * torch.tensor(dy)).sum().backward()
        dl, db, dm = o.compose_bwd(dy, base, lora, m, n, s, add_base=add_base)
        np.testing.assert_allclose(dl, tl.grad.numpy(), rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(db, tb.grad.numpy(), rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(dm, tm.grad.numpy(), rtol=1e-12, atol=1e-14)
    # no tokens: the magnitude gradient is an empty sum
    dl, db, dm = o.compose_bwd(dy[:0], base[:0], lora[:0], m, n, s)
    assert dl.shape == (0, 6) and np.all(dm == 0)


# ------------------------------------------------------------------ norm backward


def _norm_bwd_fraction_factored(d, n, W0, A, B, s):
    """The factored gradients, exactly: c_i = d_i / n_i,
    d_B_i = s c_i (U_i + s B_i G) with U = W0 A^T, G = A A^T, and
    d_A = s (c B)^T W0 + s^2 (B^T diag(c) B) A."""
    out, inn = W0.shape
    r = A.shape[0]
    F = lambda M: [[Fraction(float(v)) for v in row] for row in M]
    W, Af, Bf = F(W0), F(A), F(B)
    c = [Fraction(float(di)) / Fraction(float(ni)) for di, ni in zip(d, n)]
    sf = Fraction(float(s))
    G = [[sum(Af[j][k] * Af[l][k] for k in range(inn)) for l in range(r)] for j in range(r)]
    U = [[sum(W[i][k] * Af[j][k] for k in range(inn)) for j in range(r)] for i in range(out)]
    dB = [[sf * c[i] * (U[i][j] + sf * sum(Bf[i][l] * G[l][j] for l in range(r))) for j in range(r)]
          for i in range(out)]
    M = [[sum(Bf[i][j] * c[i] * Bf[i][l] for i in range(out)) for l in range(r)] for j in range(r)]
    dA = [[sf * sum(c[i] * Bf[i][j] * W[i][k] for i in range(out))
           + sf * sf * sum(M[j][l] * Af[l][k] for l in range(r)) for k in range(inn)] for j in range(r)]
    return dA, dB


def pin_norm_bwd(o, seed=10):
    """weight_norm_bwd against: exact rational arithmetic of the factored
    formulas (a different formula from the oracle's dense chain rule); central
    finite differences of weight_norm (itself pinned above); torch.autograd in
    fp64 through torch's own vector norm; the bilinearity identity
    <A, d_A> = <B, d_B> (V depends on A and B only through B A, so scaling
    either by t moves V alike); and B = 0 and r = 1 closed forms."""
    rng = np.random.default_rng(seed)
    # exact rational check on bf16-exact inputs with an arbitrary positive n
    for out, inn, r in [(3, 5, 2), (4, 3, 3)]:
        W0 = _bf16_exact(rng, (out, inn), 0.5)
        A = _bf16_exact(rng, (r, inn), 0.5)
        B = _bf16_exact(rng, (out, r), 0.5)
        d = _bf16_exact(rng, (out,), 1.0)
        n = np.abs(_bf16_exact(rng, (out,), 1.0)) + 0.25
        s = 1.5
        dA, dB = (np.asarray(x, np.float64) for x in o.weight_norm_bwd(d, n, W0, A, B, s))
        assert dA.shape == (r, inn) and dB.shape == (out, r)
        eA, eB = _norm_bwd_fraction_factored(d, n, W0, A, B, s)
        for got, exact in ((dA, eA), (dB, eB)):
            ex = np.array([[float(v) for v in row] for row in exact])
            np.testing.assert_allclose(got, ex, rtol=1e-12, atol=1e-14)
    # finite differences of the (pinned) forward norm, with the true n
    out, inn, r = 5, 6, 3
    W0 = rng.standard_normal((out, inn))
    A = rng.standard_normal((r, inn)) * 0.7
    B = rng.standard_normal((out, r)) * 0.7
    d = rng.standard_normal(out)
    s = 0.8
    n = o.weight_norm(W0, A, B, s)
    dA, dB = o.weight_norm_bwd(d, n, W0, A, B, s)
    L = lambda A_, B_: float(np.sum(d * o.weight_norm(W0, A_, B_, s)))
    eps = 1e-6
    for (j, k) in [(0, 0), (1, 4), (2, 5)]:
        e = np.zeros_like(A); e[j, k] = eps
        fd = (L(A + e, B) - L(A - e, B)) / (2 * eps)
        assert abs(dA[j, k] - fd) <= 1e-7 * max(1.0, abs(fd)), (j, k, dA[j, k], fd)
    for (i, j) in [(0, 0), (2, 1), (4, 2)]:
        e = np.zeros_like(B); e[i, j] = eps
        fd = (L(A, B + e) - L(A, B - e)) / (2 * eps)
        assert abs(dB[i, j] - fd) <= 1e-7 * max(1.0, abs(fd)), (i, j, dB[i, j], fd)
    # torch autograd through torch's vector norm
    tA = torch.tensor(A, requires_grad=True)
    tB = torch.tensor(B, requires_grad=True)
    tn = torch.linalg.vector_norm(torch.tensor(W0) + s * (tB @ tA), dim=1)
    (tn * torch.tensor(d)).sum().backward()
    np.testing.assert_allclose(dA, tA.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dB, tB.grad.numpy(), rtol=1e-12, atol=1e-13)
    # bilinearity: <A, d_A> = <B, d_B>
    a, b = float(np.sum(A * dA)), float(np.sum(B * dB))
    assert abs(a - b) <= 1e-12 * (abs(a) + abs(b) + 1e-300), (a, b)
    # B = 0: d_A = 0 and d_B_i = s (d_i / n_i) W0_i A^T; n = ||W0_i|| (library norm)
    Bz = np.zeros_like(B)
    nz = np.linalg.norm(W0, axis=1)
    dA0, dB0 = o.weight_norm_bwd(d, nz, W0, A, Bz, s)
    assert np.all(np.asarray(dA0) == 0.0)
    np.testing.assert_allclose(dB0, s * (d / nz)[:, None] * (W0 @ A.T), rtol=1e-13, atol=1e-15)
    # r = 1: d_B_i = s c_i (w_i . a + s b_i |a|^2), d_A = s sum_i c_i b_i (w_i + s b_i a)
    a1 = rng.standard_normal((1, inn))
    b1 = rng.standard_normal((out, 1))
    n1 = o.weight_norm(W0, a1, b1, s)
    c = d / n1
    dA1, dB1 = o.weight_norm_bwd(d, n1, W0, a1, b1, s)
    ref_B = s * c * (W0 @ a1[0] + s * b1[:, 0] * np.dot(a1[0], a1[0]))
    ref_A = s * np.sum((c * b1[:, 0])[:, None] * (W0 + s * b1[:, 0][:, None] * a1[0][None, :]), axis=0)
    np.testing.assert_allclose(np.asarray(dB1)[:, 0], ref_B, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(np.asarray(dA1)[0], ref_A, rtol=1e-12, atol=1e-14)
    # a zero norm row contributes nothing
    n0 = n.copy(); n0[1] = 0.0
    dA2, dB2 = o.weight_norm_bwd(d, n0, W0, A, B, s)
    assert np.all(np.asarray(dB2)[1] == 0.0) and np.all(np.isfinite(dA2))
    d_one = d.copy(); d_one[1] = 0.0
    np.testing.assert_allclose(dA2, o.weight_norm_bwd(d_one, n, W0, A, B, s)[0], rtol=1e-13, atol=1e-15)


ALL_PINS = [
    pin_norm_exact_bruteforce,
    pin_norm_special_cases,
    pin_norm_golden,
    pin_norm_invariances,
    pin_row_sqnorm,
    pin_norm_cached,
    pin_compose_golden,
    pin_compose_closed_forms,
    pin_lora_compose_exact,
    pin_lora_compose_bwd,
    pin_compose_bwd_finite_differences,
    pin_compose_bwd_autograd,
    pin_norm_bwd,
]
