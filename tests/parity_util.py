"""Tolerances of the parity tests, derived from the arithmetic.

* Norm (fp32 output): relative 1e-5 of the oracle's fp64 value.  Where the terms
  cancel, fp32 arithmetic cannot hold a relative bound, so an element also
  passes when |n_gpu^2 - n^2| is within 2^-16 of the term mass (about 2^8 fp32
  ulps of it: the split-K fp32 partials, and the two-term split of G, whose
  ~16 significant bits per element bound the Gram term's error by 2^-16 of
  its absolute sum).  The mass adds the absolute values of every product
  inside each term: base + 2s sum_j |B_ij| (|W0_i| |A_j|^T) +
  s^2 |B_i| |A A^T| |B_i|^T.  The values |cross| and Gram alone understate it
  where the terms of the quadratic form B_i G B_i^T cancel (a row of B with
  mixed signs against a G with large off-diagonal entries, as for a short
  input axis).
* Compose outputs and gradients (stored bf16/fp16): within 2 bf16 ulps of the
  oracle value (bf16) or 1e-3 relative (fp16).  fp32 intermediates bound the
  absolute error by a few fp32 ulps of the term mass, not of the result, so an
  element where the terms cancel also passes when |delta| <= 2^-22 * mass
  (4 fp32 ulps of the mass), plus half the dtype's subnormal spacing.
* Compose with lora = h B^T formed inside: the same, with the floor raised to
  3 (r + 4) 2^-24 of the term mass |(g-1) base| + |g s| sum_k |h_k B_k| (+ |base|):
  an fp32 sum of r exact products errs by at most (r - 1) 2^-24 of their
  absolute sum, the compose adds 4 roundings, and the final rounding to the
  storage dtype at most doubles that where the floor decides.
* Magnitude gradient (fp32): |delta| <= 1e-5 * sum_t |dy * (base + s*lora)| / n
  (condition-aware: the reduction order differs from the oracle's, so several
  fp32 results are correct).
"""
from __future__ import annotations

import numpy as np

BF16_MIN_EXP = -126
F16_SUB_HALF = 2.0**-25  # half the fp16 subnormal spacing
BF16_SUB_HALF = 2.0**-134


def representable_nonzero(ref: np.ndarray, dtype: str) -> np.ndarray:
    """Where the exact value rounds to a nonzero storage value (round to nearest
    even: strictly above half the smallest subnormal)."""
    half = F16_SUB_HALF if dtype == "fp16" else BF16_SUB_HALF
    return np.abs(ref) > half


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, BF16_MIN_EXP)
    return np.where(a > 0, 2.0 ** (e - 7), 2.0**-133)


def compose_ok(gpu: np.ndarray, ref: np.ndarray, mass: np.ndarray, dtype: str, floor_rel: float = 2.0**-22):
    """Boolean mask of passing elements and the mask of those passing only on the floor."""
    err = np.abs(gpu - ref)
    floor = floor_rel * mass
    if dtype == "bf16":
        main = err <= 2.0 * bf16_ulp(ref)
        floor = floor + BF16_SUB_HALF
    else:
        main = err <= 1e-3 * np.abs(ref)
        floor = floor + F16_SUB_HALF
    ok = main | (err <= floor)
    return ok, ok & ~main


def assert_compose(gpu, ref, mass, dtype, what, floor_rel: float = 2.0**-22):
    ok, floor_only = compose_ok(gpu, ref, mass, dtype, floor_rel)
    if not ok.all():
        bad = np.argwhere(~ok)[:5]
        vals = [(tuple(int(i) for i in b), float(gpu[tuple(b)]), float(ref[tuple(b)])) for b in bad]
        raise AssertionError(f"{what}: {(~ok).sum()} of {ok.size} elements out of tolerance, e.g. {vals}")
    return int(floor_only.sum())


def assert_norm(gpu, ref, mass, what, rtol=1e-5):
    gpu = np.asarray(gpu, np.float64)
    rel_ok = np.abs(gpu - ref) <= rtol * np.abs(ref)
    cancel_ok = np.abs(gpu * gpu - ref * ref) <= 2.0**-16 * mass
    ok = rel_ok | cancel_ok
    if not ok.all():
        bad = np.argwhere(~ok)[:5, 0]
        raise AssertionError(f"{what}: {(~ok).sum()} of {ok.size} rows out of tolerance, e.g. "
                             f"{[(int(i), float(gpu[i]), float(ref[i])) for i in bad]}")
    return int((ok & ~rel_ok).sum())


def assert_dmag(gpu, ref, cond, what):
    gpu = np.asarray(gpu, np.float64)
    ok = np.abs(gpu - ref) <= 1e-5 * cond + 1e-30
    if not ok.all():
        bad = np.argwhere(~ok)[:5, 0]
        raise AssertionError(f"{what}: {(~ok).sum()} of {ok.size} columns out of tolerance, e.g. "
                             f"{[(int(i), float(gpu[i]), float(ref[i]), float(cond[i])) for i in bad]}")


def norm_term_mass(W0, A, B, s):
    """Absolute mass of the three terms per row, in fp64 (scale of the
    cancellation floor): base + the absolute sums of the cross and Gram terms'
    products."""
    aW, aA, aB = np.abs(W0), np.abs(A), np.abs(B)
    base = np.sum(W0 * W0, axis=1)
    cross = 2.0 * s * np.sum(aB * (aW @ aA.T), axis=1)
    gram = s * s * np.sum((aB @ np.abs(A @ A.T)) * aB, axis=1)
    return base + cross + gram
