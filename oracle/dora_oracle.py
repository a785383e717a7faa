"""CPU fp64 oracle of the DoRA hot path.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The product path (the HIP library and its Python binding)
never calls it, and it shares no code with that path.

Source of truth: the press summary of arXiv:2603.22276 ("AI training
breakthrough: Anthropic team cracks the memory bottleneck of large-model
fine-tuning", techwalker.com/2026/0401/3182870).  The page prints no equations
with numbers; it names the operations:

* the DoRA weight norm, taken per output row of W0 + s*B*A (paragraph on the
  "factored norm", and the Q&A on why DoRA needs so much memory).  The factored
  method splits it into base, cross and Gram terms and reaches *the same result*
  by algebra, so the oracle is the plain definition: form W0 + s*B*A densely in
  fp64 and take Euclidean row norms.
* the magnitude compose in its stable form (g - 1) * base + g * s * lora, with
  g = m / n per output feature (paragraph on numerical stability near g = 1).
  The formula is the adapter's delta; ``add_base`` adds base to it.
* the backward of that compose, including the magnitude gradient, which is a
  reduction over tokens (paragraph on the convergence study: the dmag reduction
  order).  The norm n is treated as a constant in the backward.
* the compose with the adapter's second projection fused in (the page's
  paragraph on where the speedup comes from: fewer memory accesses): given
  h = x A^T [T x r] and B [out x r], lora = h B^T is formed inside the compose
  and never stored; ``lora_compose_fwd`` is the compose forward of that product,
  and ``lora_compose_bwd`` its backward with respect to base, B and m, which
  never needs lora or d_lora stored.
* the cached base term the page lists as future work (paragraph on
  limitations): W0 is frozen, so ||W0_i||^2 can be computed once and reused.
  ``row_sqnorm`` is that per-row square norm; ``weight_norm_cached`` is the
  weight norm with its base term taken from a given cache c instead of W0,
  n_i^2 = c_i + (||W0_i + s*(BA)_i||^2 - ||W0_i||^2), the difference written
  out densely as 2s<W0_i, (BA)_i> + s^2 ||(BA)_i||^2.
* the backward of the weight norm itself, for a caller that does not detach
  n (the page is silent on whether the norm is differentiated; the detached
  reading is the main one, this is the alternative).  ``weight_norm_bwd``
  gives the gradients of L = sum_i dn_i * n_i with respect to A and B (W0 is
  frozen), written from the dense definition: with V = W0 + s*B*A and
  n_i = ||V_i||, dn_i/dV_i = V_i / n_i, so dV = (dn/n) * V row-wise,
  d_B = s * dV A^T and d_A = s * B^T dV.

Everything is computed in fp64 from the exact values of the inputs: bf16/fp16
tensors and fp32 vectors convert to fp64 without rounding, and ``s`` is the fp32
scale the kernels receive.  numpy's matmul, sum and sqrt are the only library
steps.  No blocking, fusion or reordering beyond the definitions.

Readings of points the page leaves open (also listed in the design notes):
W0 is [out x in], A [r x in], B [out x r] (nn.Linear orientation); the norm is
L2 over the input axis; g = m / n with m, n fp32 per output feature; the
compose output is the delta unless add_base; n is detached in the backward.
"""
from __future__ import annotations

import numpy as np


def as_f64(t) -> np.ndarray:
    """Exact fp64 copy of a torch tensor (bf16, fp16, fp32) or numpy array."""
    if hasattr(t, "detach"):
        return t.detach().cpu().double().numpy()
    return np.asarray(t, dtype=np.float64)


def weight_norm(W0, A, B, s) -> np.ndarray:
    """n_i = || W0_i + s * (B A)_i ||_2 for every output row i.

    The dense definition of the DoRA weight norm (summary page, paragraph on the
    factored norm: base + cross + Gram terms give the same value as this).
    Shapes: W0 [out x in], A [r x in], B [out x r]; returns fp64 [out].
    Passing a row subset of W0 and B gives the norms of those rows.
    """
    W0, A, B = as_f64(W0), as_f64(A), as_f64(B)
    s = float(s)
    V = W0 + s * (B @ A)  # the out x in matrix the GPU path never forms
    return np.sqrt(np.sum(V * V, axis=1))


def row_sqnorm(W0) -> np.ndarray:
    """c_i = ||W0_i||^2 = sum_k W0_ik^2 per output row: the base term of the
    norm, a function of the frozen W0 alone (summary page, paragraph on
    limitations and future work: cache it).  Returns fp64 [out]."""
    W0 = as_f64(W0)
    return np.sum(W0 * W0, axis=1)


def weight_norm_cached(base_sq, W0, A, B, s) -> np.ndarray:
    """The weight norm with a cached base term c (= base_sq):

        n_i = sqrt(max(c_i + 2 s <W0_i, (BA)_i> + s^2 ||(BA)_i||^2, 0))

    With c_i = ||W0_i||^2 this is ||W0_i + s (BA)_i||_2; any other c shifts
    n_i^2 by c_i - ||W0_i||^2.  BA is formed densely in fp64; a negative n^2
    is clamped to 0.  base_sq: [out] (fp32 as the kernels receive it, or
    fp64); returns fp64 [out].
    """
    c = as_f64(base_sq)
    W0, A, B = as_f64(W0), as_f64(A), as_f64(B)
    s = float(s)
    V = B @ A
    n2 = c + 2.0 * s * np.sum(W0 * V, axis=1) + s * s * np.sum(V * V, axis=1)
    return np.sqrt(np.maximum(n2, 0.0))


def weight_norm_bwd(d_norm, norm, W0, A, B, s):
    """Gradients of L = sum_i d_norm_i * n_i with respect to A and B, where
    n_i = || W0_i + s * (B A)_i ||_2 and W0 is frozen.

    Chain rule through the dense definition: V = W0 + s * B A, dn_i/dV_i =
    V_i / n_i, so dV = (d_norm / norm)[:, None] * V; then d_B = s * dV A^T
    [out x r] and d_A = s * B^T dV [r x in].  ``norm`` is the n the caller
    holds (the forward's fp32 result, or any positive values): it is used as
    given, not recomputed.  Rows with n_i = 0 give no gradient (the zero
    subgradient, which is what a library norm's backward takes at 0).
    d_norm, norm: [out].  Returns fp64 (d_A [r x in], d_B [out x r]).
    """
    W0, A, B = as_f64(W0), as_f64(A), as_f64(B)
    d, n = as_f64(d_norm), as_f64(norm)
    s = float(s)
    c = np.zeros_like(n)
    nz = n != 0.0
    c[nz] = d[nz] / n[nz]
    dV = c[:, None] * (W0 + s * (B @ A))  # the out x in matrix the GPU path never forms
    return s * (B.T @ dV), s * (dV @ A.T)


def scale_factor(m, n) -> np.ndarray:
    """g = m / n per output feature (summary page, paragraph on stability near g = 1)."""
    return as_f64(m) / as_f64(n)


def compose_fwd(base, lora, m, n, s, add_base: bool = False) -> np.ndarray:
    """y = (g - 1) * base + g * s * lora, g = m / n broadcast over tokens.

    The stable compose form of the summary page (paragraph on numerical
    stability).  With ``add_base`` the output is base + that delta, which is
    the full DoRA layer output g * (base + s * lora).
    base, lora: [T x out]; m, n: [out].  Returns fp64 [T x out], unrounded.
    """
    base, lora = as_f64(base), as_f64(lora)
    g = scale_factor(m, n)
    s = float(s)
    y = (g - 1.0) * base + g * s * lora
    if add_base:
        y = y + base
    return y


def lora_compose_fwd(base, h, B, m, n, s, add_base: bool = False) -> np.ndarray:
    """compose_fwd with lora = h B^T: y = (g - 1) * base + g * s * (h B^T) (+ base).

    h: [T x r] (x A^T in the storage dtype), B: [out x r], base: [T x out].
    The product is exact fp64 from the exact input values.  Returns fp64
    [T x out], unrounded.
    """
    lora = as_f64(h) @ as_f64(B).T
    return compose_fwd(base, lora, m, n, s, add_base)


def lora_compose_bwd(dy, base, h, B, m, n, s, add_base: bool = False):
    """Backward of lora_compose_fwd for L = sum(dy * y), n held fixed:

        d_base = (g - 1) * dy, or g * dy with add_base
        d_B    = (g * s * dy)^T h                          [out x r]
        d_mag  = sum_t dy_tj * (base_tj + s * (h B^T)_tj) / n_j

    d_B is the gradient of the adapter's second projection through
    lora = h B^T (d_lora = g * s * dy, then d_lora^T h).  Returns fp64
    (d_base [T x out], d_B [out x r], d_mag [out]).
    """
    dy, base, h, B = as_f64(dy), as_f64(base), as_f64(h), as_f64(B)
    n = as_f64(n)
    g = scale_factor(m, n)
    s = float(s)
    lora = h @ B.T
    d_lora = g * s * dy
    d_base = (g if add_base else (g - 1.0)) * dy
    d_B = d_lora.T @ h
    d_mag = np.sum(dy * (base + s * lora), axis=0) / n
    return d_base, d_B, d_mag


def compose_bwd(dy, base, lora, m, n, s, add_base: bool = False):
    """Gradients of L = sum(dy * y) for the compose above, with n held fixed.

    d_lora = g * s * dy
    d_base = (g - 1) * dy, or g * dy with add_base
    d_mag_j = sum_t dy_tj * (base_tj + s * lora_tj) / n_j   (reduction over tokens)

    The magnitude gradient is the token reduction the summary page mentions in
    its convergence paragraph.  Returns fp64 (d_lora [T x out], d_base [T x out],
    d_mag [out]).
    """
    dy, base, lora = as_f64(dy), as_f64(base), as_f64(lora)
    n = as_f64(n)
    g = scale_factor(m, n)
    s = float(s)
    d_lora = g * s * dy
    d_base = (g if add_base else (g - 1.0)) * dy
    d_mag = np.sum(dy * (base + s * lora), axis=0) / n
    return d_lora, d_base, d_mag
