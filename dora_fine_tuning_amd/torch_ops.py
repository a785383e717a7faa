"""PyTorch integration of the DoRA hot path: custom operators and a DoRA linear layer.

The press summary of arXiv:2603.22276 describes the fused kernels as a PyTorch
custom operator, which compiled graphs keep without breaks (paragraph on
framework compatibility). It also describes a three-tier dispatch (paragraph
on the dispatch tiers): training runs the fused forward and the fused
backward, inference runs the forward kernel alone, and whatever the kernels
cannot take goes to eager PyTorch.

This module registers:

* ``dora_amd::weight_norm`` -- the factored norm ||W0 + s*B*A|| per output row
  (fp32).  Callers that treat the norm as a constant (the usual DoRA reading)
  pass detached A and B.  Otherwise its autograd formula is
  ``dora_amd::weight_norm_backward``, the factored backward into A and B (W0
  is frozen and gets no gradient); ``weight_norm_cached`` has the same formula.
* ``dora_amd::lora_compose`` -- the compose with the adapter's second
  projection fused in: from h = x A^T and B it forms lora = h B^T inside the
  kernel and never stores it.  Its autograd formula is
  ``dora_amd::lora_compose_backward`` (d_base, d_B and d_mag without lora or
  d_lora), plus d_h = dy (g s .* B), a GEMM done by torch.
* ``dora_amd::row_sqnorm`` and ``dora_amd::weight_norm_cached`` -- the cached
  base term the page proposes as future work (W0 is frozen): ||W0_i||^2 once,
  then the norm that takes it instead of re-deriving it from W0.
* ``dora_amd::compose`` -- the stable compose (g - 1)*base + g*s*lora
  (+ base), g = m / n. Its autograd formula is the fused backward
  ``dora_amd::compose_backward``, which gives the gradients of base, lora and
  the magnitude m.
* ``DoRALinear`` -- a linear layer with frozen W0 and trainable A, B and m:
  y = x W0^T + compose(x W0^T, x A^T B^T, m, n, s), with n = ||W0 + s*B*A||
  detached by default.  With ``detach_norm=False`` the gradient also flows
  through n: the compose's formula gives dL/dn = -(m / n) * d_mag (L depends on
  n only through g = m / n; this [out]-sized product is the one step of the
  chain done by torch), and the norm's formula turns it into d_A and d_B.

Tiers (paragraph on the dispatch tiers): autograd records the compose only
when a gradient is needed (training: the fused forward, then the fused
backward); under ``torch.no_grad()`` or ``torch.inference_mode()`` the forward
kernel runs alone.  ``DoRALinear`` runs the compose with the second projection
fused in on both tiers, so lora = x A^T B^T is never stored.  The third tier
is eager PyTorch for inputs the kernels do not take: tensors on the CPU, matrix
dtypes other than bf16/fp16 (fp32), and a call the library refuses with
DORA_UNSUPPORTED.  Those run the plain, unfused torch form of each operator
(dense B A for the norm, the compose written out elementwise), computed in
fp32.  Supported inputs on a HIP device always take the kernels; a missing
library raises on import, it never falls back.

On that path every operator is argument marshalling around the C ABI
(``binding``); the arithmetic runs in the HIP kernels.
"""
from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F

from . import binding

Tensor = torch.Tensor


# ---------------------------------------------------------------- eager tier
#
# The plain PyTorch form of each operator, for inputs the kernels do not take
# (the page's fallback tier).  fp32 arithmetic, outputs in the matrices' dtype.


def _kernels_take(*mats: Tensor) -> bool:
    """True when the kernels take these matrix arguments: all on a HIP device,
    in bf16 or fp16."""
    return all(t.device.type == "cuda" and t.dtype in binding.DTYPE_CODE for t in mats)


def _unsupported(e: Exception) -> bool:
    return isinstance(e, binding.DoraError) and e.status == binding.DORA_UNSUPPORTED


def _eager_weight_norm(W0, A, B, s):
    V = W0.float() + s * (B.float() @ A.float())
    return torch.linalg.vector_norm(V, dim=1)


def _eager_row_sqnorm(W0):
    W = W0.float()
    return (W * W).sum(dim=1)


def _eager_weight_norm_cached(W0, A, B, base_sq, s):
    V = B.float() @ A.float()
    n2 = base_sq.float() + 2.0 * s * (W0.float() * V).sum(dim=1) + (s * s) * (V * V).sum(dim=1)
    return torch.sqrt(torch.clamp(n2, min=0.0))


def _eager_weight_norm_backward(W0, A, B, norm, d_norm, s):
    n, d = norm.float(), d_norm.float()
    c = torch.where(n != 0, d / torch.where(n != 0, n, torch.ones_like(n)), torch.zeros_like(n))
    dV = c[:, None] * (W0.float() + s * (B.float() @ A.float()))
    return (s * (B.float().t() @ dV)).to(A.dtype), (s * (dV @ A.float().t())).to(B.dtype)


def _scales(mag, norm):
    m, n = mag.float(), norm.float()
    return m / n, (m - n) / n  # g and g - 1 (the subtraction is exact near g = 1)


def _eager_compose(base, lora, mag, norm, s, add_base):
    g, gm1 = _scales(mag, norm)
    b = base.float()
    y = gm1 * b + g * s * lora.float()
    return (y + b if add_base else y).to(base.dtype)


def _eager_compose_backward(dy, base, lora, mag, norm, s, add_base, want_base):
    g, gm1 = _scales(mag, norm)
    d = dy.float()
    d_lora = (g * s * d).to(dy.dtype)
    d_base = ((g if add_base else gm1) * d).to(dy.dtype) if want_base else dy.new_empty((0,))
    d_mag = (d * (base.float() + s * lora.float())).sum(dim=0) / norm.float()
    return d_lora, d_base, d_mag


def _eager_lora_compose(base, h, B, mag, norm, s, add_base):
    return _eager_compose(base, h.float() @ B.float().t(), mag, norm, s, add_base)


def _eager_lora_compose_backward(dy, base, h, B, mag, norm, s, add_base, want_base):
    g, gm1 = _scales(mag, norm)
    d, hf, Bf = dy.float(), h.float(), B.float()
    E = d.t() @ hf  # dy^T h
    d_base = ((g if add_base else gm1) * d).to(dy.dtype) if want_base else dy.new_empty((0,))
    d_B = ((g * s)[:, None] * E).to(B.dtype)
    d_mag = ((d * base.float()).sum(dim=0) + s * (Bf * E).sum(dim=1)) / norm.float()
    return d_base, d_B, d_mag


# --------------------------------------------------------------------------- norm


@torch.library.custom_op("dora_amd::weight_norm", mutates_args=(), device_types="cuda")
def weight_norm(W0: Tensor, A: Tensor, B: Tensor, s: float) -> Tensor:
    """||W0_i + s * B_i A||_2 per output row i, fp32, via the factored kernels."""
    if not _kernels_take(W0, A, B):
        return _eager_weight_norm(W0, A, B, s)
    return binding.dora_norm_factored(W0.contiguous(), A.contiguous(), B.contiguous(), s)


@weight_norm.register_fake
def _weight_norm_fake(W0, A, B, s):
    return W0.new_empty((W0.shape[0],), dtype=torch.float32)


@torch.library.custom_op("dora_amd::row_sqnorm", mutates_args=(), device_types="cuda")
def row_sqnorm(W0: Tensor) -> Tensor:
    """||W0_i||^2 per output row, fp32."""
    if not _kernels_take(W0):
        return _eager_row_sqnorm(W0)
    return binding.dora_row_sqnorm(W0.contiguous())


@row_sqnorm.register_fake
def _row_sqnorm_fake(W0):
    return W0.new_empty((W0.shape[0],), dtype=torch.float32)


@torch.library.custom_op("dora_amd::weight_norm_cached", mutates_args=(), device_types="cuda")
def weight_norm_cached(W0: Tensor, A: Tensor, B: Tensor, base_sq: Tensor, s: float) -> Tensor:
    """The weight norm with the base term ||W0_i||^2 taken from base_sq."""
    if not _kernels_take(W0, A, B):
        return _eager_weight_norm_cached(W0, A, B, base_sq, s)
    return binding.dora_norm_factored_cached(W0.contiguous(), A.contiguous(), B.contiguous(),
                                             base_sq.contiguous().float(), s)


@weight_norm_cached.register_fake
def _weight_norm_cached_fake(W0, A, B, base_sq, s):
    return W0.new_empty((W0.shape[0],), dtype=torch.float32)


@torch.library.custom_op("dora_amd::weight_norm_backward", mutates_args=(), device_types="cuda")
def weight_norm_backward(W0: Tensor, A: Tensor, B: Tensor, norm: Tensor, d_norm: Tensor,
                         s: float) -> tuple[Tensor, Tensor]:
    """(d_A, d_B) of sum(d_norm * n) for n = ||W0 + s*B*A|| (norm: the forward's n)."""
    if not _kernels_take(W0, A, B):
        return _eager_weight_norm_backward(W0, A, B, norm, d_norm, s)
    return binding.dora_norm_bwd(W0.contiguous(), A.contiguous(), B.contiguous(), norm.contiguous().float(),
                                 d_norm.contiguous().float(), s)


@weight_norm_backward.register_fake
def _weight_norm_backward_fake(W0, A, B, norm, d_norm, s):
    return torch.empty_like(A), torch.empty_like(B)


def _norm_setup(ctx, inputs, output):
    W0, A, B = inputs[0], inputs[1], inputs[2]
    ctx.save_for_backward(W0, A, B, output)
    ctx.s = inputs[-1]
    ctx.n_inputs = len(inputs)


def _norm_grad(ctx, d_norm):
    W0, A, B, n = ctx.saved_tensors
    need_a, need_b = ctx.needs_input_grad[1], ctx.needs_input_grad[2]
    if ctx.needs_input_grad[0]:
        raise RuntimeError("dora_amd: W0 is frozen; the weight-norm backward gives gradients of A and B only")
    d_A = d_B = None
    if need_a or need_b:
        d_A, d_B = weight_norm_backward(W0, A, B, n, d_norm, ctx.s)
    return (None, d_A if need_a else None, d_B if need_b else None) + (None,) * (ctx.n_inputs - 3)


weight_norm.register_autograd(_norm_grad, setup_context=_norm_setup)
weight_norm_cached.register_autograd(_norm_grad, setup_context=_norm_setup)


# ------------------------------------------------------------------------ compose


@torch.library.custom_op("dora_amd::compose", mutates_args=(), device_types="cuda")
def compose(base: Tensor, lora: Tensor, mag: Tensor, norm: Tensor, s: float, add_base: bool) -> Tensor:
    """(g - 1) * base + g * s * lora, plus base when add_base, with g = mag / norm per column."""
    if not _kernels_take(base, lora):
        return _eager_compose(base, lora, mag, norm, s, add_base)
    return binding.dora_compose_fwd(base.contiguous(), lora.to(base.dtype).contiguous(), mag.contiguous().float(),
                                    norm.contiguous().float(), s, add_base=add_base)


@compose.register_fake
def _compose_fake(base, lora, mag, norm, s, add_base):
    return torch.empty_like(base)


@torch.library.custom_op("dora_amd::compose_backward", mutates_args=(), device_types="cuda")
def compose_backward(dy: Tensor, base: Tensor, lora: Tensor, mag: Tensor, norm: Tensor, s: float, add_base: bool,
                     want_base: bool) -> tuple[Tensor, Tensor, Tensor]:
    """(d_lora, d_base, d_mag) of the compose.  With want_base false the kernel
    does not write d_base and an empty tensor stands in for it."""
    if not _kernels_take(dy, base, lora):
        return _eager_compose_backward(dy, base, lora, mag, norm, s, add_base, want_base)
    d_lora, d_base, d_mag = binding.dora_compose_bwd(dy.contiguous(), base.contiguous(), lora.contiguous(),
                                                     mag.contiguous().float(), norm.contiguous().float(), s,
                                                     add_base=add_base, want_d_base=want_base)
    if d_base is None:
        d_base = dy.new_empty((0,))
    return d_lora, d_base, d_mag


@compose_backward.register_fake
def _compose_backward_fake(dy, base, lora, mag, norm, s, add_base, want_base):
    d_base = torch.empty_like(dy) if want_base else dy.new_empty((0,))
    return torch.empty_like(dy), d_base, mag.new_empty(mag.shape)


@torch.library.custom_op("dora_amd::lora_compose", mutates_args=(), device_types="cuda")
def lora_compose(base: Tensor, h: Tensor, B: Tensor, mag: Tensor, norm: Tensor, s: float, add_base: bool) -> Tensor:
    """(g - 1) * base + g * s * (h B^T), plus base when add_base; lora never stored."""
    if not _kernels_take(base, h, B):
        return _eager_lora_compose(base, h, B, mag, norm, s, add_base)
    return binding.dora_lora_compose_fwd(base.contiguous(), h.contiguous(), B.contiguous(), mag.contiguous().float(),
                                         norm.contiguous().float(), s, add_base=add_base)


@lora_compose.register_fake
def _lora_compose_fake(base, h, B, mag, norm, s, add_base):
    return torch.empty_like(base)


def _compose_setup(ctx, inputs, output):
    base, lora, mag, norm, s, add_base = inputs
    ctx.save_for_backward(base, lora, mag, norm)
    ctx.s = s
    ctx.add_base = add_base


def _compose_grad(ctx, dy):
    base, lora, mag, norm = ctx.saved_tensors
    want_base = bool(ctx.needs_input_grad[0])
    d_lora, d_base, d_mag = compose_backward(dy, base, lora, mag, norm, ctx.s, ctx.add_base, want_base)
    # a norm that is not detached: L depends on n only through g = m / n, so
    # dL/dn = -(m / n) * d_mag, with d_mag = sum_t dy (base + s lora) / n
    d_norm = -(mag / norm) * d_mag if ctx.needs_input_grad[3] else None
    return (d_base if want_base else None,
            d_lora if ctx.needs_input_grad[1] else None,
            d_mag if ctx.needs_input_grad[2] else None,
            d_norm, None, None)


compose.register_autograd(_compose_grad, setup_context=_compose_setup)


@torch.library.custom_op("dora_amd::lora_compose_backward", mutates_args=(), device_types="cuda")
def lora_compose_backward(dy: Tensor, base: Tensor, h: Tensor, B: Tensor, mag: Tensor, norm: Tensor, s: float,
                          add_base: bool, want_base: bool) -> tuple[Tensor, Tensor, Tensor]:
    """(d_base, d_B, d_mag) of ``lora_compose``, lora and d_lora never formed.
    With want_base false the kernel does not write d_base and an empty tensor
    stands in for it."""
    if not _kernels_take(dy, base, h, B):
        return _eager_lora_compose_backward(dy, base, h, B, mag, norm, s, add_base, want_base)
    try:
        d_base, d_B, d_mag = binding.dora_lora_compose_bwd(dy.contiguous(), base.contiguous(), h.contiguous(),
                                                           B.contiguous(), mag.contiguous().float(),
                                                           norm.contiguous().float(), s, add_base=add_base,
                                                           want_d_base=want_base)
    except binding.DoraError as e:
        if not _unsupported(e):  # a shape the library refuses (its slow path would be too slow): eager tier
            raise
        return _eager_lora_compose_backward(dy, base, h, B, mag, norm, s, add_base, want_base)
    if d_base is None:
        d_base = dy.new_empty((0,))
    return d_base, d_B, d_mag


@lora_compose_backward.register_fake
def _lora_compose_backward_fake(dy, base, h, B, mag, norm, s, add_base, want_base):
    d_base = torch.empty_like(dy) if want_base else dy.new_empty((0,))
    return d_base, torch.empty_like(B), mag.new_empty(mag.shape)


def _lora_compose_setup(ctx, inputs, output):
    base, h, B, mag, norm, s, add_base = inputs
    ctx.save_for_backward(base, h, B, mag, norm)
    ctx.s = s
    ctx.add_base = add_base


def _lora_compose_grad(ctx, dy):
    base, h, B, mag, norm = ctx.saved_tensors
    need = ctx.needs_input_grad
    d_base, d_B, d_mag = lora_compose_backward(dy, base, h, B, mag, norm, ctx.s, ctx.add_base, bool(need[0]))
    # the gradient of h through lora = h B^T: d_lora B = dy (g s .* B), the
    # caller's GEMM (a [T x out] by [out x r] product), with g s folded into B
    d_h = None
    if need[1]:
        gsB = ((mag / norm) * ctx.s)[:, None] * B.float()
        d_h = (dy @ gsB.to(dy.dtype))
    d_norm = -(mag / norm) * d_mag if need[4] else None
    return (d_base if need[0] else None, d_h, d_B if need[2] else None, d_mag if need[3] else None, d_norm,
            None, None)


lora_compose.register_autograd(_lora_compose_grad, setup_context=_lora_compose_setup)


# The eager tier is also each operator's kernel for CPU tensors.
weight_norm.register_kernel("cpu")(_eager_weight_norm)
row_sqnorm.register_kernel("cpu")(_eager_row_sqnorm)
weight_norm_cached.register_kernel("cpu")(_eager_weight_norm_cached)
weight_norm_backward.register_kernel("cpu")(_eager_weight_norm_backward)
compose.register_kernel("cpu")(_eager_compose)
compose_backward.register_kernel("cpu")(_eager_compose_backward)
lora_compose.register_kernel("cpu")(_eager_lora_compose)
lora_compose_backward.register_kernel("cpu")(_eager_lora_compose_backward)


# -------------------------------------------------------------------------- layer


class DoRALinear(torch.nn.Module):
    """DoRA-adapted linear layer: frozen W0 [out x in], trainable A [r x in],
    B [out x r] and magnitude m [out] (fp32); scale s = alpha / sqrt(r) (rsLoRA).

    Initialisation follows LoRA/DoRA practice: B = 0 and m = ||W0|| per row,
    so the layer starts out equal to x W0^T.  A is drawn from N(0, 1/in).  On a
    HIP device m is taken from the factored norm itself, so g = m / n is exactly
    1 at B = 0 and the first output equals x W0^T bit for bit.

    W0 is frozen, so its row square norms are computed once (on the first norm
    on a HIP device) and kept in the buffer ``weight_sqnorm``; the norm then
    takes its base term from there.  After changing ``weight``, call
    ``refresh_weight_cache()``.

    ``detach_norm`` (default True) treats n as a constant in the backward; with
    False the gradients of A and B also carry the path through n, by the
    factored norm backward.
    """

    def __init__(self, in_features: int, out_features: int, r: int, alpha: float = 32.0,
                 weight: Tensor | None = None, dtype: torch.dtype = torch.bfloat16, device=None,
                 detach_norm: bool = True):
        super().__init__()
        self.detach_norm = detach_norm
        if dtype not in (torch.bfloat16, torch.float16, torch.float32):
            raise ValueError(f"unsupported dtype {dtype}; bf16 and fp16 (HIP kernels) and fp32 (eager tier) are")
        self.in_features, self.out_features, self.r = in_features, out_features, r
        self.s = float(np.float32(alpha / math.sqrt(r)))
        if weight is None:
            weight = torch.randn(out_features, in_features, device=device) / math.sqrt(in_features)
        self.register_buffer("weight", weight.to(device=device, dtype=dtype).contiguous())
        self.lora_A = torch.nn.Parameter(
            (torch.randn(r, in_features, device=device) / math.sqrt(in_features)).to(dtype))
        self.lora_B = torch.nn.Parameter(torch.zeros(out_features, r, device=device, dtype=dtype))
        self.magnitude = torch.nn.Parameter(self.weight.float().norm(dim=1))
        self.register_buffer("weight_sqnorm", None)
        if self.weight.is_cuda:
            self.reset_magnitude()

    @torch.no_grad()
    def refresh_weight_cache(self) -> None:
        """Recompute ||W0_i||^2 (after ``weight`` changed)."""
        self.weight_sqnorm = row_sqnorm(self.weight)

    @torch.no_grad()
    def reset_magnitude(self) -> None:
        """m = ||W0 + s*B*A|| per row (the DoRA initialisation of the magnitude)."""
        self.magnitude.copy_(self.weight_norm())

    def weight_norm(self) -> Tensor:
        """n = ||W0 + s*B*A|| per output row (base term from the cache); detached
        unless the layer was built with ``detach_norm=False``."""
        if self.weight_sqnorm is None or self.weight_sqnorm.device != self.weight.device:
            self.refresh_weight_cache()
        A, B = (self.lora_A.detach(), self.lora_B.detach()) if self.detach_norm else (self.lora_A, self.lora_B)
        return weight_norm_cached(self.weight, A, B, self.weight_sqnorm, self.s)

    def forward(self, x: Tensor) -> Tensor:
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.in_features)
        base = F.linear(x2, self.weight)
        h = F.linear(x2, self.lora_A)
        # lora = h B^T is formed inside the compose kernel on both tiers; on the
        # training tier autograd records it and its backward (lora_compose_backward)
        # never forms lora or d_lora either, so nothing T x out is saved for lora
        y = lora_compose(base, h, self.lora_B, self.magnitude, self.weight_norm(), self.s, True)
        return y.reshape(*lead, self.out_features)
