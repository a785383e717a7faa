"""Parity of the cached-base norm entry points with the CPU fp64 oracle.

dora_row_sqnorm gives ||W0_i||^2 once (W0 is frozen); dora_norm_factored_cached
takes it as the norm's base term.  Tolerances:

* row square norm (fp32 output): each fp32 partial sum holds at most
  ceil(in/256) + 1 squares (every square is exact in fp32), the partials are
  combined in fp64 and rounded once, so the relative error is at most
  (ceil(in/256) + 2) * 2^-24; the test allows one more 2^-24.
* cached norm: the norm's own tolerance (relative 1e-5, or 2^-16 of the term
  mass where the terms cancel), with the cache as the base term.
"""
import math
import sys

import numpy as np
import pytest
import torch

import parity_util as PU
from dora_fine_tuning_amd import synth
from oracle import dora_oracle as O

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def lib():
    assert torch.cuda.is_available(), "GPU parity tests need a HIP device"
    from dora_fine_tuning_amd import binding

    return binding


def f64(t):
    return t.detach().cpu().double().numpy()


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def sqnorm_rtol(in_):
    return (math.ceil(in_ / 256) + 3) * 2.0**-24


def cached_mass(c, W0, A, B, s):
    """c + |cross| + Gram per row (scale of the cancellation floor)."""
    cross = 2.0 * s * np.sum(B * (W0 @ A.T), axis=1)
    gram = s * s * np.sum((B @ (A @ A.T)) * B, axis=1)
    return np.abs(c) + np.abs(cross) + np.abs(gram)


def unaligned_copy(t):
    """The same values at an address 2 bytes past a 16-byte boundary (general path)."""
    flat = torch.empty(t.numel() + 8, dtype=t.dtype, device=DEV)
    v = flat[1:1 + t.numel()].view(t.shape)
    v.copy_(t.to(DEV))
    assert v.data_ptr() % 16 != 0
    return v


SQ_SHAPES = [(300, 520), (257, 1000), (130, 75), (5, 0), (1, 8), (64, 2056), (33, 8200), (1000, 16)]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("shape", SQ_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_row_sqnorm(lib, shape, dtype):
    out, in_ = shape
    cfg = synth.custom("sqnorm", out, in_, 8, 1)
    W0, _, _ = synth.weights(cfg, dtype)
    ref = O.row_sqnorm(W0)
    variants = [("aligned", W0.to(DEV))] + ([("unaligned", unaligned_copy(W0))] if W0.numel() else [])
    for tag, dev_w in variants:
        got = f64(lib.dora_row_sqnorm(dev_w))
        np.testing.assert_allclose(got, ref, rtol=sqnorm_rtol(in_), atol=0, err_msg=f"{shape} {dtype} {tag}")


def test_row_sqnorm_zero_rows_and_determinism(lib):
    cfg = synth.custom("sqnorm0", 200, 1024, 8, 1)
    W0, _, _ = synth.weights(cfg)
    W0[7] = 0
    W0[150] = 0
    d = W0.to(DEV)
    a, b = lib.dora_row_sqnorm(d), lib.dora_row_sqnorm(d)
    assert torch.equal(a, b)
    assert a[7].item() == 0.0 and a[150].item() == 0.0


CACHED_SHAPES = [(300, 520, 24), (257, 1000, 136), (130, 75, 13), (64, 64, 0), (5, 0, 8), (200, 264, 296),
                 (150, 128, 504), (90, 100, 300)]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("shape", CACHED_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_norm_cached_small(lib, shape, dtype):
    out, in_, r = shape
    cfg = synth.custom("norm_cached", out, in_, r, 1)
    W0, A, B = synth.weights(cfg, dtype)
    s = cfg.s
    W0d, Ad, Bd = W0.to(DEV), A.to(DEV), B.to(DEV)
    c = lib.dora_row_sqnorm(W0d)
    W, Af, Bf = f64(W0), f64(A), f64(B)
    # the true base term, then an arbitrary cache (the norm must take it as given)
    for tag, cache in (("row_sqnorm", c), ("1.5x cache", c * 1.5)):
        n_gpu = f64(lib.dora_norm_factored_cached(W0d, Ad, Bd, cache, s))
        cf = f64(cache)
        ref = O.weight_norm_cached(cf, W0, A, B, s)
        PU.assert_norm(n_gpu, ref, cached_mass(cf, W, Af, Bf, s), f"cached norm {shape} {dtype} {tag}")
    # with the true cache the result is the plain norm, within the norm's tolerance
    n_plain = O.weight_norm(W0, A, B, s)
    n_gpu = f64(lib.dora_norm_factored_cached(W0d, Ad, Bd, c, s))
    PU.assert_norm(n_gpu, n_plain, PU.norm_term_mass(W, Af, Bf, s), f"cached vs plain {shape} {dtype}")


def test_norm_cached_clamps_negative(lib):
    """A zero cache with rows where the adapter cancels most of W0
    (W0 = -0.8 s B A, so ||W0 + s B A||^2 - ||W0||^2 = -0.6 ||s B A||^2 < 0):
    n = 0 there, and positive on the other rows."""
    cfg = synth.custom("norm_cached_neg", 64, 256, 16, 1)
    W0, A, B = synth.weights(cfg)
    B = (B.float() * 40).to(B.dtype)
    W0 = W0.float()
    W0[::2] = -0.8 * cfg.s * (B.float()[::2] @ A.float())
    W0 = W0.to(torch.bfloat16)
    W0d, Ad, Bd = W0.to(DEV), A.to(DEV), B.to(DEV)
    zero = torch.zeros(64, dtype=torch.float32, device=DEV)
    n_gpu = f64(lib.dora_norm_factored_cached(W0d, Ad, Bd, zero, cfg.s))
    ref = O.weight_norm_cached(np.zeros(64), W0, A, B, cfg.s)
    assert np.all(ref[::2] == 0) and np.all(ref[1::2] > 0)
    PU.assert_norm(n_gpu, ref, cached_mass(np.zeros(64), f64(W0), f64(A), f64(B), cfg.s), "clamp")
    assert np.all(n_gpu[::2] == 0.0)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_norm_cached_wide_config(lib, dtype):
    """The module out = in = 8192, r = 384 in the benchmark's launch
    configuration: every row of the cached norm against the oracle, with the
    cache from dora_row_sqnorm checked on every row too."""
    cfg = synth.CONFIGS["wide_8192_r384"]
    log(f"[cached] wide {dtype}: generating")
    W0, A, B = synth.weights(cfg, dtype)
    W0d, Ad, Bd = W0.to(DEV), A.to(DEV), B.to(DEV)
    c = lib.dora_row_sqnorm(W0d)
    c_ref = O.row_sqnorm(W0)
    np.testing.assert_allclose(f64(c), c_ref, rtol=sqnorm_rtol(cfg.in_), atol=0)
    n_gpu = f64(lib.dora_norm_factored_cached(W0d, Ad, Bd, c, cfg.s))
    ref = O.weight_norm_cached(f64(c), W0, A, B, cfg.s)
    W, Af, Bf = f64(W0), f64(A), f64(B)
    PU.assert_norm(n_gpu, ref, cached_mass(f64(c), W, Af, Bf, cfg.s), f"wide cached {dtype}")
    n_plain = f64(lib.dora_norm_factored(W0d, Ad, Bd, cfg.s))
    log(f"[cached] wide {dtype}: ok; max |cached - plain| / plain = {np.max(np.abs(n_gpu - n_plain) / n_plain):.2e}")
