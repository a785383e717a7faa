"""Parity of the small-adapter norm paths with the CPU fp64 oracle.

For r <= 32 and at least 128 strips of 32 rows (out >= 4065) the 16-byte path
takes one launch in which every workgroup streams a 32-row strip of W0 over
the whole input axis and forms the Gram matrix A A^T itself.  The shapes here
are above that row threshold and ragged in every direction that kernel tiles:
the last strip (out % 32), the last K stage (in % 64, down to a single
partial stage) and the rank tile (r % 32).  The shapes with 32 < r <= 64 take
the split-K W stream instead, whose rank panel leaves out the DMA of panel
rows past r; they check that path at a partly filled rank tile.  Tolerance:
the norm's own (relative 1e-5, or 2^-16 of the term mass where terms cancel).
"""
import sys

import numpy as np
import pytest
import torch

import parity_util as PU
from dora_fine_tuning_amd import synth
from oracle import dora_oracle as O

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

STRIP_SHAPES = [
    (4113, 200, 8),    # ragged last strip and K stage, narrowest rank
    (4096, 72, 24),    # two K stages, the second 8 wide
    (4133, 136, 40),   # second rank tile partly filled
    (4096, 8, 64),     # one partial K stage, full second rank tile
    (4160, 1000, 56),
    (4097, 520, 32),   # one full rank tile, a single row in the last strip
    (4096, 4096, 16),  # the attention projection's shape at a small rank
]


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


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("shape", STRIP_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_norm_strip(lib, shape, dtype):
    out, in_, r = shape
    log(f"[strip] {shape} {dtype}")
    cfg = synth.custom("norm_strip", out, in_, r, 1)
    W0, A, B = synth.weights(cfg, dtype)
    s = cfg.s
    W0d, Ad, Bd = W0.to(DEV), A.to(DEV), B.to(DEV)
    n_gpu = f64(lib.dora_norm_factored(W0d, Ad, Bd, s))
    ref = O.weight_norm(W0, A, B, s)
    W, Af, Bf = f64(W0), f64(A), f64(B)
    PU.assert_norm(n_gpu, ref, PU.norm_term_mass(W, Af, Bf, s), f"strip norm {shape} {dtype}")
    # the cached-base variant: an arbitrary cache is taken as the base term
    cache = torch.from_numpy((np.sum(W * W, axis=1) * 1.25).astype(np.float32)).to(DEV)
    cf = f64(cache)
    n_c = f64(lib.dora_norm_factored_cached(W0d, Ad, Bd, cache, s))
    ref_c = O.weight_norm_cached(cf, W0, A, B, s)
    cross = 2.0 * s * np.sum(Bf * (W @ Af.T), axis=1)
    gram = s * s * np.sum((Bf @ (Af @ Af.T)) * Bf, axis=1)
    PU.assert_norm(n_c, ref_c, np.abs(cf) + np.abs(cross) + np.abs(gram), f"strip cached {shape} {dtype}")
    # deterministic: a second call gives the same bits
    assert np.array_equal(f64(lib.dora_norm_factored(W0d, Ad, Bd, s)), n_gpu)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_norm_strip_large_adapter(lib, dtype):
    """B 30x larger than at initialisation: the Gram term carries most of n^2,
    so an error in the in-kernel Gram tile (a transposed or misplaced block)
    shows."""
    cfg = synth.custom("norm_strip_big_B", 4128, 392, 32, 1)
    W0, A, B = synth.weights(cfg, dtype)
    B = (B.float() * 30).to(B.dtype)
    n_gpu = f64(lib.dora_norm_factored(W0.to(DEV), A.to(DEV), B.to(DEV), cfg.s))
    ref = O.weight_norm(W0, A, B, cfg.s)
    W, Af, Bf = f64(W0), f64(A), f64(B)
    gram = cfg.s**2 * np.sum((Bf @ (Af @ Af.T)) * Bf, axis=1)
    assert np.median(gram / ref**2) > 0.5
    PU.assert_norm(n_gpu, ref, PU.norm_term_mass(W, Af, Bf, cfg.s), f"strip big B {dtype}")


@pytest.mark.parametrize("r", [24, 40])
def test_norm_strip_exact_cancellation(lib, r):
    """W0 = -s B A with dyadic entries (every product and sum exact): n = 0 on
    those rows and the known residual on every third row."""
    rng = np.random.default_rng(17 + r)
    out, in_, s = 4101, 136, 2.0
    A = rng.choice([-1.0, -0.5, 0.0, 0.5, 1.0], size=(r, in_))
    B = rng.choice([-0.25, 0.0, 0.25, 0.5], size=(out, r))
    W0 = -s * (B @ A)
    W0[::3] += 0.125
    t = lambda a: torch.tensor(a, dtype=torch.bfloat16)
    assert np.array_equal(t(W0).double().numpy(), W0)
    n_gpu = f64(lib.dora_norm_factored(t(W0).to(DEV), t(A).to(DEV), t(B).to(DEV), s))
    ref = O.weight_norm(W0, A, B, s)
    np.testing.assert_array_equal(ref[1::3], 0.0)
    PU.assert_norm(n_gpu, ref, PU.norm_term_mass(W0, A, B, s), f"strip cancellation r {r}")
    np.testing.assert_allclose(n_gpu[::3], np.sqrt(in_ * 2.0**-6), rtol=1e-6)


@pytest.mark.parametrize("r", [16, 64])
def test_norm_strip_b_zero_is_plain_row_norm(lib, r):
    cfg = synth.custom("strip_bzero", 4096, 1024, r, 1)
    W0, A, B = synth.weights(cfg)
    n_gpu = f64(lib.dora_norm_factored(W0.to(DEV), A.to(DEV), torch.zeros_like(B).to(DEV), cfg.s))
    np.testing.assert_allclose(n_gpu, np.linalg.norm(f64(W0), axis=1), rtol=1e-6)
