"""Seeded synthetic inputs for the DoRA hot path.

This module is the only code shared by the oracle-side tests and the HIP path's
callers (tests, benchmark, smoke check).  It draws random tensors and builds the
adapter-module shapes; it holds none of the method's arithmetic (no norm, no
compose, no gradient).  The two things it does compute are input-recipe steps
that sit outside the method:

* ``base = x @ W0^T``, ``h = x @ A^T`` and ``lora = h @ B^T`` -- the caller's own
  GEMMs that feed the compose (the pages' compose takes these products as
  given);
* ``m = n * (1 + eps)`` -- the magnitude vector of a module whose scale factor
  g = m / n sits at a chosen distance from 1.  ``n`` is passed in by the caller.

Distributions follow the adapter shapes of the paper summary's workloads
(an 8192-dim module at rank 384, rsLoRA scaling, bf16 training; page
"Anthropic team cracks the fine-tuning memory bottleneck", paragraphs on memory
and on the convergence study): W0 ~ N(0, 0.02), A ~ N(0, 1/sqrt(in)),
B ~ N(0, 0.01), x ~ N(0, 1), dy ~ N(0, 1), where N(mu, sigma) names the standard
deviation.  Random draws use numpy's PCG64 seeded per (config, tensor), in
fp32, then rounded to the storage dtype with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}
DTYPE_CODES = {"bf16": 0, "fp16": 1}

# tensor ids mixed into the seed
_TID = {"W0": 1, "A": 2, "B": 3, "x": 4, "dy": 5, "eps": 6, "sign": 7}


@dataclasses.dataclass(frozen=True)
class ModuleConfig:
    """One adapter module: W0 [out x in], A [r x in], B [out x r], T tokens."""

    name: str
    out: int
    in_: int
    r: int
    T: int
    eps_kind: str  # "normal" | "signed_uniform"
    eps_scale: float
    index: int  # seed namespace
    alpha: float = 32.0

    @property
    def s(self) -> float:
        """rsLoRA scale alpha / sqrt(r), as the fp32 value passed to the kernels."""
        return float(np.float32(self.alpha / math.sqrt(self.r))) if self.r > 0 else 0.0

    def seed(self, tensor: str, salt: int = 0) -> int:
        return 1000 * self.index + _TID[tensor] + 100_000 * salt


def _cfg(name, out, in_, r, T, eps_kind, eps_scale, index):
    return ModuleConfig(name, out, in_, r, T, eps_kind, eps_scale, index)


# The workloads: a tiny module, an attention projection, the 8192-wide module of
# the memory case (g inside the bf16 collapse region), an MLP up-projection of a
# ~32B model, and a rank sweep on the 8192-wide module.
CONFIGS = {
    "tiny": _cfg("tiny", 512, 512, 16, 256, "normal", 1e-3, 1),
    "attn_proj": _cfg("attn_proj", 4096, 4096, 64, 4096, "normal", 1e-3, 2),
    "wide_8192_r384": _cfg("wide_8192_r384", 8192, 8192, 384, 8192, "signed_uniform", 2.0**-8, 3),
    "mlp_up_27648x5120": _cfg("mlp_up_27648x5120", 27648, 5120, 512, 10240, "normal", 1e-3, 4),
}
for _r in (16, 64, 128, 384, 512, 768):
    CONFIGS[f"sweep_r{_r}"] = _cfg(f"sweep_r{_r}", 8192, 8192, _r, 8192, "normal", 2.0**-10, 50 + _r)


def custom(name, out, in_, r, T, eps_kind="normal", eps_scale=1e-3, index=900):
    """A config of arbitrary shape (tests of ragged tiles and edge cases)."""
    return ModuleConfig(name, out, in_, r, T, eps_kind, eps_scale, index)


def _normal(seed: int, shape, sigma: float) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return a


def to_dtype(a: np.ndarray, dtype: str) -> torch.Tensor:
    """fp32 numpy -> torch CPU tensor in the storage dtype (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DTYPES[dtype])


def weights(cfg: ModuleConfig, dtype: str = "bf16", salt: int = 0):
    """W0 [out x in], A [r x in], B [out x r] as CPU tensors in ``dtype``."""
    W0 = to_dtype(_normal(cfg.seed("W0", salt), (cfg.out, cfg.in_), 0.02), dtype)
    A = to_dtype(_normal(cfg.seed("A", salt), (cfg.r, cfg.in_), 1.0 / math.sqrt(max(cfg.in_, 1))), dtype)
    B = to_dtype(_normal(cfg.seed("B", salt), (cfg.out, cfg.r), 0.01), dtype)
    return W0, A, B


def activations(cfg: ModuleConfig, dtype: str = "bf16", salt: int = 0):
    """x [T x in] and the upstream gradient dy [T x out] as CPU tensors."""
    x = to_dtype(_normal(cfg.seed("x", salt), (cfg.T, cfg.in_), 1.0), dtype)
    dy = to_dtype(_normal(cfg.seed("dy", salt), (cfg.T, cfg.out), 1.0), dtype)
    return x, dy


def magnitude_eps(cfg: ModuleConfig, salt: int = 0) -> np.ndarray:
    """Relative offset eps of m from n, per output feature (fp64).

    ``normal``: eps ~ N(0, eps_scale).  ``signed_uniform``: |eps| ~ U(0, eps_scale)
    with a random sign, so g - 1 spans the bf16 collapse band.
    """
    rng = np.random.Generator(np.random.PCG64(cfg.seed("eps", salt)))
    if cfg.eps_kind == "normal":
        return rng.standard_normal(cfg.out) * cfg.eps_scale
    if cfg.eps_kind == "signed_uniform":
        mag = rng.uniform(0.0, cfg.eps_scale, cfg.out)
        sign = np.where(rng.random(cfg.out) < 0.5, -1.0, 1.0)
        return mag * sign
    raise ValueError(cfg.eps_kind)


def magnitude(n, eps: np.ndarray) -> np.ndarray:
    """m = n * (1 + eps) rounded to fp32; ``n`` is any per-row norm the caller holds."""
    n = np.asarray(n, dtype=np.float64)
    return (n * (1.0 + eps)).astype(np.float32)


def base_and_h(x, W0, A, device="cpu"):
    """base = x W0^T and the adapter's first projection h = x A^T, in x's dtype
    (the inputs of the compose with the second projection fused in); the same
    GEMMs as base_and_lora."""
    dt = x.dtype
    if str(device) == "cpu":
        xf = x.float()
        return (xf @ W0.float().t()).to(dt), (xf @ A.float().t()).to(dt)
    xd, Wd, Ad = (t.to(device) for t in (x, W0, A))
    return torch.nn.functional.linear(xd, Wd), torch.nn.functional.linear(xd, Ad)


def base_and_lora(x, W0, A, B, device="cpu"):
    """The caller's two GEMMs: base = x W0^T, lora = (x A^T) B^T, in x's dtype.

    On CPU the products run in fp32 and are rounded once; on a GPU they are
    torch's own bf16/fp16 GEMMs.  The x A^T intermediate is rounded to the dtype,
    as a LoRA branch stores it.
    """
    dt = x.dtype
    if str(device) == "cpu":
        xf = x.float()
        base = (xf @ W0.float().t()).to(dt)
        xa = (xf @ A.float().t()).to(dt)
        lora = (xa.float() @ B.float().t()).to(dt)
        return base, lora
    xd, Wd, Ad, Bd = (t.to(device) for t in (x, W0, A, B))
    base = torch.nn.functional.linear(xd, Wd)
    xa = torch.nn.functional.linear(xd, Ad)
    lora = torch.nn.functional.linear(xa, Bd)
    return base, lora
