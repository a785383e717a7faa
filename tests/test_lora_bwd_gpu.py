"""Parity of dora_lora_compose_bwd (the backward of the compose with lora =
h B^T fused in) with the CPU fp64 oracle, through the C ABI.

Tolerances, from the arithmetic:
* d_base (elementwise): 2 bf16 ulps (bf16) or 1e-3 relative (fp16).
* d_B = g s (dy^T h): the token sum runs as MFMA accumulation in fp32 over at
  most T/16 steps of 16 exact products plus the ordered sum of the slices, so
  it errs by at most (T/16 + 80) 2^-24 of g s sum_t |dy h|; the floor is three
  times that (the final rounding at most doubles it where the floor decides),
  beside the 2 ulps / 1e-3 of the value.
* d_mag: 1e-5 of sum_t |dy (base + s lora)| / n, or the chain bound
  (T/16 + 96) 2^-24 of the term mass (sum_t |dy base| + s sum_k |B| sum_t |dy h|) / n
  that the fused path's sums obey (the lora term is sum_k B (dy^T h)).
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


def case(T, out, r, dtype, seed):
    rng = np.random.default_rng(2000 + seed)
    to = lambda a: synth.to_dtype(a.astype(np.float32), dtype)
    dy = to(rng.standard_normal((T, out)))
    base = to(rng.standard_normal((T, out)) * 0.3)
    h = to(rng.standard_normal((T, r)))
    B = to(rng.standard_normal((out, r)) * 0.05)
    n = rng.uniform(0.5, 2.0, out).astype(np.float32)
    m = (n * (1 + rng.normal(0, 1e-3, out))).astype(np.float32)
    s = float(np.float32(32.0 / np.sqrt(max(r, 1))))
    return dy, base, h, B, m, n, s


def check(lib, dy, base, h, B, m, n, s, dtype, what, cols=None, rows=None):
    T, out = dy.shape
    r = h.shape[1]
    dyd, bd, hd, Bd = dy.to(DEV), base.to(DEV), h.to(DEV), B.to(DEV)
    md, nd = torch.from_numpy(m).to(DEV), torch.from_numpy(n).to(DEV)
    cols = np.arange(out) if cols is None else cols
    rows = np.arange(T) if rows is None else rows
    dyf, bf, hf, Bf = f64(dy), f64(base), f64(h), f64(B)
    g = m.astype(np.float64) / n.astype(np.float64)
    for add_base in (False, True):
        d_base, d_B, d_mag = lib.dora_lora_compose_bwd(dyd, bd, hd, Bd, md, nd, s, add_base=add_base)
        # oracle on the sampled columns (all tokens) and rows
        dyc, bc = dyf[:, cols], bf[:, cols]
        rb, rB, rm = O.lora_compose_bwd(dyc, bc, hf, Bf[cols], m[cols], n[cols], s, add_base=add_base)
        got_b = f64(d_base)[:, cols]
        PU.assert_compose(got_b[rows], rb[rows], np.abs(rb[rows]), dtype, f"{what} d_base add_base={add_base}")
        mass_B = np.abs(g[cols] * s)[:, None] * (np.abs(dyc).T @ np.abs(hf))
        PU.assert_compose(f64(d_B)[cols], rB, mass_B, dtype, f"{what} d_B", 3.0 * (T / 16 + 80) * 2.0**-24)
        cond = np.sum(np.abs(dyc * (bc + s * (hf @ Bf[cols].T))), axis=0) / n[cols]
        mass_m = (np.sum(np.abs(dyc * bc), axis=0) + s * np.sum(np.abs(Bf[cols]) * (np.abs(dyc).T @ np.abs(hf)), axis=1)) / n[cols]
        err = np.abs(f64(d_mag)[cols] - rm)
        ok = (err <= 1e-5 * cond + 1e-30) | (err <= (T / 16 + 96) * 2.0**-24 * mass_m)
        assert ok.all(), f"{what} d_mag: {(~ok).sum()} of {ok.size} columns out of tolerance"
        del d_base, d_B, d_mag


SMALL = [
    (300, 520, 24),    # ragged columns, rank and token slice
    (257, 1000, 136),  # two rank blocks of 128, ragged
    (513, 264, 384),   # the main workload's rank
    (1000, 256, 512),  # two rank blocks of 256
    (70, 4104, 64),    # many column blocks, few tokens
    (2048, 128, 16),   # long token axis: several token slices
    (1, 8, 8),
    (50, 517, 13),     # out and r not multiples of 8: general path
    (33, 16, 0),       # r = 0: general path, d_mag from base alone
]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_lora_bwd_small(lib, shape, dtype):
    T, out, r = shape
    dy, base, h, B, m, n, s = case(T, out, r, dtype, sum(shape))
    check(lib, dy, base, h, B, m, n, s, dtype, f"{shape} {dtype}")


def test_lora_bwd_no_d_base_empty_tokens_determinism(lib):
    T, out, r = 300, 264, 40
    dy, base, h, B, m, n, s = case(T, out, r, "bf16", 3)
    dyd, bd, hd, Bd = dy.to(DEV), base.to(DEV), h.to(DEV), B.to(DEV)
    md, nd = torch.from_numpy(m).to(DEV), torch.from_numpy(n).to(DEV)
    a = lib.dora_lora_compose_bwd(dyd, bd, hd, Bd, md, nd, s)
    b = lib.dora_lora_compose_bwd(dyd, bd, hd, Bd, md, nd, s, want_d_base=False)
    assert b[0] is None
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    c = lib.dora_lora_compose_bwd(dyd, bd, hd, Bd, md, nd, s)
    assert all(torch.equal(x, y) for x, y in zip(a, c))
    z = lib.dora_lora_compose_bwd(dyd[:0], bd[:0], hd[:0], Bd, md, nd, s)
    assert torch.count_nonzero(z[1]).item() == 0 and torch.count_nonzero(z[2]).item() == 0


def test_lora_bwd_matches_unfused_gradients(lib):
    """Against the unfused chain on the GPU: compose backward on a stored lora,
    then d_B = d_lora^T h.  The unfused chain rounds lora and d_lora to bf16
    (relative error at most 2^-9 per element, round to nearest), which moves
    its d_B and d_mag by at most 2^-9 of their absolute sums; the fused path
    keeps both in fp32.  So the two agree to 2^-8 in the Frobenius norm."""
    T, out, r = 512, 512, 64
    dy, base, h, B, m, n, s = case(T, out, r, "bf16", 11)
    dyd, bd, hd, Bd = dy.to(DEV), base.to(DEV), h.to(DEV), B.to(DEV)
    md, nd = torch.from_numpy(m).to(DEV), torch.from_numpy(n).to(DEV)
    lora = (hd.float() @ Bd.float().t()).to(torch.bfloat16)
    d_lora, d_base_u, d_mag_u = lib.dora_compose_bwd(dyd, bd, lora, md, nd, s)
    dB_u = d_lora.float().t() @ hd.float()
    d_base, d_B, d_mag = lib.dora_lora_compose_bwd(dyd, bd, hd, Bd, md, nd, s)
    assert torch.equal(d_base, d_base_u)
    rel = lambda a, b: float((a.float() - b.float()).norm() / b.float().norm())
    print(f"fused against unfused: d_B {rel(d_B, dB_u):.2e}, d_mag {rel(d_mag, d_mag_u):.2e}", flush=True)
    assert rel(d_B, dB_u) < 2.0**-8
    assert rel(d_mag, d_mag_u) < 2.0**-8


FULL = [("attn_proj", "bf16"), ("wide_8192_r384", "bf16"), ("wide_8192_r384", "fp16"),
        ("mlp_up_27648x5120", "bf16"), ("sweep_r16", "bf16"), ("sweep_r768", "fp16")]


@pytest.mark.parametrize("name,dtype", FULL, ids=lambda v: str(v))
def test_lora_bwd_full_config(lib, name, dtype):
    """A workload module at full size (the wide one, out = in = 8192, r = 384,
    T = 8192, is the benchmark's), in the benchmark's launch configuration: 64
    sampled output columns (all tokens) for d_B and d_mag, 64 sampled token
    rows of d_base."""
    cfg = synth.CONFIGS[name]
    log(f"[lora-bwd] {name} {dtype}: generating")
    W0, A, B = synth.weights(cfg, dtype)
    x, dy = synth.activations(cfg, dtype)
    base, h = synth.base_and_h(x, W0, A, device=DEV)
    del x, W0
    n = (np.linalg.norm(f64(B), axis=1) + 1.0).astype(np.float32)
    m = synth.magnitude(n, synth.magnitude_eps(cfg))
    rng = np.random.default_rng(cfg.index + 1)
    cols = np.unique(np.concatenate([[0, cfg.out - 1], rng.choice(cfg.out, 62, replace=False)]))
    rows = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, 62, replace=False)]))
    check(lib, dy, base.cpu(), h.cpu(), B, m, n, cfg.s, dtype, f"{name} {dtype}", cols=cols, rows=rows)
    log(f"[lora-bwd] {name} {dtype}: ok")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_lora_bwd_all_elements_wide(lib, dtype):
    """The wide module (out = in = 8192, r = 384, T = 8192) in the benchmark's
    launch configuration: every element of d_base, every element of d_B and
    every d_mag column against the oracle."""
    name = "wide_8192_r384"
    cfg = synth.CONFIGS[name]
    W0, A, B = synth.weights(cfg, dtype)
    x, dy = synth.activations(cfg, dtype)
    base, h = synth.base_and_h(x, W0, A, device=DEV)
    del x, W0
    n = (np.linalg.norm(f64(B), axis=1) + 1.0).astype(np.float32)
    m = synth.magnitude(n, synth.magnitude_eps(cfg))
    check(lib, dy, base.cpu(), h.cpu(), B, m, n, cfg.s, dtype, f"{name} {dtype} all elements")
    log(f"[lora-bwd] {name} {dtype}: every element of d_base and d_B and every d_mag column ok")
