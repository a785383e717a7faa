"""Parity of dora_lora_compose_fwd (the compose with lora = h B^T formed
inside, h = x A^T) with the CPU fp64 oracle, through the C ABI.

Tolerance: 2 bf16 ulps (bf16) or 1e-3 relative (fp16) of the oracle value, or
the floor 3 (r + 4) 2^-24 of the term mass where the terms cancel (derivation
in parity_util).
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


def floor_rel(r):
    return 3.0 * (r + 4) * 2.0**-24


def mass(base, h, B, m, n, s, add_base):
    g = np.asarray(m, np.float64) / np.asarray(n, np.float64)
    lm = np.abs(h) @ np.abs(B).T
    return np.abs((g - 1) * base) + np.abs(g * s) * lm + (np.abs(base) if add_base else 0)


def case(T, out, r, dtype, seed):
    cfg = synth.custom("lora_compose", out, 64, r, T, index=700 + seed)
    rng = np.random.default_rng(1000 + seed)
    to = lambda a: synth.to_dtype(a.astype(np.float32), dtype)
    base = to(rng.standard_normal((T, out)) * 0.3)
    h = to(rng.standard_normal((T, r)))
    B = to(rng.standard_normal((out, r)) * 0.05)
    n = (rng.uniform(0.5, 2.0, out)).astype(np.float32)
    m = (n * (1 + rng.normal(0, 1e-3, out))).astype(np.float32)
    return base, h, B, m, n, cfg.s


def check(lib, base, h, B, m, n, s, dtype, what, add_base_modes=(False, True), dev_inputs=None):
    bd, hd, Bd = dev_inputs if dev_inputs else (base.to(DEV), h.to(DEV), B.to(DEV))
    md, nd = torch.from_numpy(m).to(DEV), torch.from_numpy(n).to(DEV)
    bf, hf, Bf = f64(base), f64(h), f64(B)
    for add_base in add_base_modes:
        y = lib.dora_lora_compose_fwd(bd, hd, Bd, md, nd, s, add_base=add_base)
        ref = O.lora_compose_fwd(bf, hf, Bf, m, n, s, add_base=add_base)
        PU.assert_compose(f64(y), ref, mass(bf, hf, Bf, m, n, s, add_base), dtype, f"{what} add_base={add_base}",
                          floor_rel(hf.shape[1]))


SMALL = [
    (300, 520, 24),    # ragged token and column tiles, one K stage with a tail
    (257, 1000, 136),  # several K stages, ragged tail
    (513, 264, 384),   # the main workload's rank, ragged
    (70, 4104, 64),    # many column tiles
    (256, 256, 16),    # one exact tile
    (1, 8, 8),
    (33, 8, 0),        # r = 0: the compose of lora = 0
    (50, 517, 13),     # out and r not multiples of 8: general path
    (40, 96, 1000),    # K longer than the ring
]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_lora_compose_small(lib, shape, dtype):
    T, out, r = shape
    base, h, B, m, n, s = case(T, out, r, dtype, sum(shape))
    check(lib, base, h, B, m, n, s, dtype, f"{shape} {dtype}")


def test_lora_compose_unaligned_and_in_place(lib):
    """A base 2 bytes off a 16-byte boundary takes the general path; y may be base."""
    T, out, r = 64, 136, 40
    base, h, B, m, n, s = case(T, out, r, "bf16", 5)
    flat = torch.empty(T * out + 8, dtype=torch.bfloat16, device=DEV)
    bu = flat[1:1 + T * out].view(T, out)
    bu.copy_(base.to(DEV))
    assert bu.data_ptr() % 16 != 0
    check(lib, base, h, B, m, n, s, "bf16", "unaligned", dev_inputs=(bu, h.to(DEV), B.to(DEV)))
    md, nd = torch.from_numpy(m).to(DEV), torch.from_numpy(n).to(DEV)
    want = lib.dora_lora_compose_fwd(base.to(DEV), h.to(DEV), B.to(DEV), md, nd, s, add_base=True)
    inplace = base.to(DEV)
    got = lib.dora_lora_compose_fwd(inplace, h.to(DEV), B.to(DEV), md, nd, s, add_base=True, y=inplace)
    assert got.data_ptr() == inplace.data_ptr()
    assert torch.equal(got, want)


def test_lora_compose_determinism_and_identity(lib):
    """Bitwise repeatable; with B = 0 and m = n the delta is exactly zero and
    add_base returns base bit for bit."""
    T, out, r = 300, 520, 48
    base, h, B, m, n, s = case(T, out, r, "bf16", 9)
    bd, hd, Bd = base.to(DEV), h.to(DEV), B.to(DEV)
    md, nd = torch.from_numpy(m).to(DEV), torch.from_numpy(n).to(DEV)
    a = lib.dora_lora_compose_fwd(bd, hd, Bd, md, nd, s)
    b = lib.dora_lora_compose_fwd(bd, hd, Bd, md, nd, s)
    assert torch.equal(a, b)
    zB = torch.zeros_like(Bd)
    y = lib.dora_lora_compose_fwd(bd, hd, zB, nd, nd, s, add_base=True)
    assert torch.equal(y, bd)
    y = lib.dora_lora_compose_fwd(bd, hd, zB, nd, nd, s)
    assert torch.count_nonzero(y).item() == 0


FULL = [("attn_proj", "bf16"), ("wide_8192_r384", "bf16"), ("wide_8192_r384", "fp16"),
        ("mlp_up_27648x5120", "bf16"), ("sweep_r16", "bf16"), ("sweep_r768", "fp16")]


@pytest.mark.parametrize("name,dtype", FULL, ids=lambda v: str(v))
def test_lora_compose_full_config(lib, name, dtype):
    """A workload module at full size (the wide one, out = in = 8192, r = 384,
    T = 8192, is the benchmark's), in the benchmark's launch configuration: 96
    sampled token rows, every column, against the oracle; and the near-unity
    check (h = 0: the correction alone, nonzero wherever the oracle's is and
    the dtype can hold it)."""
    cfg = synth.CONFIGS[name]
    log(f"[lora-fused] {name} {dtype}: generating")
    W0, A, B = synth.weights(cfg, dtype)
    x, _ = synth.activations(cfg, dtype)
    base, h = synth.base_and_h(x, W0, A, device=DEV)
    del x, W0
    n = np.linalg.norm(f64(B), axis=1) + 1.0
    n32 = n.astype(np.float32)
    m = synth.magnitude(n, synth.magnitude_eps(cfg))
    md, nd, Bd = torch.from_numpy(m).to(DEV), torch.from_numpy(n32).to(DEV), B.to(DEV)
    rng = np.random.default_rng(cfg.index)
    rows = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, 94, replace=False)]))
    ri = torch.from_numpy(rows).to(DEV)
    br, hr, Bf = f64(base[ri]), f64(h[ri]), f64(B)
    for add_base in (False, True):
        y = lib.dora_lora_compose_fwd(base, h, Bd, md, nd, cfg.s, add_base=add_base)
        ref = O.lora_compose_fwd(br, hr, Bf, m, n32, cfg.s, add_base=add_base)
        fo = PU.assert_compose(f64(y[ri]), ref, mass(br, hr, Bf, m, n32, cfg.s, add_base), dtype,
                               f"{name} fused add_base={add_base}", floor_rel(cfg.r))
        log(f"[lora-fused] {name} {dtype} add_base={add_base}: ok ({fo} floor-only elements)")
        del y
    z = torch.zeros_like(h)
    y = f64(lib.dora_lora_compose_fwd(base, z, Bd, md, nd, cfg.s)[ri])
    ref = O.lora_compose_fwd(br, np.zeros_like(hr), Bf, m, n32, cfg.s)
    g = m.astype(np.float64) / n32.astype(np.float64)
    near = np.abs(g - 1) < 2.0**-8
    assert near.any()
    want = PU.representable_nonzero(ref, dtype)[:, near]
    assert np.all((y != 0)[:, near] == want)
    log(f"[lora-fused] {name} {dtype}: near-unity correction nonzero in all {int(want.sum())} representable elements")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_lora_compose_all_elements_wide(lib, dtype):
    """The wide module (out = in = 8192, r = 384, T = 8192) in the benchmark's
    launch configuration: every element of y, delta and full output, against
    the oracle, which walks token chunks of 512 rows."""
    name = "wide_8192_r384"
    cfg = synth.CONFIGS[name]
    W0, A, B = synth.weights(cfg, dtype)
    x, _ = synth.activations(cfg, dtype)
    base, h = synth.base_and_h(x, W0, A, device=DEV)
    del x, W0
    n = np.linalg.norm(f64(B), axis=1) + 1.0
    n32 = n.astype(np.float32)
    m = synth.magnitude(n, synth.magnitude_eps(cfg))
    md, nd, Bd = torch.from_numpy(m).to(DEV), torch.from_numpy(n32).to(DEV), B.to(DEV)
    Bf = f64(B)
    for add_base in (False, True):
        y = lib.dora_lora_compose_fwd(base, h, Bd, md, nd, cfg.s, add_base=add_base)
        fo = 0
        for t0 in range(0, cfg.T, 512):
            t1 = min(t0 + 512, cfg.T)
            bc, hc = f64(base[t0:t1]), f64(h[t0:t1])
            ref = O.lora_compose_fwd(bc, hc, Bf, m, n32, cfg.s, add_base=add_base)
            fo += PU.assert_compose(f64(y[t0:t1]), ref, mass(bc, hc, Bf, m, n32, cfg.s, add_base), dtype,
                                    f"{name} fused rows {t0}:{t1} add_base={add_base}", floor_rel(cfg.r))
        log(f"[lora-fused] {name} {dtype} add_base={add_base}: all {cfg.T * cfg.out} elements ok "
            f"({fo} floor-only elements)")
        del y
