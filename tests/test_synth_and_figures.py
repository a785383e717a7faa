"""Seeded input recipe and the memory figures the summary page prints."""
import json
import math
import os

import numpy as np
import pytest
import torch

from dora_fine_tuning_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_configs_shapes_and_scale():
    c = synth.CONFIGS["wide_8192_r384"]
    assert (c.out, c.in_, c.r, c.T) == (8192, 8192, 384, 8192)
    assert c.s == float(np.float32(32 / math.sqrt(384)))
    assert synth.CONFIGS["tiny"].s == 8.0
    assert synth.CONFIGS["mlp_up_27648x5120"].out == 27648
    assert {synth.CONFIGS[f"sweep_r{r}"].r for r in (16, 64, 128, 384, 512, 768)} == {16, 64, 128, 384, 512, 768}


def test_seeded_and_distributed():
    c = synth.custom("t", 256, 512, 32, 64)
    W0, A, B = synth.weights(c)
    W0b, _, _ = synth.weights(c)
    assert torch.equal(W0, W0b)  # seeded
    assert W0.dtype == torch.bfloat16 and W0.shape == (256, 512)
    assert abs(W0.float().std().item() - 0.02) < 0.002
    assert abs(A.float().std().item() - 1 / math.sqrt(512)) < 0.005
    assert abs(B.float().std().item() - 0.01) < 0.002
    x, dy = synth.activations(c, "fp16")
    assert x.dtype == torch.float16 and dy.shape == (64, 256)
    assert abs(dy.float().std().item() - 1.0) < 0.05


def test_bf16_rounding_is_rne():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 in bf16; RNE picks the even 1.0
    a = np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8)], np.float32)
    got = synth.to_dtype(a, "bf16").float().numpy()
    np.testing.assert_array_equal(got, [1.0, 1 + 2**-6, -1.0])


def test_magnitude_eps_recipes():
    c3 = synth.CONFIGS["wide_8192_r384"]
    e = synth.magnitude_eps(c3)
    assert np.all(np.abs(e) <= 2.0**-8) and (e < 0).any() and (e > 0).any()
    c5 = synth.CONFIGS["sweep_r64"]
    e5 = synth.magnitude_eps(c5)
    assert abs(e5.std() - 2.0**-10) < 2e-4
    n = np.full(8, 2.0)
    m = synth.magnitude(n, np.zeros(8))
    assert m.dtype == np.float32 and np.all(m == 2.0)


def test_base_and_lora_cpu_shapes():
    c = synth.custom("t", 48, 40, 8, 24)
    W0, A, B = synth.weights(c)
    x, _ = synth.activations(c)
    base, lora = synth.base_and_lora(x, W0, A, B)
    assert base.shape == (24, 48) and lora.shape == (24, 48) and base.dtype == torch.bfloat16


def _closed_form(f):
    if f["closed_form"].startswith("out*in / (out*r + r*r)"):
        return f["out"] * f["in"] / (f["out"] * f["r"] + f["r"] ** 2)
    if f["closed_form"].startswith("2 * out*in * 4"):
        return 2 * f["out"] * f["in"] * 4 / 2**20
    if f["closed_form"].startswith("out*in * 4"):
        return f["out"] * f["in"] * 4 / 2**20
    if f["closed_form"].startswith("out * 4"):
        return f["out"] * 4 / 2**10
    raise KeyError(f["closed_form"])


@pytest.mark.parametrize("idx", range(4))
def test_memory_figures_printed_on_the_page(idx):
    f = json.load(open(os.path.join(GOLDEN, "memory_figures.json")))["figures"][idx]
    v = _closed_form(f)
    assert abs(v - f["value"]) <= f["rel_tol"] * f["value"] + 1e-12, (f, v)
