"""PyTorch integration: custom operators, autograd through the fused compose,
and the DoRA linear layer.  Gradients are checked against the fp64 oracle
(compose) and against a float64 CPU evaluation of the dense DoRA formula with
the norm detached (layer)."""
import numpy as np
import pytest
import torch

from dora_fine_tuning_amd import synth
from oracle import dora_oracle as O
from parity_util import assert_compose, assert_dmag

torch_ops = pytest.importorskip("dora_fine_tuning_amd.torch_ops")

gpu = pytest.mark.gpu


def test_layer_rejects_other_dtypes():
    with pytest.raises(ValueError):
        torch_ops.DoRALinear(8, 8, 2, dtype=torch.float64)


# ------------------------------------------------------------------ eager tier (CPU)


def test_eager_tier_ops_match_oracle():
    """CPU tensors take the eager tier (plain torch, fp32): every operator
    against the fp64 oracle.  fp32 arithmetic over bf16 inputs bounds the
    error well below these tolerances."""
    rng = np.random.default_rng(21)
    T, out, in_, r, s = 40, 48, 64, 8, 2.5
    bf = lambda a: torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16)
    W0, A, B = bf(rng.normal(0, 0.02, (out, in_))), bf(rng.normal(0, 0.125, (r, in_))), bf(rng.normal(0, 0.05, (out, r)))
    n_ref = O.weight_norm(W0, A, B, s)
    np.testing.assert_allclose(torch_ops.weight_norm(W0, A, B, s).double().numpy(), n_ref, rtol=1e-5)
    sq = torch_ops.row_sqnorm(W0)
    np.testing.assert_allclose(sq.double().numpy(), O.row_sqnorm(W0), rtol=1e-5)
    np.testing.assert_allclose(torch_ops.weight_norm_cached(W0, A, B, sq, s).double().numpy(),
                               O.weight_norm_cached(sq, W0, A, B, s), rtol=1e-5)
    n32 = torch.from_numpy(n_ref.astype(np.float32))
    dn = torch.from_numpy(rng.normal(0, 1, out).astype(np.float32))
    dA, dB = torch_ops.weight_norm_backward(W0, A, B, n32, dn, s)
    rA, rB = O.weight_norm_bwd(dn, n32, W0, A, B, s)
    np.testing.assert_allclose(dA.double().numpy(), rA, rtol=2e-2, atol=2e-2 * np.abs(rA).max())
    np.testing.assert_allclose(dB.double().numpy(), rB, rtol=2e-2, atol=2e-2 * np.abs(rB).max())

    base, lora, dy = bf(rng.normal(0, 1, (T, out))), bf(rng.normal(0, 0.3, (T, out))), bf(rng.normal(0, 1, (T, out)))
    m = torch.from_numpy(synth.magnitude(n_ref, rng.uniform(-2**-8, 2**-8, out)))
    for add_base in (False, True):
        bg, lg, mg = (t.clone().requires_grad_() for t in (base, lora, m))
        y = torch_ops.compose(bg, lg, mg, n32, s, add_base)
        y.backward(dy)
        y_ref = O.compose_fwd(base, lora, m, n32, s, add_base)
        dl_ref, db_ref, dm_ref = O.compose_bwd(dy, base, lora, m, n32, s, add_base)
        g = m.double().numpy() / n32.double().numpy()
        b64, l64 = O.as_f64(base), O.as_f64(lora)
        mass = np.abs((g - 1) * b64) + np.abs(g * s * l64) + (np.abs(b64) if add_base else 0)
        assert_compose(y.detach().float().numpy(), y_ref, mass, "bf16", "eager y")
        assert_compose(lg.grad.float().numpy(), dl_ref, np.abs(dl_ref), "bf16", "eager d_lora")
        assert_compose(bg.grad.float().numpy(), db_ref, np.abs(db_ref), "bf16", "eager d_base")
        cond = np.sum(np.abs(O.as_f64(dy) * (b64 + s * l64)), axis=0) / n32.double().numpy()
        assert_dmag(mg.grad.numpy(), dm_ref, cond, "eager d_mag")
    h = bf(rng.normal(0, 1, (T, r)))
    y = torch_ops.lora_compose(base, h, B, m, n32, s, True)
    y_ref = O.lora_compose_fwd(base, h, B, m, n32, s, True)
    np.testing.assert_allclose(y.double().numpy(), y_ref, rtol=2e-2, atol=1e-2)
    d_base, d_B, d_mag = torch_ops.lora_compose_backward(dy, base, h, B, m, n32, s, False, True)
    rb, rB2, rm = O.lora_compose_bwd(dy, base, h, B, m, n32, s, False)
    np.testing.assert_allclose(d_base.double().numpy(), rb, rtol=2e-2, atol=1e-6)
    np.testing.assert_allclose(d_B.double().numpy(), rB2, rtol=2e-2, atol=2e-2 * np.abs(rB2).max())
    np.testing.assert_allclose(d_mag.double().numpy(), rm, rtol=1e-4, atol=1e-4 * np.abs(rm).max())


def test_eager_tier_layer_matches_dense_reference():
    """DoRALinear on the CPU (eager tier), forward and backward, against the
    float64 dense evaluation with the norm detached and not detached."""
    torch.manual_seed(4)
    for detach in (True, False):
        layer = torch_ops.DoRALinear(96, 80, 8, dtype=torch.float32, detach_norm=detach)
        with torch.no_grad():
            layer.lora_B.normal_(0.0, 0.05)
            layer.magnitude.mul_(1.0 + 0.01 * torch.randn_like(layer.magnitude))
        x = torch.randn(30, 96).requires_grad_()
        y = layer(x)
        dy = (y.detach() + 0.1 * torch.randn_like(y))
        y.backward(dy)
        ref = _dense_reference if detach else _dense_reference_full
        out = ref(x, layer.weight, layer.lora_A, layer.lora_B, layer.magnitude, layer.s, dy)
        y_ref, dx_ref, dA_ref, dB_ref, dm_ref = out[:5]
        assert _rel(y, y_ref) < 1e-5 and _rel(x.grad, dx_ref) < 1e-5
        assert _rel(layer.lora_A.grad, dA_ref) < 1e-4 and _rel(layer.lora_B.grad, dB_ref) < 1e-4
        assert _rel(layer.magnitude.grad, dm_ref) < 1e-5


def _compile_check(layer, x):
    """The layer under torch.compile (fullgraph, aot_eager backend: torch's
    own autograd-traced graph, no code generation) gives no graph break and
    the eager layer's outputs and gradients."""
    import torch._dynamo

    torch._dynamo.reset()
    y_eager = layer(x)  # fills the base-term cache outside the compiled region
    explain = torch._dynamo.explain(layer)(x)
    assert explain.graph_break_count == 0, explain.break_reasons
    compiled = torch.compile(layer, fullgraph=True, backend="aot_eager")
    xg = x.detach().clone().requires_grad_()
    y = compiled(xg)
    dy = torch.randn_like(y)
    y.backward(dy)
    grads = [p.grad.clone() for p in (layer.lora_A, layer.lora_B, layer.magnitude)]
    for p in (layer.lora_A, layer.lora_B, layer.magnitude):
        p.grad = None
    xe = x.detach().clone().requires_grad_()
    y_eager = layer(xe)
    y_eager.backward(dy)
    assert torch.equal(y.detach(), y_eager.detach())
    assert torch.equal(xg.grad, xe.grad)
    for g, p in zip(grads, (layer.lora_A, layer.lora_B, layer.magnitude)):
        assert torch.equal(g, p.grad)


def test_compile_without_graph_breaks_cpu():
    torch.manual_seed(5)
    for detach in (True, False):
        layer = torch_ops.DoRALinear(64, 48, 8, dtype=torch.float32, detach_norm=detach)
        with torch.no_grad():
            layer.lora_B.normal_(0.0, 0.05)
        _compile_check(layer, torch.randn(2, 10, 64))


def _compose_inputs(T, out, dtype, seed):
    cfg = synth.custom("torch_ops", out, 64, 8, T, index=seed)
    g = np.random.default_rng(seed)
    base = torch.from_numpy(g.standard_normal((T, out)).astype(np.float32)).to(dtype)
    lora = torch.from_numpy(g.standard_normal((T, out)).astype(np.float32) * 0.5).to(dtype)
    dy = torch.from_numpy(g.standard_normal((T, out)).astype(np.float32)).to(dtype)
    n = np.abs(g.standard_normal(out)).astype(np.float32) + 0.5
    m = synth.magnitude(n, g.uniform(-2**-8, 2**-8, out))
    return base, lora, dy, torch.from_numpy(m), torch.from_numpy(n), cfg.s


@gpu
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("add_base", [False, True])
def test_compose_autograd_matches_oracle(dtype, add_base):
    dev = torch.device("cuda:0")
    base, lora, dy, m, n, s = _compose_inputs(300, 264, dtype, 7)
    bg, lg, mg = (t.to(dev).requires_grad_() for t in (base, lora, m))
    y = torch_ops.compose(bg, lg, mg, n.to(dev), s, add_base)
    y.backward(dy.to(dev))
    kind = "bf16" if dtype == torch.bfloat16 else "fp16"
    b64, l64, dy64 = (O.as_f64(t.float().numpy()) for t in (base, lora, dy))
    y_ref = O.compose_fwd(b64, l64, O.as_f64(m.numpy()), O.as_f64(n.numpy()), s, add_base)
    dl_ref, db_ref, dm_ref = O.compose_bwd(dy64, b64, l64, O.as_f64(m.numpy()), O.as_f64(n.numpy()), s, add_base)
    g = m.double().numpy() / n.double().numpy()
    mass_y = np.abs((g - 1) * b64) + np.abs(g * s * l64) + (np.abs(b64) if add_base else 0)
    assert_compose(y.detach().float().cpu().numpy(), y_ref, mass_y, kind, "y")
    assert_compose(lg.grad.float().cpu().numpy(), dl_ref, np.abs(dl_ref), kind, "d_lora")
    assert_compose(bg.grad.float().cpu().numpy(), db_ref, np.abs(db_ref), kind, "d_base")
    cond = np.sum(np.abs(dy64 * (b64 + s * l64)), axis=0) / n.double().numpy()
    assert_dmag(mg.grad.cpu().numpy(), dm_ref, cond, "d_mag")


@gpu
@pytest.mark.parametrize("add_base", [False, True])
def test_lora_compose_autograd_matches_oracle(add_base):
    # the fused pair through autograd: d_base, d_B and d_mag from the kernels
    # (lora never formed), d_h = dy (g s .* B) from torch's GEMM
    dev = torch.device("cuda:0")
    T, out, r = 300, 264, 24
    rng = np.random.default_rng(11)
    to = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)
    base, h, B, dy = to(rng.normal(0, 0.3, (T, out))), to(rng.normal(0, 1, (T, r))), to(rng.normal(0, 0.05, (out, r))), \
        to(rng.normal(0, 1, (T, out)))
    n = torch.from_numpy(rng.uniform(0.5, 2.0, out).astype(np.float32))
    m = n * (1 + torch.from_numpy(rng.normal(0, 1e-3, out).astype(np.float32)))
    s = 32 / np.sqrt(r)
    bg, hg, Bg, mg = (t.to(dev).requires_grad_() for t in (base, h, B, m))
    y = torch_ops.lora_compose(bg, hg, Bg, mg, n.to(dev), s, add_base)
    y.backward(dy.to(dev))
    b64, h64, B64, dy64 = (O.as_f64(t.float().numpy()) for t in (base, h, B, dy))
    m64, n64 = O.as_f64(m.numpy()), O.as_f64(n.numpy())
    y_ref = O.lora_compose_fwd(b64, h64, B64, m64, n64, s, add_base)
    db_ref, dB_ref, dm_ref = O.lora_compose_bwd(dy64, b64, h64, B64, m64, n64, s, add_base)
    g = m64 / n64
    dh_ref = (g * s * dy64) @ B64
    assert _rel(y, torch.from_numpy(y_ref)) < 1e-2
    assert_compose(bg.grad.float().cpu().numpy(), db_ref, np.abs(db_ref), "bf16", "d_base")
    assert _rel(Bg.grad, torch.from_numpy(dB_ref)) < 1e-2
    assert _rel(hg.grad, torch.from_numpy(dh_ref)) < 1e-2
    # d_mag: 1e-5 of the condition, or the fused path's chain bound (its lora
    # term is sum_k B (dy^T h), an MFMA sum over the tokens)
    cond = np.sum(np.abs(dy64 * (b64 + s * (h64 @ B64.T))), axis=0) / n64
    mass_m = (np.sum(np.abs(dy64 * b64), axis=0) + s * np.sum(np.abs(B64) * (np.abs(dy64).T @ np.abs(h64)), axis=1)) / n64
    err = np.abs(mg.grad.cpu().double().numpy() - dm_ref)
    assert np.all((err <= 1e-5 * cond) | (err <= (T / 16 + 96) * 2.0**-24 * mass_m)), "d_mag"


@gpu
def test_compose_grad_base_skipped_when_not_needed():
    dev = torch.device("cuda:0")
    base, lora, dy, m, n, s = _compose_inputs(64, 64, torch.bfloat16, 3)
    lg = lora.to(dev).requires_grad_()
    y = torch_ops.compose(base.to(dev), lg, m.to(dev), n.to(dev), s, False)
    y.backward(dy.to(dev))
    assert lg.grad is not None and lg.grad.shape == lora.shape


@gpu
def test_opcheck():
    dev = torch.device("cuda:0")
    base, lora, dy, m, n, s = _compose_inputs(64, 64, torch.bfloat16, 5)
    args = (base.to(dev).requires_grad_(), lora.to(dev).requires_grad_(), m.to(dev).requires_grad_(), n.to(dev), s,
            False)
    torch.library.opcheck(torch_ops.compose, args,
                          test_utils=("test_schema", "test_autograd_registration", "test_faketensor"))
    W0, A, B = (t.to(dev) for t in synth.weights(synth.CONFIGS["tiny"]))
    torch.library.opcheck(torch_ops.weight_norm, (W0, A, B, 1.5), test_utils=("test_schema", "test_faketensor"))
    torch.library.opcheck(torch_ops.row_sqnorm, (W0,), test_utils=("test_schema", "test_faketensor"))
    h = torch.randn(64, 16, device=dev, dtype=torch.bfloat16)
    B2 = 0.1 * torch.randn(64, 16, device=dev, dtype=torch.bfloat16)
    torch.library.opcheck(torch_ops.lora_compose, (base.to(dev), h, B2, m.to(dev), n.to(dev), s, True),
                          test_utils=("test_schema", "test_faketensor"))
    torch.library.opcheck(torch_ops.lora_compose, (base.to(dev).requires_grad_(), h.clone().requires_grad_(),
                                                   B2.clone().requires_grad_(), m.to(dev).requires_grad_(),
                                                   n.to(dev), s, False),
                          test_utils=("test_schema", "test_autograd_registration", "test_faketensor"))
    torch.library.opcheck(torch_ops.lora_compose_backward, (dy.to(dev), base.to(dev), h, B2, m.to(dev), n.to(dev), s,
                                                            False, True),
                          test_utils=("test_schema", "test_faketensor"))
    sq = torch_ops.row_sqnorm(W0)
    torch.library.opcheck(torch_ops.weight_norm_cached, (W0, A, B, sq, 1.5),
                          test_utils=("test_schema", "test_faketensor"))
    Ag, Bg = A.clone().requires_grad_(), B.clone().requires_grad_()
    torch.library.opcheck(torch_ops.weight_norm, (W0, Ag, Bg, 1.5),
                          test_utils=("test_schema", "test_autograd_registration", "test_faketensor"))
    n = torch_ops.weight_norm(W0, A, B, 1.5)
    dn = torch.randn_like(n)
    torch.library.opcheck(torch_ops.weight_norm_backward, (W0, A, B, n, dn, 1.5),
                          test_utils=("test_schema", "test_faketensor"))


@gpu
def test_layer_caches_the_base_term():
    """DoRALinear keeps ||W0_i||^2 and takes its norm with that base term; the
    result is the plain factored norm within the norm's tolerance, and a
    refresh after changing W0 follows the new weight."""
    dev = torch.device("cuda:0")
    torch.manual_seed(2)
    layer = torch_ops.DoRALinear(512, 384, 16, device=dev)
    with torch.no_grad():
        layer.lora_B.normal_(0.0, 0.02)
    n = layer.weight_norm()
    assert layer.weight_sqnorm is not None and layer.weight_sqnorm.dtype == torch.float32
    W, A, B = (t.detach().float().cpu().numpy() for t in (layer.weight, layer.lora_A, layer.lora_B))
    np.testing.assert_allclose(layer.weight_sqnorm.double().cpu().numpy(), O.row_sqnorm(W), rtol=1e-6)
    np.testing.assert_allclose(n.double().cpu().numpy(), O.weight_norm(W, A, B, layer.s), rtol=1e-5)
    plain = torch_ops.weight_norm(layer.weight, layer.lora_A.detach(), layer.lora_B.detach(), layer.s)
    np.testing.assert_allclose(n.double().cpu().numpy(), plain.double().cpu().numpy(), rtol=2e-5)
    with torch.no_grad():
        layer.weight.mul_(2.0)
    layer.refresh_weight_cache()
    W2 = layer.weight.float().cpu().numpy()
    np.testing.assert_allclose(layer.weight_norm().double().cpu().numpy(), O.weight_norm(W2, A, B, layer.s), rtol=1e-5)


def _dense_reference(x, W0, A, B, m, s, dy):
    """float64 CPU: y = x W0^T + (g-1) x W0^T + g s x A^T B^T with n detached; grads of A, B, m, x."""
    xd, W0d, Ad, Bd, md = (t.detach().double().cpu().requires_grad_() for t in (x, W0, A, B, m))
    W0d.requires_grad_(False)
    n = torch.from_numpy(O.weight_norm(*(t.detach().float().cpu().numpy() for t in (W0, A, B)), s))
    g = md / n
    base = xd @ W0d.T
    lora = (xd @ Ad.T) @ Bd.T
    y = base + (g - 1) * base + g * s * lora
    y.backward(dy.double().cpu())
    return y.detach(), xd.grad, Ad.grad, Bd.grad, md.grad, n


def _rel(a, b):
    a, b = a.detach().double().cpu(), b.detach().double().cpu()
    return float((a - b).norm() / b.norm().clamp_min(1e-300))


@gpu
def test_dora_linear_forward_backward():
    dev = torch.device("cuda:0")
    torch.manual_seed(0)
    layer = torch_ops.DoRALinear(320, 256, 16, alpha=32.0, device=dev)
    with torch.no_grad():
        layer.lora_B.normal_(0.0, 0.02)
        layer.magnitude.mul_(1.0 + 0.01 * torch.randn_like(layer.magnitude))
    x = torch.randn(3, 70, 320, device=dev, dtype=torch.bfloat16).requires_grad_()
    y = layer(x)
    dy = torch.randn_like(y)
    y.backward(dy)
    y_ref, dx_ref, dA_ref, dB_ref, dm_ref, n_ref = _dense_reference(
        x.reshape(-1, 320), layer.weight, layer.lora_A, layer.lora_B, layer.magnitude, layer.s, dy.reshape(-1, 256))
    # the layer's norm is the factored kernel's, to fp32 rounding
    np.testing.assert_allclose(layer.weight_norm().double().cpu().numpy(), n_ref.numpy(), rtol=1e-5)
    # bf16 GEMM outputs and inputs bound the rest
    assert _rel(y.reshape(-1, 256), y_ref) < 2e-2
    assert _rel(x.grad.reshape(-1, 320), dx_ref) < 2e-2
    assert _rel(layer.lora_A.grad, dA_ref) < 3e-2
    assert _rel(layer.lora_B.grad, dB_ref) < 3e-2
    assert _rel(layer.magnitude.grad, dm_ref) < 2e-2
    assert layer.weight.grad is None


@gpu
def test_dora_linear_starts_as_base_layer_and_inference_tier():
    dev = torch.device("cuda:0")
    torch.manual_seed(1)
    layer = torch_ops.DoRALinear(256, 192, 8, device=dev)
    x = torch.randn(50, 256, device=dev, dtype=torch.bfloat16)
    base = torch.nn.functional.linear(x, layer.weight)
    with torch.no_grad():
        y0 = layer(x)
    # B = 0 and m = n exactly: g - 1 = 0 and s*lora = 0, so y is base bit for bit
    assert torch.equal(y0, base)
    with torch.no_grad():
        layer.lora_B.normal_(0.0, 0.05)
    with torch.inference_mode():
        y_inf = layer(x)
    assert y_inf.grad_fn is None
    y_train = layer(x.requires_grad_())
    assert y_train.grad_fn is not None
    # both tiers form lora inside the same compose kernel (the training tier
    # records it for autograd): the outputs agree with the dense fp64 layer
    W, A, B, m = (t.detach().double().cpu() for t in (layer.weight, layer.lora_A, layer.lora_B, layer.magnitude))
    n = torch.from_numpy(O.weight_norm(W.numpy(), A.numpy(), B.numpy(), layer.s))
    xd = x.detach().double().cpu()
    ref = (m / n) * (xd @ W.T + layer.s * (xd @ A.T) @ B.T)
    assert _rel(y_inf, ref) < 1e-2 and _rel(y_train, ref) < 1e-2
    assert torch.equal(y_inf, y_train.detach())


def _dense_reference_full(x, W0, A, B, m, s, dy):
    """float64 CPU, norm NOT detached: n = ||W0 + s B A|| inside the graph."""
    xd, W0d, Ad, Bd, md = (t.detach().double().cpu().requires_grad_() for t in (x, W0, A, B, m))
    W0d.requires_grad_(False)
    n = torch.linalg.vector_norm(W0d + s * (Bd @ Ad), dim=1)
    g = md / n
    base = xd @ W0d.T
    y = g * (base + s * ((xd @ Ad.T) @ Bd.T))
    y.backward(dy.double().cpu())
    return y.detach(), xd.grad, Ad.grad, Bd.grad, md.grad


@gpu
def test_dora_linear_norm_not_detached():
    dev = torch.device("cuda:0")
    torch.manual_seed(3)
    layer = torch_ops.DoRALinear(256, 192, 16, alpha=32.0, device=dev, detach_norm=False)
    with torch.no_grad():
        layer.lora_B.normal_(0.0, 0.05)
        layer.magnitude.mul_(1.0 + 0.01 * torch.randn_like(layer.magnitude))
    x = torch.randn(2, 40, 256, device=dev, dtype=torch.bfloat16).requires_grad_()
    y = layer(x)
    # dy close to y (the gradient of |y|^2 / 2): the sums over tokens of dy * y
    # that drive the path through n then add up instead of cancelling
    dy = (y.detach().float() + 0.1 * torch.randn(y.shape, device=dev)).to(y.dtype)
    y.backward(dy)
    y_ref, dx_ref, dA_ref, dB_ref, dm_ref = _dense_reference_full(
        x.reshape(-1, 256), layer.weight, layer.lora_A, layer.lora_B, layer.magnitude, layer.s, dy.reshape(-1, 192))
    _, _, dA_det, dB_det, _, _ = _dense_reference(
        x.reshape(-1, 256), layer.weight, layer.lora_A, layer.lora_B, layer.magnitude, layer.s, dy.reshape(-1, 192))
    assert _rel(y.reshape(-1, 192), y_ref) < 2e-2
    assert _rel(x.grad.reshape(-1, 256), dx_ref) < 2e-2
    assert _rel(layer.magnitude.grad, dm_ref) < 2e-2
    # the path through n changes the adapter gradients by more than the tolerance,
    # so these checks tell the two readings apart
    assert _rel(dA_det, dA_ref) > 0.1 and _rel(dB_det, dB_ref) > 0.1
    assert _rel(layer.lora_A.grad, dA_ref) < 3e-2
    assert _rel(layer.lora_B.grad, dB_ref) < 3e-2
    assert layer.weight.grad is None


@gpu
def test_compile_without_graph_breaks_gpu():
    dev = torch.device("cuda:0")
    torch.manual_seed(6)
    for detach in (True, False):
        layer = torch_ops.DoRALinear(256, 192, 16, device=dev, detach_norm=detach)
        with torch.no_grad():
            layer.lora_B.normal_(0.0, 0.05)
        _compile_check(layer, torch.randn(3, 20, 256, device=dev, dtype=torch.bfloat16))


@gpu
def test_supported_inputs_always_take_the_kernels(monkeypatch):
    """bf16/fp16 tensors on the GPU reach the C ABI for every operator of the
    layer's forward and backward (norm not detached, so the norm backward too);
    the eager tier is not entered (its functions raise if called)."""
    from dora_fine_tuning_amd import binding

    dev = torch.device("cuda:0")
    calls = {}
    for name in ("dora_norm_factored_cached", "dora_row_sqnorm", "dora_lora_compose_fwd", "dora_lora_compose_bwd",
                 "dora_norm_bwd", "dora_compose_fwd", "dora_compose_bwd", "dora_norm_factored"):
        fn = getattr(binding, name)

        def counted(*a, _fn=fn, _name=name, **k):
            calls[_name] = calls.get(_name, 0) + 1
            return _fn(*a, **k)

        monkeypatch.setattr(binding, name, counted)
    for name in [n for n in dir(torch_ops) if n.startswith("_eager_")]:
        def boom(*a, _name=name, **k):
            raise AssertionError(f"eager tier entered: {_name}")

        monkeypatch.setattr(torch_ops, name, boom)
    for dtype in (torch.bfloat16, torch.float16):
        layer = torch_ops.DoRALinear(256, 192, 16, device=dev, dtype=dtype, detach_norm=False)
        with torch.no_grad():
            layer.lora_B.normal_(0.0, 0.05)
        x = torch.randn(40, 256, device=dev, dtype=dtype).requires_grad_()
        layer(x).backward(torch.randn(40, 192, device=dev, dtype=dtype))
        base, lora, dy, m, n, s = _compose_inputs(64, 64, dtype, 9)
        lg = lora.to(dev).requires_grad_()
        torch_ops.compose(base.to(dev), lg, m.to(dev), n.to(dev), s, False).backward(dy.to(dev))
        torch_ops.weight_norm(*(t.to(dev) for t in synth.weights(synth.CONFIGS["tiny"], "bf16" if dtype == torch.bfloat16 else "fp16")), 1.5)
    for name in ("dora_norm_factored_cached", "dora_row_sqnorm", "dora_lora_compose_fwd", "dora_lora_compose_bwd",
                 "dora_norm_bwd", "dora_compose_fwd", "dora_compose_bwd", "dora_norm_factored"):
        assert calls.get(name, 0) >= 2, (name, calls)


@gpu
def test_eager_tier_for_fp32_on_the_gpu():
    """fp32 matrices on the GPU are not a kernel dtype: the operators take the
    eager tier there and agree with the oracle."""
    dev = torch.device("cuda:0")
    base, lora, dy, m, n, s = _compose_inputs(50, 72, torch.float32, 13)
    y = torch_ops.compose(base.to(dev), lora.to(dev), m.to(dev), n.to(dev), s, True)
    y_ref = O.compose_fwd(base, lora, m, n, s, True)
    np.testing.assert_allclose(y.double().cpu().numpy(), y_ref, rtol=1e-5, atol=1e-6)


@gpu
def test_compose_backward_takes_non_contiguous_inputs():
    """A transposed (non-contiguous) base and lora pass through the forward and
    the backward alike (the saved originals are made contiguous for the kernel)."""
    dev = torch.device("cuda:0")
    base, lora, dy, m, n, s = _compose_inputs(64, 96, torch.bfloat16, 17)
    bt = base.t().contiguous().to(dev).t()  # [T x out] view of an [out x T] buffer
    lt = lora.t().contiguous().to(dev).t()
    assert not bt.is_contiguous() and not lt.is_contiguous()
    bg, lg = bt.detach().requires_grad_(), lt.detach().requires_grad_()
    y = torch_ops.compose(bg, lg, m.to(dev), n.to(dev), s, False)
    y.backward(dy.to(dev))
    dl_ref, db_ref, _ = O.compose_bwd(dy, base, lora, m, n, s, False)
    assert_compose(lg.grad.float().cpu().numpy(), dl_ref, np.abs(dl_ref), "bf16", "d_lora non-contiguous")
    assert_compose(bg.grad.float().cpu().numpy(), db_ref, np.abs(db_ref), "bf16", "d_base non-contiguous")
