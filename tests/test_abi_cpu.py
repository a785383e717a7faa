"""The C-ABI library on the host: it loads, exports every entry point the header
declares, answers workspace queries inside the factored memory bound, and
rejects invalid arguments before any launch (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

from dora_fine_tuning_amd import binding, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = binding.LIB
OK, INVALID, UNSUPPORTED = binding.DORA_OK, binding.DORA_INVALID_ARG, binding.DORA_UNSUPPORTED


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "dora.h")).read()
    return re.findall(r"DORA_API\s+[\w\s\*]+?\b(dora_\w+)\s*\(", text)


def test_header_declarations_are_exported():
    names = declared_symbols()
    assert set(names) == set(binding.EXPORTS), names
    raw = ctypes.CDLL(binding.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_version():
    v = binding.dora_version()
    assert "gfx950" in v and "dora_fine_tuning_amd" in v


def bound(out, r):
    return 4 * (out * r + r * r) + 64 * out


@pytest.mark.parametrize("name", sorted(synth.CONFIGS))
def test_norm_workspace_within_factored_bound(name):
    c = synth.CONFIGS[name]
    for dt in (0, 1):
        ws = LIB.dora_norm_workspace_bytes(c.out, c.in_, c.r, dt)
        assert 0 < ws <= bound(c.out, c.r), (name, ws, bound(c.out, c.r))
    # the 8192 x 8192 rank-384 module: scratch far below one dense fp32 out x in buffer
    if name == "wide_8192_r384":
        assert LIB.dora_norm_workspace_bytes(8192, 8192, 384, 0) < 8192 * 8192 * 4 / 15


def test_norm_workspace_bound_over_shapes():
    # every rank from 1 to 4 * out on small modules (r > out included), and a
    # spread of ranks on larger ones, in both dtypes and on both paths
    # (in % 8 selects whether the 16-byte path's plan is also considered)
    for out in (1, 2, 7, 8, 33, 64):
        for in_ in (0, 8, 100, 4096):
            for r in range(0, 4 * out + 1):
                for dt in (0, 1):
                    ws = LIB.dora_norm_workspace_bytes(out, in_, r, dt)
                    assert ws <= bound(out, r), (out, in_, r, dt, ws, bound(out, r))
    for out in (128, 129, 1000, 4096, 27648):
        for in_ in (0, 8, 100, 4096, 8192):
            for r in (0, 1, 8, 16, 64, 130, 384, 768, 1000, 2048, 4 * out):
                ws = LIB.dora_norm_workspace_bytes(out, in_, r, 0)
                assert ws <= bound(out, r), (out, in_, r, ws, bound(out, r))
    # shapes where r is large against out (the Gram kernel then writes G'hi/G'lo itself)
    for out, in_, r in ((64, 64, 1000), (33, 64, 200), (8, 8192, 768), (1, 16, 4)):
        assert LIB.dora_norm_workspace_bytes(out, in_, r, 0) <= bound(out, r)


def test_workspace_queries_invalid():
    assert LIB.dora_norm_workspace_bytes(-1, 8, 8, 0) == 0
    assert LIB.dora_norm_workspace_bytes(8, 8, 8, 7) == 0
    assert LIB.dora_norm_workspace_bytes(0, 8, 8, 0) == 0
    assert LIB.dora_compose_bwd_workspace_bytes(0, 8) == 0
    # 16-token blocks while 64-token blocks would give under 512 workgroups
    # (256 threads of 8 columns per workgroup), else 64-token blocks
    assert LIB.dora_compose_bwd_workspace_bytes(64, 8) == 4 * 8 * 4
    assert LIB.dora_compose_bwd_workspace_bytes(65, 8) == 5 * 8 * 4
    assert LIB.dora_compose_bwd_workspace_bytes(4096, 4096) == 256 * 4096 * 4  # 2 x 64 = 128 workgroups at 64
    assert LIB.dora_compose_bwd_workspace_bytes(8192, 8192) == 128 * 8192 * 4  # 4 x 128 = 512 at 64
    assert LIB.dora_compose_bwd_workspace_bytes(10240, 27648) == 160 * 27648 * 4


P = 1 << 20  # fake, never dereferenced: every call below fails validation first


def _status(ret, want, fragment):
    assert ret == want, (ret, binding.dora_last_error())
    assert fragment in binding.dora_last_error()


def test_norm_validation():
    ws = LIB.dora_norm_workspace_bytes(64, 64, 8, 0)
    _status(LIB.dora_norm_factored(P, P, P, 64, 64, 8, 1.0, 5, P * 2, P * 3, ws, None), UNSUPPORTED, "dtype")
    _status(LIB.dora_norm_factored(P, P, P, -1, 64, 8, 1.0, 0, P * 2, P * 3, ws, None), INVALID, "negative")
    _status(LIB.dora_norm_factored(None, P, P, 64, 64, 8, 1.0, 0, P * 2, P * 3, ws, None), INVALID, "W0")
    _status(LIB.dora_norm_factored(P, None, P, 64, 64, 8, 1.0, 0, P * 2, P * 3, ws, None), INVALID, "A")
    _status(LIB.dora_norm_factored(P, P, None, 64, 64, 8, 1.0, 0, P * 2, P * 3, ws, None), INVALID, "B")
    _status(LIB.dora_norm_factored(P, P, P, 64, 64, 8, 1.0, 0, None, P * 3, ws, None), INVALID, "norm_out")
    _status(LIB.dora_norm_factored(P, P, P, 64, 64, 8, 1.0, 0, P * 2, P * 3, ws - 1, None), INVALID, "workspace")
    _status(LIB.dora_norm_factored(P, P, P, 64, 64, 8, 1.0, 0, P * 2, None, ws, None), INVALID, "NULL")
    _status(LIB.dora_norm_factored(P * 8, P * 9, P * 10, 64, 64, 8, 1.0, 0, P * 8 + 4, P * 3, ws, None),
            INVALID, "overlaps")
    # out == 0 is a no-op that succeeds without touching the device
    assert LIB.dora_norm_factored(None, None, None, 0, 64, 8, 1.0, 0, None, None, 0, None) == OK
    assert binding.dora_last_error() == ""


def test_norm_cached_validation():
    ws = LIB.dora_norm_workspace_bytes(64, 64, 8, 0)
    _status(LIB.dora_norm_factored_cached(P, P, P, P * 4, 64, 64, 8, 1.0, 5, P * 2, P * 3, ws, None), UNSUPPORTED,
            "dtype")
    _status(LIB.dora_norm_factored_cached(P, P, P, None, 64, 64, 8, 1.0, 0, P * 2, P * 3, ws, None), INVALID,
            "base_sq")
    _status(LIB.dora_norm_factored_cached(P, P, P, P * 2 + 4, 64, 64, 8, 1.0, 0, P * 2, P * 3, ws, None), INVALID,
            "base_sq overlaps")
    _status(LIB.dora_norm_factored_cached(P, P, P, P * 3 + 8, 64, 64, 8, 1.0, 0, P * 2, P * 3, ws, None), INVALID,
            "base_sq overlaps")
    _status(LIB.dora_norm_factored_cached(P, P, P, P * 4, 64, 64, 8, 1.0, 0, None, P * 3, ws, None), INVALID,
            "norm_out")
    assert LIB.dora_norm_factored_cached(None, None, None, None, 0, 64, 8, 1.0, 0, None, None, 0, None) == OK


def test_row_sqnorm_validation():
    _status(LIB.dora_row_sqnorm(P, 64, 64, 7, P * 2, None), UNSUPPORTED, "dtype")
    _status(LIB.dora_row_sqnorm(P, -1, 64, 0, P * 2, None), INVALID, "negative")
    _status(LIB.dora_row_sqnorm(None, 64, 64, 0, P * 2, None), INVALID, "W0")
    _status(LIB.dora_row_sqnorm(P, 64, 64, 0, None, None), INVALID, "sq_out")
    _status(LIB.dora_row_sqnorm(P, 64, 64, 0, P + 64, None), INVALID, "overlaps")
    far = 1 << 46
    _status(LIB.dora_row_sqnorm(far, 1 << 34, 1, 0, 2 * far, None), UNSUPPORTED, "workgroups")
    assert LIB.dora_row_sqnorm(None, 0, 64, 0, None, None) == OK


def test_compose_fwd_validation():
    _status(LIB.dora_compose_fwd(P, P * 2, P * 3, P * 4, 1.0, 8, 8, 3, 0, P * 5, None), UNSUPPORTED, "dtype")
    _status(LIB.dora_compose_fwd(P, P * 2, P * 3, P * 4, 1.0, -8, 8, 0, 0, P * 5, None), INVALID, "negative")
    _status(LIB.dora_compose_fwd(P, None, P * 3, P * 4, 1.0, 8, 8, 0, 0, P * 5, None), INVALID, "NULL")
    _status(LIB.dora_compose_fwd(P, P * 2, P * 3, P * 4, 1.0, 8, 8, 0, 0, P + 2, None), INVALID, "partially")
    _status(LIB.dora_compose_fwd(P, P * 2, P * 3, P * 4, 1.0, 8, 8, 0, 0, P * 3, None), INVALID, "mag")
    assert LIB.dora_compose_fwd(None, None, None, None, 1.0, 0, 8, 0, 0, None, None) == OK
    assert LIB.dora_compose_fwd(None, None, None, None, 1.0, 8, 0, 0, 0, None, None) == OK


def test_compose_bwd_validation():
    T, out = 64, 16
    ws = LIB.dora_compose_bwd_workspace_bytes(T, out)
    args = dict(dy=P, base=P * 2, lora=P * 3, mag=P * 4, norm=P * 5, d_lora=P * 6, d_base=P * 7, d_mag=P * 8,
                ws=P * 9)

    def call(dtype=0, T=T, ws_bytes=ws, **kw):
        a = dict(args, **kw)
        return LIB.dora_compose_bwd(a["dy"], a["base"], a["lora"], a["mag"], a["norm"], 1.0, T, out, dtype, 0,
                                    a["d_lora"], a["d_base"], a["d_mag"], a["ws"], ws_bytes, None)

    _status(call(dtype=9), UNSUPPORTED, "dtype")
    _status(call(T=-1), INVALID, "negative")
    _status(call(d_mag=None), INVALID, "d_mag")
    _status(call(dy=None), INVALID, "NULL")
    _status(call(ws_bytes=ws - 4), INVALID, "workspace")
    _status(call(ws=None), INVALID, "workspace is NULL")
    _status(call(d_base=P * 6 + 2), INVALID, "d_lora and d_base overlap")
    _status(call(d_lora=P + 2), INVALID, "partially overlaps")
    _status(call(ws=P * 2), INVALID, "workspace overlaps")
    _status(call(d_mag=P * 2 + 8), INVALID, "d_mag overlaps")
    assert LIB.dora_compose_bwd(None, None, None, None, None, 1.0, 8, 0, 0, 0, None, None, None, None, 0, None) == OK


def test_lora_compose_fwd_validation():
    def call(base=P, h=P * 2, B=P * 3, mag=P * 4, norm=P * 5, y=P * 6, T=64, out=16, r=8, dtype=0):
        return LIB.dora_lora_compose_fwd(base, h, B, mag, norm, 1.0, T, out, r, dtype, 0, y, None)

    _status(call(dtype=4), UNSUPPORTED, "dtype")
    _status(call(r=-1), INVALID, "negative")
    _status(call(base=None), INVALID, "NULL")
    _status(call(h=None), INVALID, "h or B")
    _status(call(y=P + 2), INVALID, "partially")
    _status(call(y=P * 2 + 8), INVALID, "y overlaps")
    _status(call(y=P * 4), INVALID, "y overlaps")
    # r == 0 needs no h or B; empty sizes are no-ops
    # 2^40 tokens x 256 columns need 2^32 workgroups; far-apart fake pointers
    # keep the overlap checks quiet (nothing is launched)
    _status(LIB.dora_lora_compose_fwd(1 << 49, None, None, 1 << 50, (1 << 50) + (1 << 20), 1.0, 1 << 40, 1 << 8, 0,
                                      0, 0, 1 << 51, None), UNSUPPORTED, "workgroups")
    assert LIB.dora_lora_compose_fwd(None, None, None, None, None, 1.0, 0, 16, 8, 0, 0, None, None) == OK
    assert LIB.dora_lora_compose_fwd(None, None, None, None, None, 1.0, 16, 0, 8, 0, 0, None, None) == OK


def test_lora_compose_bwd_validation():
    T, out, r = 64, 16, 8
    ws = LIB.dora_lora_compose_bwd_workspace_bytes(T, out, r)
    assert ws > 0

    def call(dy=P, base=P * 2, h=P * 3, B=P * 4, mag=P * 5, norm=P * 6, d_base=P * 7, d_B=P * 8, d_mag=P * 9,
             w=P * 10, ws_bytes=ws, dtype=0, T=T):
        return LIB.dora_lora_compose_bwd(dy, base, h, B, mag, norm, 1.0, T, out, r, dtype, 0, d_base, d_B, d_mag, w,
                                         ws_bytes, None)

    _status(call(dtype=3), UNSUPPORTED, "dtype")
    _status(call(T=-1), INVALID, "negative")
    _status(call(d_mag=None), INVALID, "d_mag")
    _status(call(base=None), INVALID, "dy or base")
    _status(call(B=None), INVALID, "B or d_B")
    _status(call(h=None), INVALID, "h is NULL")
    _status(call(d_base=P + 2), INVALID, "overlaps an input")
    _status(call(d_B=P * 7 + 4), INVALID, "outputs overlap")
    _status(call(ws_bytes=ws - 16), INVALID, "workspace of")
    _status(call(w=None), INVALID, "workspace is NULL")
    _status(call(w=P * 2), INVALID, "workspace overlaps")
    assert LIB.dora_lora_compose_bwd(None, None, None, None, None, None, 1.0, 8, 0, 8, 0, 0, None, None, None, None, 0,
                                     None) == OK
    assert LIB.dora_lora_compose_bwd_workspace_bytes(0, 8, 8) == 0


def test_lora_compose_bwd_slow_path_limit():
    """Off the fast path (here: an unaligned dy), the slow path runs T * r
    products in order per output column; above 2^20 the call is refused with
    UNSUPPORTED before any launch, at or below it the arguments pass validation
    (checked with far-apart fake pointers and out = 0 would be a no-op, so use
    a shape whose only failure is the limit)."""
    out = 8

    def call(T, r):
        # pointers 2^34 bytes apart: no overlap for any of these sizes
        p = [(k + 1) << 34 for k in range(10)]
        return LIB.dora_lora_compose_bwd(p[0] + 2, p[1], p[2], p[3], p[4], p[5], 1.0, T, out, r, 0, 0, p[6], p[7],
                                         p[8], p[9], 1 << 30, None)

    _status(call(8192, 384), UNSUPPORTED, "slow path")
    _status(call((1 << 20) // 128 + 1, 128), UNSUPPORTED, "slow path")


def test_compose_bwd_noalloc_validation():
    """The entry point without a workspace: the argument checks of
    dora_compose_bwd, and sizes whose partials exceed its 24 MiB scratch are
    refused (UNSUPPORTED) before any device call."""
    T, out = 64, 16
    call = lambda dtype=0, T=T, out=out, d_mag=P * 9, base=P * 2: LIB.dora_compose_bwd_noalloc(
        P, base, P * 3, P * 4, P * 5, 1.0, T, out, dtype, 0, P * 6, P * 7, d_mag, None)
    _status(call(dtype=4), UNSUPPORTED, "dtype")
    _status(call(T=-1), INVALID, "negative")
    # 16-token blocks of 8192 columns: 2^21 tokens need 2^17 blocks x 32 KiB = 4 GiB of partials
    far = [(k + 1) << 42 for k in range(10)]
    _status(LIB.dora_compose_bwd_noalloc(far[0], far[1], far[2], far[3], far[4], 1.0, 1 << 21, 8192, 0, 0, far[5],
                                         far[6], far[7], None), UNSUPPORTED, "scratch")
    # the largest workload module fits: 10240 tokens x 27648 columns (17.7 MB of partials)
    assert LIB.dora_compose_bwd_workspace_bytes(10240, 27648) <= 24 << 20
    assert LIB.dora_compose_bwd_noalloc(None, None, None, None, None, 1.0, 8, 0, 0, 0, None, None, None, None) == OK


def test_compose_rejects_grids_beyond_one_launch():
    # 2^36 tokens of 8 columns: the forward would need 2^34 workgroups.  Far-apart
    # fake pointers keep the overlap checks quiet; nothing is launched.
    T, out, far = 1 << 36, 8, 1 << 46
    p = [far * k for k in range(1, 10)]
    _status(LIB.dora_compose_fwd(p[0], p[1], p[2], p[3], 1.0, T, out, 0, 0, p[4], None), UNSUPPORTED, "workgroups")
    ws = LIB.dora_compose_bwd_workspace_bytes(T, out)
    _status(LIB.dora_compose_bwd(p[0], p[1], p[2], p[3], p[4], 1.0, T, out, 0, 0, p[5], p[6], p[7], p[8], ws, None),
            UNSUPPORTED, "workgroups")


def test_binding_rejects_host_tensors():
    import torch

    W0 = torch.zeros(8, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="HIP device"):
        binding.dora_norm_factored(W0, W0, W0, 1.0)
    with pytest.raises(ValueError, match="dtype"):
        binding.dora_compose_fwd(W0.float(), W0.float(), None, None, 1.0)


def test_norm_bwd_validation():
    ws = LIB.dora_norm_bwd_workspace_bytes(64, 64, 8, 0)
    assert ws > 0 and LIB.dora_norm_bwd_workspace_bytes(64, 64, 8, 7) == 0
    assert LIB.dora_norm_bwd_workspace_bytes(-1, 64, 8, 0) == 0
    # W0 P, A 2P, B 3P, norm 4P, d_norm 5P, d_A 6P, d_B 7P, ws 8P
    args = lambda **k: [k.get(n, d) for n, d in (("W0", P), ("A", P * 2), ("B", P * 3), ("norm", P * 4),
                                                 ("d_norm", P * 5), ("out", 64), ("in_", 64), ("r", 8), ("s", 1.0),
                                                 ("dt", 0), ("d_A", P * 6), ("d_B", P * 7), ("ws", P * 8),
                                                 ("wsb", ws), ("stream", None))]
    _status(LIB.dora_norm_bwd(*args(dt=3)), UNSUPPORTED, "dtype")
    _status(LIB.dora_norm_bwd(*args(out=-1)), INVALID, "negative")
    _status(LIB.dora_norm_bwd(*args(A=None)), INVALID, "A or d_A")
    _status(LIB.dora_norm_bwd(*args(d_norm=None)), INVALID, "d_norm")
    _status(LIB.dora_norm_bwd(*args(W0=None)), INVALID, "W0")
    # sizes the 16-byte path cannot take go to the general path, whose (smaller)
    # workspace is still checked before any launch
    ws_gen = LIB.dora_norm_bwd_workspace_bytes(64, 60, 12, 0)
    assert ws_gen > 0
    _status(LIB.dora_norm_bwd(*args(in_=60, r=12, wsb=3)), INVALID, "workspace")
    _status(LIB.dora_norm_bwd(*args(wsb=ws - 1)), INVALID, "workspace")
    _status(LIB.dora_norm_bwd(*args(ws=None)), INVALID, "workspace is NULL")
    _status(LIB.dora_norm_bwd(*args(d_B=P * 3 + 64)), INVALID, "overlaps")
    _status(LIB.dora_norm_bwd(*args(d_A=P * 7 + 16)), INVALID, "overlap")
    _status(LIB.dora_norm_bwd(*args(ws=P + 1024)), INVALID, "overlaps")
    assert LIB.dora_norm_bwd(*args(r=0, W0=None, A=None, B=None)) == OK


def test_norm_bwd_workspace_is_factored():
    # O(out*r + in*r + r*r) scratch, well under the dense out x in transient
    # (V and dV in bf16) at every workload shape.  The row slices of the
    # contractions are sized for one workgroup per CU (256 CUs, 128-column
    # blocks), which adds at most r * 4 bytes per row of 256 * 128 rows (the
    # bound allows 2r * 4).
    for c in synth.CONFIGS.values():
        ws = LIB.dora_norm_bwd_workspace_bytes(c.out, c.in_, c.r, 0)
        dense = 2 * 2 * c.out * c.in_
        bound = 24 * (c.out * c.r + c.in_ * c.r + c.r * c.r) + 8 * c.r * 256 * 128 + 4 * c.out + 4096
        assert 0 < ws <= bound, (c.name, ws, bound)
        if c.out * c.in_ >= 4096 * 4096:
            assert ws < dense / 2, (c.name, ws, dense)
    assert LIB.dora_norm_bwd_workspace_bytes(64, 64, 0, 0) == 0
    assert LIB.dora_norm_bwd_workspace_bytes(0, 64, 8, 0) == 0
