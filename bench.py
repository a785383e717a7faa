#!/usr/bin/env python3
"""Benchmark of the DoRA hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input at the
8192 x 8192, rank-384 module (T = 8192 tokens, bf16): the factored weight norm,
the compose forward and the compose backward with the magnitude gradient.  All
inputs are resident in HBM before timing starts.  Kernels run on torch's current
stream, so torch.cuda.Event pairs around each call time exactly that call's
kernels.

Timing protocol: each kernel call of a step runs cold -- right before it a
1 GiB read-only pass evicts L2 and the 256 MB last-level cache (no dirty lines
are left behind), so its inputs come from HBM -- and HIP events on the launch
stream bracket the call alone (not the evicting read).  ``ms_per_step`` is the
wall time of a whole step, evicting reads included.

Prints one JSON line.  ``value`` is the cold compose fwd+bwd throughput in GB/s
of algorithmic bytes (reads of base, lora, dy and writes of y, d_lora, d_base,
plus the fp32 vectors); the factored norm time is reported beside it, and the
same three calls run back to back without evicting reads (as in a training
step where the backward directly follows the forward) are reported in
``in_step``.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
                    [--copy-calibration] [--in-step-reps N]
"""
from __future__ import annotations

import argparse
import concurrent.futures
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from dora_fine_tuning_amd import binding, synth  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
WORKLOAD = "wide_8192_r384"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "compose_bwd_wide_8192_r384_traffic.json")
COMPOSE_SRCS = [os.path.join(ROOT, "dora_fine_tuning_amd", "csrc", f)
                for f in ("compose.hip", "compose_kernels.hpp", "dora_common.hpp")]


def compose_bytes(T, out, e=2):
    """Algorithmic bytes per call: fwd reads base+lora and writes y; bwd reads dy,
    base, lora and writes d_lora, d_base; plus the fp32 m, n (and d_mag) vectors."""
    fwd = 3 * e * T * out + 8 * out
    bwd = 5 * e * T * out + 12 * out
    return fwd, bwd


def norm_work(out, in_, r, e=2):
    byts = e * (out * in_ + r * in_ + out * r) + 4 * out
    flops = 2 * out * in_ * r + 2 * r * r * in_ + 2 * out * r * r
    return byts, flops


def kernel_traffic(bwd_launch_bytes):
    """HBM traffic of the compose backward from committed rocprofv3 counter runs,
    or None when there are none or the kernel source changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = json.load(open(TRAFFIC_FILE))
    h = hashlib.sha256()
    for f in COMPOSE_SRCS:
        with open(f, "rb") as fh:
            h.update(fh.read())
    if rec.get("source_sha256") != h.hexdigest():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(cfg, W0, A, B, base, lora, dy, chunk_tokens, seconds):
    """The CPU fp64 oracle timed on a bounded sample of the same workload, on
    all host cores available to this process.

    The compose forward + backward oracle runs on chunks of ``chunk_tokens``
    token rows (cycling through all T rows), one chunk per worker thread at a
    time on ``len(os.sched_getaffinity(0))`` threads (numpy's elementwise
    kernels release the GIL), until about ``seconds`` of wall time have
    passed; its rate is the bytes of the finished chunks over that wall time.
    The oracle functions are called unchanged.  The dense fp64 norm oracle runs
    three times over all rows (median; BLAS matmul on its own threads).  The
    inputs are copied to host memory before any timing."""
    from oracle import dora_oracle as O

    cores = len(os.sched_getaffinity(0))
    norm_t = []
    for _ in range(3):
        t = time.perf_counter()
        n = O.weight_norm(W0, A, B, cfg.s)
        norm_t.append(time.perf_counter() - t)
    norm_s = float(np.median(norm_t))
    m = synth.magnitude(n, synth.magnitude_eps(cfg))
    n32 = n.astype(np.float32)
    bh, lh, dh = base.cpu(), lora.cpu(), dy.cpu()
    T = bh.shape[0]
    starts = list(range(0, T, chunk_tokens))
    torch_threads = torch.get_num_threads()
    torch.set_num_threads(1)  # one core per worker: no nested intra-op threads in the tensor conversions

    def work(t0):
        t1 = min(t0 + chunk_tokens, T)
        bs, ls, ds = bh[t0:t1], lh[t0:t1], dh[t0:t1]
        O.compose_fwd(bs, ls, m, n32, cfg.s)
        O.compose_bwd(ds, bs, ls, m, n32, cfg.s)
        return t1 - t0

    # Keep freed arrays in the allocator's heap (no unmapping and re-faulting of
    # fresh pages for every temporary of every chunk, which serialises threads
    # on the address-space lock); the defaults are restored afterwards.
    try:
        import ctypes

        libc = ctypes.CDLL("libc.so.6")
        M_TRIM_THRESHOLD, M_MMAP_THRESHOLD = -1, -3
        libc.mallopt(M_MMAP_THRESHOLD, 1 << 30)
        libc.mallopt(M_TRIM_THRESHOLD, 1 << 30)
    except OSError:  # pragma: no cover
        libc = None
    done_tokens, k = 0, 0
    try:
        with concurrent.futures.ThreadPoolExecutor(max_workers=cores) as ex:
            t = time.perf_counter()
            pending = set()
            while True:
                while len(pending) < cores and time.perf_counter() - t < seconds:
                    pending.add(ex.submit(work, starts[k % len(starts)]))
                    k += 1
                if not pending:
                    break
                finished, pending = concurrent.futures.wait(pending, return_when=concurrent.futures.FIRST_COMPLETED)
                done_tokens += sum(f.result() for f in finished)
            comp_s = time.perf_counter() - t
    finally:
        torch.set_num_threads(torch_threads)
        if libc is not None:
            libc.mallopt(M_MMAP_THRESHOLD, 128 * 1024)
            libc.mallopt(M_TRIM_THRESHOLD, 128 * 1024)
    fb, bb = compose_bytes(done_tokens, cfg.out)
    try:
        from threadpoolctl import threadpool_info

        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    return {
        "value": (fb + bb) / comp_s / 1e9,
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"compose fwd+bwd (numpy fp64) over {done_tokens} token rows ({done_tokens / T:.1f} passes over "
                  f"the {T} x {cfg.out} workload, chunks of {chunk_tokens} rows on {cores} worker threads): "
                  f"{comp_s:.1f} s wall; factored-norm oracle (dense fp64, BLAS matmul on {blas_threads} threads) "
                  f"on all {cfg.out} rows, median of 3: {norm_s:.2f} s",
        "norm_us": norm_s * 1e6,
        "norm_threads": blas_threads,
    }


SWEEP = [("attn_proj", "bf16"), ("wide_8192_r384", "bf16"), ("wide_8192_r384", "fp16"),
         ("mlp_up_27648x5120", "bf16")] + [(f"sweep_r{r}", dt) for r in (16, 64, 128, 384, 512, 768)
                                           for dt in ("bf16", "fp16")]
MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16


def sweep(reps, only=None, cpu_seconds=0.0):
    """One JSON line per workload config: the factored norm and the compose
    forward and backward, timed in the step's order (norm, fwd, bwd) with HIP
    events, median over ``reps`` steps after 3 warm-up steps, against their
    rooflines (norm: max of its HBM and MFMA times; compose: HBM).  With
    ``cpu_seconds`` > 0 the line also carries the CPU oracle timed on the same
    config (``cpu_baseline``: the norm over all rows, and about ``cpu_seconds``
    of compose work)."""
    dev = torch.device("cuda:0")
    for name, dtype in SWEEP:
        if only and name not in only:
            continue
        cfg = synth.CONFIGS[name]
        T, out, in_, r, s = cfg.T, cfg.out, cfg.in_, cfg.r, cfg.s
        W0c, Ac, Bc = synth.weights(cfg, dtype)
        xc, dyc = synth.activations(cfg, dtype)
        W0, A, B = W0c.to(dev), Ac.to(dev), Bc.to(dev)
        base, lora = synth.base_and_lora(xc, W0c, Ac, Bc, device=dev)
        dy = dyc.to(dev)
        del xc, dyc
        norm = torch.empty(out, dtype=torch.float32, device=dev)
        ws_n = torch.empty(max(binding.dora_norm_workspace_bytes(out, in_, r, W0.dtype), 1), dtype=torch.uint8,
                           device=dev)
        binding.dora_norm_factored(W0, A, B, s, norm_out=norm, workspace=ws_n)
        mag = torch.from_numpy(synth.magnitude(norm.cpu().numpy(), synth.magnitude_eps(cfg))).to(dev)
        y, d_lora, d_base = torch.empty_like(base), torch.empty_like(base), torch.empty_like(base)
        d_mag = torch.empty(out, dtype=torch.float32, device=dev)
        ws_b = torch.empty(max(binding.dora_compose_bwd_workspace_bytes(T, out), 1), dtype=torch.uint8, device=dev)
        evs = []
        for k in range(3 + reps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            e[0].record()
            binding.dora_norm_factored(W0, A, B, s, norm_out=norm, workspace=ws_n)
            e[1].record()
            binding.dora_compose_fwd(base, lora, mag, norm, s, y=y)
            e[2].record()
            binding.dora_compose_bwd(dy, base, lora, mag, norm, s, d_lora=d_lora, d_base=d_base, d_mag=d_mag,
                                     workspace=ws_b)
            e[3].record()
            if k >= 3:
                evs.append(e)
        torch.cuda.synchronize()
        med = lambda i: float(np.median([e[i].elapsed_time(e[i + 1]) for e in evs])) * 1e3
        n_us, f_us, b_us = med(0), med(1), med(2)
        nb, nf = norm_work(out, in_, r)
        fb, bb = compose_bytes(T, out)
        n_roof_us = max(nb / (HBM_PEAK_GBS * 1e3), nf / (MFMA_PEAK_TFLOPS * 1e6))
        line = {
            "config": name, "dtype": dtype, "out": out, "in": in_, "r": r, "T": T,
            "norm_us": round(n_us, 2), "norm_tflops": round(nf / (n_us * 1e-6) / 1e12, 1),
            "norm_bound": "mfma" if nf / (MFMA_PEAK_TFLOPS * 1e6) > nb / (HBM_PEAK_GBS * 1e3) else "hbm",
            "norm_roofline_us": round(n_roof_us, 2), "norm_frac_roofline": round(n_roof_us / n_us, 4),
            "compose_fwd_us": round(f_us, 2), "compose_fwd_gbs": round(fb / (f_us * 1e-6) / 1e9, 1),
            "compose_bwd_us": round(b_us, 2), "compose_bwd_gbs": round(bb / (b_us * 1e-6) / 1e9, 1),
            "compose_frac_hbm_peak": round((fb + bb) / ((f_us + b_us) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "reps": reps,
        }
        if cpu_seconds > 0:
            cb = cpu_baseline(cfg, W0c, Ac, Bc, base, lora, dy, 128, cpu_seconds)
            line["cpu_oracle"] = {"norm_us": round(cb["norm_us"], 1), "norm_threads": cb["norm_threads"],
                                  "compose_gbs": round(cb["value"], 3), "compose_cores": cb["cores"],
                                  "sample": cb["sample"]}
        print(json.dumps(line), flush=True)
        del W0, A, B, base, lora, dy, y, d_lora, d_base, ws_n, ws_b
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-chunk-tokens", type=int, default=128, help="token rows per oracle compose call")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="seconds of oracle compose work to time")
    ap.add_argument("--in-step-reps", type=int, default=20,
                    help="steps timed without evicting reads (the backward right after the forward); 0 skips")
    ap.add_argument("--cached-reps", type=int, default=10,
                    help="steps timing the norm with a cached base term (W0 frozen); 0 skips")
    ap.add_argument("--fused-reps", type=int, default=20,
                    help="calls timing the compose with lora = h B^T fused in, against GEMM + compose; 0 skips")
    ap.add_argument("--norm-bwd-reps", type=int, default=10,
                    help="calls timing the weight-norm backward (non-detached norm), against the dense torch form; 0 skips")
    ap.add_argument("--torch-reps", type=int, default=10,
                    help="compose forward+backward timed through the PyTorch custom operator and autograd")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 1 GiB device copy first (reference dispatch for byte counters)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the step: one JSON line per workload config (norm and compose vs rooflines)")
    ap.add_argument("--sweep-only", default="", help="comma-separated config names to restrict --sweep to")
    ap.add_argument("--sweep-cpu-seconds", type=float, default=1.0,
                    help="seconds of oracle compose work per --sweep config (with the oracle norm); 0 skips")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.sweep:
        sweep(max(args.steps // 5, 5), [c for c in args.sweep_only.split(",") if c], args.sweep_cpu_seconds)
        return

    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS[WORKLOAD]
    T, out, in_, r, s = cfg.T, cfg.out, cfg.in_, cfg.r, cfg.s

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    W0c, Ac, Bc = synth.weights(cfg)
    xc, dyc = synth.activations(cfg)
    W0, A, B = W0c.to(dev), Ac.to(dev), Bc.to(dev)
    base, lora = synth.base_and_lora(xc, W0c, Ac, Bc, device=dev)
    h = torch.nn.functional.linear(xc.to(dev), A) if args.fused_reps > 0 else None  # x A^T, the adapter's first projection
    dy = dyc.to(dev)
    del xc
    norm = torch.empty(out, dtype=torch.float32, device=dev)
    ws_norm = torch.empty(binding.dora_norm_workspace_bytes(out, in_, r), dtype=torch.uint8, device=dev)
    binding.dora_norm_factored(W0, A, B, s, norm_out=norm, workspace=ws_norm)
    mag = torch.from_numpy(synth.magnitude(norm.cpu().numpy(), synth.magnitude_eps(cfg))).to(dev)
    y = torch.empty_like(base)
    d_lora = torch.empty_like(base)
    d_base = torch.empty_like(base)
    d_mag = torch.empty(out, dtype=torch.float32, device=dev)
    ws_bwd = torch.empty(max(binding.dora_compose_bwd_workspace_bytes(T, out), 1), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    # 1 GiB read-only pass: evicts L2 and the 256 MB last-level cache without
    # leaving dirty lines, so the next kernel's inputs come from HBM
    flush_buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)

    def flush():
        flush_buf.view(torch.int64).sum()

    def step(ev):
        flush()
        ev[0].record()
        binding.dora_norm_factored(W0, A, B, s, norm_out=norm, workspace=ws_norm)
        ev[1].record()
        flush()
        ev[2].record()
        binding.dora_compose_fwd(base, lora, mag, norm, s, y=y)
        ev[3].record()
        flush()
        ev[4].record()
        binding.dora_compose_bwd(dy, base, lora, mag, norm, s, d_lora=d_lora, d_base=d_base, d_mag=d_mag,
                                 workspace=ws_bwd)
        ev[5].record()

    mk = lambda n: [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for _ in range(args.warmup):
        step(mk(6))
    evs = [mk(6) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    norm_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    fwd_ms = np.array([e[2].elapsed_time(e[3]) for e in evs])
    bwd_ms = np.array([e[4].elapsed_time(e[5]) for e in evs])

    # The same three calls back to back without evicting reads, as in a
    # training step whose backward directly follows its forward: the backward
    # then reads part of base and lora from the last-level cache, where the
    # forward left them.
    in_step = None
    if args.in_step_reps > 0:
        evw = []
        for k in range(3 + args.in_step_reps):
            e = mk(4)
            e[0].record()
            binding.dora_norm_factored(W0, A, B, s, norm_out=norm, workspace=ws_norm)
            e[1].record()
            binding.dora_compose_fwd(base, lora, mag, norm, s, y=y)
            e[2].record()
            binding.dora_compose_bwd(dy, base, lora, mag, norm, s, d_lora=d_lora, d_base=d_base, d_mag=d_mag,
                                     workspace=ws_bwd)
            e[3].record()
            if k >= 3:
                evw.append(e)
        torch.cuda.synchronize()
        wm = lambda i: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evw])) * 1e3
        fb0, bb0 = compose_bytes(T, out)
        in_step = {"norm_us": round(wm(0), 2), "compose_fwd_us": round(wm(1), 2), "compose_bwd_us": round(wm(2), 2),
                   "compose_gbs": round((fb0 + bb0) / ((wm(1) + wm(2)) * 1e-6) / 1e9, 1),
                   "compose_frac_hbm_peak": round((fb0 + bb0) / ((wm(1) + wm(2)) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                   "reps": args.in_step_reps}

    def timed(call, reps, cold=True):
        """Median HIP-event time of ``call`` over ``reps`` calls after 3 warm-up
        calls, each call after an evicting read when ``cold``."""
        evl = []
        for k in range(3 + reps):
            if cold:
                flush()
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record()
            call()
            a1.record()
            if k >= 3:
                evl.append((a0, a1))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in evl])) * 1e3

    # The norm with its base term cached (W0 is frozen): the row square norms
    # once, then the factored norm that takes them, timed in the step's place
    # (before the compose forward and backward) so the caches hold what they do
    # in the step.
    cached = None
    if args.cached_reps > 0:
        sq = torch.empty(out, dtype=torch.float32, device=dev)
        sq_us = timed(lambda: binding.dora_row_sqnorm(W0, sq_out=sq), args.cached_reps)
        n_c = torch.empty_like(norm)
        nc_us = timed(lambda: binding.dora_norm_factored_cached(W0, A, B, sq, s, norm_out=n_c, workspace=ws_norm),
                      args.cached_reps)
        cached = {"norm_us": round(nc_us, 2), "row_sqnorm_us": round(sq_us, 2),
                  "max_rel_vs_norm": float(((n_c - norm).abs() / norm).max().item()),
                  "reps": args.cached_reps}
        del sq, n_c

    # The compose forward with lora = h B^T formed inside the kernel, against the
    # unfused pair it replaces (torch's lora GEMM h B^T, then the compose
    # forward), each timed over the same number of calls.
    fused = None
    if args.fused_reps > 0:
        y2 = torch.empty_like(base)
        lora2 = torch.empty_like(base)

        R = args.fused_reps
        f_us = timed(lambda: binding.dora_lora_compose_fwd(base, h, B, mag, norm, s, y=y2), R)
        g_us = timed(lambda: torch.mm(h, B.t(), out=lora2), R)
        u_us = timed(lambda: (torch.mm(h, B.t(), out=lora2), binding.dora_compose_fwd(base, lora2, mag, norm, s, y=y2)),
                     R)
        fb = 2 * 2 * T * out + 2 * (T * r + out * r) + 8 * out
        ff = 2.0 * T * out * r
        fused = {"fused_us": round(f_us, 2), "unfused_us": round(u_us, 2), "lora_gemm_us": round(g_us, 2),
                 "algorithmic_bytes": fb, "flops": ff,
                 "fused_gbs": round(fb / (f_us * 1e-6) / 1e9, 1),
                 "fused_frac_hbm_peak": round(fb / (f_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                 "fused_tflops": round(ff / (f_us * 1e-6) / 1e12, 1),
                 "reps": args.fused_reps}
        # Its backward: d_base, d_B = g s (dy^T h) and d_mag in one pass over dy
        # and base, against the unfused backward (the compose backward reading a
        # stored lora and writing d_lora, then torch's GEMM d_B = d_lora^T h).
        db2, dB2, dm2 = torch.empty_like(base), torch.empty_like(B), torch.empty_like(mag)
        dl2 = torch.empty_like(base)
        ws_lb = torch.empty(max(binding.dora_lora_compose_bwd_workspace_bytes(T, out, r), 1), dtype=torch.uint8,
                            device=dev)
        torch.mm(h, B.t(), out=lora2)
        fbw_us = timed(lambda: binding.dora_lora_compose_bwd(dy, base, h, B, mag, norm, s, d_base=db2, d_B=dB2,
                                                             d_mag=dm2, workspace=ws_lb), R)
        ubw_us = timed(lambda: (binding.dora_compose_bwd(dy, base, lora2, mag, norm, s, d_lora=dl2, d_base=db2,
                                                         d_mag=dm2, workspace=ws_bwd),
                                torch.mm(dl2.t(), h, out=dB2)), R)
        bb = 3 * 2 * T * out + 2 * (T * r + 2 * out * r) + 12 * out
        fused["bwd"] = {"fused_us": round(fbw_us, 2), "unfused_us": round(ubw_us, 2), "algorithmic_bytes": bb,
                        "flops": ff, "fused_gbs": round(bb / (fbw_us * 1e-6) / 1e9, 1),
                        "fused_frac_hbm_peak": round(bb / (fbw_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                        "fused_tflops": round(ff / (fbw_us * 1e-6) / 1e12, 1)}
        del y2, lora2, db2, dB2, dm2, dl2, ws_lb

    # The weight-norm backward for a non-detached norm (d_A, d_B from dL/dn),
    # against the dense form in torch bf16 that forms V = W0 + s B A:
    # dV = (dn / n) V, d_B = s dV A^T, d_A = s B^T dV.
    norm_bwd = None
    if args.norm_bwd_reps > 0:
        d_norm = (-(mag / norm) * d_mag).contiguous()  # dL/dn of the DoRA layer: -g d_mag
        dA_o, dB_o = torch.empty_like(A), torch.empty_like(B)
        ws_nb = torch.empty(max(binding.dora_norm_bwd_workspace_bytes(out, in_, r), 1), dtype=torch.uint8,
                            device=dev)

        nb_us = timed(lambda: binding.dora_norm_bwd(W0, A, B, norm, d_norm, s, d_A=dA_o, d_B=dB_o,
                                                      workspace=ws_nb), args.norm_bwd_reps)
        cB = (d_norm / norm).to(torch.bfloat16)

        def dense():
            V = torch.addmm(W0, B, A, alpha=s)
            dV = V * cB[:, None]
            return torch.mm(dV, A.t()) * s, torch.mm(B.t().contiguous(), dV) * s

        dn_us = timed(dense, args.norm_bwd_reps)
        nbf = 4.0 * out * in_ * r + 4.0 * r * r * in_ + 4.0 * out * r * r
        nbb = 2 * (out * in_ + 2 * r * in_ + 2 * out * r) + 8 * out
        norm_bwd = {"us": round(nb_us, 2), "dense_torch_us": round(dn_us, 2), "algorithmic_flops": nbf,
                    "algorithmic_bytes": nbb, "tflops": round(nbf / (nb_us * 1e-6) / 1e12, 1),
                    "frac_mfma_peak": round(nbf / (nb_us * 1e-6) / 2.5e15, 4),
                    "workspace_bytes": int(ws_nb.numel()), "dense_transient_bytes": 2 * 2 * out * in_,
                    "reps": args.norm_bwd_reps}
        del dA_o, dB_o, ws_nb

    # The same compose forward + backward driven through the PyTorch custom
    # operator and autograd (dora_amd::compose), against the direct calls above.
    torch_us = None
    if args.torch_reps > 0:
        from dora_fine_tuning_amd import torch_ops

        bg, lg, mg = base.detach().requires_grad_(), lora.detach().requires_grad_(), mag.detach().requires_grad_()
        def fwd_bwd():
            bg.grad = lg.grad = mg.grad = None
            torch_ops.compose(bg, lg, mg, norm, s, False).backward(dy)

        torch_us = timed(fwd_bwd, args.torch_reps)
        del bg, lg, mg

    fwd_b, bwd_b = compose_bytes(T, out)
    comp_ms = fwd_ms.mean() + bwd_ms.mean()
    value = (fwd_b + bwd_b) / (comp_ms * 1e-3) / 1e9
    nb, nf = norm_work(out, in_, r)
    bwd_gbs = bwd_b / (bwd_ms.mean() * 1e-3) / 1e9
    traffic = kernel_traffic(bwd_b)

    res = {
        "metric": "DoRA compose fwd+bwd GB/s (% HBM peak); factored-norm us at 8192^2 r=384",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"DoRA module out=8192 in=8192 r=384 T=8192 tokens, bf16, s=32/sqrt(r)",
                   "out": out, "in": in_, "r": r, "T": T},
        "compose_frac_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "timing": "each kernel call after a 1 GiB cache-evicting read (cold); HIP events bracket the call alone; "
                  "ms_per_step includes the three evicting reads of a step",
        "norm_us": round(float(norm_ms.mean()) * 1e3, 2),
        "norm_tflops": round(nf / (norm_ms.mean() * 1e-3) / 1e12, 1),
        "norm_frac_mfma_peak": round(nf / (norm_ms.mean() * 1e-3) / 2.5e15, 4),
        # the factored norm's scratch against its O(out r + r^2) bound and the dense fp32 transient it avoids
        "norm_workspace": {"bytes": ws_norm.numel(), "bound_bytes": 4 * (out * r + r * r) + 64 * out,
                           "dense_fp32_bytes": 4 * out * in_},
        "compose_bwd_workspace_bytes": ws_bwd.numel(),
        "norm_cached_base": cached,
        "lora_fused_fwd": fused,
        "norm_bwd": norm_bwd,
        "compose_fwd_us": round(float(fwd_ms.mean()) * 1e3, 2),
        "compose_bwd_us": round(float(bwd_ms.mean()) * 1e3, 2),
        "in_step": in_step,
        "torch_compose": ({"fwd_bwd_us": round(torch_us, 2),
                           "direct_fwd_bwd_us": round(float(fwd_ms.mean() + bwd_ms.mean()) * 1e3, 2),
                           "reps": args.torch_reps} if torch_us is not None else None),
        "roofline": {
            "kernel": "dora_compose_bwd (compose_bwd_vec + dmag_finalize)",
            "bound": "hbm",
            "achieved": round(bwd_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(bwd_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": bwd_b,
            "avg_launch_us": round(float(bwd_ms.mean()) * 1e3, 2),
            "launch": "cold",
        },
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, W0c, Ac, Bc, base, lora, dy, args.cpu_chunk_tokens, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
