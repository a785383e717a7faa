// C ABI of the DoRA hot path: argument validation, workspace queries, launch
// selection (16-byte fast path or general path) and the per-thread error string.
// Every check runs before the first HIP call, so invalid calls touch no device.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "../../include/dora.h"
#include "compose_kernels.hpp"
#include "lora_compose_kernels.hpp"
#include "noalloc_kernels.hpp"
#include "norm_bwd_kernels.hpp"
#include "norm_kernels.hpp"

#ifndef DORA_VERSION_STRING
#define DORA_VERSION_STRING "0.1.0"
#endif

namespace {

thread_local std::string g_err;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return status;
}

int ok() {
  g_err.clear();
  return DORA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(DORA_HIP_ERROR, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Two byte ranges [p, p + n) and [q, q + m) that overlap without being the same buffer.
bool partial_overlap(const void* p, size_t n, const void* q, size_t m) {
  if (!p || !q || n == 0 || m == 0) return false;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  if (a == b && n == m) return false;
  return a < b + m && b < a + n;
}

bool any_overlap(const void* p, size_t n, const void* q, size_t m) {
  if (!p || !q || n == 0 || m == 0) return false;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + m && b < a + n;
}

bool valid_dtype(int dtype) { return dtype == DORA_BF16 || dtype == DORA_F16; }

// Longest serial chain (T * r products per thread) the slow path of
// dora_lora_compose_bwd is allowed to run.
constexpr int64_t kLoraBwdGeneralMaxSerial = int64_t(1) << 20;

// Validation and launch shared by the two norm entry points (base_sq: the
// cached base term, or NULL to compute it).
int norm_call(const char* fn, const void* W0, const void* A, const void* B, const float* base_sq, int64_t out,
              int64_t in, int64_t r, float s, int dtype, float* norm_out, void* ws, size_t ws_bytes,
              hipStream_t stream) {
  if (!valid_dtype(dtype)) return fail(DORA_UNSUPPORTED, "%s: unknown dtype %d", fn, dtype);
  if (out < 0 || in < 0 || r < 0)
    return fail(DORA_INVALID_ARG, "%s: negative size (out=%lld in=%lld r=%lld)", fn, (long long)out, (long long)in,
                (long long)r);
  if (out == 0) return ok();
  if (!norm_out) return fail(DORA_INVALID_ARG, "%s: norm_out is NULL", fn);
  if (in > 0 && !W0) return fail(DORA_INVALID_ARG, "%s: W0 is NULL", fn);
  if (r > 0 && in > 0 && !A) return fail(DORA_INVALID_ARG, "%s: A is NULL", fn);
  if (r > 0 && !B) return fail(DORA_INVALID_ARG, "%s: B is NULL", fn);
  const size_t need = dora::norm_workspace_bytes(out, in, r, dtype);
  if (ws_bytes < need) return fail(DORA_INVALID_ARG, "%s: workspace of %zu bytes, %zu needed", fn, ws_bytes, need);
  if (need > 0 && !ws) return fail(DORA_INVALID_ARG, "%s: workspace is NULL", fn);
  const size_t e = 2;
  const size_t nb = static_cast<size_t>(out) * 4;
  if (any_overlap(norm_out, nb, ws, need) || any_overlap(norm_out, nb, W0, out * in * e) ||
      any_overlap(norm_out, nb, B, out * r * e) || any_overlap(norm_out, nb, A, r * in * e))
    return fail(DORA_INVALID_ARG, "%s: norm_out overlaps an input or the workspace", fn);
  if (any_overlap(ws, need, W0, out * in * e) || any_overlap(ws, need, A, r * in * e) ||
      any_overlap(ws, need, B, out * r * e))
    return fail(DORA_INVALID_ARG, "%s: workspace overlaps an input", fn);
  if (base_sq && (any_overlap(base_sq, nb, norm_out, nb) || any_overlap(base_sq, nb, ws, need)))
    return fail(DORA_INVALID_ARG, "%s: base_sq overlaps norm_out or the workspace", fn);
  // 16-byte path: 16-byte rows and pointers, and buffer byte offsets below
  // 2^31 within a panel of at most 512 rows of in (< 2^21) or r elements
  const bool vec = (in % 8 == 0) && (r % 8 == 0) && aligned16(W0) && aligned16(A) && aligned16(B) &&
                   aligned16(ws) && in < (int64_t(1) << 21) && r <= (int64_t(1) << 20);
  const dora::NormPlan plan = dora::make_norm_plan(out, in, r, dtype, vec);
  if (dora::norm_max_grid(plan) > INT32_MAX)
    return fail(DORA_UNSUPPORTED, "%s: out=%lld r=%lld needs more workgroups than one launch holds", fn,
                (long long)out, (long long)r);
  dora::NormArgs a{W0, A, B, s, norm_out, ws, stream, base_sq};
  return hip_status(dora::launch_norm(plan, a), fn);
}

// Validation and launch shared by the compose backward entry points (ws: the
// caller's workspace, or the library's own scratch for the no-allocation one).
int compose_bwd_call(const char* fn, const void* dy, const void* base, const void* lora, const float* mag, const float* norm, float s,
                     int64_t T, int64_t out, int dtype, int add_base, void* d_lora, void* d_base, float* d_mag,
                     void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!valid_dtype(dtype)) return fail(DORA_UNSUPPORTED, "%s: unknown dtype %d", fn, dtype);
  if (T < 0 || out < 0)
    return fail(DORA_INVALID_ARG, "%s: negative size (T=%lld out=%lld)", fn, (long long)T, (long long)out);
  if (out == 0) return ok();
  if (!norm || !d_mag) return fail(DORA_INVALID_ARG, "%s: norm or d_mag is NULL", fn);
  if (T > 0 && (!dy || !base || !lora || !mag || !d_lora))
    return fail(DORA_INVALID_ARG, "%s: NULL pointer argument", fn);
  const size_t need = dora_compose_bwd_workspace_bytes(T, out);
  if (ws_bytes < need) return fail(DORA_INVALID_ARG, "%s: workspace of %zu bytes, %zu needed", fn, ws_bytes, need);
  if (need > 0 && !ws) return fail(DORA_INVALID_ARG, "%s: workspace is NULL", fn);
  const size_t mb = static_cast<size_t>(T) * out * 2, vb = static_cast<size_t>(out) * 4;
  if (any_overlap(d_lora, mb, d_base, mb)) return fail(DORA_INVALID_ARG, "%s: d_lora and d_base overlap", fn);
  const void* ins[3] = {dy, base, lora};
  for (const void* p : ins) {
    if (partial_overlap(d_lora, mb, p, mb) || partial_overlap(d_base, mb, p, mb))
      return fail(DORA_INVALID_ARG, "%s: an output partially overlaps an input", fn);
    if (any_overlap(ws, need, p, mb)) return fail(DORA_INVALID_ARG, "%s: workspace overlaps an input", fn);
  }
  if (any_overlap(ws, need, d_lora, mb) || any_overlap(ws, need, d_base, mb) || any_overlap(ws, need, d_mag, vb) ||
      any_overlap(ws, need, norm, vb) || any_overlap(ws, need, mag, vb))
    return fail(DORA_INVALID_ARG, "%s: workspace overlaps an argument", fn);
  if (any_overlap(d_mag, vb, d_lora, mb) || any_overlap(d_mag, vb, d_base, mb) || any_overlap(d_mag, vb, dy, mb) ||
      any_overlap(d_mag, vb, base, mb) || any_overlap(d_mag, vb, lora, mb) || partial_overlap(d_mag, vb, norm, vb) ||
      partial_overlap(d_mag, vb, mag, vb))
    return fail(DORA_INVALID_ARG, "%s: d_mag overlaps another argument", fn);
  dora::ComposeArgs a{};
  a.dtype = dtype;
  a.T = T;
  a.out = out;
  a.s = s;
  a.add_base = add_base ? 1 : 0;
  a.mag = mag;
  a.norm = norm;
  a.dy = dy;
  a.base = base;
  a.lora = lora;
  a.d_lora = d_lora;
  a.d_base = d_base;
  a.d_mag = d_mag;
  a.partial = static_cast<float*>(ws);
  a.stream = stream;
  const bool vec = (out % 8 == 0) && aligned16(dy) && aligned16(base) && aligned16(lora) && aligned16(d_lora) &&
                   (d_base == nullptr || aligned16(d_base)) && aligned16(mag) && aligned16(norm) && aligned16(ws);
  if (dora::compose_max_grid(T, out, vec) > INT32_MAX)
    return fail(DORA_UNSUPPORTED, "%s: T=%lld x out=%lld needs more workgroups than one launch holds", fn,
                (long long)T, (long long)out);
  return hip_status(dora::launch_compose_bwd(a, vec), fn);
}

}  // namespace

extern "C" {

const char* dora_last_error(void) { return g_err.c_str(); }

const char* dora_version(void) { return "dora_fine_tuning_amd " DORA_VERSION_STRING " (HIP, gfx950)"; }

size_t dora_norm_workspace_bytes(int64_t out, int64_t in, int64_t r, int dtype) {
  if (out < 0 || in < 0 || r < 0 || !valid_dtype(dtype)) return 0;
  return dora::norm_workspace_bytes(out, in, r, dtype);
}

int dora_norm_factored(const void* W0, const void* A, const void* B, int64_t out, int64_t in, int64_t r, float s,
                       int dtype, float* norm_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  return norm_call("dora_norm_factored", W0, A, B, nullptr, out, in, r, s, dtype, norm_out, ws, ws_bytes, stream);
}

int dora_norm_factored_cached(const void* W0, const void* A, const void* B, const float* base_sq, int64_t out,
                              int64_t in, int64_t r, float s, int dtype, float* norm_out, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  if (out > 0 && !base_sq) return fail(DORA_INVALID_ARG, "dora_norm_factored_cached: base_sq is NULL");
  return norm_call("dora_norm_factored_cached", W0, A, B, base_sq, out, in, r, s, dtype, norm_out, ws, ws_bytes,
                   stream);
}

int dora_row_sqnorm(const void* W0, int64_t out, int64_t in, int dtype, float* sq_out, hipStream_t stream) {
  if (!valid_dtype(dtype)) return fail(DORA_UNSUPPORTED, "dora_row_sqnorm: unknown dtype %d", dtype);
  if (out < 0 || in < 0)
    return fail(DORA_INVALID_ARG, "dora_row_sqnorm: negative size (out=%lld in=%lld)", (long long)out, (long long)in);
  if (out == 0) return ok();
  if (!sq_out) return fail(DORA_INVALID_ARG, "dora_row_sqnorm: sq_out is NULL");
  if (in > 0 && !W0) return fail(DORA_INVALID_ARG, "dora_row_sqnorm: W0 is NULL");
  if (any_overlap(sq_out, static_cast<size_t>(out) * 4, W0, static_cast<size_t>(out) * in * 2))
    return fail(DORA_INVALID_ARG, "dora_row_sqnorm: sq_out overlaps W0");
  if ((out + 3) / 4 > INT32_MAX)
    return fail(DORA_UNSUPPORTED, "dora_row_sqnorm: out=%lld needs more workgroups than one launch holds",
                (long long)out);
  const bool vec = (in % 8 == 0) && aligned16(W0);
  return hip_status(dora::launch_row_sqnorm(W0, out, in, dtype, vec, sq_out, stream), "dora_row_sqnorm");
}

int dora_compose_fwd(const void* base, const void* lora, const float* mag, const float* norm, float s, int64_t T,
                     int64_t out, int dtype, int add_base, void* y, hipStream_t stream) {
  if (!valid_dtype(dtype)) return fail(DORA_UNSUPPORTED, "dora_compose_fwd: unknown dtype %d", dtype);
  if (T < 0 || out < 0)
    return fail(DORA_INVALID_ARG, "dora_compose_fwd: negative size (T=%lld out=%lld)", (long long)T, (long long)out);
  if (T == 0 || out == 0) return ok();
  if (!base || !lora || !mag || !norm || !y) return fail(DORA_INVALID_ARG, "dora_compose_fwd: NULL pointer argument");
  const size_t mb = static_cast<size_t>(T) * out * 2, vb = static_cast<size_t>(out) * 4;
  if (partial_overlap(y, mb, base, mb) || partial_overlap(y, mb, lora, mb))
    return fail(DORA_INVALID_ARG, "dora_compose_fwd: y partially overlaps base or lora");
  if (any_overlap(y, mb, mag, vb) || any_overlap(y, mb, norm, vb))
    return fail(DORA_INVALID_ARG, "dora_compose_fwd: y overlaps mag or norm");
  dora::ComposeArgs a{};
  a.dtype = dtype;
  a.T = T;
  a.out = out;
  a.s = s;
  a.add_base = add_base ? 1 : 0;
  a.mag = mag;
  a.norm = norm;
  a.base = base;
  a.lora = lora;
  a.y = y;
  a.stream = stream;
  const bool vec = (out % 8 == 0) && aligned16(base) && aligned16(lora) && aligned16(y) && aligned16(mag) &&
                   aligned16(norm);
  if (dora::compose_max_grid(T, out, vec) > INT32_MAX)
    return fail(DORA_UNSUPPORTED, "dora_compose_fwd: T=%lld x out=%lld needs more workgroups than one launch holds",
                (long long)T, (long long)out);
  return hip_status(dora::launch_compose_fwd(a, vec), "dora_compose_fwd");
}

int dora_lora_compose_fwd(const void* base, const void* h, const void* B, const float* mag, const float* norm, float s,
                          int64_t T, int64_t out, int64_t r, int dtype, int add_base, void* y, hipStream_t stream) {
  const char* fn = "dora_lora_compose_fwd";
  if (!valid_dtype(dtype)) return fail(DORA_UNSUPPORTED, "%s: unknown dtype %d", fn, dtype);
  if (T < 0 || out < 0 || r < 0)
    return fail(DORA_INVALID_ARG, "%s: negative size (T=%lld out=%lld r=%lld)", fn, (long long)T, (long long)out,
                (long long)r);
  if (T == 0 || out == 0) return ok();
  if (!base || !mag || !norm || !y) return fail(DORA_INVALID_ARG, "%s: NULL pointer argument", fn);
  if (r > 0 && (!h || !B)) return fail(DORA_INVALID_ARG, "%s: h or B is NULL", fn);
  const size_t mb = static_cast<size_t>(T) * out * 2, vb = static_cast<size_t>(out) * 4;
  const size_t hb = static_cast<size_t>(T) * r * 2, bb = static_cast<size_t>(out) * r * 2;
  if (partial_overlap(y, mb, base, mb)) return fail(DORA_INVALID_ARG, "%s: y partially overlaps base", fn);
  if (any_overlap(y, mb, h, hb) || any_overlap(y, mb, B, bb) || any_overlap(y, mb, mag, vb) ||
      any_overlap(y, mb, norm, vb))
    return fail(DORA_INVALID_ARG, "%s: y overlaps h, B, mag or norm", fn);
  const bool vec = (out % 8 == 0) && out < (int64_t(1) << 22) && (r % 8 == 0) && r <= (int64_t(1) << 20) &&
                   aligned16(base) && (r == 0 || (aligned16(h) && aligned16(B))) && aligned16(mag) &&
                   aligned16(norm) && aligned16(y);
  if (dora::lora_fwd_max_grid(T, out, vec) > INT32_MAX)
    return fail(DORA_UNSUPPORTED, "%s: T=%lld x out=%lld needs more workgroups than one launch holds", fn,
                (long long)T, (long long)out);
  dora::LoraFwdArgs a{dtype, T, out, r, s, add_base ? 1 : 0, base, h, B, mag, norm, y, stream};
  return hip_status(dora::launch_lora_fwd(a, vec), fn);
}

size_t dora_lora_compose_bwd_workspace_bytes(int64_t T, int64_t out, int64_t r) {
  if (T <= 0 || out <= 0 || r < 0) return 0;
  return dora::lora_bwd_workspace_bytes(T, out, r);
}

int dora_lora_compose_bwd(const void* dy, const void* base, const void* h, const void* B, const float* mag,
                          const float* norm, float s, int64_t T, int64_t out, int64_t r, int dtype, int add_base,
                          void* d_base, void* d_B, float* d_mag, void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* fn = "dora_lora_compose_bwd";
  if (!valid_dtype(dtype)) return fail(DORA_UNSUPPORTED, "%s: unknown dtype %d", fn, dtype);
  if (T < 0 || out < 0 || r < 0)
    return fail(DORA_INVALID_ARG, "%s: negative size (T=%lld out=%lld r=%lld)", fn, (long long)T, (long long)out,
                (long long)r);
  if (out == 0) return ok();
  if (!mag || !norm || !d_mag) return fail(DORA_INVALID_ARG, "%s: mag, norm or d_mag is NULL", fn);
  if (T > 0 && (!dy || !base)) return fail(DORA_INVALID_ARG, "%s: dy or base is NULL", fn);
  if (r > 0 && (!B || !d_B)) return fail(DORA_INVALID_ARG, "%s: B or d_B is NULL", fn);
  if (T > 0 && r > 0 && !h) return fail(DORA_INVALID_ARG, "%s: h is NULL", fn);
  const size_t mb = static_cast<size_t>(T) * out * 2, vb = static_cast<size_t>(out) * 4;
  const size_t hb = static_cast<size_t>(T) * r * 2, bb = static_cast<size_t>(out) * r * 2;
  const void* ins[6] = {dy, base, h, B, mag, norm};
  const size_t insz[6] = {mb, mb, hb, bb, vb, vb};
  const void* outs[3] = {d_base, d_B, d_mag};
  const size_t outsz[3] = {mb, bb, vb};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 6; ++i)
      if (any_overlap(outs[o], outsz[o], ins[i], insz[i]))
        return fail(DORA_INVALID_ARG, "%s: an output overlaps an input", fn);
    for (int q = o + 1; q < 3; ++q)
      if (any_overlap(outs[o], outsz[o], outs[q], outsz[q])) return fail(DORA_INVALID_ARG, "%s: outputs overlap", fn);
  }
  const bool vec = T >= 1 && (out % 8 == 0) && (r % 8 == 0) && r >= 8 && r <= (int64_t(1) << 20) && aligned16(dy) &&
                   aligned16(base) && aligned16(h) && aligned16(B) && (d_base == nullptr || aligned16(d_base)) &&
                   aligned16(d_B) && aligned16(mag) && aligned16(norm) && aligned16(ws);
  if (vec) {
    const size_t need = dora::lora_bwd_workspace_bytes(T, out, r);
    if (ws_bytes < need) return fail(DORA_INVALID_ARG, "%s: workspace of %zu bytes, %zu needed", fn, ws_bytes, need);
    if (!ws) return fail(DORA_INVALID_ARG, "%s: workspace is NULL", fn);
    for (int i = 0; i < 6; ++i)
      if (any_overlap(ws, need, ins[i], insz[i])) return fail(DORA_INVALID_ARG, "%s: workspace overlaps an input", fn);
    for (int o = 0; o < 3; ++o)
      if (any_overlap(ws, need, outs[o], outsz[o]))
        return fail(DORA_INVALID_ARG, "%s: workspace overlaps an output", fn);
    if (dora::lora_bwd_max_slice_bytes(T, out, r) >= (int64_t(1) << 31))
      return fail(DORA_UNSUPPORTED, "%s: T=%lld out=%lld r=%lld: a token slice spans 2 GiB or more", fn,
                  (long long)T, (long long)out, (long long)r);
  }
  // The slow path gives each output column to one thread, which walks all T x r
  // products of its d_B row in order: refuse shapes where that serial chain
  // would be long (a cliff of orders of magnitude against the fast path), so
  // the caller can take another route (the PyTorch layer's eager tier).
  if (!vec && T * r > kLoraBwdGeneralMaxSerial)
    return fail(DORA_UNSUPPORTED,
                "%s: T=%lld out=%lld r=%lld misses the fast path (out and r multiples of 8, 8 <= r, 16-byte aligned "
                "pointers and workspace) and T*r exceeds the slow path's limit of %lld",
                fn, (long long)T, (long long)out, (long long)r, (long long)kLoraBwdGeneralMaxSerial);
  if (dora::lora_bwd_max_grid(T, out, r, vec) > INT32_MAX)
    return fail(DORA_UNSUPPORTED, "%s: out=%lld needs more workgroups than one launch holds", fn, (long long)out);
  dora::LoraBwdArgs a{dtype, T, out, r, s, add_base ? 1 : 0, dy, base, h, B, mag, norm, d_base, d_B, d_mag, ws, stream};
  return hip_status(dora::launch_lora_bwd(a, vec), fn);
}

size_t dora_norm_bwd_workspace_bytes(int64_t out, int64_t in, int64_t r, int dtype) {
  if (out < 0 || in < 0 || r < 0 || !valid_dtype(dtype)) return 0;
  return dora::norm_bwd_workspace_bytes(out, in, r, dtype);
}

int dora_norm_bwd(const void* W0, const void* A, const void* B, const float* norm, const float* d_norm, int64_t out,
                  int64_t in, int64_t r, float s, int dtype, void* d_A, void* d_B, void* ws, size_t ws_bytes,
                  hipStream_t stream) {
  const char* fn = "dora_norm_bwd";
  if (!valid_dtype(dtype)) return fail(DORA_UNSUPPORTED, "%s: unknown dtype %d", fn, dtype);
  if (out < 0 || in < 0 || r < 0)
    return fail(DORA_INVALID_ARG, "%s: negative size (out=%lld in=%lld r=%lld)", fn, (long long)out, (long long)in,
                (long long)r);
  if (r == 0) return ok();
  if (in > 0 && (!A || !d_A)) return fail(DORA_INVALID_ARG, "%s: A or d_A is NULL", fn);
  if (out > 0 && (!B || !d_B || !norm || !d_norm)) return fail(DORA_INVALID_ARG, "%s: B, d_B, norm or d_norm is NULL", fn);
  if (out > 0 && in > 0 && !W0) return fail(DORA_INVALID_ARG, "%s: W0 is NULL", fn);
  const bool vec = in % 8 == 0 && r % 8 == 0 && in < (int64_t(1) << 21) && r <= (int64_t(1) << 20) &&
                   aligned16(W0) && aligned16(A) && aligned16(B) && aligned16(d_A) && aligned16(d_B) &&
                   aligned16(ws);
  const dora::NormBwdPlan plan = dora::make_norm_bwd_plan(out, in, r, dtype, vec);
  const size_t need = plan.bytes;
  if (ws_bytes < need) return fail(DORA_INVALID_ARG, "%s: workspace of %zu bytes, %zu needed", fn, ws_bytes, need);
  if (need > 0 && !ws) return fail(DORA_INVALID_ARG, "%s: workspace is NULL", fn);
  const size_t e = 2, vb = static_cast<size_t>(out) * 4;
  const void* ins[5] = {W0, A, B, norm, d_norm};
  const size_t insz[5] = {out * in * e, r * in * e, out * r * e, vb, vb};
  const void* outs[3] = {d_A, d_B, ws};
  const size_t outsz[3] = {r * in * e, out * r * e, need};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 5; ++i)
      if (any_overlap(outs[o], outsz[o], ins[i], insz[i]))
        return fail(DORA_INVALID_ARG, "%s: an output or the workspace overlaps an input", fn);
    for (int q = o + 1; q < 3; ++q)
      if (any_overlap(outs[o], outsz[o], outs[q], outsz[q]))
        return fail(DORA_INVALID_ARG, "%s: outputs or the workspace overlap", fn);
  }
  if (plan.max_grid > INT32_MAX)
    return fail(DORA_UNSUPPORTED, "%s: out=%lld in=%lld r=%lld needs more workgroups than one launch holds", fn,
                (long long)out, (long long)in, (long long)r);
  if (plan.max_slice_bytes >= (int64_t(1) << 31))
    return fail(DORA_UNSUPPORTED, "%s: out=%lld in=%lld r=%lld: a row slice spans 2 GiB or more", fn, (long long)out,
                (long long)in, (long long)r);
  dora::NormBwdArgs a{dtype, W0, A, B, norm, d_norm, s, d_A, d_B, ws, stream};
  return hip_status(dora::launch_norm_bwd(plan, a), fn);
}

size_t dora_compose_bwd_workspace_bytes(int64_t T, int64_t out) {
  if (T <= 0 || out <= 0) return 0;
  return dora::compose_bwd_workspace(T, out);
}

int dora_compose_bwd(const void* dy, const void* base, const void* lora, const float* mag, const float* norm, float s,
                     int64_t T, int64_t out, int dtype, int add_base, void* d_lora, void* d_base, float* d_mag,
                     void* ws, size_t ws_bytes, hipStream_t stream) {
  return compose_bwd_call("dora_compose_bwd", dy, base, lora, mag, norm, s, T, out, dtype, add_base, d_lora, d_base,
                          d_mag, ws, ws_bytes, stream);
}

int dora_compose_bwd_noalloc(const void* dy, const void* base, const void* lora, const float* mag, const float* norm,
                             float s, int64_t T, int64_t out, int dtype, int add_base, void* d_lora, void* d_base,
                             float* d_mag, hipStream_t stream) {
  const char* fn = "dora_compose_bwd_noalloc";
  if (!valid_dtype(dtype)) return fail(DORA_UNSUPPORTED, "%s: unknown dtype %d", fn, dtype);
  if (T < 0 || out < 0)
    return fail(DORA_INVALID_ARG, "%s: negative size (T=%lld out=%lld)", fn, (long long)T, (long long)out);
  if (out == 0) return ok();
  const size_t need = dora_compose_bwd_workspace_bytes(T, out);
  if (need > dora::kNoAllocScratchBytes)
    return fail(DORA_UNSUPPORTED, "%s: T=%lld out=%lld needs %zu bytes of scratch, above this entry point's %zu; "
                "use dora_compose_bwd with a workspace", fn, (long long)T, (long long)out, need,
                dora::kNoAllocScratchBytes);
  void* scratch = nullptr;
  if (need > 0) {
    const hipError_t e = dora::noalloc_scratch(stream, &scratch);
    if (e != hipSuccess) return fail(DORA_HIP_ERROR, "%s: scratch address: %s", fn, hipGetErrorString(e));
  }
  return compose_bwd_call(fn, dy, base, lora, mag, norm, s, T, out, dtype, add_base, d_lora, d_base, d_mag, scratch,
                          need, stream);
}

}  // extern "C"
