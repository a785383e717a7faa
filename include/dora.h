/*
 * dora.h -- C ABI of the DoRA adapter hot path on AMD Instinct MI355X (gfx950).
 *
 * DoRA (weight-decomposed low-rank adaptation) scales each output row of the
 * adapted weight W0 + s*B*A by g = m / n, where m is a trained magnitude and
 * n = ||W0_i + s*B_i*A||_2 is the weight norm of that row.  This library
 * provides the three operations that the press summary of arXiv:2603.22276
 * ("AI training breakthrough: Anthropic team cracks the memory bottleneck of
 * large-model fine-tuning", techwalker.com/2026/0401/3182870) singles out:
 *
 *   dora_norm_factored  the weight norm as base + cross + Gram terms, never
 *                       forming the out x in matrix B*A (paragraph on the
 *                       "factored norm");
 *   dora_compose_fwd    the fused magnitude compose in its stable form
 *                       (g-1)*base + g*s*lora with fp32 intermediates
 *                       (paragraphs on the fused kernel and on stability near
 *                       g = 1; the forward-only inference tier);
 *   dora_compose_bwd    its fused backward with the magnitude-gradient token
 *                       reduction (paragraphs on the three-tier dispatch and on
 *                       the convergence study's dmag reduction).
 *
 * and the compose with the adapter's second projection fused in, so that lora
 * is never stored (the page's account of where the fused kernel's gains come
 * from: fewer memory accesses):
 *
 *   dora_lora_compose_fwd      y = (g-1)*base + g*s*(h*B^T), h = x*A^T;
 *   dora_lora_compose_bwd      its backward: d_base, d_B and d_mag from dy,
 *                              base and h, without lora or d_lora;
 *
 * for a caller that does not treat the norm as a constant:
 *
 *   dora_norm_bwd              d_A and d_B of the weight norm, from dL/dn,
 *                              without forming B*A;
 *
 * and, for the cached base norm the page lists as future work (W0 is frozen):
 *
 *   dora_row_sqnorm            ||W0_i||^2 per row, computed once;
 *   dora_norm_factored_cached  the weight norm with that cache as its base term.
 *
 * Conventions shared by every entry point
 *  - Matrices are row-major and contiguous.  W0 is [out x in], A is [r x in],
 *    B is [out x r] (nn.Linear orientation); base, lora, y, dy, d_lora and
 *    d_base are [T x out] (T tokens).  Vectors mag (m), norm (n) and d_mag are
 *    fp32 [out].
 *  - dtype selects the storage type of every matrix argument: DORA_BF16 or
 *    DORA_F16.  Arithmetic is fp32 throughout; each stored output is rounded
 *    once, to nearest even.
 *  - All data pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or synchronises: each call enqueues its kernels on
 *    `stream` and returns.  Scratch memory is passed in by the caller (size from
 *    the *_workspace_bytes queries), so no call makes a transient allocation.
 *  - Return value: DORA_OK, or a status below.  Arguments are validated before
 *    any launch; on a non-zero status nothing was enqueued (except
 *    DORA_HIP_ERROR, reported by the launch itself).  dora_last_error() gives
 *    the message of the calling thread's last failure.
 *  - Any sizes are accepted.  The fast paths need 16-byte aligned pointers and
 *    row lengths that are multiples of 8 elements (for the norm also
 *    in < 2^21); other cases take a slower general path with the same
 *    accuracy (its summation order differs, so results are not bitwise equal
 *    to the fast path's).
 *  - Results are deterministic: no floating-point atomics, fixed reduction
 *    orders, so repeated calls give bitwise identical outputs.
 */
#ifndef DORA_H_
#define DORA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifndef DORA_API
#define DORA_API __attribute__((visibility("default")))
#endif

#ifdef __cplusplus
extern "C" {
#endif

/*
 * DORA_UNSUPPORTED marks arguments that are valid but that this library does
 * not take; a caller can route such a call elsewhere (the page's eager tier):
 *  - an unknown dtype code;
 *  - sizes whose launch grid would exceed one grid dimension's limit;
 *  - on the fast paths of dora_lora_compose_bwd and dora_norm_bwd, a token or
 *    row slice that would span 2 GiB or more;
 *  - dora_lora_compose_bwd with a shape or pointers its fast path cannot take
 *    and T * r above 2^20 (its slow path runs T * r products in order in one
 *    thread per output column);
 *  - dora_compose_bwd_noalloc with sizes whose partials exceed its scratch.
 */
enum dora_status {
  DORA_OK = 0,
  DORA_INVALID_ARG = 1, /* null pointer, negative size, workspace too small, bad alias */
  DORA_UNSUPPORTED = 2, /* valid arguments this library does not take (listed above) */
  DORA_HIP_ERROR = 3    /* a kernel launch failed (message from the HIP runtime) */
};

enum dora_dtype { DORA_BF16 = 0, DORA_F16 = 1 };

/*
 * Bytes of device workspace dora_norm_factored needs for these sizes.
 * The scratch is O(out*r + r*r): split-K partial sums of G = A*A^T, the
 * two-term split of (s/2)*G in the storage dtype, and per-split row partials.
 * For every shape it stays within 4*(out*r + r*r) + 64*out bytes, region
 * alignment included (the factored norm's memory bound, paragraph on the
 * factored norm): where the Gram partials would not fit, one K split writes
 * the split of (s/2)*G directly.  Returns 0 for invalid sizes (negative) or an
 * unknown dtype.
 */
DORA_API size_t dora_norm_workspace_bytes(int64_t out, int64_t in, int64_t r, int dtype);

/*
 * norm_out[i] = || W0_i + s * B_i * A ||_2, i in [0, out), in fp32.
 *
 * Computed as sqrt(base_i + cross_i + gram_i) with
 *   base_i  = sum_k W0_ik^2,
 *   cross_i = 2 s * sum_j B_ij * U_ij,   U = W0 * A^T   [out x r],
 *   gram_i  = s^2 * B_i * G * B_i^T,     G = A * A^T    [r x r],
 * (summary page, paragraph on the factored norm).  U and G are dense MFMA
 * contractions with fp32 accumulation; U never leaves the registers.  A
 * negative sum from rounding is clamped to 0.  The norm is a plain value: the
 * backward of the compose treats it as a constant.  With in and r multiples of
 * 8, 16-byte aligned matrices, r <= 32 and out >= 4065 the call is a single
 * launch that forms G itself and leaves ws untouched; the workspace query
 * does not depend on this.
 *
 * W0, A, B: device, dtype.  A and B may be NULL when r == 0.  norm_out: device
 * fp32 [out].  ws: device scratch of at least dora_norm_workspace_bytes(...)
 * bytes, contents undefined on entry and exit; ws may be NULL when that size is
 * 0.  out == 0 is a no-op; in == 0 gives n = 0.
 */
DORA_API int dora_norm_factored(const void* W0, const void* A, const void* B, int64_t out, int64_t in,
                       int64_t r, float s, int dtype, float* norm_out, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/*
 * sq_out[i] = ||W0_i||^2 = sum_k W0_ik^2, i in [0, out), in fp32: the base term
 * of the weight norm on its own.  W0 is frozen during fine-tuning, so this is
 * the cache the summary page proposes as future work (paragraph on
 * limitations: cache the base norm); compute it once and pass it to
 * dora_norm_factored_cached.  One read of W0; squares accumulate in fp32
 * partial sums of at most ceil(in/256) + 1 terms, combined in fp64 and rounded
 * once.
 *
 * W0: device, dtype, [out x in].  sq_out: device fp32 [out], not overlapping
 * W0.  out == 0 is a no-op; in == 0 gives 0.
 */
DORA_API int dora_row_sqnorm(const void* W0, int64_t out, int64_t in, int dtype, float* sq_out,
                             hipStream_t stream);

/*
 * dora_norm_factored with the base term taken from a cache:
 *   norm_out[i] = sqrt(max(base_sq[i] + cross_i + gram_i, 0)),
 * cross_i and gram_i as in dora_norm_factored (summary page, paragraph on
 * limitations: the cached base norm).  With base_sq from dora_row_sqnorm on the
 * same W0 this is ||W0_i + s * B_i * A||_2; the pass over W0 for the cross term
 * then skips the squares.  Same arguments, workspace and errors as
 * dora_norm_factored, plus base_sq: device fp32 [out], not overlapping
 * norm_out or ws (NULL is INVALID_ARG unless out == 0).
 */
DORA_API int dora_norm_factored_cached(const void* W0, const void* A, const void* B, const float* base_sq,
                                       int64_t out, int64_t in, int64_t r, float s, int dtype, float* norm_out,
                                       void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * y = (g - 1) * base + g * s * lora, g_j = mag_j / norm_j broadcast over the T
 * rows (summary page, paragraph on stability near g = 1).  g - 1 is formed as
 * (mag - norm) / norm, whose subtraction is exact when mag/norm is in [1/2, 2],
 * so the base correction is nonzero wherever mag != norm and base != 0.  With
 * add_base != 0, y = base + that delta (the full layer output) in the same
 * pass.  One read of base and lora, one write of y.
 *
 * base, lora, y: device, dtype, [T x out].  mag, norm: device fp32 [out].
 * y may be the same buffer as base or lora (in place); no other overlap.
 * T == 0 or out == 0 is a no-op.  norm_j == 0 follows IEEE division.
 */
DORA_API int dora_compose_fwd(const void* base, const void* lora, const float* mag, const float* norm, float s,
                     int64_t T, int64_t out, int dtype, int add_base, void* y, hipStream_t stream);

/*
 * dora_compose_fwd with the adapter's second projection fused in:
 *   y = (g - 1) * base + g * s * (h * B^T)   (+ base when add_base != 0),
 * where h = x * A^T is the adapter's first projection [T x r] and B is
 * [out x r] (summary page: the fused kernel's gains come from fewer memory
 * accesses).  lora = h * B^T is accumulated in fp32 by MFMA and never stored:
 * one read of base, one write of y, and h and B read per tile (they are small).
 * g - 1 is formed as in dora_compose_fwd; one rounding per output.
 *
 * base, y: device, dtype, [T x out]; h: [T x r]; B: [out x r]; mag, norm:
 * device fp32 [out].  y may be the same buffer as base; no other overlap with
 * an input.  h and B may be NULL when r == 0 (then y is the compose of
 * lora = 0).  T == 0 or out == 0 is a no-op.  The fast path needs out and r
 * multiples of 8, out < 2^22, r <= 2^20 and 16-byte aligned pointers; other
 * cases take a slow path (one thread per output element).
 */
DORA_API int dora_lora_compose_fwd(const void* base, const void* h, const void* B, const float* mag,
                                   const float* norm, float s, int64_t T, int64_t out, int64_t r, int dtype,
                                   int add_base, void* y, hipStream_t stream);

/*
 * Bytes of device workspace dora_norm_bwd needs for these sizes (either
 * path): on the fast path the Gram scratch of the norm, c [out] fp32, the
 * hi/lo pair of s*c*B [out x 2r] and of an r x r product [r x 2r] in the
 * storage dtype, and one fp32 region of row-slice partials of size
 * O(out*r + in*r) reused by the steps in turn.
 * Returns 0 for negative sizes or an unknown dtype.
 */
DORA_API size_t dora_norm_bwd_workspace_bytes(int64_t out, int64_t in, int64_t r, int dtype);

/*
 * Backward of the weight norm n_i = ||W0_i + s * B_i * A||_2 for a caller
 * that does not treat n as a constant (the summary page's paragraph on the
 * factored norm gives its base, cross and Gram parts; the page does not say
 * whether n is differentiated, and dora_compose_bwd takes it as constant).
 * Given dL/dn = d_norm, with c_i = d_norm_i / norm_i (0 where norm_i == 0):
 *   d_B_i = s * c_i * (U_i + s * B_i * G),          U = W0 * A^T, G = A * A^T
 *   d_A   = s * (c .* B)^T * W0 + s^2 * (B^T * diag(c) * B) * A
 * which is s * B^T * dV and s * dV * A^T for dV = c .* (W0 + s * B * A), with
 * the out x in matrix B * A never formed.  W0 is frozen: it gets no gradient.
 * For the DoRA layer, L depends on n only through g = m / n, so
 * d_norm_j = -(m_j / n_j) * d_mag_j with d_mag from dora_compose_bwd.
 * U, G and the two contractions over the out rows run on MFMA with fp32
 * accumulation; the computed operands s*c*B and the r x r product enter them as
 * hi/lo pairs of the storage dtype.  Each output is rounded once.
 *
 * W0: device, dtype, [out x in]; A, d_A: [r x in]; B, d_B: [out x r]; norm
 * (the forward's n) and d_norm: device fp32 [out].  No output overlaps an
 * input, the other output or ws.  ws: at least dora_norm_bwd_workspace_bytes
 * bytes.  r == 0 is a no-op; out == 0 gives d_A = 0; in == 0 gives d_B = 0.
 * The fast path needs in and r multiples of 8, in < 2^21, r <= 2^20 and
 * 16-byte aligned matrix and workspace pointers; other cases take a slow
 * general path (one thread per output element, every sum in order in fp32,
 * no hi/lo operands).
 * In fp16 the fast path stores column j of s*c*B times a power of two
 * sigma_j that puts that column's largest magnitude in [1/2, 1) (sigma_j
 * within 2^-60 .. 2^60; two extra small launches), carries sigma_j on every
 * operand column that feeds row j of d_A, and divides it out of that row in
 * fp32, so a small d_norm, a small B or a single small column of B does not
 * push the operands into fp16's subnormal range.  Entries of the r x r product
 * s*B^T*(c*B) beyond fp16's range (65504) after that scaling still overflow.
 * bf16 has fp32's exponent range and takes sigma_j = 1.
 */
DORA_API int dora_norm_bwd(const void* W0, const void* A, const void* B, const float* norm, const float* d_norm,
                           int64_t out, int64_t in, int64_t r, float s, int dtype, void* d_A, void* d_B, void* ws,
                           size_t ws_bytes, hipStream_t stream);

/* Bytes of device workspace dora_lora_compose_bwd needs (fp32 slices of dy^T h and column partials). */
DORA_API size_t dora_lora_compose_bwd_workspace_bytes(int64_t T, int64_t out, int64_t r);

/*
 * Backward of dora_lora_compose_fwd for L = sum(dy * y), with norm held
 * constant, never forming lora or d_lora = g * s * dy:
 *   d_base = (g - 1) * dy         (add_base == 0)
 *          = g * dy               (add_base != 0)
 *   d_B    = (g * s * dy)^T h = g * s * (dy^T h)       [out x r]
 *   d_mag_j = (sum_t dy_tj * base_tj + s * sum_k B_jk (dy^T h)_jk) / norm_j,
 * which equals sum_t dy_tj * (base_tj + s * (h B^T)_tj) / norm_j (summary page:
 * the training tier's fused backward; gains from fewer memory accesses).
 * dy^T h is an MFMA contraction over the tokens with fp32 accumulation, its
 * token slices added in a fixed order; d_mag sums its partials in fp64.  The
 * gradient of h, d_lora * B = dy * (g * s * B), is the caller's GEMM.
 *
 * dy, base, d_base: device, dtype, [T x out]; d_base may be NULL (not
 * computed).  h: [T x r]; B, d_B: [out x r].  mag, norm, d_mag: device fp32
 * [out].  No output may overlap an input or another output.  ws: at least
 * dora_lora_compose_bwd_workspace_bytes(T, out, r) bytes on the fast path
 * (out and r multiples of 8, 8 <= r <= 2^20, T >= 1, 16-byte aligned
 * pointers); other cases take a slow path (one thread per output column) and
 * need no workspace; the slow path refuses (DORA_UNSUPPORTED) shapes with
 * T * r > 2^20.  out == 0 is a no-op; T == 0 gives d_B = 0 and d_mag = 0.
 */
DORA_API int dora_lora_compose_bwd(const void* dy, const void* base, const void* h, const void* B, const float* mag,
                                   const float* norm, float s, int64_t T, int64_t out, int64_t r, int dtype,
                                   int add_base, void* d_base, void* d_B, float* d_mag, void* ws, size_t ws_bytes,
                                   hipStream_t stream);

/* Bytes of device workspace dora_compose_bwd needs (per-token-block fp32 partial sums). */
DORA_API size_t dora_compose_bwd_workspace_bytes(int64_t T, int64_t out);

/*
 * Backward of dora_compose_fwd for L = sum(dy * y), with norm held constant:
 *   d_lora = g * s * dy
 *   d_base = (g - 1) * dy         (add_base == 0)
 *          = g * dy               (add_base != 0)
 *   d_mag_j = sum_t dy_tj * (base_tj + s * lora_tj) / norm_j
 * (summary page: fused backward of the training tier; the magnitude gradient is
 * a token reduction whose order may differ from an eager implementation).  The
 * reduction is fixed-order: fp32 partial sums over blocks of tokens, combined
 * in fp64 in a second kernel, so d_mag is bitwise reproducible.
 *
 * dy, base, lora, d_lora, d_base: device, dtype, [T x out]; d_base may be NULL
 * (not computed).  mag, norm, d_mag: device fp32 [out].  d_lora may be the same
 * buffer as dy or lora; d_base may be the same buffer as dy or base; d_lora
 * and d_base must differ.  ws: at least dora_compose_bwd_workspace_bytes(T,
 * out) bytes.  out == 0 is a no-op; T == 0 writes d_mag = 0 / norm.
 */
DORA_API int dora_compose_bwd(const void* dy, const void* base, const void* lora, const float* mag,
                     const float* norm, float s, int64_t T, int64_t out, int dtype, int add_base,
                     void* d_lora, void* d_base, float* d_mag, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/*
 * dora_compose_bwd for callers that cannot allocate device memory (code under
 * stream or graph capture, tight serving loops, harnesses that forbid
 * allocation): same arguments, results and errors, without the workspace.
 * The magnitude-gradient partials go to a scratch array of 24 MiB that the
 * library holds on each GPU it runs on from load until process exit; this
 * call allocates and frees nothing.  Sizes whose partials need more
 * (dora_compose_bwd_workspace_bytes(T, out) > 24 MiB) return DORA_UNSUPPORTED
 * before any launch.  Every call on a GPU shares that GPU's array, so calls
 * that overlap in time on one GPU (on different streams, or from different
 * threads) race on it: serialise them.  The array keeps the last call's
 * partials; each call overwrites every partial it reads.  The first call on a
 * device looks up the array's address there (hipGetSymbolAddress).
 */
DORA_API int dora_compose_bwd_noalloc(const void* dy, const void* base, const void* lora, const float* mag,
                                      const float* norm, float s, int64_t T, int64_t out, int dtype, int add_base,
                                      void* d_lora, void* d_base, float* d_mag, hipStream_t stream);

/* Message of the calling thread's last non-OK status ("" if none).  Valid until the next call. */
DORA_API const char* dora_last_error(void);

/* Library build string (version, target architecture). */
DORA_API const char* dora_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DORA_H_ */
