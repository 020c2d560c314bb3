/*
 * ptgq.h - per-token-group 8-bit activation quantization on MI355X (gfx950).
 *
 * C ABI of libptgq.so.  Plain pointers and sizes only.
 *
 * What the library computes (the method of the pages this library follows):
 *   for every row and every contiguous group of G elements of that row,
 *     amax  = max |y|                          (y = x, or silu(gate) * up)
 *     r     = max(amax, eps) / qmax            (qmax 448 for e4m3, 127 for int8;
 *                                               IEEE fp32 division)
 *     scale = r            (fp32 format)       multiplier inv = 1 / r (IEEE)
 *           | 2^ceil(log2 r) (UE8M0 format)    stored as the biased exponent byte
 *                                               e; multiplier 2^(127-e), exact
 *     code  = narrow(y * inv)                  round-to-nearest-even, saturated
 *                                               (e4m3: +-448; int8: [-128,127]);
 *                                               a negative value rounding to 0
 *                                               gives e4m3 code 0x80
 *   Sources: sglang #30924 review page, implementation breakdown (the trait
 *   set: in/out dtype, group size, fp32 or UE8M0 scale, row- or column-major
 *   scale, fused silu_and_mul, flat or masked schedule) and key source
 *   snippets (ref_fp8_ue8m0); sglang #27449 PR body, summary (group sizes,
 *   scale formats, fused silu+mul, masked scheduler); sglang #34257 review
 *   page, key source snippets (per-token kernel, reciprocal multiply,
 *   saturating narrowing); vllm #41326 review page, key source snippets
 *   (packed column-major UE8M0 words).
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *     library never allocates, frees or keeps a tensor; outputs are written in
 *     place.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *     asynchronous on that stream and never synchronize the host, so they may
 *     be captured into a HIP graph, the first call on a device included.  The
 *     fused calls large enough to read a SiLU lookup table (one for bf16
 *     gates, 32 KiB, one for fp16 gates, 144 KiB) build both tables on their
 *     own stream the first time (one small kernel, stream-ordered; other
 *     streams then wait for it on the device); a call captured before the
 *     tables exist evaluates SiLU directly instead (same results, slower).
 *     ptgq_init does that set-up ahead of time.
 *   - The library's only device memory of its own is those tables; no entry
 *     point allocates or frees memory.
 *   - Arguments are validated on the host before anything is launched.  A
 *     negative return value means nothing was launched and nothing written.
 *   - Sizes are int64.  A call with zero rows (M == 0, E == 0, or K == 0)
 *     returns PTGQ_OK and launches nothing.
 *   - Inputs must not alias outputs.  Concurrent calls writing the same
 *     outputs race, as any two kernels would.
 *   - NaN or infinite inputs give unspecified (but in-bounds) outputs.
 *   - When the fp32 multiplier 1 / r overflows to +inf (a scale r below about
 *     2^-128: a per-token row, or a group with fp32 scales and eps below
 *     ~1.3e-36, whose largest magnitude is below ~1.3e-36, normal values
 *     included), a zero element gives the zero code of its sign and every
 *     other element saturates; the same holds for a zero product in
 *     ptgq_requant_fp8.  (The pages leave this corner open; the quotient
 *     y / r of a zero is zero.)
 *
 * Scale tensor layouts (ng = K / G groups per row, rows_pad = ceil(rows/4)*4):
 *   PTGQ_ROW_MAJOR + PTGQ_SCALE_F32    float   [rows][ng]
 *   PTGQ_ROW_MAJOR + PTGQ_SCALE_UE8M0  uint8   [rows][ng]
 *   PTGQ_COL_MAJOR + PTGQ_SCALE_F32    float   [ng][rows_pad]
 *   PTGQ_COL_MAJOR + PTGQ_SCALE_UE8M0  uint32  [ceil(ng/4)][rows_pad]; group g
 *                  of row m is byte g%4 (little-endian) of word
 *                  (g/4)*rows_pad + m  (vllm #41326 review page, key source
 *                  snippets, all-zero test; sglang #35593 review page,
 *                  implementation breakdown: column-major [E, M, hidden/128])
 *   In flat calls the column-major pad slots (rows rows..rows_pad-1) and the
 *   unused bytes of a partial packed word are written as zero.
 */
#ifndef PTGQ_H
#define PTGQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exported symbols of libptgq.so (everything else in it is hidden). */
#if defined(__GNUC__)
#define PTGQ_API __attribute__((visibility("default")))
#else
#define PTGQ_API
#endif

/* Return codes. */
enum ptgq_status {
    PTGQ_OK = 0,
    PTGQ_EINVAL = -1,       /* a size, enum or pointer argument is invalid      */
    PTGQ_EALIGN = -2,       /* a pointer is not aligned as required            */
    PTGQ_EUNSUPPORTED = -3, /* valid arguments, combination not implemented    */
    PTGQ_ELAUNCH = -4,      /* the HIP launch failed (hipGetLastError)          */
    PTGQ_EDEVICE = -5       /* no usable HIP device / device query failed       */
};

enum ptgq_in_dtype { PTGQ_BF16 = 0, PTGQ_FP16 = 1, PTGQ_FP32 = 2 };
enum ptgq_out_dtype { PTGQ_E4M3 = 0, PTGQ_INT8 = 1 };
enum ptgq_scale_fmt { PTGQ_SCALE_F32 = 0, PTGQ_SCALE_UE8M0 = 1 };
enum ptgq_scale_layout { PTGQ_ROW_MAJOR = 0, PTGQ_COL_MAJOR = 1 };

/*
 * ptgq_quant - flat per-token-group quantization of x [M, K] (or of
 * silu(gate) * up for x = [M, 2K] = gate | up when fuse_silu_mul != 0).
 *
 *   x          device, in_dtype (PTGQ_BF16, PTGQ_FP16, or PTGQ_FP32 when not
 *              fused), row-major contiguous [M, K] or [M, 2K]; 16-byte
 *              aligned.  fp32 input is the trait the pages list beside the
 *              16-bit ones (sglang #34257 review page, key source snippets:
 *              float, half and bfloat16 instantiations).
 *   group_size G in {16, 32, 64, 128}; K % G == 0.
 *   out_dtype  PTGQ_E4M3 (OCP e4m3fn codes) or PTGQ_INT8 (two's complement).
 *   scale_fmt, scale_layout  see the layouts above.
 *   eps        floor of the group absmax (finite, >= +0.0; -0.0 is rejected;
 *              e.g. 1e-10).
 *   q          device uint8 [M, K] codes; 16-byte aligned.
 *   s          device scale tensor of ptgq_scale_bytes(M, K, G, fmt, layout)
 *              bytes; 4-byte aligned.
 * Sources: sglang #30924 review page, implementation breakdown (flat
 * schedule); sglang #27449 PR body, summary (naive scheduler over [M, K]).
 * Errors: PTGQ_EINVAL (M < 0, K < 0, G not allowed, K % G, bad enum, NULL
 * pointer with M*K > 0, eps not finite, negative or -0.0), PTGQ_EALIGN,
 * PTGQ_EUNSUPPORTED (fp32 input with fuse_silu_mul, K >= 2^29, sizes beyond
 * 32-bit task counts), PTGQ_ELAUNCH, PTGQ_EDEVICE.
 */
PTGQ_API int ptgq_quant(const void *x, int in_dtype, int64_t M, int64_t K, int group_size,
               int fuse_silu_mul, int out_dtype, int scale_fmt, int scale_layout, float eps,
               void *q, void *s, void *stream);

/*
 * ptgq_quant_padded - ptgq_quant into a padded code buffer: q holds q_rows >=
 * M rows of K bytes, as consumers that load q in 4-row-aligned tiles allocate
 * it; rows M .. q_rows-1 are written as zero in the same launch (so they hold
 * no stale bytes).  Rows 0 .. M-1 and the scales are exactly ptgq_quant's
 * (scale layouts still use rows = M).  With M == 0 only the zero fill runs, and
 * x and s are not used.
 * Source: vllm #41326 review page, implementation breakdown (zero-filling the
 * TMA-aligned extra rows of output_q after quantization) and key source
 * snippets (the kernel's output_q extent beside tma_aligned_mn).
 * Errors: as ptgq_quant, plus PTGQ_EINVAL for q_rows < M and
 * PTGQ_EUNSUPPORTED for q_rows >= 2^31.
 */
PTGQ_API int ptgq_quant_padded(const void *x, int in_dtype, int64_t M, int64_t K,
                               int group_size, int fuse_silu_mul, int out_dtype, int scale_fmt,
                               int scale_layout, float eps, void *q, int64_t q_rows, void *s,
                               void *stream);

/*
 * ptgq_quant_masked - the masked expert-parallel MoE layout.
 *
 *   x          device [E, tokens_pad, K] (or [E, tokens_pad, 2K] fused),
 *              in_dtype as above; 16-byte aligned.
 *   masked_m   device int32 [E]: expert e quantizes its rows
 *              t < min(max(masked_m[e], 0), tokens_pad).  Read on the device;
 *              the host never waits for it.
 *   expected_m host hint of the typical masked_m (<= 0: unknown).  It only
 *              sizes the launch; results never depend on it.
 *   q          device uint8 [E, tokens_pad, K]; 16-byte aligned.
 *   s          device, E consecutive per-expert scale tensors, each of
 *              ptgq_scale_bytes(tokens_pad, K, G, fmt, layout) bytes (so the
 *              column-major form is [E][ng or ceil(ng/4)][pad4(tokens_pad)]).
 *   Rows at or past masked_m are neither read nor written, in q or in s
 *   (column-major pad slots included): the caller's contents stay.  The live
 *   rows of all experts are spread evenly over the launch, whatever their
 *   distribution over experts.
 * Sources: sglang #30924 review page, implementation breakdown (masked_m and
 * expected_m); sglang #27449 PR body, summary and validation (masked layout
 * scheduler, [num_experts, tokens_pad, hidden*2] with silu+mul); sglang
 * #35593 review page, key source snippets (rows past masked_m untouched).
 * Errors: as ptgq_quant, plus PTGQ_EINVAL for E < 0, tokens_pad < 0 or a NULL
 * masked_m with E > 0, and PTGQ_EUNSUPPORTED for E > 4096.
 */
PTGQ_API int ptgq_quant_masked(const void *x, int in_dtype, int64_t E, int64_t tokens_pad, int64_t K,
                      int group_size, int fuse_silu_mul, const int32_t *masked_m,
                      int64_t expected_m, int out_dtype, int scale_fmt, int scale_layout,
                      float eps, void *q, void *s, void *stream);

/*
 * ptq_quant_fp8 - whole-row per-token e4m3: scale[m] = max_k |x[m,k]| / 448
 * (no floor), multiplier 0 when the scale is 0, codes narrowed with
 * saturation.
 *
 *   x   device [M, K] in_dtype in {PTGQ_BF16, PTGQ_FP16, PTGQ_FP32},
 *       row-major contiguous; 16-byte aligned.  K % 4 == 0.
 *   q   device uint8 [M, K] e4m3 codes; 16-byte aligned.
 *   s   device float [M]; 4-byte aligned.
 *   q and s may be the first M rows of longer buffers (serving code pads its
 *   outputs): only rows 0 .. M-1 are written (sglang #34257 review page, key
 *   source snippets, the host contract on output rows).
 * Sources: sglang #34257 review page, key source snippets (warp kernel and
 * its dispatch by token count), implementation breakdown (hidden % 4 == 0).
 * Errors: PTGQ_EINVAL (M < 0, K < 0, K % 4, bad dtype, NULL pointer),
 * PTGQ_EALIGN, PTGQ_ELAUNCH, PTGQ_EDEVICE.
 */
PTGQ_API int ptq_quant_fp8(const void *x, int in_dtype, int64_t M, int64_t K, void *q, float *s,
                  void *stream);

/*
 * ptgq_requant_fp8 - per-token-group fp8 -> per-tensor fp8 requantization
 * on the masked layout: for expert e and rows t < min(max(masked_m[e], 0), T)
 * (every row when masked_m is NULL),
 *   out[e][t][k] = e4m3_sat((decode(x[e][t][k]) * s) * (1 / output_scale[0]))
 * with s = x_scale[e*scale_stride_e + t*scale_stride_t + (k/G)*scale_stride_g],
 * each product one fp32 rounding (1 / output_scale is an IEEE division),
 * narrowed round-to-nearest-even with saturation to +-448.  Rows past
 * masked_m keep out's contents.
 *
 *   x             device uint8 [E, T, K] e4m3 codes; 16-byte aligned.
 *   group_size    G in {16, 32, 64, 128} (the pages use 128); K % G == 0, so
 *                 K need only be G-aligned (e.g. 3584, 1152).
 *   x_scale       device float group scales; strides in elements, >= 0 (the
 *                 DeepEP layout [E, T, K/128] with its last two dims
 *                 column-major is se = T*(K/128), st = 1, sg = T).
 *   masked_m      device int32 [E] or NULL; expected_m: launch hint (<= 0:
 *                 unknown), never changes results.
 *   output_scale  device float [1], the per-tensor output scale.
 *   out           device uint8 [E, T, K]; 16-byte aligned; must not be x.
 * Source: sglang #35593 review page (key source snippets: the requant kernel
 * and its test; implementation breakdown: 128-aligned hidden sizes).
 * Errors: PTGQ_EINVAL (negative sizes or strides, G, K % G, NULL pointer,
 * out == x), PTGQ_EALIGN, PTGQ_EUNSUPPORTED (E > 4096, T*K >= 2^31, a scale
 * span of 2^30 elements or more, sizes beyond 32-bit task counts),
 * PTGQ_ELAUNCH, PTGQ_EDEVICE.
 */
PTGQ_API int ptgq_requant_fp8(const uint8_t *x, int64_t E, int64_t T, int64_t K, int group_size,
                              const float *x_scale, int64_t scale_stride_e,
                              int64_t scale_stride_t, int64_t scale_stride_g,
                              const int32_t *masked_m, int64_t expected_m,
                              const float *output_scale, uint8_t *out, void *stream);

/*
 * ptgq_dequant - group dequantization, the inverse of ptgq_quant:
 *   y[m][k] = round_out(decode(q[m][k]) * scale(m, k / G))
 * decode is the e4m3 value of the code (OCP e4m3fn; 0x7F / 0xFF are NaN) or
 * the int8 value; the product is one fp32 rounding (exact for UE8M0 scales
 * unless it falls below the normal range); round_out is round-to-nearest-even
 * to bf16 / fp16 (overflowing to infinity) or nothing for fp32.  A UE8M0
 * scale byte e stands for 2^(e - 127) (e == 0: 2^-127, e == 255: infinity).
 *
 *   q             device uint8 [M, K] codes of code_dtype (PTGQ_E4M3 or
 *                 PTGQ_INT8); row-major; 16-byte aligned.
 *   group_size    G in {16, 32, 64, 128}; K % G == 0.
 *   s             device scales of M rows in scale_fmt / scale_layout, exactly
 *                 as ptgq_quant writes them (layout table above; pad slots are
 *                 not read); fp32 scales 4-byte aligned.
 *   out_dtype     PTGQ_BF16, PTGQ_FP16 or PTGQ_FP32.
 *   y             device [M, K] of out_dtype; 16-byte aligned; must not alias
 *                 q or s.
 * Sources: sglang #35593 review page, key source snippets (the test's
 * reference multiplies the codes, as float, by the group scales repeated over
 * each group); sglang #30924 review page, implementation breakdown (fp32-scale
 * results are verified through their dequantization).
 * Errors: PTGQ_EINVAL (M < 0, K < 0, G not allowed, K % G, bad enum, NULL
 * pointer, y aliasing q or s), PTGQ_EALIGN, PTGQ_EUNSUPPORTED (K >= 2^29,
 * sizes beyond 32-bit task counts or scale spans), PTGQ_ELAUNCH, PTGQ_EDEVICE.
 */
PTGQ_API int ptgq_dequant(const uint8_t *q, int code_dtype, int64_t M, int64_t K, int group_size,
                          const void *s, int scale_fmt, int scale_layout, int out_dtype, void *y,
                          void *stream);

/*
 * ptgq_scale_bytes - size in bytes of the scale tensor for `rows` rows of K
 * elements in groups of group_size, in the given format and layout (see the
 * layout table above).  Returns 0 for invalid arguments.  Host only; no
 * device access.
 */
PTGQ_API size_t ptgq_scale_bytes(int64_t rows, int64_t K, int group_size, int scale_fmt,
                        int scale_layout);

/* ptgq_status_string - static English text of a return code.  Host only. */
PTGQ_API const char *ptgq_status_string(int status);

/*
 * ptgq_init - optional: make `device` (a HIP ordinal) ready now: query its
 * compute-unit count and build its SiLU lookup tables on the default stream,
 * then wait on the host until the build has finished (the one call of the
 * library that blocks the host; not to be called while a stream captures).
 * Calls captured into a HIP graph after it use the tables.  A failed
 * initialization is not remembered: a later call tries again.  Returns
 * PTGQ_OK or PTGQ_EDEVICE.
 */
PTGQ_API int ptgq_init(int device);

#ifdef __cplusplus
}
#endif

#endif /* PTGQ_H */
