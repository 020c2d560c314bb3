/*
 * ptgq_diag.h - diagnostics of libptgq.so: single-step device probes, a
 * no-arithmetic stream, the launch-geometry report and its overrides.
 *
 * Not part of the quantization interface (include/ptgq.h): these calls exist
 * so that tests can check the device arithmetic over whole input spaces
 * against a reference, and so that measurements can compare the kernels with
 * a plain stream and sweep the launch geometry.  Return codes and the stream
 * convention are those of ptgq.h.
 */
#ifndef PTGQ_DIAG_H
#define PTGQ_DIAG_H

#include <stddef.h>
#include <stdint.h>

#include "ptgq.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Single-step device probes, for checking the device arithmetic against
 * a reference over whole input spaces.  They run exactly the device code the
 * quantization kernels use for that step.
 *
 * ptgq_probe_e4m3: out[i] = e4m3 code of v[i] (round-to-nearest-even,
 *   saturated to +-448, signed zero kept).  v device float [n], out device
 *   uint8 [n]; both 4-byte aligned.
 * ptgq_probe_silu_mul: out[i] = silu(g[i]) * u[i] in fp32, where g, u are
 *   device arrays of in_dtype (PTGQ_BF16 or PTGQ_FP16) bit patterns [n]
 *   and out is device float [n].  path 0: the direct evaluation (e^-g
 *   correctly rounded to fp32 from an fp64 polynomial, the fp32 add, the
 *   quotient from an fp64 reciprocal rounded to fp32, the fp32 multiply);
 *   path 1: the lookup of g / (1 + e^-g) that large fused calls use (bf16:
 *   the closed forms outside the table; fp16: the direct evaluation for
 *   gates of magnitude 8 or more), followed by the multiply.
 * Errors: PTGQ_EINVAL (n < 0, NULL pointer, bad dtype or path), PTGQ_ELAUNCH,
 * PTGQ_EDEVICE.
 */
PTGQ_API int ptgq_probe_e4m3(const float *v, uint8_t *out, int64_t n, void *stream);
PTGQ_API int ptgq_probe_silu_mul(const void *g, const void *u, int in_dtype, int path,
                                 float *out, int64_t n, void *stream);

/*
 * ptgq_probe_scale - the scale step of the quantization kernels alone: for
 * i < n, amax = the fp32 value with bit pattern first_bits + i (every one of
 * them non-negative and finite: first_bits + n <= 0x7F800000), floored by eps
 * and divided by qmax (448 for PTGQ_E4M3, 127 for PTGQ_INT8), in scale_fmt:
 *   PTGQ_SCALE_F32    scale_out float [n] = r, inv_out[i] = 1 / r (0 if r = 0)
 *   PTGQ_SCALE_UE8M0  scale_out uint8 [n] = exponent byte e, inv_out[i] =
 *                     2^(127 - e)
 * inv_out (device float [n]) may be NULL.  Source of the definition: sglang
 * #30924 review page, key source snippets (ref_fp8_ue8m0); sglang #34257
 * review page, key source snippets (reciprocal, zero for a zero scale).
 * Errors: PTGQ_EINVAL (bad enum, eps, n < 0, range past +inf, NULL
 * scale_out), PTGQ_EALIGN, PTGQ_ELAUNCH, PTGQ_EDEVICE.
 */
PTGQ_API int ptgq_probe_scale(uint32_t first_bits, int64_t n, float eps, int out_dtype,
                              int scale_fmt, void *scale_out, float *inv_out, void *stream);

/*
 * ptgq_probe_int8 - the int8 narrowing of the quantization kernels alone:
 * out[i] = code of the fp32 value with bit pattern (first_bits + i) mod 2^32
 * (round to nearest, ties to even, saturated to [-128, 127]; NaN patterns
 * give unspecified codes).  n <= 2^32; out device int8 [n].
 * Errors: PTGQ_EINVAL, PTGQ_ELAUNCH, PTGQ_EDEVICE.
 */
PTGQ_API int ptgq_probe_int8(uint32_t first_bits, int64_t n, int8_t *out, void *stream);

/*
 * ptgq_probe_stream - a stream with the plain quantization kernel's traffic
 * and launch geometry and no arithmetic: reads n 16-bit elements of x and
 * writes the low byte of each to q (2 bytes read per byte written, as a
 * 16-bit quantization's codes, without the scales).  Its rate is what the
 * memory system gives that access pattern.  n % 1024 == 0; x and q device,
 * 16-byte aligned.
 * Errors: PTGQ_EINVAL, PTGQ_EALIGN, PTGQ_EUNSUPPORTED, PTGQ_ELAUNCH,
 * PTGQ_EDEVICE.
 */
PTGQ_API int ptgq_probe_stream(const void *x, int64_t n, uint8_t *q, void *stream);

/*
 * ptgq_diag_fastdiv - host only: q[i] = floor(n[i] / d) by the
 * multiply-high division the kernels use for task indices (Granlund and
 * Montgomery 1994), for checking it.  n[i] < 2^31; d >= 1.
 * Returns PTGQ_OK or PTGQ_EINVAL.
 */
PTGQ_API int ptgq_diag_fastdiv(uint32_t d, const uint32_t *n, uint32_t *q, int64_t count);

/*
 * ptgq_plan_group - diagnostics and tests of the launch-geometry chooser:
 * the launch a ptgq_quant / ptgq_quant_padded call (E = 0; q_rows = rows of
 * the code buffer, >= rows) or a ptgq_quant_masked call (E >= 1 experts of
 * rows = tokens_pad rows, sized for expected_m) would make on a device of
 * `cus` compute units.  Tiny calls spread one-slab tasks over the compute
 * units; larger unfused flat ones use two-slab tasks on a grid of one wave
 * per task dealt to the XCDs in chunks; fused and masked calls a capped grid
 * whose persistent blocks loop over the tasks (the pages size their launch by
 * token count the same way: the sglang #34257 review page, key source
 * snippets, dispatch; `expected_m` of the sglang #30924 review page,
 * implementation breakdown).  Makes no HIP call and touches no device;
 * honours the ptgq_set_tuning overrides.
 *   out: host array of 9, written with: blocks in the grid, threads per
 *        block, slabs (512 consecutive elements of a row) per task, tasks per
 *        row (row tasks; ceil(slabs per row / slabs per task)), tasks in all
 *        (masked: the expected ones), blocks per XCD chunk of the block ->
 *        task mapping (0: one contiguous range per XCD), SiLU lookup table
 *        (0/1), uncapped grid (0/1), flat-slab tasks (0 none; 1 the tensor's
 *        whole-row slabs taken as one sequence, tasks crossing row ends; 2
 *        slabs of several rows shorter than a slab; 3 slabs of the flattened
 *        tensor, for other rows that are not whole slabs, fused included;
 *        4 chunk tasks of 128 output elements of a row, for small fused
 *        calls on the direct SiLU path, tasks per row then counting chunks;
 *        masked calls: 0, or 3 for slabs of each expert's flattened live
 *        rows); all zero when nothing would be launched.
 * Returns PTGQ_OK, PTGQ_EINVAL (invalid shape, cus < 1, out NULL) or
 * PTGQ_EUNSUPPORTED, as the calls would for the same shape.
 */
PTGQ_API int ptgq_plan_group(int in_dtype, int64_t E, int64_t rows, int64_t K, int group_size,
                             int fuse_silu_mul, int64_t expected_m, int64_t q_rows, int cus,
                             int64_t *out);

/*
 * ptgq_set_tuning - diagnostics only: override one decision of the launch
 * geometry chooser for the whole process (value -1 restores the automatic
 * choice). Knobs: 0 slabs per task (quantization: 1 or 2, one slab = 512
 * elements of a row; dequantization: 1 or 4 sub-slabs), 1 waves per block
 * (group, requantization and dequantization kernels 1..4, not the fused
 * SiLU-table kernels, which always run 16;
 * per-token one-block-per-row mode: waves per row, 1..8; per-token one-wave-
 * per-row mode: rows per block, 1..4), 2 resident blocks per compute unit
 * (grid cap), 3 per-token mode (0 one wave per row, 1 one block per row, 2
 * two-pass block, 3 persistent waves walking the rows), 4 fused SiLU
 * path (0 direct evaluation, 1 LDS lookup table), 5 blocks per XCD chunk of
 * the block-to-task mappings of the flat quantization, dequantization and
 * requantization kernels and of the per-token one-block-per-row mode (0 one
 * contiguous range per XCD, or for the per-token mode block b takes row b), 6
 * grid of the flat quantization, requantization and dequantization kernels (0
 * capped: resident blocks loop over the tasks; 1 uncapped: one wave per
 * task), 7 two-slab tasks of unfused flat calls whose K is a multiple of 512
 * (0 row tasks; 1 flat-slab tasks, which cross row ends; automatic: flat-slab
 * tasks for an odd number of slabs per row) and the slabs of rows that are
 * not whole slabs (0 row tasks; otherwise automatic: multi-row or flattened
 * slabs); masked calls: 0 row tasks, 1 flattened slabs of each expert's live
 * rows, automatic: those for rows that are not whole slabs and for unfused
 * rows of an odd number of slabs; fused flat calls: 0 slab tasks, 2 chunk
 * tasks whenever the SiLU table is not read, automatic: chunk tasks for
 * small calls (knob 0 set also selects slab tasks).
 * Results never depend on these; only speed does. Not synchronized with calls
 * running on other host threads. Returns PTGQ_OK or PTGQ_EINVAL.
 */
PTGQ_API int ptgq_set_tuning(int knob, int64_t value);

#ifdef __cplusplus
}
#endif

#endif /* PTGQ_DIAG_H */
