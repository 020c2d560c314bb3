/*
 * CPU oracle for per-token-group 8-bit activation quantization.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: it is used by the test-suite, by the smoke check and
 * by the CPU-baseline leg of the benchmark, to decide whether the GPU library
 * is right.  It shares no code, header, table or constant generator with the
 * HIP library; the two meet only at the byte level of their outputs.
 *
 * It is deliberately plain: one thread, IEEE binary32 arithmetic (x86-64 SSE,
 * round-to-nearest), compiled with -O2 -fno-fast-math -ffp-contract=off, no
 * SIMD intrinsics, no blocking or reordering.  Every function follows the
 * definition on the source pages step by step; each cites the passage it
 * follows.  Page names used in citations:
 *   [sglang #30924]  review page "unify per_token_group_quant into a
 *                    trait-driven JIT kernel"
 *   [sglang #34257]  review page "per-token FP8 quant migrated to JIT"
 *   [sglang #35593]  review page "W4AFP8 requant kernel accepts 128-aligned
 *                    hidden sizes"
 *   [sglang #27449]  GitHub PR body "port per_token_group_quant_8bit_v2 to JIT"
 *   [vllm #41326]    review page "Blackwell register-resident FP8 group quant"
 *
 * Readings the pages leave open (each is listed with its reason in the design
 * notes of the repository):
 *   - eps is applied once, before the division by qmax (the formula of
 *     [sglang #30924] key source snippets, ref_fp8_ue8m0), not again after it.
 *   - all divisions are IEEE round-to-nearest fp32 divisions.
 *   - fp32-scale codes use v = y * fl(1/r), the reciprocal-multiply form of
 *     the per-token kernel in [sglang #34257] key source snippets.
 *   - SiLU uses a correctly rounded binary32 exp; every other step of
 *     silu(g)*u is one IEEE fp32 operation.
 *   - a zero value times an infinite multiplier (fl(1/r) overflowed: r below
 *     about 2^-128) is a zero of the value's sign, not NaN; a non-zero value
 *     times it saturates.
 *   - e4m3 narrowing is round-to-nearest-even with saturation to +-448
 *     ([sglang #35593] key source snippets, satfinite conversion); a negative
 *     value that rounds to zero keeps its sign (code 0x80).
 *   - column-major scale pad slots (rows M..M_pad-1, unused bytes of a
 *     partial packed word) are zero in flat calls; masked calls touch nothing
 *     in rows at or past masked_m.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

/* Argument codes of this oracle (its own; the Python wrapper maps names). */
enum { OR_BF16 = 0, OR_FP16 = 1, OR_FP32 = 2 };
enum { OR_E4M3 = 0, OR_INT8 = 1 };
enum { OR_SCALE_F32 = 0, OR_SCALE_UE8M0 = 1 };
enum { OR_ROW_MAJOR = 0, OR_COL_MAJOR = 1 };

static float f32_from_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

/* ------------------------------------------------------------------------ */
/* Step 1: decode the 16-bit input to fp32 (both conversions are exact).     */
/* ------------------------------------------------------------------------ */

/* bfloat16 is the top half of a binary32 pattern. */
static float decode_bf16(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static float decode_fp16(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double mag;
    if (e == 0)
        mag = ldexp((double)m, -24);               /* subnormal: m * 2^-24 */
    else if (e == 31)
        mag = m ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + m), e - 25);   /* (1 + m/1024) * 2^(e-15) */
    return (float)(sign ? -mag : mag);
}

static float decode_elem(const void *x, int dtype, int64_t idx)
{
    if (dtype == OR_BF16) return decode_bf16(((const uint16_t *)x)[idx]);
    if (dtype == OR_FP16) return decode_fp16(((const uint16_t *)x)[idx]);
    return ((const float *)x)[idx];
}

/* ------------------------------------------------------------------------ */
/* Narrowing to 8 bits.                                                      */
/* ------------------------------------------------------------------------ */

/* OCP e4m3 ("fn"): bias 7, no infinities, 0x7F/0xFF are NaN, largest finite
 * value 448 (code 0x7E); code = E<<3 | m; E = 0 holds the subnormals m*2^-9,
 * E >= 1 holds (8+m) * 2^(E-10).  Codes 0..126 are the non-negative finite
 * values in increasing order. */
static double e4m3_table[127];
static int e4m3_table_ready = 0;

static void e4m3_build_table(void)
{
    for (int c = 0; c < 127; ++c) {
        int E = c >> 3, m = c & 7;
        e4m3_table[c] = (E == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), E - 10);
    }
    e4m3_table_ready = 1;
}

/* Round to the nearest finite e4m3 value, ties to the even code, saturate
 * to +-448; the sign of a value that rounds to zero is kept.
 * ([sglang #35593] key source snippets: satfinite RN conversion clamps to 448
 * where a plain cast would give NaN.)  All comparisons are exact in double. */
static uint8_t e4m3_rne_sat(float v)
{
    if (!e4m3_table_ready) e4m3_build_table();
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a >= 448.0) return sign | 0x7E;
    /* largest code lo with value(lo) <= a; lo <= 125 because a < 448 */
    int lo = 0, hi = 126;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (e4m3_table[mid] <= a) lo = mid; else hi = mid - 1;
    }
    double below = a - e4m3_table[lo];
    double above = e4m3_table[lo + 1] - a;
    int c;
    if (below < above) c = lo;
    else if (above < below) c = lo + 1;
    else c = (lo & 1) ? lo + 1 : lo;          /* tie: even mantissa LSB */
    return (uint8_t)(sign | c);
}

/* int8: round to nearest integer, ties to even, then clamp to [-128, 127]. */
static int8_t int8_rne_sat(float v)
{
    double x = v;
    double f = floor(x);
    double frac = x - f;                     /* exact */
    double r;
    if (frac > 0.5) r = f + 1.0;
    else if (frac < 0.5) r = f;
    else r = (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
    if (r > 127.0) r = 127.0;
    if (r < -128.0) r = -128.0;
    return (int8_t)r;
}

/* ------------------------------------------------------------------------ */
/* Step 2 (fused variants only): silu(gate) * up in fp32.                    */
/* ------------------------------------------------------------------------ */

/* Correctly rounded binary32 e^x.  The double result of the C library is
 * within about one double ulp of e^x, far closer than any binary32 rounding
 * boundary for the 16-bit inputs this path takes; the test-suite checks the
 * result against a 60-digit decimal evaluation for every bf16 and fp16 input. */
static float exp_cr(float x) { return (float)exp((double)x); }

/* silu(g) * u = (g / (1 + e^-g)) * u, each operation one fp32 rounding.
 * ([sglang #30924] implementation breakdown: fused silu_and_mul trait;
 * the fp32 evaluation follows the configuration of the fused workload.) */
static float silu_mul(float g, float u)
{
    float e = exp_cr(-g);
    float d = 1.0f + e;
    float s = g / d;
    return s * u;
}

/* ------------------------------------------------------------------------ */
/* Steps 3-6: scale of one group.                                           */
/* ------------------------------------------------------------------------ */

typedef struct {
    float r;        /* fp32 scale, = max(amax, eps) / qmax            */
    uint8_t ue8m0;  /* exponent byte of the power-of-two ceiling of r */
    float inv;      /* the multiplier the codes are made with         */
} group_scale;

/* [sglang #30924] key source snippets (ref_fp8_ue8m0): amax floored by eps,
 * divided by the format maximum; UE8M0 takes the exponent field of that
 * quotient and adds one when its fraction is non-zero; the multiplier
 * 2^(127-e) is rebuilt exactly from the bit pattern (254-e)<<23.
 * [sglang #34257] key source snippets: the fp32 form multiplies by the
 * reciprocal, which is zero when the scale is zero. */
static group_scale make_scale(float amax, float eps, float qmax, int ue8m0)
{
    group_scale gs;
    float a = (amax > eps) ? amax : eps;
    gs.r = a / qmax;
    if (!ue8m0) {
        gs.ue8m0 = 0;
        gs.inv = (gs.r == 0.0f) ? 0.0f : 1.0f / gs.r;
    } else {
        uint32_t b = bits_from_f32(gs.r);
        uint32_t e = ((b >> 23) & 0xFFu) + ((b & 0x7FFFFFu) != 0u);
        gs.ue8m0 = (uint8_t)e;
        gs.inv = f32_from_bits((254u - e) << 23);
    }
    return gs;
}

/* The value narrowed for y: v = y * inv, one fp32 rounding, except that a
 * zero y gives v = y.  The two differ only when inv is infinite, which
 * happens when fl(1/r) overflows (r below about 2^-128: an fp32 scale with a
 * floor eps below about 1.3e-36, or a per-token row whose largest magnitude is
 * below that): the product 0 * inf would be NaN, while the quotient y / r the
 * codes stand for is exactly zero.  So a zero keeps its sign (e4m3 0x00 or
 * 0x80) and a non-zero y times an infinite multiplier saturates.  (The pages
 * leave this corner open; [sglang #34257] key source snippets guard only the
 * all-zero row, by a zero multiplier.) */
static float scaled(float y, float inv)
{
    return (y == 0.0f) ? y : y * inv;
}

static uint8_t quantize(float y, float inv, int out_dtype)
{
    float v = scaled(y, inv);
    if (out_dtype == OR_E4M3) return e4m3_rne_sat(v);
    return (uint8_t)int8_rne_sat(v);
}

/* ------------------------------------------------------------------------ */
/* Scale tensor layouts.                                                     */
/*   row-major fp32:    float  [rows][ng]                                    */
/*   row-major UE8M0:   uint8  [rows][ng]                                    */
/*   col-major fp32:    float  [ng][rows_pad],  rows_pad = ceil(rows/4)*4    */
/*   col-major UE8M0:   uint32 [ceil(ng/4)][rows_pad], group g of row m in   */
/*                      byte g%4 (little-endian) of word (g/4)*rows_pad + m  */
/* ([vllm #41326] key source snippets, the all-zero test, spells out the     */
/* packed index; [sglang #30924] implementation breakdown names the layout   */
/* trait; [sglang #35593] implementation breakdown gives the col-major       */
/* per-expert scale shape.)                                                  */
/* ------------------------------------------------------------------------ */

static int64_t pad4(int64_t n) { return (n + 3) / 4 * 4; }

size_t oracle_scale_bytes(int64_t rows, int64_t K, int G, int scale_fmt, int scale_layout)
{
    int64_t ng = K / G;
    if (scale_layout == OR_ROW_MAJOR)
        return (size_t)(rows * ng * (scale_fmt == OR_SCALE_F32 ? 4 : 1));
    if (scale_fmt == OR_SCALE_F32)
        return (size_t)(ng * pad4(rows) * 4);
    return (size_t)(((ng + 3) / 4) * pad4(rows) * 4);
}

static void store_scale(void *s, int64_t rows, int64_t ng, int64_t m, int64_t g,
                        const group_scale *gs, int scale_fmt, int scale_layout)
{
    if (scale_layout == OR_ROW_MAJOR) {
        if (scale_fmt == OR_SCALE_F32) ((float *)s)[m * ng + g] = gs->r;
        else ((uint8_t *)s)[m * ng + g] = gs->ue8m0;
    } else {
        int64_t rp = pad4(rows);
        if (scale_fmt == OR_SCALE_F32) ((float *)s)[g * rp + m] = gs->r;
        else ((uint8_t *)s)[((g / 4) * rp + m) * 4 + (g % 4)] = gs->ue8m0;
    }
}

/* Zero the bytes of row m's packed words that no group uses (ng % 4 != 0). */
static void zero_packed_tail(void *s, int64_t rows, int64_t ng, int64_t m)
{
    int64_t rp = pad4(rows);
    for (int64_t g = ng; g % 4 != 0; ++g)
        ((uint8_t *)s)[((g / 4) * rp + m) * 4 + (g % 4)] = 0;
}

/* ------------------------------------------------------------------------ */
/* One row of the group quantizer.                                          */
/* ------------------------------------------------------------------------ */

static void quant_row(const void *x, int in_dtype, int64_t row_in, int64_t K, int G, int fuse,
                      int out_dtype, int scale_fmt, int scale_layout, float eps,
                      uint8_t *q, int64_t row_out, void *s, int64_t s_rows, int64_t s_row)
{
    const float qmax = (out_dtype == OR_E4M3) ? 448.0f : 127.0f;
    const int64_t ng = K / G;
    const int64_t in_width = fuse ? 2 * K : K;
    float y[128];
    for (int64_t g = 0; g < ng; ++g) {
        /* steps 1-2: the group's fp32 values */
        for (int k = 0; k < G; ++k) {
            int64_t col = g * G + k;
            if (fuse) {
                float gate = decode_elem(x, in_dtype, row_in * in_width + col);
                float up = decode_elem(x, in_dtype, row_in * in_width + K + col);
                y[k] = silu_mul(gate, up);
            } else {
                y[k] = decode_elem(x, in_dtype, row_in * in_width + col);
            }
        }
        /* step 3: group absmax (exact, order-free) */
        float amax = 0.0f;
        for (int k = 0; k < G; ++k) {
            float a = fabsf(y[k]);
            if (a > amax) amax = a;
        }
        /* steps 4-6 */
        group_scale gs = make_scale(amax, eps, qmax, scale_fmt == OR_SCALE_UE8M0);
        /* step 7: codes */
        for (int k = 0; k < G; ++k)
            q[row_out * K + g * G + k] = quantize(y[k], gs.inv, out_dtype);
        /* step 8: scale */
        store_scale(s, s_rows, ng, s_row, g, &gs, scale_fmt, scale_layout);
    }
    if (scale_layout == OR_COL_MAJOR && scale_fmt == OR_SCALE_UE8M0)
        zero_packed_tail(s, s_rows, ng, s_row);
}

static int check_common(int in_dtype, int64_t K, int G, int out_dtype, int scale_fmt,
                        int scale_layout)
{
    if (in_dtype != OR_BF16 && in_dtype != OR_FP16 && in_dtype != OR_FP32) return -1;
    if (G != 16 && G != 32 && G != 64 && G != 128) return -1;
    if (K < 0 || K % G != 0) return -1;
    if (out_dtype != OR_E4M3 && out_dtype != OR_INT8) return -1;
    if (scale_fmt != OR_SCALE_F32 && scale_fmt != OR_SCALE_UE8M0) return -1;
    if (scale_layout != OR_ROW_MAJOR && scale_layout != OR_COL_MAJOR) return -1;
    return 0;
}

/* Flat group quantization of x [M, K] (or [M, 2K] gate|up when fused) into
 * q [M, K] codes and the scale tensor s (whole buffer written, pad slots 0).
 * ([sglang #30924] implementation breakdown; [sglang #27449] summary: the
 * flat scheduler over [M, K].) */
int oracle_ptgq(const void *x, int in_dtype, int64_t M, int64_t K, int G, int fuse,
                int out_dtype, int scale_fmt, int scale_layout, float eps,
                uint8_t *q, void *s)
{
    if (check_common(in_dtype, K, G, out_dtype, scale_fmt, scale_layout) || M < 0) return -1;
    if (fuse && in_dtype == OR_FP32) return -1;   /* fused calls take 16-bit inputs */
    if (scale_layout == OR_COL_MAJOR)
        memset(s, 0, oracle_scale_bytes(M, K, G, scale_fmt, scale_layout));
    for (int64_t m = 0; m < M; ++m)
        quant_row(x, in_dtype, m, K, G, fuse, out_dtype, scale_fmt, scale_layout, eps,
                  q, m, s, M, m);
    return 0;
}

/* Masked (expert-parallel MoE) layout: x [E, T, K or 2K], q [E, T, K], the
 * scale tensor is one per-expert block of oracle_scale_bytes(T, ...) bytes.
 * Expert e quantizes rows t < min(max(masked_m[e], 0), T); every other byte
 * of q and s is left as it was.  ([sglang #30924] implementation breakdown:
 * masked_m / expected_m; [sglang #35593] key source snippets: rows past
 * masked_m keep the caller's sentinel.) */
int oracle_ptgq_masked(const void *x, int in_dtype, int64_t E, int64_t T, int64_t K, int G,
                       int fuse, const int32_t *masked_m, int out_dtype, int scale_fmt,
                       int scale_layout, float eps, uint8_t *q, void *s)
{
    if (check_common(in_dtype, K, G, out_dtype, scale_fmt, scale_layout) || E < 0 || T < 0)
        return -1;
    if (fuse && in_dtype == OR_FP32) return -1;
    const size_t sb = oracle_scale_bytes(T, K, G, scale_fmt, scale_layout);
    const int64_t in_width = fuse ? 2 * K : K;
    const size_t in_elem = in_dtype == OR_FP32 ? 4 : 2;
    for (int64_t e = 0; e < E; ++e) {
        int64_t live = masked_m[e];
        if (live < 0) live = 0;
        if (live > T) live = T;
        const uint8_t *xe = (const uint8_t *)x + (size_t)(e * T * in_width) * in_elem;
        uint8_t *qe = q + e * T * K;
        uint8_t *se = (uint8_t *)s + (size_t)e * sb;
        for (int64_t t = 0; t < live; ++t)
            quant_row(xe, in_dtype, t, K, G, fuse, out_dtype, scale_fmt, scale_layout, eps,
                      qe, t, se, T, t);
    }
    return 0;
}

/* Whole-row per-token e4m3: scale = rowmax / 448 with no floor, multiplier
 * zero when the scale is zero, codes narrowed with saturation (a zero element
 * gives a zero code of its sign even when the multiplier overflowed, as in
 * scaled() above).
 * ([sglang #34257] key source snippets, the warp kernel.) */
int oracle_ptq_fp8(const void *x, int in_dtype, int64_t M, int64_t K, uint8_t *q, float *s)
{
    if (in_dtype != OR_BF16 && in_dtype != OR_FP16 && in_dtype != OR_FP32) return -1;
    if (M < 0 || K < 0) return -1;
    for (int64_t m = 0; m < M; ++m) {
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(decode_elem(x, in_dtype, m * K + k));
            if (a > amax) amax = a;
        }
        float r = amax / 448.0f;
        float inv = (r == 0.0f) ? 0.0f : 1.0f / r;
        s[m] = r;
        for (int64_t k = 0; k < K; ++k)
            q[m * K + k] = e4m3_rne_sat(scaled(decode_elem(x, in_dtype, m * K + k), inv));
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Per-token-group fp8 -> per-tensor fp8 requantization (masked layout).     */
/* ------------------------------------------------------------------------ */

/* Value of an e4m3 code (finite codes; 0x7F / 0xFF are NaN). */
static float e4m3_decode(uint8_t c)
{
    if (!e4m3_table_ready) e4m3_build_table();
    if ((c & 0x7F) == 0x7F) return NAN;
    const float mag = (float)e4m3_table[c & 0x7F];
    return (c & 0x80) ? -mag : mag;
}

/* For expert e and rows t < min(max(masked_m[e], 0), T) (every row when
 * masked_m is NULL): out[e][t][k] = e4m3_sat((dec(x[e][t][k]) * s) * inv) with
 * s = x_scale[e*se + t*st + (k/G)*sg] and inv = 1 / output_scale, each product
 * one fp32 rounding (a zero product keeps its sign whatever inv, as in
 * scaled() above); rows past masked_m keep out's contents.
 * ([sglang #35593] key source snippets: dequantize by the group scale, then
 * multiply by the reciprocal of the per-tensor output scale, saturating RN
 * narrowing; implementation breakdown: 128-wide scale groups, column-major
 * [E, M, hidden/128] scales, rows past masked_m untouched.) */
int oracle_requant_fp8(const uint8_t *x, int64_t E, int64_t T, int64_t K, int G,
                       const float *x_scale, int64_t se, int64_t st, int64_t sg,
                       const int32_t *masked_m, float output_scale, uint8_t *out)
{
    if (E < 0 || T < 0 || K < 0 || G <= 0 || K % G != 0) return -1;
    const float inv = 1.0f / output_scale;
    for (int64_t e = 0; e < E; ++e) {
        int64_t live = masked_m ? masked_m[e] : T;
        if (live < 0) live = 0;
        if (live > T) live = T;
        for (int64_t t = 0; t < live; ++t) {
            for (int64_t k = 0; k < K; ++k) {
                const int64_t i = (e * T + t) * K + k;
                const float s = x_scale[e * se + t * st + (k / G) * sg];
                const float h = e4m3_decode(x[i]) * s;
                out[i] = e4m3_rne_sat(scaled(h, inv));
            }
        }
    }
    return 0;
}

float oracle_e4m3_decode(uint8_t c) { return e4m3_decode(c); }

/* ------------------------------------------------------------------------ */
/* Dequantization: codes x group scales -> bf16 / fp16 / fp32.               */
/* ------------------------------------------------------------------------ */

/* Round a finite or infinite fp32 to the nearest bf16 (ties to even),
 * overflowing to infinity from the midpoint above the largest finite value. */
static uint16_t bf16_rne(float v)
{
    uint32_t b = bits_from_f32(v);
    if (isnan(v)) return (uint16_t)((b >> 16) | 0x40);
    uint16_t lo = (uint16_t)(b >> 16);                 /* truncated magnitude */
    uint16_t hi = (uint16_t)(lo + 1);
    double a = fabs((double)v);
    double alo = fabs((double)decode_bf16(lo));
    double ahi = fabs((double)decode_bf16(hi));
    /* Past the largest finite bf16 the next step up is infinity; IEEE rounds
     * as if the exponent range went on, i.e. towards 2^128. */
    if (isinf(ahi) && !isinf(alo)) ahi = ldexp(1.0, 128);
    if ((b & 0xFFFFu) == 0) return lo;
    double dlo = a - alo, dhi = ahi - a;
    if (dlo < dhi) return lo;
    if (dhi < dlo) return hi;
    return (lo & 1) ? hi : lo;
}

/* Round a finite fp32 to the nearest IEEE binary16 (ties to even),
 * overflowing to infinity from 65520 up. */
static uint16_t fp16_rne(float v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs((double)v);
    if (isnan(v)) return 0x7E00;
    if (a >= 65520.0) return sign | 0x7C00;
    int e = (a > 0) ? (int)floor(log2(a)) : -14;
    if (e < -14) e = -14;
    if (a >= ldexp(1.0, e + 1)) e += 1;             /* guard the log2 rounding */
    if (e > -14 && a < ldexp(1.0, e)) e -= 1;
    double ulp = ldexp(1.0, e - 10);
    double n = a / ulp;                             /* exact: a has <= 24 bits */
    double f = floor(n), frac = n - f;
    double r = (frac > 0.5) ? f + 1 : (frac < 0.5) ? f : (fmod(f, 2.0) == 0 ? f : f + 1);
    /* r * ulp, re-encoded: subnormals have exponent field 0 */
    double val = r * ulp;
    if (val == 0) return sign;
    int E = (int)floor(log2(val));
    if (val < ldexp(1.0, E)) E -= 1;
    if (E < -14) return sign | (uint16_t)(val / ldexp(1.0, -24));
    uint16_t m = (uint16_t)(val / ldexp(1.0, E - 10) - 1024.0);
    return sign | (uint16_t)((E + 15) << 10) | m;
}

static float scale_of(const void *s, int64_t rows, int64_t ng, int64_t m, int64_t g,
                      int scale_fmt, int scale_layout)
{
    if (scale_fmt == OR_SCALE_F32) {
        const float *f = (const float *)s;
        return scale_layout == OR_ROW_MAJOR ? f[m * ng + g] : f[g * pad4(rows) + m];
    }
    const uint8_t *b = (const uint8_t *)s;
    uint8_t e = scale_layout == OR_ROW_MAJOR ? b[m * ng + g]
                                             : b[((g / 4) * pad4(rows) + m) * 4 + (g % 4)];
    return f32_from_bits(e == 0 ? 0x00400000u : (uint32_t)e << 23);   /* 2^(e-127) */
}

/* y[m][k] = round_out(fl(decode(q[m][k]) * scale(m, k/G))): the product is one
 * fp32 rounding (exact for UE8M0 scales unless it underflows), then rounded
 * to the output dtype (round-to-nearest-even).  ([sglang #35593] key source
 * snippets, the test's reference: codes as float times the repeated group
 * scales; [sglang #30924] implementation breakdown: fp32-scale results are
 * checked by their dequantization.) */
int oracle_dequant(const uint8_t *q, int code_dtype, int64_t M, int64_t K, int G, const void *s,
                   int scale_fmt, int scale_layout, int out_dtype, void *y)
{
    if (M < 0 || K < 0 || G <= 0 || K % G != 0) return -1;
    if (code_dtype != OR_E4M3 && code_dtype != OR_INT8) return -1;
    const int64_t ng = K / G;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t k = 0; k < K; ++k) {
            const uint8_t c = q[m * K + k];
            const float d = code_dtype == OR_E4M3 ? e4m3_decode(c) : (float)(int8_t)c;
            const float v = d * scale_of(s, M, ng, m, k / G, scale_fmt, scale_layout);
            if (out_dtype == OR_BF16) ((uint16_t *)y)[m * K + k] = bf16_rne(v);
            else if (out_dtype == OR_FP16) ((uint16_t *)y)[m * K + k] = fp16_rne(v);
            else ((float *)y)[m * K + k] = v;
        }
    }
    return 0;
}

void oracle_bf16_rne_vec(const float *v, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_rne(v[i]);
}
void oracle_fp16_rne_vec(const float *v, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = fp16_rne(v[i]);
}

/* ------------------------------------------------------------------------ */
/* Element helpers, exported so that the tests can pin each step alone.      */
/* ------------------------------------------------------------------------ */

uint8_t oracle_e4m3(float v) { return e4m3_rne_sat(v); }
int8_t oracle_int8(float v) { return int8_rne_sat(v); }
float oracle_exp(float x) { return exp_cr(x); }
float oracle_silu_mul(float g, float u) { return silu_mul(g, u); }
float oracle_decode(uint16_t h, int dtype)
{
    return dtype == OR_FP16 ? decode_fp16(h) : decode_bf16(h);
}

/* Vector forms of the helpers (plain loops), so that exhaustive pins over
 * millions of values do not pay a foreign-call per element. */
void oracle_e4m3_vec(const float *v, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = e4m3_rne_sat(v[i]);
}
void oracle_int8_vec(const float *v, int8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = int8_rne_sat(v[i]);
}
void oracle_exp_vec(const float *x, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = exp_cr(x[i]);
}
void oracle_silu_mul_vec(const float *g, const float *u, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = silu_mul(g[i], u[i]);
}
void oracle_decode_vec(const uint16_t *h, int dtype, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_decode(h[i], dtype);
}

/* The scale step alone over many absmax values (for exhaustive device
 * probes): r, the UE8M0 byte and the multiplier of make_scale. */
void oracle_scale_vec(const float *amax, int64_t n, float eps, int out_dtype, int ue8m0,
                      float *r, uint8_t *e, float *inv)
{
    const float qmax = (out_dtype == OR_E4M3) ? 448.0f : 127.0f;
    for (int64_t i = 0; i < n; ++i) {
        group_scale gs = make_scale(amax[i], eps, qmax, ue8m0);
        if (r) r[i] = gs.r;
        if (e) e[i] = gs.ue8m0;
        if (inv) inv[i] = gs.inv;
    }
}
