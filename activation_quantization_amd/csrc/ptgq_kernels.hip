// Device kernels of libptgq: per-token-group 8-bit activation quantization
// for gfx950 (CDNA4, wave64).
//
// Design (see the layout notes in include/ptgq.h):
//   * A "slab" is one 16-byte load per lane across a wave: 64 x 8 sixteen-bit
//     elements = 512 consecutive elements of one row.  Each lane owns 8
//     consecutive elements, so a group of G elements is held by G/8 adjacent
//     lanes (2, 4, 8 or 16) and every load instruction of the wave reads one
//     contiguous kilobyte.  A task is 1..4 slabs of one row; all loads of a
//     task are issued before any arithmetic so each lane keeps several 16-byte
//     requests in flight.
//   * The group absmax is reduced with DPP lane moves inside the lane cluster
//     (quad_perm xor1, xor2, row_half_mirror, row_mirror: at most 4 steps, no
//     LDS, no barrier); every lane of the cluster then derives the scale and
//     multiplier itself.
//   * Codes are narrowed by the gfx950 packed fp32 -> OCP e4m3 conversion after
//     clamping to +-448 (round-to-nearest-even; saturation by the clamp), or by
//     round-to-nearest-even plus clamping for int8, and stored 8 bytes per lane,
//     contiguous across the wave.
//   * Packed column-major UE8M0 scales: the 4 groups sharing a 32-bit word sit
//     in the same slab; their leader lanes' bytes are gathered by lane
//     permutes and one lane stores the word.
//   * Blocks are remapped so that each of the 8 XCDs walks a contiguous range
//     of tasks (rows), which keeps the scattered column-major scale words of
//     neighbouring rows in one L2.
//
// Arithmetic follows the definition step by step in IEEE fp32 (the library is
// built without fast-math and without FP contraction; fp32 division is the
// correctly rounded sequence, denormals are kept):
//   sglang #30924 review page, key source snippets (ref_fp8_ue8m0): floor the
//   absmax by eps, divide by 448, UE8M0 = exponent field plus one if the
//   fraction is non-zero, multiplier rebuilt from (254 - e) << 23;
//   sglang #34257 review page, key source snippets: reciprocal multiply, zero
//   multiplier for a zero scale, clamp to +-448 before narrowing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ptgq_internal.h"

namespace ptgq {

// --------------------------------------------------------------------------
// Element widening (exact).
// --------------------------------------------------------------------------

__device__ __forceinline__ float fp16_to_f32(uint32_t h)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xFFFFu));
}

// 8 sixteen-bit elements in a uint4 -> 8 floats.
template <int IN>
__device__ __forceinline__ void widen8(const uint4 r, float (&f)[8])
{
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (IN == IN_BF16) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        } else {
            f[2 * i] = fp16_to_f32(w[i]);
            f[2 * i + 1] = fp16_to_f32(w[i] >> 16);
        }
    }
}

// --------------------------------------------------------------------------
// Maxima of non-negative floats, taken on their bit patterns (which order
// exactly like the values), so no NaN canonicalization is needed and each
// DPP step folds into one v_max_u32_dpp (old value 0, the identity).
// --------------------------------------------------------------------------

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_umax(uint32_t v)
{
    const uint32_t o =
        (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
    return v > o ? v : o;
}

// All lanes of each aligned LANES-lane cluster end with the cluster maximum.
template <int LANES>
__device__ __forceinline__ uint32_t cluster_max_bits(uint32_t v)
{
    if constexpr (LANES >= 2) v = dpp_umax<0xB1>(v);    // quad_perm [1,0,3,2]
    if constexpr (LANES >= 4) v = dpp_umax<0x4E>(v);    // quad_perm [2,3,0,1]
    if constexpr (LANES >= 8) v = dpp_umax<0x141>(v);   // row_half_mirror
    if constexpr (LANES >= 16) v = dpp_umax<0x140>(v);  // row_mirror
    if constexpr (LANES >= 32) {
        // rows 0 <-> 1 and 2 <-> 3: ds_swizzle bit mode, lane ^ 16 within 32
        const uint32_t o = (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);
        v = v > o ? v : o;
    }
    return v;
}

// Wave maximum, returned wave-uniform: row maxima, then row_bcast:15 into
// rows 1 and 3 and row_bcast:31 into rows 2 and 3, so lane 63 holds the lot.
__device__ __forceinline__ uint32_t wave_max_bits(uint32_t v)
{
    v = cluster_max_bits<16>(v);
    v = dpp_umax<0x142, 0xA>(v);                        // row_bcast:15
    v = dpp_umax<0x143, 0xC>(v);                        // row_bcast:31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// |x| maximum of 8 sixteen-bit floats (bf16 or fp16) held in 4 dwords, as the
// fp32 bit pattern of that maximum: magnitudes of both formats order like
// their bit patterns, so packed u16 maxima of (bits & 0x7FFF) suffice.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_umax16(uint32_t a, uint32_t b)
{
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}

template <int IN>
__device__ __forceinline__ uint32_t absmax8_bits(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3)
{
    const uint32_t m = pk_umax16(pk_umax16(w0 & 0x7FFF7FFFu, w1 & 0x7FFF7FFFu),
                                 pk_umax16(w2 & 0x7FFF7FFFu, w3 & 0x7FFF7FFFu));
    const uint32_t lo = m & 0xFFFFu, hi = m >> 16;
    const uint32_t h = lo > hi ? lo : hi;
    if constexpr (IN == IN_BF16)
        return h << 16;
    else
        return __float_as_uint(fp16_to_f32(h));
}

// |x| maximum of fp32 values, as a bit pattern: gfx950's three-operand
// IEEE maximum with |.| source modifiers, 4 instructions for 8 values.  For
// non-NaN values this is the largest magnitude exactly (-0 counts as +0);
// NaN propagates.
__device__ __forceinline__ uint32_t absmax_bits(const float (&y)[8])
{
    float m = __builtin_elementwise_maximum(__builtin_fabsf(y[0]), __builtin_fabsf(y[1]));
#pragma unroll
    for (int k = 2; k < 8; ++k) m = __builtin_elementwise_maximum(m, __builtin_fabsf(y[k]));
    return __float_as_uint(m);
}

__device__ __forceinline__ uint32_t absmax4_bits(const float (&y)[4])
{
    float m = __builtin_elementwise_maximum(__builtin_fabsf(y[0]), __builtin_fabsf(y[1]));
    m = __builtin_elementwise_maximum(m, __builtin_fabsf(y[2]));
    m = __builtin_elementwise_maximum(m, __builtin_fabsf(y[3]));
    return __float_as_uint(m);
}

// --------------------------------------------------------------------------
// Scale of one group: r = max(amax, eps) / qmax; fp32 multiplier 1/r (0 if
// r == 0), or UE8M0 byte e and exact multiplier 2^(127 - e).
// --------------------------------------------------------------------------

// UE8M0 without a division.  For a normal a with fl(a / qmax) normal (a at or
// above qmax * 2^-126), write a = 1.f * 2^(E-127) and qmax = 1.q * 2^EQ: the
// quotient's exponent field is E - EQ when 1.f >= 1.q and E - EQ - 1 when
// 1.f < 1.q, its fraction is zero only when 1.f == 1.q, and rounding the
// quotient to fp32 never carries it onto a power of two (no fp32 a lies within
// half an ulp below a power-of-two multiple of qmax).  Hence
//   e = E - EQ + (f > q).
// Checked against the division for every fp32 a at or above the threshold.
template <int OUT>
struct Ue8m0Consts;
template <>
struct Ue8m0Consts<OUT_E4M3> {  // 448 = 1.75 * 2^8
    static constexpr uint32_t EQ = 8, FQ = 0x600000u, THRESHOLD = 0x04E00000u;
};
template <>
struct Ue8m0Consts<OUT_INT8> {  // 127 = 1.984375 * 2^6
    static constexpr uint32_t EQ = 6, FQ = 0x7E0000u, THRESHOLD = 0x03FE0000u;
};

template <int OUT>
__device__ __forceinline__ uint32_t ue8m0_byte(float a, float qmax)
{
    using C = Ue8m0Consts<OUT>;
    const uint32_t b = __float_as_uint(a);
    uint32_t e = (b >> 23) - C::EQ + ((b & 0x7FFFFFu) > C::FQ ? 1u : 0u);
    if (b < C::THRESHOLD) {  // tiny a (eps below ~1e-35): exponent of the quotient
        const uint32_t rb = __float_as_uint(a / qmax);
        e = ((rb >> 23) & 0xFFu) + ((rb & 0x7FFFFFu) != 0u ? 1u : 0u);
    }
    return e;
}

struct Scale {
    float inv;       // multiplier applied to y
    float r;         // fp32 scale
    uint32_t e;      // UE8M0 byte
};

// `amax_bits` and `eps_bits`: bit patterns of non-negative floats (eps >= +0).
template <int OUT>
__device__ __forceinline__ Scale group_scale(uint32_t amax_bits, uint32_t eps_bits, bool ue8m0)
{
    const float qmax = (OUT == OUT_E4M3) ? 448.0f : 127.0f;
    Scale sc;
    const float a = __uint_as_float(amax_bits > eps_bits ? amax_bits : eps_bits);
    if (!ue8m0) {
        sc.r = a / qmax;
        sc.e = 0;
        sc.inv = (sc.r == 0.0f) ? 0.0f : 1.0f / sc.r;
    } else {
        sc.r = 0.0f;
        sc.e = ue8m0_byte<OUT>(a, qmax);
        sc.inv = __uint_as_float((254u - sc.e) << 23);
    }
    return sc;
}

// v = y * inv, one fp32 rounding per element, except that a zero y keeps its
// value (and sign) when inv is infinite.  fl(1/r) overflows for a scale r
// below about 2^-128 (an fp32 scale with no floor, or one under ~1.3e-36):
// the quotient y / r of a zero is then still zero, where the product 0 * inf
// would be NaN; every other y times inf saturates when narrowed.  A finite
// multiplier already gives y * inv == y for a zero y, so:
//   MUL_PLAIN  the caller knows inv is finite (UE8M0 multipliers, or a
//              uniform multiplier tested beforehand);
//   MUL_CHECK  per-lane multipliers: the fix-up runs only when some lane of
//              the wave holds an infinite one (a scalar branch);
//   MUL_FIX    the caller knows inv is infinite.
enum { MUL_PLAIN = 0, MUL_CHECK = 1, MUL_FIX = 2 };

template <int MODE, int N>
__device__ __forceinline__ void scale_by(const float (&y)[N], float inv, float (&v)[N])
{
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] = y[k] * inv;
    if constexpr (MODE == MUL_FIX) {
#pragma unroll
        for (int k = 0; k < N; ++k) v[k] = (y[k] == 0.0f) ? y[k] : v[k];
    } else if constexpr (MODE == MUL_CHECK) {
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(inv == __builtin_inff()) != 0, 0)) {
#pragma unroll
            for (int k = 0; k < N; ++k) v[k] = (y[k] == 0.0f) ? y[k] : v[k];
        }
    }
}

// Runs body(std::integral_constant<int, MUL_FIX or MUL_PLAIN>) for a
// wave-uniform multiplier: one scalar branch instead of a test per vector.
template <class Body>
__device__ __forceinline__ void with_uniform_multiplier(float inv, Body &&body)
{
    if (__builtin_expect(inv == __builtin_inff(), 0))
        body(std::integral_constant<int, MUL_FIX>{});
    else
        body(std::integral_constant<int, MUL_PLAIN>{});
}

// --------------------------------------------------------------------------
// Narrowing.
// --------------------------------------------------------------------------

// 4 floats -> 4 OCP e4m3 codes (byte i = code of value i), round to nearest
// even.  CLAMP saturates to +-448 first; without it the caller guarantees
// |v| <= 448 (true for UE8M0 scales: 2^(e-127) >= max(amax, eps) / 448
// exactly).  -0 and negative values that round to zero keep the sign bit.
template <bool CLAMP>
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d)
{
    if constexpr (CLAMP) {
        a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
        b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
        c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
        d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
    }
    int p = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    p = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, p, true);
    return (uint32_t)p;
}

// int8 code of v in the low byte of the result: v is clamped to [-128, 127]
// (the same as rounding first, the bounds being integers), then 1.5 * 2^23
// is added.  The sum lies in [2^23, 2^24), where the fp32 ulp is 1, and the
// offset is even, so round-to-nearest-even of the sum is the offset plus
// rne(v): the sum's low byte is the two's-complement code.  (Checked against
// rint + clamp + convert for every non-NaN fp32 value.)
__device__ __forceinline__ uint32_t int8_bits(float v)
{
    return __float_as_uint(__builtin_amdgcn_fmed3f(v, -128.0f, 127.0f) + 12582912.0f);
}

// 4 floats -> 4 int8 codes (byte i = code of value i), round to nearest
// even, saturated; two byte permutes (selector 0x0C: a zero byte).
__device__ __forceinline__ uint32_t int8x4(float a, float b, float c, float d)
{
    const uint32_t ab = __builtin_amdgcn_perm(int8_bits(b), int8_bits(a), 0x0C0C0400u);
    const uint32_t cd = __builtin_amdgcn_perm(int8_bits(d), int8_bits(c), 0x04000C0Cu);
    return ab | cd;
}

template <int OUT, bool CLAMP>
__device__ __forceinline__ uint32_t narrow4(const float (&v)[4])
{
    if constexpr (OUT == OUT_E4M3)
        return e4m3x4<CLAMP>(v[0], v[1], v[2], v[3]);
    else
        return int8x4(v[0], v[1], v[2], v[3]);
}

template <int OUT, bool CLAMP>
__device__ __forceinline__ uint2 narrow8(const float (&v)[8])
{
    uint2 o;
    if constexpr (OUT == OUT_E4M3) {
        o.x = e4m3x4<CLAMP>(v[0], v[1], v[2], v[3]);
        o.y = e4m3x4<CLAMP>(v[4], v[5], v[6], v[7]);
    } else {
        o.x = int8x4(v[0], v[1], v[2], v[3]);
        o.y = int8x4(v[4], v[5], v[6], v[7]);
    }
    return o;
}

// --------------------------------------------------------------------------
// Direct SiLU for 16-bit gates: s(g) = g / (1 + e), e = e^-g correctly
// rounded to fp32, the add and the quotient correctly rounded fp32 steps.
//
// e: Cody and Waite's reduction -g = k ln 2 + r (ln 2 split into a 32-bit
// head and a tail, so k * head is exact; |r| <= ln 2 / 2), the Taylor
// polynomial of e^r of degree 9 by Horner's rule, all fp64 FMAs, scaled by
// 2^k and rounded once to fp32.  For each of the 128 768 finite bf16 and
// fp16 gates its relative error (at most 2^-36.6) is smaller than the
// distance of e^-g from the nearest fp32 rounding midpoint, so the rounding
// is the correct one: a host simulation of these fp64 steps gives the
// correctly rounded e^-g for every gate (degree 8 does not), and the device
// probe compares every gate against the oracle.  Gates outside [-100, 120]
// are clamped to it: e^-g then rounds to +inf (g < -88.73) or to 0
// (g > 103.98) either way.
//
// The quotient: g times the reciprocal of d in fp64 (the hardware
// reciprocal, about 2^-24.4 relative error, then one Newton step, which
// squares it), rounded to fp32.  The fp64 product is within 2^-48.5 of
// g / d, and over all gates no quotient that is not itself an fp32 value
// lies within 2^-48 of an fp32 midpoint, so the rounding equals the IEEE
// fp32 division (also checked for every gate by the probe).  d = +inf (g < -88.73): the
// reciprocal is 0 and the Newton term NaN, which the max turns into -1, so
// s = g * 0 = -0, the IEEE quotient.
// --------------------------------------------------------------------------

__device__ __forceinline__ float silu_s(float g)
{
    const float gc = __builtin_amdgcn_fmed3f(g, -100.0f, 120.0f);
    const double x = -(double)gc;
    const double k = __builtin_rint(x * 0x1.71547652b82fep+0);       // x / ln 2
    double r = __builtin_fma(-k, 0x1.62e42fee00000p-1, x);           // ln 2, head
    r = __builtin_fma(-k, 0x1.a39ef35793c76p-33, r);                  // ln 2, tail
    double p = 0x1.71de3a556c734p-19;                                 // 1/9!
    p = __builtin_fma(p, r, 0x1.a01a01a01a01ap-16);                   // 1/8!
    p = __builtin_fma(p, r, 0x1.a01a01a01a01ap-13);                   // 1/7!
    p = __builtin_fma(p, r, 0x1.6c16c16c16c17p-10);                   // 1/6!
    p = __builtin_fma(p, r, 0x1.1111111111111p-7);                    // 1/5!
    p = __builtin_fma(p, r, 0x1.5555555555555p-5);                    // 1/4!
    p = __builtin_fma(p, r, 0x1.5555555555555p-3);                    // 1/3!
    p = __builtin_fma(p, r, 0.5);
    p = __builtin_fma(p, r, 1.0);
    p = __builtin_fma(p, r, 1.0);
    const float e = (float)__builtin_ldexp(p, (int)k);
    const double d = (double)(1.0f + e);
    const double y0 = __builtin_amdgcn_rcp(d);
    const double t = __builtin_fmax(__builtin_fma(-d, y0, 1.0), -1.0);
    return (float)((double)g * __builtin_fma(y0, t, y0));
}

// --------------------------------------------------------------------------
// SiLU lookup for bf16 gates.  s(g) depends on the 16 bits of g only.
// Outside |g| in [2^-25, 2^7) it has a closed form that the IEEE steps reach
// exactly: |g| < 2^-25 gives e^-g rounded to 1, so s = g/2; g >= 2^7 gives
// e^-g rounded to 0, so s = g; g <= -2^7 gives e^-g = +inf, so s = -0.  The
// 2 x 32 binades in between (8192 values) are tabulated by the direct
// evaluation above, on the device, once per device.
// --------------------------------------------------------------------------

constexpr uint32_t kTabElo = 127 - 25;   // biased exponent of 2^-25
constexpr uint32_t kTabEhi = 127 + 6;    // biased exponent of [2^6, 2^7)
constexpr uint32_t kTabNE = kTabEhi - kTabElo + 1;
constexpr int kSiluTab = 2 * kTabNE * 128;   // 8192 floats = 32 KiB

__device__ float g_silu_table[kSiluTab];

// SiLU lookup for fp16 gates: magnitudes below 8 (bit patterns below 0x4800:
// the subnormals and the 17 binades 2^-14 .. 2^2), both signs, 36 864
// values (144 KiB), tabulated by the direct evaluation; the entry of gate h
// is (h & 0x7FFF) + (sign ? 0x4800 : 0).  Larger gates, rare in activations,
// are evaluated directly.
constexpr uint32_t kTab16Mag = 0x4800;
constexpr int kSiluTab16 = 2 * (int)kTab16Mag;   // 36864 floats = 144 KiB

__device__ float g_silu_table16[kSiluTab16];

// Floats of the lookup table of a gate type.
template <int IN>
constexpr int table_floats()
{
    return IN == IN_BF16 ? kSiluTab : kSiluTab16;
}

// Both tables: threads [0, kSiluTab) the bf16 one, the next kSiluTab16 the
// fp16 one.
__global__ __launch_bounds__(256) void silu_table_init_kernel()
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < kSiluTab) {
        const uint32_t sign = (uint32_t)i / (kTabNE * 128);
        const uint32_t E = kTabElo + ((uint32_t)i / 128) % kTabNE;
        const uint32_t h = (sign << 15) | (E << 7) | ((uint32_t)i & 127u);
        g_silu_table[i] = silu_s(__uint_as_float(h << 16));
    } else if (i < kSiluTab + kSiluTab16) {
        const uint32_t j = (uint32_t)(i - kSiluTab);
        const uint32_t h = ((j / kTab16Mag) << 15) | (j % kTab16Mag);
        g_silu_table16[j] = silu_s(fp16_to_f32(h));
    }
}

__device__ __forceinline__ float silu_s_lookup(uint32_t h, const float *tab)
{
    const uint32_t E = (h >> 7) & 0xFFu;
    const uint32_t sign = (h >> 15) & 1u;
    const float g = __uint_as_float(h << 16);
    const uint32_t Ec = E < kTabElo ? kTabElo : (E > kTabEhi ? kTabEhi : E);
    const float t = tab[((sign * kTabNE + (Ec - kTabElo)) << 7) | (h & 0x7Fu)];
    const float big = sign ? -0.0f : g;
    return E < kTabElo ? g * 0.5f : (E > kTabEhi ? big : t);
}

// Two bf16 gates packed in a dword -> LDS byte offsets of their table entries
// (valid when both gates' magnitudes lie in the tabulated binades; `in_range`
// says whether they do).  The table index of a gate is
// (|bits| - Elo*128) + sign*NE*128 with NE*128 = 4096 = (bit 15) >> 3, so the
// two 16-bit halves are clamped with packed u16 min/max and the rest is done
// on the whole dword without any carry crossing the halves.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void silu_pair_offsets(uint32_t w, uint32_t &off_lo, uint32_t &off_hi,
                                                  bool &in_range)
{
    constexpr uint32_t lo = kTabElo << 7;
    constexpr uint32_t hi = ((kTabEhi + 1) << 7) - 1;
    static_assert(kTabNE * 128 == 4096, "sign offset is bit 15 >> 3");
    const uint32_t mag = w & 0x7FFF7FFFu;
    const u16x2 lo2 = {(unsigned short)lo, (unsigned short)lo};
    const u16x2 hi2 = {(unsigned short)hi, (unsigned short)hi};
    const uint32_t c = __builtin_bit_cast(
        uint32_t, __builtin_elementwise_min(__builtin_elementwise_max(
                                                __builtin_bit_cast(u16x2, mag), lo2), hi2));
    in_range = c == mag;
    const uint32_t idx = ((c - lo * 0x10001u) | ((w & 0x80008000u) >> 3)) << 2;
    off_lo = idx & 0xFFFFu;
    off_hi = idx >> 16;
}

__device__ __forceinline__ float lds_f32_at(const float *tab, uint32_t byte_off)
{
    return *reinterpret_cast<const float *>(reinterpret_cast<const char *>(tab) + byte_off);
}

// Two fp16 gates packed in a dword -> byte offsets of their fp16-table
// entries, each magnitude first clamped into the table (packed u16 min) so
// that every offset lies inside it; `in_range` says whether both gates are
// tabulated.  The two entry indices stay below 2^16, so they are formed on
// the whole dword without a carry crossing the halves.
__device__ __forceinline__ void silu16_pair_offsets(uint32_t w, uint32_t &off_lo,
                                                    uint32_t &off_hi, bool &in_range)
{
    const uint32_t mag = w & 0x7FFF7FFFu;
    const u16x2 top = {(unsigned short)(kTab16Mag - 1), (unsigned short)(kTab16Mag - 1)};
    const uint32_t c = __builtin_bit_cast(
        uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, mag), top));
    in_range = c == mag;
    const uint32_t idx = c + ((w >> 15) & 0x00010001u) * kTab16Mag;
    off_lo = (idx & 0xFFFFu) << 2;
    off_hi = (idx >> 16) << 2;
}

// --------------------------------------------------------------------------
// Group quantization tasks.
//   A task is UMAX consecutive slabs of one row: slabs [j*UMAX, j*UMAX+UMAX)
//   of row m; a slab is 512 consecutive elements of the row, one 16-byte load
//   per lane.  Loads and code stores go through per-row buffer resources, so
//   a slab or lane past the end of the row reads zeros without touching
//   memory and its code store is dropped by the hardware range check: a task
//   has no branches.  The next task's loads are issued before the current
//   task is processed (two buffers), so each wave keeps its loads in flight
//   while it computes and stores.
// --------------------------------------------------------------------------

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Cache policy of the streaming accesses: non-temporal ("nt"), since every
// input byte is read once and every code byte written once.  Measured on
// MI355X for this 2:1 read/write mix: 6.4 TB/s non-temporal against 5.9 TB/s
// with the default policy.  Scale words keep the default policy so that the
// partial lines of neighbouring rows merge in L2.
constexpr int kStreamPolicy = 2;
// Code stores of the flat SiLU-table kernel (persistent 16-wave blocks) keep
// the default policy: measured on MI355X, fused [8192, 2*4096] 29.3 us with
// non-temporal code stores, 28.6 us with the default (or sc0 / sc1) policy.
// Every other kernel's code stores are non-temporal (the masked SiLU-table
// kernel: 13.4 us non-temporal, 13.7 us default).
constexpr int kTableStorePolicy = 0;
// Dequantized output (two or four bytes written per byte read): system-scope
// (sc1) non-temporal stores, measured 57.4 -> 56.9 us at [16384, 7168] -> bf16
// (default policy: 59.7 us).
constexpr int kDequantStorePolicy = 16 | 2;
// and its code loads keep the default policy (57.0 -> 56.4 us against
// non-temporal code loads).
constexpr int kDequantLoadPolicy = 0;

// Raw (unstructured) buffer resource over [base, base + bytes); the third
// dword selects 32-bit data format, as gfx9 raw buffers expect.
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes,
                                             0x00020000);
}

// A task's loads: per slab, 16 bytes per lane of the input (gate) half and,
// when fused, of the up half; fp32 input takes 32 bytes per lane (g, then gh).
template <int UMAX>
struct TaskBuf {
    u32x4 g[UMAX];
    u32x4 gh[UMAX];
    u32x4 u[UMAX];
};

// Where a task lives.  `xb` / `qb` are the base of the region the task's
// input (gate half when fused) and codes are addressed from, `xrange` /
// `qrange` that region's bytes (loads past it read zeros, stores past it are
// dropped by the buffer range check), and `c0` the offset, in elements, of
// the task's first slab from the bases.  The region is the task's row (its
// last task may run past the row end), extended for a flat-slab task by the
// slab that crosses into the next row.  `codes` is the number of elements of
// the task (fewer than UMAX slabs at the end of a row, or of the tensor).
// `sbase` is the scale tensor of the rows (flat: the whole tensor; masked:
// the expert's); `m` and `j` are the row and the slab index within that row
// of the first slab.  Row tasks keep all their slabs in row m; flat-slab
// tasks move on to row m + 1 when a slab index reaches spr.  (Measured on
// MI355X, same addresses, bf16 -> e4m3: buffer descriptors based at the row
// are faster than descriptors based at each task, [256, 7168] 3.0 against
// 3.19 us, or one descriptor over the whole tensor, [4096, 7168] 15.4
// against 15.9 us.)
struct TaskLoc {
    const char *xb;
    uint8_t *qb;
    uint8_t *sbase;
    uint32_t xrange;
    uint32_t qrange;
    uint32_t c0;
    uint32_t codes;
    int64_t m;
    int j;
    int next_row;   // flat-slab tasks: first slab (0..UMAX) that lies in row m + 1
    uint32_t row0;  // fused slabs of the flattened tensor: the row `xb` points at
};

// `live` false: the loads are issued over an empty range (zeros, no memory
// traffic), so that every path through the task loop issues the same loads
// and the wait counts stay exact.
template <int IN, bool FUSE, int UMAX, int FS = 0>
__device__ __forceinline__ void load_task(const GroupArgs &a, const TaskLoc &t, int lane,
                                          bool live, TaskBuf<UMAX> &b)
{
    constexpr int ES = IN == IN_FP32 ? 4 : 2;   // input element bytes
    constexpr int pol = kStreamPolicy;
    const uint32_t bytes = live ? t.xrange : 0u;
    const rsrc_t rg = make_rsrc(t.xb, bytes);
    if constexpr (FUSE && FS == 3) {
        // slabs of the flattened output: a lane's 8 elements lie in one row
        // (8 divides G, which divides K); their gate and up halves sit at
        // column c of row r's [gate | up] input, r counted from row0
        const uint32_t K = (uint32_t)a.K;
#pragma unroll
        for (int s = 0; s < UMAX; ++s) {
            const uint32_t e = ((uint32_t)t.m + s) * kSlab + (uint32_t)lane * 8;   // < 2^31
            const uint32_t r = fastdiv(e, a.k_div);
            const uint32_t off = ((r - t.row0) * 2 * K + (e - r * K)) * 2;
            b.g[s] = __builtin_amdgcn_raw_buffer_load_b128(rg, off, 0, pol);
            b.u[s] = __builtin_amdgcn_raw_buffer_load_b128(rg, off + K * 2, 0, pol);
        }
        return;
    }
    // 16-bit: lane l holds elements 8l..8l+7 of a slab; fp32: 4l..4l+3 (g)
    // and 256+4l..256+4l+3 (gh), so every load instruction reads one
    // contiguous KiB
    const uint32_t off = t.c0 * ES + (uint32_t)lane * 16;
#pragma unroll
    for (int s = 0; s < UMAX; ++s) {
        b.g[s] = __builtin_amdgcn_raw_buffer_load_b128(rg, off + s * kSlab * ES, 0, pol);
        if constexpr (IN == IN_FP32)
            b.gh[s] = __builtin_amdgcn_raw_buffer_load_b128(rg, off + s * kSlab * ES + 1024, 0, pol);
    }
    if constexpr (FUSE) {
        static_assert(IN != IN_FP32, "fused calls take 16-bit inputs");
        const rsrc_t ru = make_rsrc(t.xb + a.K * ES, bytes);
#pragma unroll
        for (int s = 0; s < UMAX; ++s)
            b.u[s] = __builtin_amdgcn_raw_buffer_load_b128(ru, off + s * kSlab * 2, 0, pol);
    }
}

__device__ __forceinline__ uint4 as_uint4(u32x4 v) { return make_uint4(v.x, v.y, v.z, v.w); }

// The scale of group f of the tensor's group sequence (slabs of the
// flattened tensor): group f % ng of row f / ng, a multiply-high division
// (f < 2^31).  A packed column-major word may take its groups from two slabs
// (two waves), so its bytes are stored one by one; the lane of a row's last
// group also zeroes the unused bytes of the row's last, partial word.
template <bool UE8M0>
__device__ __forceinline__ void flat_group_scale(const GroupArgs &a, uint8_t *se, uint32_t f,
                                                 const Scale &sc)
{
    const uint32_t mr = fastdiv(f, a.ng_div);
    const uint32_t gr = f - mr * (uint32_t)a.ng;
    if constexpr (UE8M0) {
        if (a.scale_layout == LAYOUT_COL) {
            uint8_t *wb = se + ((int64_t)(gr >> 2) * a.rows_pad + mr) * 4;
            wb[gr & 3] = (uint8_t)sc.e;
            if (gr + 1 == (uint32_t)a.ng)
                for (uint32_t b = (gr & 3) + 1; b < 4; ++b) wb[b] = 0;
        } else {
            se[f] = (uint8_t)sc.e;
        }
    } else if (a.scale_layout == LAYOUT_ROW) {
        reinterpret_cast<float *>(se)[f] = sc.r;
    } else {
        reinterpret_cast<float *>(se)[(int64_t)gr * a.rows_pad + mr] = sc.r;
    }
}

// Fused calls of a few slabs, which are latency-bound: one wave per chunk of
// kChunk output elements of a row, two per lane, so that the SiLU work of a
// wave, its critical path, is a quarter of a slab's and spreads over four
// times as many waves.  A row has tpr chunks, the last one possibly short (G
// divides K).  A group is G/2 adjacent lanes; its leader stores the scale
// into the layout's slot.
// A chunk task's row: its input row (gate half first), its code row, the
// scale tensor it writes, its row index m in that tensor, and the chunk's
// first column.
struct ChunkLoc {
    const char *xr;
    uint8_t *qr;
    uint8_t *s;
    uint32_t m;
    uint32_t c0;
};

// Flat schedule: task t is chunk t % tpr of row t / tpr (spr = tpr).
struct FlatChunkMap {
    __device__ __forceinline__ ChunkLoc operator()(const GroupArgs &a, int t, int /*lane*/)
    {
        const uint32_t m = fastdiv((uint32_t)t, a.spr_div);
        const uint32_t c0 = ((uint32_t)t - m * (uint32_t)a.spr) * (uint32_t)kChunk;
        ChunkLoc l;
        l.xr = static_cast<const char *>(a.x) + (uint64_t)m * a.in_stride;
        l.qr = a.q + (uint64_t)m * a.K;
        l.s = static_cast<uint8_t *>(a.s);
        l.m = m;
        l.c0 = c0;
        return l;
    }
};

template <int IN, int G, int OUT, int SF, class Map>
__device__ __forceinline__ void run_chunk_tasks(const GroupArgs &a, Map map, int first, int n,
                                                int stride, int lane)
{
    constexpr int LPG = G / 2;                           // lanes per group (8..64)
    constexpr bool ue8m0 = SF == SCALE_UE8M0;
    constexpr int pol = kStreamPolicy;
    static_assert(IN != IN_FP32, "fused calls take 16-bit inputs");
    const uint32_t K = (uint32_t)a.K;
    for (int t = first; t < n; t += stride) {
        const ChunkLoc l = map(a, t, lane);
        const uint32_t c0 = l.c0;
        const uint32_t cnt = K - c0 < (uint32_t)kChunk ? K - c0 : (uint32_t)kChunk;
        const char *xr = l.xr + c0 * 2;
        const uint32_t wg =
            __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(xr, cnt * 2), lane * 4, 0, pol);
        const uint32_t wu = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(xr + K * 2, cnt * 2),
                                                                 lane * 4, 0, pol);
        float y[2];
        if constexpr (IN == IN_BF16) {
            y[0] = silu_s(__uint_as_float(wg << 16)) * __uint_as_float(wu << 16);
            y[1] = silu_s(__uint_as_float(wg & 0xFFFF0000u)) *
                   __uint_as_float(wu & 0xFFFF0000u);
        } else {
            y[0] = silu_s(fp16_to_f32(wg)) * fp16_to_f32(wu);
            y[1] = silu_s(fp16_to_f32(wg >> 16)) * fp16_to_f32(wu >> 16);
        }
        uint32_t amax = __float_as_uint(
            __builtin_elementwise_maximum(__builtin_fabsf(y[0]), __builtin_fabsf(y[1])));
        if constexpr (LPG == 64)
            amax = wave_max_bits(amax);
        else
            amax = cluster_max_bits<LPG>(amax);
        const Scale sc = group_scale<OUT>(amax, __float_as_uint(a.eps), ue8m0);
        float v[2];
        scale_by<ue8m0 ? MUL_PLAIN : MUL_CHECK>(y, sc.inv, v);
        const float v4[4] = {v[0], v[1], 0.0f, 0.0f};
        const uint32_t codes = narrow4<OUT, !ue8m0>(v4);
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)codes, make_rsrc(l.qr + c0, cnt),
                                              lane * 2, 0, pol);
        const uint32_t col = c0 + (uint32_t)lane * 2;
        if (lane % LPG == 0 && col < K)
            flat_group_scale<ue8m0>(a, l.s, l.m * (uint32_t)a.ng + col / G, sc);
    }
}

// One slab of fp32 input: lane l holds elements 4l..4l+3 (half A, `ga`) and
// 256+4l..256+4l+3 (half B, `gb`) of the slab, so a group of G elements is
// held by G/4 adjacent lanes of one half and every lane derives two scales.
// Codes are stored 4 bytes per lane and half (each store instruction writes
// 256 contiguous bytes; stores past the row are dropped); scales go to the
// layout's slots like those of the 16-bit path.
// `slab`: index of the slab within row m; `at`: offset of the slab's first
// code from the task's first code, `c0`: offset of that from the code
// region's base, `codes`: the task's code count.
template <int G, int OUT, int SF, int SPOL, int FS = 0>
__device__ __forceinline__ void process_slab_fp32(const GroupArgs &a, const u32x4 &ga,
                                                  const u32x4 &gb, int slab, uint32_t at,
                                                  uint32_t c0, uint32_t codes, rsrc_t rq,
                                                  uint8_t *se, int64_t m, int lane)
{
    constexpr int LA = G / 4;           // lanes per group within a half (4..32)
    constexpr int GPH = 256 / G;        // groups per half (2..16)
    constexpr int GPS = kSlab / G;      // groups per slab
    constexpr bool ue8m0 = SF == SCALE_UE8M0;
    const uint32_t colA = at + (uint32_t)lane * 4;     // offsets within the task
    const uint32_t colB = colA + 256;
    const bool validA = colA < codes, validB = colB < codes;
    const float ya[4] = {__uint_as_float(ga.x), __uint_as_float(ga.y), __uint_as_float(ga.z),
                         __uint_as_float(ga.w)};
    const float yb[4] = {__uint_as_float(gb.x), __uint_as_float(gb.y), __uint_as_float(gb.z),
                         __uint_as_float(gb.w)};
    const uint32_t amA = cluster_max_bits<LA>(absmax4_bits(ya));
    const uint32_t amB = cluster_max_bits<LA>(absmax4_bits(yb));
    const Scale sA = group_scale<OUT>(amA, __float_as_uint(a.eps), ue8m0);
    const Scale sB = group_scale<OUT>(amB, __float_as_uint(a.eps), ue8m0);
    float va[4], vb[4];
    scale_by<ue8m0 ? MUL_PLAIN : MUL_CHECK>(ya, sA.inv, va);
    scale_by<ue8m0 ? MUL_PLAIN : MUL_CHECK>(yb, sB.inv, vb);
    __builtin_amdgcn_raw_buffer_store_b32(narrow4<OUT, !ue8m0>(va), rq, c0 + colA, 0, SPOL);
    __builtin_amdgcn_raw_buffer_store_b32(narrow4<OUT, !ue8m0>(vb), rq, c0 + colB, 0, SPOL);

    const int lg = lane / LA;                          // group within the half
    const bool leader = (lane % LA) == 0;
    if constexpr (FS == 3) {
        // slabs of the flattened tensor: m is the slab's index in it
        const uint32_t fA = (uint32_t)(m * GPS + lg);
        if (leader && validA) flat_group_scale<SF == SCALE_UE8M0>(a, se, fA, sA);
        if (leader && validB) flat_group_scale<SF == SCALE_UE8M0>(a, se, fA + GPH, sB);
        return;
    }
    const int64_t g0 = (int64_t)slab * GPS;            // first group of the slab
    const int64_t gA = g0 + lg, gB = g0 + GPH + lg;
    if constexpr (ue8m0) {
        if (a.scale_layout == LAYOUT_COL) {
            const uint32_t byteA = validA ? sA.e : 0u, byteB = validB ? sB.e : 0u;
            uint32_t *words = reinterpret_cast<uint32_t *>(se);
            if constexpr (GPH <= 4) {
                // G >= 64: the slab's 4 or 8 groups, read from their leaders
#pragma unroll
                for (int w = 0; w < GPS / 4; ++w) {
                    uint32_t word = 0;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int gi = 4 * w + i;      // group within the slab
                        const uint32_t bi =
                            gi < GPH ? (uint32_t)__builtin_amdgcn_readlane((int)byteA, gi * LA)
                                     : (uint32_t)__builtin_amdgcn_readlane((int)byteB,
                                                                           (gi - GPH) * LA);
                        word |= bi << (8 * i);
                    }
                    const int64_t gw = g0 + 4 * w;
                    if (lane == 0 && at < codes && gw < a.ng)
                        words[(gw >> 2) * a.rows_pad + m] = word;
                }
            } else {
                // G <= 32: each word's 4 groups lie in one half
                const uint32_t a1 = (uint32_t)__shfl((int)byteA, lane + LA);
                const uint32_t a2 = (uint32_t)__shfl((int)byteA, lane + 2 * LA);
                const uint32_t a3 = (uint32_t)__shfl((int)byteA, lane + 3 * LA);
                const uint32_t b1 = (uint32_t)__shfl((int)byteB, lane + LA);
                const uint32_t b2 = (uint32_t)__shfl((int)byteB, lane + 2 * LA);
                const uint32_t b3 = (uint32_t)__shfl((int)byteB, lane + 3 * LA);
                if (leader && (lg & 3) == 0) {
                    if (validA)
                        words[(gA >> 2) * a.rows_pad + m] = byteA | (a1 << 8) | (a2 << 16) | (a3 << 24);
                    if (validB)
                        words[(gB >> 2) * a.rows_pad + m] = byteB | (b1 << 8) | (b2 << 16) | (b3 << 24);
                }
            }
        } else if (leader) {
            if (validA) se[m * a.ng + gA] = (uint8_t)sA.e;
            if (validB) se[m * a.ng + gB] = (uint8_t)sB.e;
        }
    } else if (leader) {
        float *sf = reinterpret_cast<float *>(se);
        if (a.scale_layout == LAYOUT_ROW) {
            if (validA) sf[m * a.ng + gA] = sA.r;
            if (validB) sf[m * a.ng + gB] = sB.r;
        } else {
            if (validA) sf[gA * a.rows_pad + m] = sA.r;
            if (validB) sf[gB * a.rows_pad + m] = sB.r;
        }
    }
}

template <int IN, int G, bool FUSE, int OUT, int SF, int UMAX, bool TABLE, int SPOL,
          int FS = 0>
__device__ __forceinline__ void process_task(const GroupArgs &a, const TaskLoc &t, int lane,
                                             const TaskBuf<UMAX> &b, const float *tab)
{
    constexpr int LPG = G / 8;          // lanes per group
    constexpr int GPS = kSlab / G;      // groups per slab (>= 4)
    const rsrc_t rq = make_rsrc(t.qb, t.qrange);
    uint8_t *se = t.sbase;
    constexpr bool ue8m0 = SF == SCALE_UE8M0;
#pragma unroll
    for (int s = 0; s < UMAX; ++s) {
        // row and slab-within-row of slab s; flat-slab tasks cross into the
        // next row (whole slabs only: K is a multiple of the slab)
        int slab = t.j + s;
        int64_t m = t.m;
        if constexpr (FS) {
            // 1 when slab s lies in the next row: the sign bit of
            // next_row - s - 1, plain integer arithmetic (a comparison would
            // be materialized through a vector register)
            const int nx = (int)((uint32_t)(t.next_row - s - 1) >> 31);
            slab -= nx * a.spr;
            m += nx;
        }
        const uint32_t at = (uint32_t)s * kSlab;                    // offset in the task
        if constexpr (IN == IN_FP32) {
            process_slab_fp32<G, OUT, SF, SPOL, FS>(a, b.g[s], b.gh[s], slab, at, t.c0, t.codes,
                                                    rq, se, m, lane);
            continue;
        }
        const uint32_t col = at + (uint32_t)lane * 8;              // in the task
        const bool valid = col < t.codes;
        float y[8];
        if constexpr (FUSE && TABLE) {
            const u32x4 w = b.g[s];
            float u[8];
            widen8<IN>(as_uint4(b.u[s]), u);
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
            uint32_t off[8];
            bool in[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if constexpr (IN == IN_BF16)
                    silu_pair_offsets(ww[k], off[2 * k], off[2 * k + 1], in[k]);
                else
                    silu16_pair_offsets(ww[k], off[2 * k], off[2 * k + 1], in[k]);
            }
            if (__all(in[0] && in[1] && in[2] && in[3])) {
                // every gate of the wave is tabulated: plain lookups
#pragma unroll
                for (int k = 0; k < 8; ++k) y[k] = lds_f32_at(tab, off[k]) * u[k];
            } else if constexpr (IN == IN_BF16) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    y[2 * k] = silu_s_lookup(ww[k] & 0xFFFFu, tab) * u[2 * k];
                    y[2 * k + 1] = silu_s_lookup(ww[k] >> 16, tab) * u[2 * k + 1];
                }
            } else {
                // fp16 gates of magnitude 8 or more: the direct evaluation
                // (the clamped offsets keep every lookup inside the table)
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const uint32_t h = (k & 1) ? ww[k / 2] >> 16 : ww[k / 2] & 0xFFFFu;
                    const float t = lds_f32_at(tab, off[k]);
                    y[k] = ((h & 0x7FFFu) < kTab16Mag ? t : silu_s(fp16_to_f32(h))) * u[k];
                }
            }
        } else if constexpr (IN == IN_FP32) {
            const uint32_t w[8] = {b.g[s].x, b.g[s].y, b.g[s].z, b.g[s].w,
                                   b.gh[s].x, b.gh[s].y, b.gh[s].z, b.gh[s].w};
#pragma unroll
            for (int k = 0; k < 8; ++k) y[k] = __uint_as_float(w[k]);
        } else {
            widen8<IN>(as_uint4(b.g[s]), y);
            if constexpr (FUSE) {
                float u[8];
                widen8<IN>(as_uint4(b.u[s]), u);
#pragma unroll
                for (int k = 0; k < 8; ++k) y[k] = silu_s(y[k]) * u[k];
            }
        }
        uint32_t amax;
        if constexpr (FUSE || IN == IN_FP32)
            amax = absmax_bits(y);
        else
            amax = absmax8_bits<IN>(b.g[s].x, b.g[s].y, b.g[s].z, b.g[s].w);
        amax = cluster_max_bits<LPG>(amax);

        const Scale sc = group_scale<OUT>(amax, __float_as_uint(a.eps), ue8m0);
        float v[8];
        scale_by<ue8m0 ? MUL_PLAIN : MUL_CHECK>(y, sc.inv, v);
        const uint2 codes = narrow8<OUT, !ue8m0>(v);
        u32x2 c2;
        c2.x = codes.x;
        c2.y = codes.y;
        __builtin_amdgcn_raw_buffer_store_b64(c2, rq, t.c0 + col, 0, SPOL);  // dropped past the region

        // scales of the slab's groups
        const int lg = lane / LPG;                                  // group within slab
        const int64_t g0 = (int64_t)slab * GPS;                     // first group of slab
        const bool leader = (lane % LPG) == 0;
        if constexpr (FS == 3) {
            // slabs of the flattened tensor: slab m holds groups m * GPS ..
            // m * GPS + GPS - 1 of the tensor's group sequence (G divides K,
            // so no group crosses a row)
            if (leader && valid)
                flat_group_scale<ue8m0>(a, se, (uint32_t)(m * GPS + lg), sc);
            continue;
        }
        if constexpr (FS == 2) {
            // multi-row slabs: slab m of the sequence holds groups m * GPS ..
            // m * GPS + GPS - 1 of the tensor taken as one sequence of groups;
            // group f is group f % ng of row f / ng (ng a power of two).  A
            // packed word's groups (four, or the row's ng < 4) are consecutive
            // groups of one slab.
            const int64_t f = m * GPS + lg;
            const int64_t mr = f >> a.mr_shift;
            const int64_t gr = f & (a.ng - 1);
            if constexpr (ue8m0) {
                if (a.scale_layout == LAYOUT_COL) {
                    const uint32_t byte = sc.e;
                    const uint32_t b1 = (uint32_t)__shfl((int)byte, lane + LPG);
                    const uint32_t b2 = (uint32_t)__shfl((int)byte, lane + 2 * LPG);
                    const uint32_t b3 = (uint32_t)__shfl((int)byte, lane + 3 * LPG);
                    if (leader && valid && (gr & 3) == 0) {
                        uint32_t word = byte;
                        if (a.ng > 1) word |= b1 << 8;
                        if (a.ng > 2) word |= (b2 << 16) | (b3 << 24);
                        reinterpret_cast<uint32_t *>(se)[(gr >> 2) * a.rows_pad + mr] = word;
                    }
                } else if (leader && valid) {
                    se[f] = (uint8_t)sc.e;
                }
            } else if (leader && valid) {
                if (a.scale_layout == LAYOUT_ROW)
                    reinterpret_cast<float *>(se)[f] = sc.r;
                else
                    reinterpret_cast<float *>(se)[gr * a.rows_pad + mr] = sc.r;
            }
            continue;
        }
        if constexpr (ue8m0) {
          if (a.scale_layout == LAYOUT_COL) {
            const uint32_t byte = valid ? sc.e : 0u;
            if constexpr (G >= 64) {
                // G/8 >= 8 lanes per group: read the bytes into scalars
#pragma unroll
                for (int w = 0; w < GPS / 4; ++w) {
                    const uint32_t word =
                        (uint32_t)__builtin_amdgcn_readlane((int)byte, (4 * w + 0) * LPG) |
                        ((uint32_t)__builtin_amdgcn_readlane((int)byte, (4 * w + 1) * LPG) << 8) |
                        ((uint32_t)__builtin_amdgcn_readlane((int)byte, (4 * w + 2) * LPG) << 16) |
                        ((uint32_t)__builtin_amdgcn_readlane((int)byte, (4 * w + 3) * LPG) << 24);
                    const int64_t gw = g0 + 4 * w;
                    if (lane == 0 && at < t.codes && gw < a.ng)
                        reinterpret_cast<uint32_t *>(se)[(gw >> 2) * a.rows_pad + m] = word;
                }
            } else {
                const uint32_t b1 = (uint32_t)__shfl((int)byte, lane + LPG);
                const uint32_t b2 = (uint32_t)__shfl((int)byte, lane + 2 * LPG);
                const uint32_t b3 = (uint32_t)__shfl((int)byte, lane + 3 * LPG);
                if (leader && (lg & 3) == 0 && valid) {
                    const uint32_t word = byte | (b1 << 8) | (b2 << 16) | (b3 << 24);
                    reinterpret_cast<uint32_t *>(se)[((g0 + lg) >> 2) * a.rows_pad + m] = word;
                }
            }
          } else if (leader && valid) {
            se[m * a.ng + g0 + lg] = (uint8_t)sc.e;
          }
        } else if (leader && valid) {
            const int64_t gi = g0 + lg;
            if (a.scale_layout == LAYOUT_ROW)
                reinterpret_cast<float *>(se)[m * a.ng + gi] = sc.r;
            else
                reinterpret_cast<float *>(se)[gi * a.rows_pad + m] = sc.r;
        }
    }
}

// A row task: task j of row m (slabs j*U .. j*U+U-1 of the row) whose row
// starts at xrow (input) and qrow (codes) and whose scales live in sbase.
template <int IN, int UMAX>
__device__ __forceinline__ TaskLoc row_task(const GroupArgs &a, const char *xrow, uint8_t *qrow,
                                            uint8_t *sbase, int64_t m, int j)
{
    constexpr int ES = IN == IN_FP32 ? 4 : 2;
    // 32-bit column arithmetic: K < 2^29
    const uint32_t K = (uint32_t)a.K;
    const uint32_t c0 = (uint32_t)j * (UMAX * kSlab);   // first column of the task
    const uint32_t left = K - c0;
    TaskLoc l;
    l.xb = xrow;
    l.qb = qrow;
    l.sbase = sbase;
    l.xrange = K * ES;
    l.qrange = K;
    l.c0 = c0;
    l.codes = left < UMAX * kSlab ? left : UMAX * kSlab;
    l.m = m;
    l.j = j * UMAX;
    l.next_row = UMAX;
    return l;
}

// Flat schedule, row tasks: task t is task t % tpr of row t / tpr.  The
// quotient by a multiply-high (the integer division's instruction sequence
// lies on the path to a task's first load): measured faster for fused calls
// (bf16 [2048, 2 * 4096] 9.46 -> 9.30 us) and one-slab tasks ([256, 7168]
// 2.98 -> 2.82), but 2 % slower for the unfused two-slab tasks of [4096,
// 7168] (15.40 -> 15.72, the same at M = 16384; cause not found), which keep
// the division.
template <int IN, int UMAX, bool FUSE>
struct FlatMap {
    __device__ __forceinline__ TaskLoc operator()(const GroupArgs &a, int t, int /*lane*/)
    {
        int m;
        if constexpr (FUSE || UMAX == 1)
            m = (int)fastdiv((uint32_t)t, a.tpr_div);
        else
            m = t / a.tpr;
        return row_task<IN, UMAX>(a, static_cast<const char *>(a.x) + (int64_t)m * a.in_stride,
                                  a.q + (int64_t)m * a.K, static_cast<uint8_t *>(a.s), m,
                                  t - m * a.tpr);
    }
};

// Task of UMAX slabs from slab S of a flattened output of `total` (< 2^31)
// elements: codes S * kSlab .. up to the sequence's end (a sequence's last
// task may be short), written from q; the output's rows of K codes come from
// input rows of a.in_stride bytes from x, scales go to s.  Unfused input is
// the same flat sequence; fused lanes address the gate and up halves of their
// own rows (load_task), from row0, the row of the task's first code.  Slab s
// of the task is "row" S + s (next_row 1).
template <int IN, int UMAX, bool FUSE>
__device__ __forceinline__ TaskLoc flat_seq_loc(const GroupArgs &a, const char *x, uint8_t *q,
                                                uint8_t *s, uint32_t S, uint32_t total)
{
    constexpr int ES = IN == IN_FP32 ? 4 : 2;
    const uint32_t e0 = S * kSlab;
    const uint32_t rest = total - e0;                       // >= 1 for live tasks
    const uint32_t cnt = rest < UMAX * kSlab ? rest : UMAX * kSlab;
    TaskLoc l;
    l.qb = q + e0;
    l.sbase = s;
    l.qrange = cnt;
    l.c0 = 0;
    l.codes = cnt;
    l.m = S;
    l.j = 0;
    l.next_row = 1;
    if constexpr (FUSE) {
        const uint32_t r0 = fastdiv(e0, a.k_div);
        const uint32_t r1 = fastdiv(e0 + cnt - 1, a.k_div);
        l.xb = x + (uint64_t)r0 * a.in_stride;
        l.xrange = (r1 - r0 + 1) * (uint32_t)a.in_stride;
        l.row0 = r0;
    } else {
        l.xb = x + (uint64_t)e0 * ES;
        l.xrange = cnt * ES;
        l.row0 = 0;
    }
    return l;
}

// Flat schedule, flat-slab tasks: task t is slabs U*t .. U*t+U-1 of one
// sequence of slabs over the whole tensor, crossing row ends.  FS 1 (unfused,
// K a multiple of the slab, so input and codes are one contiguous sequence of
// whole-row slabs): no task is short except the tensor's last one; the row of
// slab S is S / spr (a wave-uniform multiply-high division), and the task is
// addressed from its first row, whose range is extended by the slab that
// crosses into the next row.  FS 2 (rows of kSlab elements, spr 1): the same
// arithmetic, clipped to the tensor, which may end inside its last slab.
// FS 3: slabs of the flattened output (flat_seq_loc).
template <int IN, int UMAX, bool FUSE, int FS>
struct FlatSlabMap {
    __device__ __forceinline__ TaskLoc operator()(const GroupArgs &a, int t, int /*lane*/)
    {
        constexpr int ES = IN == IN_FP32 ? 4 : 2;
        const uint32_t S = (uint32_t)t * UMAX;                      // first slab (< 2^31)
        if constexpr (FS == 3)
            return flat_seq_loc<IN, UMAX, FUSE>(a, static_cast<const char *>(a.x), a.q,
                                                static_cast<uint8_t *>(a.s), S,
                                                (uint32_t)a.fs_total);
        const uint32_t m = fastdiv(S, a.spr_div);
        const uint32_t j = S - m * (uint32_t)a.spr;
        const uint32_t left = (uint32_t)a.n_slabs - S;               // >= 1 for live tasks
        const uint32_t K = (uint32_t)a.fs_row;
        // the region is row m and the slabs after it up to the task's end
        // (the next row's first slab when the task crosses the row end),
        // clipped to the tensor
        const uint32_t span = j * kSlab + (left < UMAX ? left : UMAX) * kSlab;
        const int64_t rest = a.fs_total - (int64_t)m * K;          // >= 1 for live tasks
        const uint32_t reach0 = span > K ? span : K;
        const uint32_t reach = rest < (int64_t)reach0 ? (uint32_t)rest : reach0;
        TaskLoc l;
        l.xb = static_cast<const char *>(a.x) + (uint64_t)m * K * ES;
        l.qb = a.q + (uint64_t)m * K;
        l.sbase = static_cast<uint8_t *>(a.s);
        l.xrange = reach * ES;
        l.qrange = reach;
        l.c0 = j * kSlab;
        const uint32_t codes = (left < UMAX ? left : UMAX) * kSlab;
        l.codes = reach - l.c0 < codes ? reach - l.c0 : codes;
        l.m = m;
        l.j = (int)j;
        l.next_row = (int)((uint32_t)a.spr - j);     // >= UMAX: no crossing
        return l;
    }
};

// Masked schedule: the live rows of all experts, back to back, are one task
// space.  `scan` (LDS) holds the inclusive prefix sum of the experts' live row
// counts, so live row R belongs to the first expert e with scan[e] > R and is
// row R - scan[e-1] of that expert.  A wave's rows only move forward, so the
// wave keeps the current 64-expert window of the prefix sum in a register
// (lane l holds scan[chunk + l]) and searches it with one ballot; the window
// only moves forward, re-read from LDS when a search runs off its end.
struct MaskedRows {
    const int *scan;
    int E;
    int chunk;    // first expert of the window
    int base;     // scan[chunk - 1] (0 for the first window)
    int win;      // this lane's scan[chunk + lane], INT32_MAX past E

    __device__ __forceinline__ MaskedRows(const int *scan_, int E_, int lane)
        : scan(scan_), E(E_), chunk(0), base(0), win(lane < E_ ? scan_[lane] : INT32_MAX)
    {
    }

    // E <= 64: the whole prefix sum is the register window `win_` (lane l
    // holds the sum over experts 0..l); no LDS copy exists or is read.
    __device__ __forceinline__ MaskedRows(int win_, int E_, int lane)
        : scan(nullptr), E(E_), chunk(0), base(0), win(lane < E_ ? win_ : INT32_MAX)
    {
    }

    // live row R (< total live rows) -> expert e and row r within it
    __device__ __forceinline__ void locate(int R, int lane, int &e, int &r)
    {
        unsigned long long hit = __ballot(win > R);
        while (!hit && chunk + 64 < E) {                 // wave-uniform; rare
            base = __builtin_amdgcn_readlane(win, 63);
            chunk += 64;
            win = chunk + lane < E ? scan[chunk + lane] : INT32_MAX;
            hit = __ballot(win > R);
        }
        // R is below the total live rows, so the last window always hits; the
        // clamp only keeps a miss inside the experts
        const int k = hit ? (int)__builtin_ctzll(hit) : min(63, E - 1 - chunk);
        const int prev = __builtin_amdgcn_readlane(win, k > 0 ? k - 1 : 0);
        e = chunk + k;
        r = R - (k == 0 ? base : prev);
    }
};

// Tasks of UMAX slabs over `live` flattened rows of K codes (live * K < 2^31).
template <int UMAX>
__device__ __forceinline__ int slab_tasks(int live, uint32_t K)
{
    constexpr uint32_t per = (uint32_t)UMAX * kSlab;
    return (int)(((uint32_t)live * K + per - 1) / per);
}

// Inclusive prefix sum of clamp(masked_m[e], 0, rows) over e < E into LDS
// `scan` (masked_m NULL: every row of every expert is live).  SLABS (UMAX
// slabs per task): the sum is over the experts' task counts, and the clamped
// live rows go to scan[E + e].  Wave 0 only; the caller synchronizes.
template <int SLABS = 0>
__device__ __forceinline__ void masked_prefix_sum(const int32_t *masked_m, int E, int64_t rows,
                                                  int lane, int *scan, uint32_t K = 0)
{
    int carry = 0;
    for (int c = 0; c < E; c += 64) {
        int v = 0;
        if (c + lane < E) {
            v = masked_m ? masked_m[c + lane] : (int)rows;
            v = v < 0 ? 0 : (v > rows ? (int)rows : v);
            if constexpr (SLABS > 0) {
                scan[E + c + lane] = v;
                v = slab_tasks<SLABS>(v, K);
            }
        }
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(v, d);
            if (lane >= d) v += y;
        }
        if (c + lane < E) scan[c + lane] = v + carry;
        carry += __builtin_amdgcn_readlane(v, 63);
    }
}

// Inclusive prefix sum of `v` over the lanes of a wave (lane l gets the sum
// over lanes 0..l).
__device__ __forceinline__ int wave_inclusive_sum(int v, int lane)
{
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(v, d);
        if (lane >= d) v += y;
    }
    return v;
}

// clamp(masked_m[lane], 0, rows) for lane < E (every row when masked_m is
// NULL), 0 for the other lanes.  E <= 64.
__device__ __forceinline__ int live_rows_of_lane(const int32_t *masked_m, int E, int64_t rows,
                                                 int lane)
{
    int v = 0;
    if (lane < E) {
        v = masked_m ? masked_m[lane] : (int)rows;
        v = v < 0 ? 0 : (v > rows ? (int)rows : v);
    }
    return v;
}

// Row r of expert e, task j of the row.
template <int IN, int UMAX>
__device__ __forceinline__ TaskLoc masked_loc(const GroupArgs &a, int e, int r, int j)
{
    return row_task<IN, UMAX>(
        a, static_cast<const char *>(a.x) + (int64_t)e * a.x_expert_stride + (int64_t)r * a.in_stride,
        a.q + (int64_t)e * a.q_expert_stride + (int64_t)r * a.K,
        static_cast<uint8_t *>(a.s) + (int64_t)e * a.s_expert_stride, r, j);
}

template <int IN, int UMAX>
struct MaskedMap {
    MaskedRows rows;

    __device__ __forceinline__ MaskedMap(const int *scan, int E, int lane) : rows(scan, E, lane) {}
    __device__ __forceinline__ MaskedMap(int win, int E, int lane) : rows(win, E, lane) {}

    __device__ __forceinline__ TaskLoc operator()(const GroupArgs &a, int t, int lane)
    {
        const int R = (int)fastdiv((uint32_t)t, a.tpr_div);
        int e, r;
        rows.locate(R, lane, e, r);
        return masked_loc<IN, UMAX>(a, e, r, t - R * a.tpr);
    }
};
// Masked schedule in chunk tasks: task t is chunk t % tpr of live row t / tpr.
struct MaskedChunkMap {
    MaskedRows rows;

    __device__ __forceinline__ MaskedChunkMap(const int *scan, int E, int lane)
        : rows(scan, E, lane) {}
    __device__ __forceinline__ MaskedChunkMap(int win, int E, int lane) : rows(win, E, lane) {}

    __device__ __forceinline__ ChunkLoc operator()(const GroupArgs &a, int t, int lane)
    {
        const uint32_t R = fastdiv((uint32_t)t, a.spr_div);
        int e, r;
        rows.locate((int)R, lane, e, r);
        ChunkLoc l;
        l.xr = static_cast<const char *>(a.x) + (int64_t)e * a.x_expert_stride +
               (int64_t)r * a.in_stride;
        l.qr = a.q + (int64_t)e * a.q_expert_stride + (int64_t)r * a.K;
        l.s = static_cast<uint8_t *>(a.s) + (int64_t)e * a.s_expert_stride;
        l.m = (uint32_t)r;
        l.c0 = ((uint32_t)t - R * (uint32_t)a.spr) * (uint32_t)kChunk;
        return l;
    }
};

// Masked schedule in flattened slabs (rows whose length is not a multiple of
// the slab): expert e's live rows are one sequence of live_e * K codes, cut
// into tasks of UMAX slabs (its last task may be short; no task crosses
// experts), and `tasks` walks the prefix sum of the experts' task counts.
// REG (E <= 64): lane l holds expert l's live rows in `live`; else they are in
// LDS at `lrows`.
template <int IN, int UMAX, bool FUSE, bool REG>
struct MaskedSlabMap {
    MaskedRows tasks;
    int live;
    const int *lrows;

    __device__ __forceinline__ MaskedSlabMap(int win, int live_, int E, int lane)
        : tasks(win, E, lane), live(live_), lrows(nullptr)
    {
    }
    __device__ __forceinline__ MaskedSlabMap(const int *scan, int E, int lane)
        : tasks(scan, E, lane), live(0), lrows(scan + E)
    {
    }

    __device__ __forceinline__ TaskLoc operator()(const GroupArgs &a, int t, int lane)
    {
        int e, tl;
        tasks.locate(t, lane, e, tl);
        e = __builtin_amdgcn_readfirstlane(e);
        const int n = REG ? __builtin_amdgcn_readlane(live, e) : lrows[e];
        return flat_seq_loc<IN, UMAX, FUSE>(
            a, static_cast<const char *>(a.x) + (int64_t)e * a.x_expert_stride,
            a.q + (int64_t)e * a.q_expert_stride,
            static_cast<uint8_t *>(a.s) + (int64_t)e * a.s_expert_stride, (uint32_t)tl * UMAX,
            (uint32_t)n * (uint32_t)a.K);
    }
};

// The SiLU table staged into LDS in two steps, so that its global loads can
// be issued before a wave's first task loads and its LDS stores wait for the
// table alone (vector memory loads complete in issue order): table kernels
// always run 1024-lane blocks, 2 (bf16 gates) or 9 (fp16) float4 of the
// table per lane.
constexpr int kTableLanes = 1024;
static_assert(kSiluTab % (4 * kTableLanes) == 0 && kSiluTab16 % (4 * kTableLanes) == 0,
              "whole float4 per lane");
template <int IN>
struct TableRegs {
    float4 v[table_floats<IN>() / 4 / kTableLanes];   // bf16: 2, fp16: 9
};

template <bool TABLE, int IN>
__device__ __forceinline__ void table_fetch(TableRegs<IN> &r)
{
    if constexpr (TABLE) {
        const float4 *src =
            reinterpret_cast<const float4 *>(IN == IN_BF16 ? g_silu_table : g_silu_table16);
#pragma unroll
        for (int i = 0; i < table_floats<IN>() / 4 / kTableLanes; ++i)
            r.v[i] = src[threadIdx.x + kTableLanes * i];
    }
}

// Stores the fetched table and synchronizes the block (call before any early
// exit that is not block-uniform).
template <bool TABLE, int IN>
__device__ __forceinline__ void table_store(const TableRegs<IN> &r, float *tab)
{
    if constexpr (TABLE) {
        float4 *dst = reinterpret_cast<float4 *>(tab);
#pragma unroll
        for (int i = 0; i < table_floats<IN>() / 4 / kTableLanes; ++i)
            dst[threadIdx.x + kTableLanes * i] = r.v[i];
        __syncthreads();
    }
}

// Continues the task sequence t, t + stride, ... < n from task t, whose loads
// are already in flight in `cur` (location lcur); `spare` is free.  Two tasks
// are in flight at a time.  A task index past n is clamped for address
// arithmetic and loaded over an empty range.
template <int IN, int G, bool FUSE, int OUT, int SF, int UMAX, bool TABLE, int SPOL, int FS,
          class Map>
__device__ __forceinline__ void continue_tasks(const GroupArgs &a, Map &map, int t, TaskLoc lcur,
                                               TaskBuf<UMAX> &cur, TaskBuf<UMAX> &spare, int n,
                                               int stride, int lane, const float *tab)
{
    while (true) {
        const int tB = t + stride;
        const bool hasB = tB < n;
        const TaskLoc lB = map(a, hasB ? tB : t, lane);
        load_task<IN, FUSE, UMAX, FS>(a, lB, lane, hasB, spare);
        process_task<IN, G, FUSE, OUT, SF, UMAX, TABLE, SPOL, FS>(a, lcur, lane, cur, tab);
        if (!hasB) break;
        t = tB;
        const int tA = t + stride;
        const bool hasA = tA < n;
        lcur = map(a, hasA ? tA : t, lane);
        load_task<IN, FUSE, UMAX, FS>(a, lcur, lane, hasA, cur);
        process_task<IN, G, FUSE, OUT, SF, UMAX, TABLE, SPOL, FS>(a, lB, lane, spare, tab);
        if (!hasA) break;
        t = tA;
    }
}

// Tasks first, first + stride, ... < n, two at a time in flight.  Table
// kernels (STAGE) fetch the SiLU table, issue the first task's loads, then
// store the table into LDS (every wave of the block reaches that barrier,
// with or without a task), so the table copy overlaps the first HBM reads.
template <int IN, int G, bool FUSE, int OUT, int SF, int UMAX, bool TABLE, int SPOL,
          bool STAGE, bool FETCHED = false, int FS = 0, class Map>
__device__ __forceinline__ void run_tasks(const GroupArgs &a, Map map, int first, int n,
                                          int stride, int lane, float *tab,
                                          TableRegs<IN> tr = TableRegs<IN>{})
{
    const bool hasA0 = first < n;
    TaskBuf<UMAX> A, B;
    if constexpr (STAGE && !FETCHED) table_fetch<TABLE>(tr);
    const TaskLoc lA = map(a, hasA0 ? first : 0, lane);
    load_task<IN, FUSE, UMAX, FS>(a, lA, lane, hasA0, A);
    if constexpr (STAGE) table_store<TABLE>(tr, tab);
    if (!hasA0) return;
    continue_tasks<IN, G, FUSE, OUT, SF, UMAX, TABLE, SPOL, FS>(a, map, first, lA, A, B, n, stride,
                                                            lane, tab);
}

// Kernel arguments live in memory and are read by scalar loads, which the
// compiler places at each argument's first use; a prologue with branches then
// waits for several rounds of them before its first input load.  Naming the
// arguments the prologue needs in one empty asm statement at entry makes all
// those loads one batch behind one wait (no instruction is emitted).
__device__ __forceinline__ void args_in_sgprs(const GroupArgs &a)
{
    asm volatile("" ::"s"(a.x), "s"(a.q), "s"(a.s), "s"(a.K), "s"(a.in_stride),
                 "s"(a.n_tasks), "s"(a.tpr), "s"(a.tpr_div.mul), "s"(a.tpr_div.shift),
                 "s"(a.xcd_chunk), "s"(a.n_slabs), "s"(a.spr_div.mul),
                 "s"(a.spr_div.shift), "s"(a.spr), "s"(a.wpb), "s"(a.q_pad_bytes),
                 "s"(gridDim.x));
}

// XCD-aware logical block id.  Blocks are dealt to the 8 XCDs round-robin
// (block b runs on XCD b % 8).  With chunk == 0 and a grid that is a multiple
// of 8, XCD x gets the logical ids [x * nb/8, (x+1) * nb/8): one contiguous
// range of tasks, the right mapping for a capped grid whose waves loop (all
// XCDs then sweep one grid-stride window together).  With chunk C > 0 the
// ids are dealt in spans of 8C blocks, XCD x taking C consecutive ids of each
// span: for a grid much larger than the chip, the XCDs stream neighbouring
// regions of memory instead of eight far-apart ones, and the scale words of
// neighbouring rows are still written from one L2.  Ids in a last, partial
// span map to themselves.
__device__ __forceinline__ int logical_block(int b, int nb, int chunk = 0)
{
    if (chunk <= 0) return (nb & 7) == 0 ? (b & 7) * (nb >> 3) + (b >> 3) : b;
    const int span = 8 * chunk;
    if (b >= nb / span * span) return b;
    const int r = b % span;
    return (b - r) + (r & 7) * chunk + (r >> 3);
}

// FS: flat-slab tasks (FlatSlabMap) instead of row tasks (FlatMap); 4: chunk
// tasks (fused calls of few slabs).
template <int IN, int G, bool FUSE, int OUT, int SF, int UMAX, bool TABLE, int FS>
__global__ __launch_bounds__(TABLE ? 1024 : 256) void ptgq_flat_kernel(GroupArgs a)
{
    __shared__ float tab[TABLE ? table_floats<IN>() : 1];
    args_in_sgprs(a);
    const int lane = threadIdx.x & 63;
    const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wpb = TABLE ? kTableLanes / 64 : a.wpb;
    const int lb = logical_block(blockIdx.x, gridDim.x, a.xcd_chunk);
    constexpr int spol = TABLE ? kTableStorePolicy : kStreamPolicy;
    if constexpr (FS == 4) {
        static_assert(FUSE && !TABLE && UMAX == 1, "chunk tasks: fused, direct SiLU");
        run_chunk_tasks<IN, G, OUT, SF>(a, FlatChunkMap{}, lb * wpb + wib, a.n_tasks,
                                        gridDim.x * wpb, lane);
    } else if constexpr (FS) {
        static_assert(FS == 3 || (!FUSE && !TABLE), "flat-slab tasks: unfused inputs");
        static_assert(FS != 2 || IN != IN_FP32, "multi-row slabs: 16-bit inputs");
        run_tasks<IN, G, FUSE, OUT, SF, UMAX, TABLE, spol, true, false, FS>(
            a, FlatSlabMap<IN, UMAX, FUSE, FS>{}, lb * wpb + wib, a.n_tasks, gridDim.x * wpb, lane,
            tab);
    } else {
        run_tasks<IN, G, FUSE, OUT, SF, UMAX, TABLE, spol, true>(
            a, FlatMap<IN, UMAX, FUSE>{}, lb * wpb + wib, a.n_tasks, gridDim.x * wpb, lane, tab);
    }
    // code rows past M (a padded q buffer) are zero: 16 bytes per lane,
    // grid-strided over all waves
    if (a.q_pad_bytes > 0) {
        u32x4 *qp = reinterpret_cast<u32x4 *>(a.q + a.rows * a.K);
        const int64_t n16 = a.q_pad_bytes / 16;
        const u32x4 zero = {0u, 0u, 0u, 0u};
        const int64_t nl = (int64_t)gridDim.x * wpb * 64;
        for (int64_t i = ((int64_t)lb * wpb + wib) * 64 + lane; i < n16; i += nl)
            __builtin_nontemporal_store(zero, qp + i);
    }
    // column-major pad slots (rows M .. rows_pad-1) are zero
    if (a.pad_cols > 0 && lb == 0 && wib == 0) {
        uint32_t *s = static_cast<uint32_t *>(a.s);
        const int64_t npad = (a.rows_pad - a.rows) * (int64_t)a.pad_cols;
        for (int64_t i = lane; i < npad; i += 64) {
            const int64_t r = a.rows + i / a.pad_cols;
            const int64_t c = i % a.pad_cols;
            s[c * a.rows_pad + r] = 0u;
        }
    }
}

// Masked layout, balanced over experts: masked_m (E values, clamped to [0,
// tokens_pad]) is summed into a prefix sum (in each wave's registers for E <=
// 64, else by wave 0 into LDS), and the grid walks the live rows of all
// experts as one task space (FS 3: the flattened slabs of each expert's live
// rows; FS 4: chunk tasks of the live rows).  Rows at or past masked_m are
// never read or written.  Dynamic LDS: E ints (FS 3: 2 E).
template <int IN, int G, bool FUSE, int OUT, int SF, int UMAX, bool TABLE, int FS>
__global__ __launch_bounds__(TABLE ? 1024 : 256) void ptgq_masked_kernel(GroupArgs a)
{
    __shared__ float tab[TABLE ? table_floats<IN>() : 1];
    extern __shared__ int scan[];
    args_in_sgprs(a);
    const int lane = threadIdx.x & 63;
    const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wpb = TABLE ? kTableLanes / 64 : a.wpb;
    const int lb = logical_block(blockIdx.x, gridDim.x);
    const int E = a.num_experts;
    if (E <= 64) {
        // Every wave reads masked_m and sums it in registers: no LDS and no
        // barrier before the first task's loads, which are issued before the
        // SiLU table is stored (every wave reaches that barrier, with or
        // without a task).
        // masked_m (never NULL here) read by every lane without a branch, so
        // that the table's loads are in flight while it arrives
        const int raw = a.masked_m[lane < E ? lane : E - 1];
        TableRegs<IN> tr;
        table_fetch<TABLE>(tr);
        __builtin_amdgcn_sched_barrier(0);   // keep both loads ahead of the wait
        const int live = lane < E ? (raw < 0 ? 0 : (raw > a.rows ? (int)a.rows : raw)) : 0;
        if constexpr (FS == 4) {
            const int win = wave_inclusive_sum(live, lane);
            const int n = __builtin_amdgcn_readlane(win, E - 1) * a.tpr;
            run_chunk_tasks<IN, G, OUT, SF>(a, MaskedChunkMap(win, E, lane), lb * wpb + wib, n,
                                            gridDim.x * wpb, lane);
        } else if constexpr (FS == 3) {
            const int win = wave_inclusive_sum(slab_tasks<UMAX>(live, (uint32_t)a.K), lane);
            const int n = __builtin_amdgcn_readlane(win, E - 1);
            run_tasks<IN, G, FUSE, OUT, SF, UMAX, TABLE, kStreamPolicy, true, true, FS>(
                a, MaskedSlabMap<IN, UMAX, FUSE, true>(win, live, E, lane), lb * wpb + wib, n,
                gridDim.x * wpb, lane, tab, tr);
        } else {
            const int win = wave_inclusive_sum(live, lane);
            const int n = __builtin_amdgcn_readlane(win, E - 1) * a.tpr;
            run_tasks<IN, G, FUSE, OUT, SF, UMAX, TABLE, kStreamPolicy, true, true>(
                a, MaskedMap<IN, UMAX>(win, E, lane), lb * wpb + wib, n, gridDim.x * wpb, lane,
                tab, tr);
        }
        return;
    }
    // More experts: the table's loads, then the prefix sum of masked_m into
    // LDS (wave 0), then the table's stores, behind one barrier.
    TableRegs<IN> tr;
    table_fetch<TABLE>(tr);
    if (wib == 0) {
        if constexpr (FS == 3)
            masked_prefix_sum<UMAX>(a.masked_m, E, a.rows, lane, scan, (uint32_t)a.K);
        else
            masked_prefix_sum(a.masked_m, E, a.rows, lane, scan);
    }
    if constexpr (TABLE) table_store<TABLE>(tr, tab);
    else __syncthreads();
    if constexpr (FS == 4) {
        const int n = scan[E - 1] * a.tpr;
        if (lb * wpb >= n) return;                // block-uniform: nothing to do
        run_chunk_tasks<IN, G, OUT, SF>(a, MaskedChunkMap(scan, E, lane), lb * wpb + wib, n,
                                        gridDim.x * wpb, lane);
    } else if constexpr (FS == 3) {
        const int n = scan[E - 1];
        if (lb * wpb >= n) return;                // block-uniform: nothing to do
        run_tasks<IN, G, FUSE, OUT, SF, UMAX, TABLE, kStreamPolicy, false, false, FS>(
            a, MaskedSlabMap<IN, UMAX, FUSE, false>(scan, E, lane), lb * wpb + wib, n,
            gridDim.x * wpb, lane, tab);
    } else {
        const int n = scan[E - 1] * a.tpr;
        if (lb * wpb >= n) return;                // block-uniform: nothing to do
        run_tasks<IN, G, FUSE, OUT, SF, UMAX, TABLE, kStreamPolicy, false>(
            a, MaskedMap<IN, UMAX>(scan, E, lane), lb * wpb + wib, n, gridDim.x * wpb, lane, tab);
    }
}

// --------------------------------------------------------------------------
// Whole-row per-token e4m3 (sglang #34257 review page, key source snippets):
// scale = rowmax / 448 with no floor, multiplier 0 for a zero row.
// A row is read once: it stays in registers between the max and the
// quantization pass (TOKEN_WAVE: one wave per row; TOKEN_BLOCK: one block of
// 1 to 8 waves per row); very long rows take the two-pass TOKEN_BLOCK_LOOP
// form.
// --------------------------------------------------------------------------

template <int IN, int VB>
struct TokVec {
    static constexpr int insz = (IN == IN_FP32) ? 4 : 2;
    static constexpr int EV = VB / insz;    // elements per vector
    using raw_t = typename std::conditional<VB == 16, uint4, uint2>::type;

    // non-temporal, like the group kernels' streaming accesses
    __device__ static __forceinline__ raw_t load(const uint8_t *p)
    {
        raw_t r;
        if constexpr (VB == 16) {
            const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
            r = make_uint4(v.x, v.y, v.z, v.w);
        } else {
            const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
            r = make_uint2(v.x, v.y);
        }
        return r;
    }
    // through a buffer descriptor: past its range the load reads zeros
    __device__ static __forceinline__ raw_t load_buf(rsrc_t rs, uint32_t off)
    {
        raw_t r;
        if constexpr (VB == 16) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kStreamPolicy);
            r = make_uint4(v.x, v.y, v.z, v.w);
        } else {
            const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, kStreamPolicy);
            r = make_uint2(v.x, v.y);
        }
        return r;
    }
    __device__ static __forceinline__ raw_t zero()
    {
        raw_t r;
        if constexpr (VB == 16) r = make_uint4(0, 0, 0, 0); else r = make_uint2(0, 0);
        return r;
    }
    __device__ static __forceinline__ void widen(const raw_t r, float (&f)[EV])
    {
        if constexpr (IN == IN_FP32) {
            const uint4 w = r;
            f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y);
            f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
        } else if constexpr (VB == 16) {
            widen8<IN>(r, f);
        } else {
            const uint32_t w[2] = {r.x, r.y};
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                if constexpr (IN == IN_BF16) {
                    f[2 * i] = __uint_as_float(w[i] << 16);
                    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
                } else {
                    f[2 * i] = fp16_to_f32(w[i]);
                    f[2 * i + 1] = fp16_to_f32(w[i] >> 16);
                }
            }
        }
    }
    // |x| maximum of the vector, as an fp32 bit pattern
    __device__ static __forceinline__ uint32_t absmax(const raw_t r)
    {
        if constexpr (IN == IN_FP32) {
            const uint4 w = r;
            const uint32_t a = (w.x & 0x7FFFFFFFu) > (w.y & 0x7FFFFFFFu) ? (w.x & 0x7FFFFFFFu)
                                                                          : (w.y & 0x7FFFFFFFu);
            const uint32_t b = (w.z & 0x7FFFFFFFu) > (w.w & 0x7FFFFFFFu) ? (w.z & 0x7FFFFFFFu)
                                                                          : (w.w & 0x7FFFFFFFu);
            return a > b ? a : b;
        } else if constexpr (VB == 16) {
            return absmax8_bits<IN>(r.x, r.y, r.z, r.w);
        } else {
            return absmax8_bits<IN>(r.x, r.y, 0u, 0u);
        }
    }

    // codes of one vector through a buffer descriptor (dropped past its range)
    __device__ static __forceinline__ void store_codes_buf(rsrc_t rs, uint32_t off,
                                                           const float (&v)[EV])
    {
        if constexpr (EV == 8) {
            u32x2 o;
            o.x = e4m3x4<true>(v[0], v[1], v[2], v[3]);
            o.y = e4m3x4<true>(v[4], v[5], v[6], v[7]);
            __builtin_amdgcn_raw_buffer_store_b64(o, rs, off, 0, kStreamPolicy);
        } else {
            __builtin_amdgcn_raw_buffer_store_b32(e4m3x4<true>(v[0], v[1], v[2], v[3]), rs, off,
                                                  0, kStreamPolicy);
        }
    }
    __device__ static __forceinline__ void store_codes(uint8_t *p, const float (&v)[EV])
    {
        if constexpr (EV == 8) {
            u32x2 o;
            o.x = e4m3x4<true>(v[0], v[1], v[2], v[3]);
            o.y = e4m3x4<true>(v[4], v[5], v[6], v[7]);
            __builtin_nontemporal_store(o, reinterpret_cast<u32x2 *>(p));
        } else {
            __builtin_nontemporal_store(e4m3x4<true>(v[0], v[1], v[2], v[3]),
                                        reinterpret_cast<uint32_t *>(p));
        }
    }
};

__device__ __forceinline__ float token_inv(float amax, float &r)
{
    r = amax / 448.0f;
    return (r == 0.0f) ? 0.0f : 1.0f / r;
}

template <int IN, int VB, int NV>
__global__ __launch_bounds__(256) void ptq_wave_kernel(TokenArgs a)
{
    using TV = TokVec<IN, VB>;
    constexpr int EV = TV::EV;
    const int lane = threadIdx.x & 63;
    const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t m = (int64_t)blockIdx.x * (blockDim.x >> 6) + wib;
    if (m >= a.M) return;                                   // wave-uniform
    const uint8_t *xr = static_cast<const uint8_t *>(a.x) + m * a.K * TV::insz;
    uint8_t *qr = a.q + m * a.K;
    typename TV::raw_t raw[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int i = lane + 64 * k;
        raw[k] = (i < a.nv) ? TV::load(xr + (int64_t)i * VB) : TV::zero();
    }
    uint32_t amax = 0;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const uint32_t m = TV::absmax(raw[k]);
        amax = amax > m ? amax : m;
    }
    float r;
    const float inv = token_inv(__uint_as_float(wave_max_bits(amax)), r);
    if (lane == 0) a.s[m] = r;
    with_uniform_multiplier(inv, [&](auto mode) {
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int i = lane + 64 * k;
            if (i < a.nv) {
                float f[EV], v[EV];
                TV::widen(raw[k], f);
                scale_by<decltype(mode)::value>(f, inv, v);
                TV::store_codes(qr + (int64_t)i * EV, v);
            }
        }
    });
}

// Persistent form of the wave-per-row kernel: a grid of a few blocks per CU
// whose waves walk the rows grid-strided, keeping the next row's loads in
// flight while they quantize the current one (so reads and writes overlap for
// the whole call instead of all rows loading first and storing last).  Loads
// and code stores go through per-row buffer resources (lanes past the row read
// zeros and store nothing).
template <int IN, int VB, int NV>
__global__ __launch_bounds__(256) void ptq_wave_loop_kernel(TokenArgs a)
{
    using TV = TokVec<IN, VB>;
    using raw_t = typename TV::raw_t;
    constexpr int EV = TV::EV;
    const int lane = threadIdx.x & 63;
    const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wpb = blockDim.x >> 6;
    const int lb = logical_block(blockIdx.x, gridDim.x);
    const uint32_t row_bytes = (uint32_t)(a.K * TV::insz);
    const int64_t W = (int64_t)gridDim.x * wpb;
    int64_t m = (int64_t)lb * wpb + wib;
    if (m >= a.M) return;                                   // wave-uniform

    auto load = [&](int64_t row, bool live, raw_t (&r)[NV]) {
        const rsrc_t rx =
            make_rsrc(static_cast<const uint8_t *>(a.x) + row * row_bytes, live ? row_bytes : 0u);
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const uint32_t off = (uint32_t)(lane + 64 * k) * VB;
            if constexpr (VB == 16) {
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, kStreamPolicy);
                r[k] = make_uint4(v.x, v.y, v.z, v.w);
            } else {
                const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rx, off, 0, kStreamPolicy);
                r[k] = make_uint2(v.x, v.y);
            }
        }
    };
    auto process = [&](int64_t row, const raw_t (&r)[NV]) {
        uint32_t amax = 0;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const uint32_t mk = TV::absmax(r[k]);
            amax = amax > mk ? amax : mk;
        }
        float rs;
        const float inv = token_inv(__uint_as_float(wave_max_bits(amax)), rs);
        if (lane == 0) a.s[row] = rs;
        const rsrc_t rq = make_rsrc(a.q + row * a.K, (uint32_t)a.K);
        with_uniform_multiplier(inv, [&](auto mode) {
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                float y[EV], f[EV];
                TV::widen(r[k], y);
                scale_by<decltype(mode)::value>(y, inv, f);
                const uint32_t off = (uint32_t)(lane + 64 * k) * EV;
                if constexpr (EV == 8) {
                    u32x2 o;
                    o.x = e4m3x4<true>(f[0], f[1], f[2], f[3]);
                    o.y = e4m3x4<true>(f[4], f[5], f[6], f[7]);
                    __builtin_amdgcn_raw_buffer_store_b64(o, rq, off, 0, kStreamPolicy);
                } else {
                    __builtin_amdgcn_raw_buffer_store_b32(e4m3x4<true>(f[0], f[1], f[2], f[3]),
                                                          rq, off, 0, kStreamPolicy);
                }
            }
        });
    };

    raw_t A[NV], B[NV];
    load(m, true, A);
    while (true) {
        const int64_t mB = m + W;
        const bool hasB = mB < a.M;
        load(hasB ? mB : m, hasB, B);
        process(m, A);
        if (!hasB) break;
        m = mB;
        const int64_t mA = m + W;
        const bool hasA = mA < a.M;
        load(hasA ? mA : m, hasA, A);
        process(m, B);
        if (!hasA) break;
        m = mA;
    }
}

// Block maximum (up to 8 waves), uniform over the block.
__device__ __forceinline__ uint32_t block_max_bits(uint32_t v, uint32_t *red)
{
    v = wave_max_bits(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    uint32_t m = red[0];
    for (int i = 1; i < (int)(blockDim.x >> 6); ++i) m = m > red[i] ? m : red[i];
    return m;
}

// One block per row (1 to 8 waves), the row held in registers: NV vectors
// per lane, lane t of the block holding vectors t, t + threads, ...  Loads
// and code stores go through buffer descriptors over the row, so vectors past
// the row read zeros and their stores are dropped (no branch per vector).
template <int IN, int VB, int NV>
__global__ __launch_bounds__(512) void ptq_block_kernel(TokenArgs a)
{
    using TV = TokVec<IN, VB>;
    constexpr int EV = TV::EV;
    __shared__ uint32_t red[8];
    asm volatile("" ::"s"(a.x), "s"(a.q), "s"(a.s), "s"(a.K), "s"(a.xcd_chunk), "s"(gridDim.x));
    const int tid = threadIdx.x;
    const int64_t m = a.xcd_chunk > 0 ? logical_block(blockIdx.x, gridDim.x, a.xcd_chunk)
                                      : (int)blockIdx.x;
    const uint32_t row_bytes = (uint32_t)(a.K * TV::insz);
    const rsrc_t rx = make_rsrc(static_cast<const uint8_t *>(a.x) + m * row_bytes, row_bytes);
    const rsrc_t rq = make_rsrc(a.q + m * a.K, (uint32_t)a.K);
    typename TV::raw_t raw[NV];
    const int nt = blockDim.x;
#pragma unroll
    for (int k = 0; k < NV; ++k) raw[k] = TV::load_buf(rx, (uint32_t)(tid + nt * k) * VB);
    uint32_t amax = 0;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const uint32_t mk = TV::absmax(raw[k]);
        amax = amax > mk ? amax : mk;
    }
    float r;
    const float inv = token_inv(__uint_as_float(block_max_bits(amax, red)), r);
    if (tid == 0) a.s[m] = r;
    with_uniform_multiplier(inv, [&](auto mode) {
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            float f[EV], v[EV];
            TV::widen(raw[k], f);
            scale_by<decltype(mode)::value>(f, inv, v);
            TV::store_codes_buf(rq, (uint32_t)(tid + nt * k) * EV, v);
        }
    });
}

template <int IN, int VB>
__global__ __launch_bounds__(256) void ptq_block_loop_kernel(TokenArgs a)
{
    using TV = TokVec<IN, VB>;
    constexpr int EV = TV::EV;
    __shared__ uint32_t red[4];
    const int tid = threadIdx.x;
    const int64_t m = blockIdx.x;
    const uint8_t *xr = static_cast<const uint8_t *>(a.x) + m * a.K * TV::insz;
    uint8_t *qr = a.q + m * a.K;
    uint32_t amax = 0;
    for (int i = tid; i < a.nv; i += 256) {
        const uint32_t mk = TV::absmax(TV::load(xr + (int64_t)i * VB));
        amax = amax > mk ? amax : mk;
    }
    float r;
    const float inv = token_inv(__uint_as_float(block_max_bits(amax, red)), r);
    if (tid == 0) a.s[m] = r;
    with_uniform_multiplier(inv, [&](auto mode) {
        for (int i = tid; i < a.nv; i += 256) {
            float f[EV], v[EV];
            TV::widen(TV::load(xr + (int64_t)i * VB), f);
            scale_by<decltype(mode)::value>(f, inv, v);
            TV::store_codes(qr + (int64_t)i * EV, v);
        }
    });
}

// --------------------------------------------------------------------------
// Per-token-group fp8 -> per-tensor fp8 requantization on the masked layout
// (sglang #35593 review page, key source snippets): each e4m3 code is decoded,
// multiplied by its group scale, then by 1 / output_scale (two fp32
// roundings), and narrowed with saturation.
//
// The live rows of an expert are contiguous in memory (rows 0 .. live-1 of
// its [T, K] block), so each expert's live codes form one flat region; a task
// is NS contiguous 1024-code sub-slabs of one region (16 codes per lane per
// sub-slab, one 16-byte load and store), crossing row ends freely: no lane idles
// on a row's ragged tail.  Tasks of all experts form one space, split over the
// grid through an LDS prefix sum of the experts' task counts (read from
// masked_m on the device); two tasks are in flight per wave.  A lane's row and
// group (hence its scale) follow from the task's first row and column.
// --------------------------------------------------------------------------

constexpr int kRqSub = 1024;

__device__ __forceinline__ void decode4_e4m3(uint32_t w, float (&f)[4])
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    f[0] = lo.x;
    f[1] = lo.y;
    f[2] = hi.x;
    f[3] = hi.y;
}

// Wave 0: live[e] = clamp(masked_m[e], 0, T) (T for every expert without
// masked_m) and scan[e] = inclusive prefix sum of ceil(live[e] * K / tcodes).
__device__ __forceinline__ void requant_task_scan(const RequantArgs &a, int lane, int *scan,
                                                  int *live)
{
    int carry = 0;
    for (int c = 0; c < a.E; c += 64) {
        int v = 0;
        if (c + lane < a.E) {
            int r = a.masked_m ? a.masked_m[c + lane] : (int)a.T;
            r = r < 0 ? 0 : (r > a.T ? (int)a.T : r);
            live[c + lane] = r;
            v = (int)(((int64_t)r * a.K + a.tcodes - 1) >>
                      __builtin_ctzll((unsigned long long)a.tcodes));   // a power of two
        }
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(v, d);
            if (lane >= d) v += y;
        }
        if (c + lane < a.E) scan[c + lane] = v + carry;
        carry += __builtin_amdgcn_readlane(v, 63);
    }
}

template <int NS>
__global__ __launch_bounds__(256) void requant_fp8_kernel(RequantArgs a)
{
    extern __shared__ int lds[];
    int *scan = lds;
    int *live = lds + a.E;
    const int lane = threadIdx.x & 63;
    const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wpb = blockDim.x >> 6;
    const int lb = logical_block(blockIdx.x, gridDim.x, a.xcd_chunk);
    // E <= 64: every wave reads masked_m and sums its experts' task counts in
    // registers (lane e: live rows of expert e, and the prefix sum), with no
    // LDS and no barrier; more experts: wave 0 builds both in LDS.
    const bool in_regs = a.E <= 64;
    int live_lane = 0, win = 0;
    if (in_regs) {
        live_lane = live_rows_of_lane(a.masked_m, a.E, a.T, lane);
        const int shift = __builtin_ctzll((unsigned long long)a.tcodes);   // a power of two
        win = wave_inclusive_sum(
            (int)(((int64_t)live_lane * a.K + a.tcodes - 1) >> shift), lane);
    } else {
        if (wib == 0) requant_task_scan(a, lane, scan, live);
        __syncthreads();
    }
    const int n = in_regs ? __builtin_amdgcn_readlane(win, a.E - 1) : scan[a.E - 1];
    if (lb * wpb >= n) return;                              // block-uniform
    MaskedRows tasks = in_regs ? MaskedRows(win, a.E, lane) : MaskedRows(scan, a.E, lane);
    const float inv = 1.0f / a.output_scale[0];
    const uint32_t K = (uint32_t)a.K;
    constexpr uint32_t TS = NS * kRqSub;
    const rsrc_t rs = make_rsrc(a.x_scale, a.s_bytes);

    struct Loc {
        int64_t base;     // code offset of the task in x and out
        uint32_t len;     // codes in the task (<= TS)
        uint32_t row0;    // row (within the expert) of the first code
        uint32_t c0;      // column of the first code
        uint32_t sexp;    // e * se: the expert's first scale element
    };
    struct Buf {
        u32x4 w[NS];
        float s[NS];
    };
    auto locate = [&](int t) {
        int e, r;
        tasks.locate(t, lane, e, r);
        Loc l;
        const uint32_t off0 = (uint32_t)r * TS;               // < T * K < 2^31
        const int live_e = in_regs ? __builtin_amdgcn_readlane(live_lane, e) : live[e];
        const uint32_t region = (uint32_t)live_e * K;
        l.len = region - off0 < TS ? region - off0 : TS;
        l.row0 = fastdiv(off0, a.k_div);
        l.c0 = off0 - l.row0 * K;
        l.base = (int64_t)e * a.T * a.K + off0;
        l.sexp = (uint32_t)e * (uint32_t)a.se;
        return l;
    };
    auto load = [&](const Loc &l, bool alive) {
        Buf b;
        const uint32_t range = alive ? l.len : 0u;
        const rsrc_t rx = make_rsrc(a.x + l.base, range);
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            const uint32_t off = k * kRqSub + lane * 16;
            b.w[k] = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, kStreamPolicy);
            uint32_t col = l.c0 + off;
            uint32_t row = l.row0;
            if (K >= TS) {
                if (col >= K) {
                    col -= K;
                    row += 1;
                }
            } else {
                // quotient from an fp32 estimate (exact operands), off by at most one
                uint32_t d = (uint32_t)((float)col * a.inv_k);
                int32_t rem = (int32_t)(col - d * K);
                if (rem < 0) {
                    d -= 1;
                    rem += (int32_t)K;
                } else if (rem >= (int32_t)K) {
                    d += 1;
                    rem -= (int32_t)K;
                }
                col = (uint32_t)rem;
                row += d;
            }
            const uint32_t sidx = l.sexp + row * (uint32_t)a.st + (col >> a.log2g) * (uint32_t)a.sg;
            const uint32_t soff = off < range ? sidx * 4 : 0xFFFFFFF0u;
            b.s[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, soff, 0, 0));
        }
        return b;
    };
    auto process = [&](const Loc &l, const Buf &b) {
        const rsrc_t ro = make_rsrc(a.out + l.base, l.len);
        with_uniform_multiplier(inv, [&](auto mode) {
#pragma unroll
            for (int k = 0; k < NS; ++k) {
                const uint32_t ww[4] = {b.w[k].x, b.w[k].y, b.w[k].z, b.w[k].w};
                u32x4 o;
                uint32_t oo[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float f[4], h[4];
                    decode4_e4m3(ww[i], f);
#pragma unroll
                    for (int j = 0; j < 4; ++j) h[j] = f[j] * b.s[k];
                    scale_by<decltype(mode)::value>(h, inv, f);
                    oo[i] = e4m3x4<true>(f[0], f[1], f[2], f[3]);
                }
                o.x = oo[0];
                o.y = oo[1];
                o.z = oo[2];
                o.w = oo[3];
                __builtin_amdgcn_raw_buffer_store_b128(o, ro, k * kRqSub + lane * 16, 0,
                                                       kStreamPolicy);
            }
        });
    };

    const int stride = gridDim.x * wpb;
    int t = lb * wpb + wib;
    if (t >= n) return;
    Loc lA = locate(t);
    Buf A = load(lA, true), B;
    while (true) {
        const int tB = t + stride;
        const bool hasB = tB < n;
        const Loc lB = locate(hasB ? tB : t);
        B = load(lB, hasB);
        process(lA, A);
        if (!hasB) break;
        t = tB;
        const int tA = t + stride;
        const bool hasA = tA < n;
        lA = locate(hasA ? tA : t);
        A = load(lA, hasA);
        process(lB, B);
        if (!hasA) break;
        t = tA;
    }
}

// --------------------------------------------------------------------------
// Dequantization: y = round_out(decode(code) * scale) per element, the
// inverse step the pages check quantized activations with (sglang #35593
// review page, key source snippets: codes as float times the group scales
// repeated over each group; sglang #30924 review page, implementation
// breakdown: fp32-scale results are checked by their dequantization).
//
// HBM-bound (1 code byte in, 2 or 4 bytes out per element).  Codes and
// outputs are contiguous [M, K], so the work is cut into flat tasks of
// NS sub-slabs that cross row ends freely; only the scale lookup needs the
// row.  A sub-slab is 64 lanes x W consecutive codes (W = 8 for 16-bit
// output, 4 for fp32), so every store instruction of the wave writes one
// contiguous 1 KiB run (16 bytes per lane).  W divides every group size and K
// is a multiple of the group size, so a lane's W codes share one row and one
// scale.  Each wave keeps two tasks in flight and walks the grid-stride
// sequence of tasks with an incremental (row, column) cursor, so no division
// happens per task.
// --------------------------------------------------------------------------

template <int OUTD>
struct DqShape {
    static constexpr int W = OUTD == IN_FP32 ? 4 : 8;   // codes per lane per sub-slab
    static constexpr int SUB = 64 * W;                    // codes per sub-slab
    static constexpr int OSZ = OUTD == IN_FP32 ? 4 : 2;  // output bytes per element
};

template <int CODE>
__device__ __forceinline__ void decode_codes4(uint32_t w, float (&f)[4])
{
    if constexpr (CODE == OUT_E4M3) {
        decode4_e4m3(w, f);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = (float)(int32_t)(int8_t)(uint8_t)(w >> (8 * i));
    }
}

// Two fp32 values to a packed pair of 16-bit values, round-to-nearest-even
// (one v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack2_out_bf16(float a, float b)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint32_t pack2_out_fp16(float a, float b)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// Position of a task: its round, first code's flat index and (row, column).
struct DqCursor {
    int32_t i;
    int64_t e;
    int64_t m;
    uint32_t c;
};

template <int CODE, int SF, int SL, int OUTD, int NS>
__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs a)
{
    using Sh = DqShape<OUTD>;
    constexpr int W = Sh::W, SUB = Sh::SUB, OSZ = Sh::OSZ;
    constexpr int TS = NS * SUB;
    const int lane = threadIdx.x & 63;
    const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wpb = blockDim.x >> 6;
    const int lb = logical_block(blockIdx.x, gridDim.x, a.xcd_chunk);
    const uint32_t K = (uint32_t)a.K;
    const int64_t total = a.M * a.K;
    const rsrc_t rs = make_rsrc(a.s, a.s_bytes);

    // Wave w's tasks: rounds 0 .. full-1 take TS codes at (i * waves + w) * TS;
    // the last round takes `last` codes (whole sub-slabs, < TS) at
    // full * waves * TS + w * last, so no wave does more than one sub-slab
    // beyond any other.
    const int64_t w = (int64_t)lb * wpb + wib;
    const int64_t e2 = a.full_end + w * a.last;   // this wave's last-round task
    auto at = [&](int32_t i, int64_t e) {
        DqCursor u;
        u.i = i;
        u.e = e;
        u.m = a.small ? (int64_t)fastdiv((uint32_t)e, a.k_div) : e / a.K;
        u.c = (uint32_t)(e - u.m * a.K);
        return u;
    };
    auto size_of = [&](const DqCursor &u) -> uint32_t {
        const int64_t cap = u.i < a.full ? TS : u.i == a.full ? a.last : 0;
        const int64_t left = total - u.e;
        return left <= 0 ? 0u : left < cap ? (uint32_t)left : (uint32_t)cap;
    };
    auto advance = [&](DqCursor u) {
        if (u.i + 1 < a.full) {
            u.i += 1;
            u.e += a.step;
            u.m += a.dm;
            u.c += a.dc;
            if (u.c >= K) {
                u.c -= K;
                u.m += 1;
            }
            return u;
        }
        if (u.i + 1 == a.full) return at(a.full, e2);
        u.i = a.full + 1;   // past the last round: empty
        return u;
    };
    DqCursor cur = a.full > 0 ? at(0, w * TS) : at(0, e2);
    if (size_of(cur) == 0) return;

    struct Task {
        DqCursor u;
        uint32_t c[NS][W / 4];
        uint32_t s[NS];  // fp32 scale bits, or the UE8M0 exponent byte
    };
    auto load = [&](Task &T) {
        T.u = cur;
        cur = advance(cur);
        const DqCursor &u = T.u;
        const uint32_t range = size_of(u);
        const rsrc_t rq = make_rsrc(a.q + (range ? u.e : 0), range);
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            const uint32_t off = k * SUB + lane * W;
            if constexpr (W == 4) {
                T.c[k][0] = __builtin_amdgcn_raw_buffer_load_b32(rq, off, 0, kDequantLoadPolicy);
            } else {
                const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rq, off, 0, kDequantLoadPolicy);
                T.c[k][0] = v.x;
                T.c[k][1] = v.y;
            }
            // row and column of this lane's codes
            uint32_t col = u.c + off;
            uint32_t m = (uint32_t)u.m;
            if (K >= (uint32_t)TS) {
                if (col >= K) {
                    col -= K;
                    m += 1;
                }
            } else {
                // quotient from an fp32 estimate (exact operands), off by at most one
                uint32_t d = (uint32_t)((float)col * a.inv_k);
                int32_t r = (int32_t)(col - d * K);
                if (r < 0) {
                    d -= 1;
                    r += (int32_t)K;
                } else if (r >= (int32_t)K) {
                    d += 1;
                    r -= (int32_t)K;
                }
                col = (uint32_t)r;
                m += d;
            }
            const uint32_t g = col >> a.log2g;
            uint32_t soff;
            if constexpr (SF == SCALE_F32) soff = (m * (uint32_t)a.st + g * (uint32_t)a.sg) * 4;
            else if constexpr (SL == LAYOUT_ROW) soff = m * (uint32_t)a.ng + g;
            else soff = ((g >> 2) * (uint32_t)a.rows_pad + m) * 4 + (g & 3);
            if (off >= range) soff = 0xFFFFFFF0u;   // past the end: read nothing
            if constexpr (SF == SCALE_F32)
                T.s[k] = __builtin_amdgcn_raw_buffer_load_b32(rs, soff, 0, 0);
            else
                T.s[k] = __builtin_amdgcn_raw_buffer_load_b8(rs, soff, 0, 0);
        }
    };
    auto process = [&](const Task &T) {
        const DqCursor &u = T.u;
        const uint32_t range = size_of(u);
        const rsrc_t ry = make_rsrc((char *)a.y + (range ? u.e * OSZ : 0), range * OSZ);
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            float sc;
            if constexpr (SF == SCALE_F32) sc = __uint_as_float(T.s[k]);
            else sc = __uint_as_float(T.s[k] == 0 ? 0x00400000u : T.s[k] << 23);   // 2^(e-127)
            float f[W];
#pragma unroll
            for (int i = 0; i < W / 4; ++i) {
                float d[4];
                decode_codes4<CODE>(T.c[k][i], d);
#pragma unroll
                for (int j = 0; j < 4; ++j) f[4 * i + j] = d[j] * sc;
            }
            u32x4 o;
            if constexpr (OUTD == IN_FP32) {
                o.x = __float_as_uint(f[0]);
                o.y = __float_as_uint(f[1]);
                o.z = __float_as_uint(f[2]);
                o.w = __float_as_uint(f[3]);
            } else if constexpr (OUTD == IN_BF16) {
                o.x = pack2_out_bf16(f[0], f[1]);
                o.y = pack2_out_bf16(f[2], f[3]);
                o.z = pack2_out_bf16(f[4], f[5]);
                o.w = pack2_out_bf16(f[6], f[7]);
            } else {
                o.x = pack2_out_fp16(f[0], f[1]);
                o.y = pack2_out_fp16(f[2], f[3]);
                o.z = pack2_out_fp16(f[4], f[5]);
                o.w = pack2_out_fp16(f[6], f[7]);
            }
            __builtin_amdgcn_raw_buffer_store_b128(o, ry, (k * SUB + lane * W) * OSZ, 0,
                                                   kDequantStorePolicy);
        }
    };

    // Two tasks in flight: the next task's loads are issued before the
    // current one is converted and stored.  An empty task loads nothing
    // (empty ranges) and ends the loop.
    Task A, B;
    load(A);
    while (true) {
        const bool hasB = size_of(cur) != 0;
        load(B);
        process(A);
        if (!hasB) break;
        const bool hasA = size_of(cur) != 0;
        load(A);
        process(B);
        if (!hasA) break;
    }
}

// --------------------------------------------------------------------------
// Probes: one step of the device arithmetic over arbitrary inputs.
// --------------------------------------------------------------------------

__global__ __launch_bounds__(256) void probe_e4m3_kernel(const float *__restrict__ v,
                                                         uint8_t *__restrict__ out, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = (uint8_t)(e4m3x4<true>(v[i], 0.0f, 0.0f, 0.0f) & 0xFFu);
}

// The scale step alone: amax = the fp32 with bit pattern first + i (a
// non-negative finite value), the group_scale of the quantization kernels.
template <int OUT, bool UE>
__global__ __launch_bounds__(256) void probe_scale_kernel(uint32_t first, int64_t n,
                                                          uint32_t eps_bits, void *scale_out,
                                                          float *inv_out)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        const Scale sc = group_scale<OUT>(first + (uint32_t)i, eps_bits, UE);
        if constexpr (UE)
            static_cast<uint8_t *>(scale_out)[i] = (uint8_t)sc.e;
        else
            static_cast<float *>(scale_out)[i] = sc.r;
        if (inv_out) inv_out[i] = sc.inv;
    }
}

// The int8 narrowing alone, over the fp32 values with bit patterns first + i
// (mod 2^32): the int8x4 of the quantization kernels.
__global__ __launch_bounds__(256) void probe_int8_kernel(uint32_t first, int64_t n,
                                                         int8_t *__restrict__ out)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        const float v = __uint_as_float(first + (uint32_t)i);
        out[i] = (int8_t)(uint8_t)(int8x4(v, 0.0f, 0.0f, 0.0f) & 0xFFu);
    }
}

// A stream with the plain quantization kernel's traffic and geometry and no
// arithmetic: each wave reads two 512-element slabs of 16-bit elements (two
// contiguous KiB per load instruction pair) and writes one byte per element
// (its low byte), 8 bytes per lane per slab; one wave per task, blocks dealt
// to the XCDs in chunks.  What it reaches is what the memory system gives
// this 2:1 read/write mix.
__global__ __launch_bounds__(256) void probe_stream_kernel(const uint16_t *x, int64_t n,
                                                           uint8_t *q, int32_t xcd_chunk)
{
    const int lane = threadIdx.x & 63;
    const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wpb = blockDim.x >> 6;
    const int64_t t = (int64_t)logical_block(blockIdx.x, gridDim.x, xcd_chunk) * wpb + wib;
    if (t * (2 * kSlab) >= n) return;                        // wave-uniform
    const rsrc_t rx = make_rsrc(x + t * (2 * kSlab), 2 * kSlab * 2);
    const rsrc_t rq = make_rsrc(q + t * (2 * kSlab), 2 * kSlab);
    u32x4 v[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
        v[s] = __builtin_amdgcn_raw_buffer_load_b128(rx, s * kSlab * 2 + lane * 16, 0,
                                                     kStreamPolicy);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        u32x2 o;
        o.x = __builtin_amdgcn_perm(v[s].y, v[s].x, 0x06040200u);
        o.y = __builtin_amdgcn_perm(v[s].w, v[s].z, 0x06040200u);
        __builtin_amdgcn_raw_buffer_store_b64(o, rq, s * kSlab + lane * 8, 0, kStreamPolicy);
    }
}

// path 0: direct evaluation; path 1: the bf16 lookup (global-memory copy of
// the table the fused kernels stage in LDS).
template <int IN>
__global__ __launch_bounds__(256) void probe_silu_kernel(const uint16_t *__restrict__ g,
                                                         const uint16_t *__restrict__ u,
                                                         float *__restrict__ out, int64_t n,
                                                         int path)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        float s, uf;
        if constexpr (IN == IN_BF16) {
            uf = __uint_as_float((uint32_t)u[i] << 16);
            if (path == 1) {
                // the fused kernels' lookup: the packed-pair offsets (gate i in
                // the low half, then in the high half, beside another gate)
                // when the gate is tabulated, else the per-gate form
                const uint32_t other = g[(i + 12345) % n];
                uint32_t lo0, hi0, lo1, hi1;
                bool in0, in1;
                silu_pair_offsets((uint32_t)g[i] | (other << 16), lo0, hi0, in0);
                silu_pair_offsets(other | ((uint32_t)g[i] << 16), lo1, hi1, in1);
                const uint32_t E = (g[i] >> 7) & 0xFFu, Eo = (other >> 7) & 0xFFu;
                const bool tabulated = E >= kTabElo && E <= kTabEhi;
                const bool both = tabulated && Eo >= kTabElo && Eo <= kTabEhi;
                if (in0 != both || in1 != both || (tabulated && lo0 != hi1))
                    s = __uint_as_float(0x7FC00000u);            // NaN: never equal
                else if (tabulated)
                    s = lds_f32_at(g_silu_table, lo0);
                else
                    s = silu_s_lookup(g[i], g_silu_table);
                (void)hi0; (void)lo1;
            } else {
                s = silu_s(__uint_as_float((uint32_t)g[i] << 16));
            }
        } else {
            uf = fp16_to_f32(u[i]);
            if (path == 1) {
                // the fp16 lookup: the packed-pair offsets (gate i in either
                // half), the table entry when the gate is tabulated, else the
                // direct evaluation
                const uint32_t other = g[(i + 12345) % n];
                uint32_t lo0, hi0, lo1, hi1;
                bool in0, in1;
                silu16_pair_offsets((uint32_t)g[i] | (other << 16), lo0, hi0, in0);
                silu16_pair_offsets(other | ((uint32_t)g[i] << 16), lo1, hi1, in1);
                const bool tabulated = (g[i] & 0x7FFFu) < kTab16Mag;
                const bool both = tabulated && (other & 0x7FFFu) < kTab16Mag;
                if (in0 != both || in1 != both || lo0 != hi1)
                    s = __uint_as_float(0x7FC00000u);            // NaN: never equal
                else if (tabulated)
                    s = lds_f32_at(g_silu_table16, lo0);
                else
                    s = silu_s(fp16_to_f32(g[i]));
                (void)hi0; (void)lo1;
            } else {
                s = silu_s(fp16_to_f32(g[i]));
            }
        }
        out[i] = s * uf;
    }
}

// --------------------------------------------------------------------------
// Launchers: runtime traits -> template instantiation.
// --------------------------------------------------------------------------

hipError_t launch_silu_table_init(hipStream_t stream)
{
    static_assert((kSiluTab + kSiluTab16) % 256 == 0, "whole blocks");
    silu_table_init_kernel<<<(kSiluTab + kSiluTab16) / 256, 256, 0, stream>>>();
    return hipGetLastError();
}

template <int IN, int G, bool FUSE, int OUT, int SF, int UMAX, bool TABLE>
static hipError_t launch_group_t(const GroupArgs &a, bool masked, unsigned grid, unsigned block,
                                 hipStream_t st)
{
    if (masked) {
        if (a.flat_slabs == 3)
            ptgq_masked_kernel<IN, G, FUSE, OUT, SF, UMAX, TABLE, 3>
                <<<grid, block, (size_t)a.num_experts * 2 * sizeof(int), st>>>(a);
        else if (a.flat_slabs == 4) {
            if constexpr (!FUSE || TABLE || UMAX != 1) return hipErrorInvalidValue;
            else
                ptgq_masked_kernel<IN, G, FUSE, OUT, SF, UMAX, TABLE, 4>
                    <<<grid, block, (size_t)a.num_experts * sizeof(int), st>>>(a);
        } else if (a.flat_slabs == 0)
            ptgq_masked_kernel<IN, G, FUSE, OUT, SF, UMAX, TABLE, 0>
                <<<grid, block, (size_t)a.num_experts * sizeof(int), st>>>(a);
        else
            return hipErrorInvalidValue;
    } else if constexpr (!FUSE && !TABLE && UMAX == 2) {
        if (a.flat_slabs == 1)
            ptgq_flat_kernel<IN, G, FUSE, OUT, SF, UMAX, TABLE, 1><<<grid, block, 0, st>>>(a);
        else if (a.flat_slabs == 2) {
            if constexpr (IN == IN_FP32) return hipErrorInvalidValue;
            else ptgq_flat_kernel<IN, G, FUSE, OUT, SF, UMAX, TABLE, 2><<<grid, block, 0, st>>>(a);
        } else if (a.flat_slabs == 3) {
            ptgq_flat_kernel<IN, G, FUSE, OUT, SF, UMAX, TABLE, 3><<<grid, block, 0, st>>>(a);
        } else if (a.flat_slabs == 0)
            ptgq_flat_kernel<IN, G, FUSE, OUT, SF, UMAX, TABLE, 0><<<grid, block, 0, st>>>(a);
        else
            return hipErrorInvalidValue;
    } else if constexpr (FUSE) {
        if (a.flat_slabs == 3)
            ptgq_flat_kernel<IN, G, FUSE, OUT, SF, UMAX, TABLE, 3><<<grid, block, 0, st>>>(a);
        else if (a.flat_slabs == 4) {
            if constexpr (TABLE || UMAX != 1) return hipErrorInvalidValue;
            else ptgq_flat_kernel<IN, G, FUSE, OUT, SF, UMAX, TABLE, 4><<<grid, block, 0, st>>>(a);
        } else if (a.flat_slabs == 0)
            ptgq_flat_kernel<IN, G, FUSE, OUT, SF, UMAX, TABLE, 0><<<grid, block, 0, st>>>(a);
        else
            return hipErrorInvalidValue;
    } else {
        if (a.flat_slabs) return hipErrorInvalidValue;
        ptgq_flat_kernel<IN, G, FUSE, OUT, SF, UMAX, TABLE, 0><<<grid, block, 0, st>>>(a);
    }
    return hipGetLastError();
}

// Task sizes: 1 or 2 slabs.  The LDS SiLU tables exist for 16-bit gates.
template <int IN, int G, bool FUSE, int OUT, int SF>
static hipError_t launch_group_u(const GroupArgs &a, bool table, bool masked, unsigned grid,
                                 unsigned block, hipStream_t st)
{
    constexpr bool T = FUSE && IN != IN_FP32;
    if (a.U != 1 && a.U != 2) return hipErrorInvalidValue;
    if (T && table)
        return a.U == 1 ? launch_group_t<IN, G, FUSE, OUT, SF, 1, T>(a, masked, grid, block, st)
                        : launch_group_t<IN, G, FUSE, OUT, SF, 2, T>(a, masked, grid, block, st);
    return a.U == 1 ? launch_group_t<IN, G, FUSE, OUT, SF, 1, false>(a, masked, grid, block, st)
                    : launch_group_t<IN, G, FUSE, OUT, SF, 2, false>(a, masked, grid, block, st);
}

template <int IN, int G, bool FUSE, int OUT>
static hipError_t launch_group_s(const GroupArgs &a, bool table, bool masked, unsigned grid,
                                 unsigned block, hipStream_t st)
{
    return a.scale_fmt == SCALE_UE8M0
               ? launch_group_u<IN, G, FUSE, OUT, SCALE_UE8M0>(a, table, masked, grid, block, st)
               : launch_group_u<IN, G, FUSE, OUT, SCALE_F32>(a, table, masked, grid, block, st);
}

template <int IN, int G, bool FUSE>
static hipError_t launch_group_o(const GroupArgs &a, int out, bool table, bool masked,
                                 unsigned grid, unsigned block, hipStream_t st)
{
    return out == OUT_E4M3
               ? launch_group_s<IN, G, FUSE, OUT_E4M3>(a, table, masked, grid, block, st)
               : launch_group_s<IN, G, FUSE, OUT_INT8>(a, table, masked, grid, block, st);
}

template <int IN, int G>
static hipError_t launch_group_f(const GroupArgs &a, bool fuse, int out, bool table, bool masked,
                                 unsigned grid, unsigned block, hipStream_t st)
{
    if constexpr (IN == IN_FP32) {   // fused calls take 16-bit inputs
        if (fuse) return hipErrorInvalidValue;
        return launch_group_o<IN, G, false>(a, out, table, masked, grid, block, st);
    } else {
        return fuse ? launch_group_o<IN, G, true>(a, out, table, masked, grid, block, st)
                    : launch_group_o<IN, G, false>(a, out, table, masked, grid, block, st);
    }
}

template <int IN>
static hipError_t launch_group_g(const GroupArgs &a, int G, bool fuse, int out, bool table,
                                 bool masked, unsigned grid, unsigned block, hipStream_t st)
{
    switch (G) {
    case 16: return launch_group_f<IN, 16>(a, fuse, out, table, masked, grid, block, st);
    case 32: return launch_group_f<IN, 32>(a, fuse, out, table, masked, grid, block, st);
    case 64: return launch_group_f<IN, 64>(a, fuse, out, table, masked, grid, block, st);
    case 128: return launch_group_f<IN, 128>(a, fuse, out, table, masked, grid, block, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_group(const GroupArgs &a, int in_dtype, int G, bool fuse, int out_dtype,
                        bool table, bool masked, unsigned grid, unsigned block,
                        hipStream_t stream)
{
    if (in_dtype == IN_BF16)
        return launch_group_g<IN_BF16>(a, G, fuse, out_dtype, table, masked, grid, block, stream);
    if (in_dtype == IN_FP16)
        return launch_group_g<IN_FP16>(a, G, fuse, out_dtype, table, masked, grid, block, stream);
    if (in_dtype == IN_FP32)
        return launch_group_g<IN_FP32>(a, G, fuse, out_dtype, false, masked, grid, block, stream);
    return hipErrorInvalidValue;
}

template <int IN, int VB>
static hipError_t launch_token_v(const TokenArgs &a, TokenMode mode, int nvl, unsigned grid,
                                 unsigned block, hipStream_t st)
{
    if (mode == TOKEN_BLOCK_LOOP) {
        ptq_block_loop_kernel<IN, VB><<<grid, block, 0, st>>>(a);
        return hipGetLastError();
    }
#define PTGQ_TOKEN_CASE(NVV)                                                   \
    case NVV:                                                                  \
        if (mode == TOKEN_WAVE)                                                \
            ptq_wave_kernel<IN, VB, NVV><<<grid, block, 0, st>>>(a);           \
        else if (mode == TOKEN_WAVE_LOOP)                                      \
            ptq_wave_loop_kernel<IN, VB, NVV><<<grid, block, 0, st>>>(a);      \
        else                                                                   \
            ptq_block_kernel<IN, VB, NVV><<<grid, block, 0, st>>>(a);          \
        return hipGetLastError();
    switch (nvl) {
        PTGQ_TOKEN_CASE(1)
        PTGQ_TOKEN_CASE(2)
        PTGQ_TOKEN_CASE(4)
        PTGQ_TOKEN_CASE(7)
        PTGQ_TOKEN_CASE(8)
        PTGQ_TOKEN_CASE(16)
    default: return hipErrorInvalidValue;
    }
#undef PTGQ_TOKEN_CASE
}

hipError_t launch_token(const TokenArgs &a, int in_dtype, int vec_bytes, TokenMode mode,
                        int nv_per_lane, unsigned grid, unsigned block, hipStream_t stream)
{
    if (in_dtype == IN_FP32)
        return vec_bytes == 16 ? launch_token_v<IN_FP32, 16>(a, mode, nv_per_lane, grid, block,
                                                             stream)
                               : hipErrorInvalidValue;
    if (in_dtype == IN_BF16)
        return vec_bytes == 16
                   ? launch_token_v<IN_BF16, 16>(a, mode, nv_per_lane, grid, block, stream)
                   : launch_token_v<IN_BF16, 8>(a, mode, nv_per_lane, grid, block, stream);
    if (in_dtype == IN_FP16)
        return vec_bytes == 16
                   ? launch_token_v<IN_FP16, 16>(a, mode, nv_per_lane, grid, block, stream)
                   : launch_token_v<IN_FP16, 8>(a, mode, nv_per_lane, grid, block, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_requant(const RequantArgs &a, unsigned grid, unsigned block, hipStream_t stream)
{
    const size_t lds = 2 * (size_t)a.E * sizeof(int);
    if (a.tcodes == kRqSub)
        requant_fp8_kernel<1><<<grid, block, lds, stream>>>(a);
    else if (a.tcodes == 2 * kRqSub)
        requant_fp8_kernel<2><<<grid, block, lds, stream>>>(a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

template <int CODE, int SF, int SL, int OUTD>
static hipError_t launch_dequant_n(const DequantArgs &a, unsigned grid, unsigned block,
                                   hipStream_t stream)
{
    switch (a.ns) {
    case 1: dequant_kernel<CODE, SF, SL, OUTD, 1><<<grid, block, 0, stream>>>(a); break;
    case 4: dequant_kernel<CODE, SF, SL, OUTD, 4><<<grid, block, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int CODE, int SF, int SL>
static hipError_t launch_dequant_o(const DequantArgs &a, int out_dtype, unsigned grid,
                                   unsigned block, hipStream_t stream)
{
    switch (out_dtype) {
    case IN_BF16: return launch_dequant_n<CODE, SF, SL, IN_BF16>(a, grid, block, stream);
    case IN_FP16: return launch_dequant_n<CODE, SF, SL, IN_FP16>(a, grid, block, stream);
    case IN_FP32: return launch_dequant_n<CODE, SF, SL, IN_FP32>(a, grid, block, stream);
    default: return hipErrorInvalidValue;
    }
}

template <int CODE>
static hipError_t launch_dequant_c(const DequantArgs &a, int scale_fmt, int scale_layout,
                                   int out_dtype, unsigned grid, unsigned block, hipStream_t stream)
{
    if (scale_fmt == SCALE_F32)   // fp32 layouts differ only in strides
        return launch_dequant_o<CODE, SCALE_F32, LAYOUT_ROW>(a, out_dtype, grid, block, stream);
    if (scale_layout == LAYOUT_ROW)
        return launch_dequant_o<CODE, SCALE_UE8M0, LAYOUT_ROW>(a, out_dtype, grid, block, stream);
    return launch_dequant_o<CODE, SCALE_UE8M0, LAYOUT_COL>(a, out_dtype, grid, block, stream);
}

hipError_t launch_dequant(const DequantArgs &a, int code_dtype, int scale_fmt, int scale_layout,
                          int out_dtype, unsigned grid, unsigned block, hipStream_t stream)
{
    if (code_dtype == OUT_E4M3)
        return launch_dequant_c<OUT_E4M3>(a, scale_fmt, scale_layout, out_dtype, grid, block,
                                          stream);
    if (code_dtype == OUT_INT8)
        return launch_dequant_c<OUT_INT8>(a, scale_fmt, scale_layout, out_dtype, grid, block,
                                          stream);
    return hipErrorInvalidValue;
}

hipError_t launch_probe_e4m3(const float *v, uint8_t *out, int64_t n, hipStream_t stream)
{
    const unsigned grid = (unsigned)((n + 255) / 256);
    probe_e4m3_kernel<<<grid, 256, 0, stream>>>(v, out, n);
    return hipGetLastError();
}

hipError_t launch_probe_scale(uint32_t first, int64_t n, float eps, int out_dtype, int scale_fmt,
                              void *scale_out, float *inv_out, hipStream_t stream)
{
    const unsigned grid = (unsigned)((n + 255) / 256);
    const uint32_t eb = __builtin_bit_cast(uint32_t, eps);
    const bool ue = scale_fmt == SCALE_UE8M0;
    if (out_dtype == OUT_E4M3) {
        if (ue) probe_scale_kernel<OUT_E4M3, true><<<grid, 256, 0, stream>>>(first, n, eb, scale_out, inv_out);
        else probe_scale_kernel<OUT_E4M3, false><<<grid, 256, 0, stream>>>(first, n, eb, scale_out, inv_out);
    } else {
        if (ue) probe_scale_kernel<OUT_INT8, true><<<grid, 256, 0, stream>>>(first, n, eb, scale_out, inv_out);
        else probe_scale_kernel<OUT_INT8, false><<<grid, 256, 0, stream>>>(first, n, eb, scale_out, inv_out);
    }
    return hipGetLastError();
}

hipError_t launch_probe_int8(uint32_t first, int64_t n, int8_t *out, hipStream_t stream)
{
    probe_int8_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(first, n, out);
    return hipGetLastError();
}

hipError_t launch_probe_stream(const void *x, int64_t n, uint8_t *q, unsigned grid,
                               int32_t xcd_chunk, hipStream_t stream)
{
    probe_stream_kernel<<<grid, 256, 0, stream>>>(static_cast<const uint16_t *>(x), n, q,
                                                  xcd_chunk);
    return hipGetLastError();
}

hipError_t launch_probe_silu(const void *g, const void *u, int in_dtype, int path, float *out,
                             int64_t n, hipStream_t stream)
{
    const unsigned grid = (unsigned)((n + 255) / 256);
    const uint16_t *gg = static_cast<const uint16_t *>(g);
    const uint16_t *uu = static_cast<const uint16_t *>(u);
    if (in_dtype == IN_BF16)
        probe_silu_kernel<IN_BF16><<<grid, 256, 0, stream>>>(gg, uu, out, n, path);
    else
        probe_silu_kernel<IN_FP16><<<grid, 256, 0, stream>>>(gg, uu, out, n, path);
    return hipGetLastError();
}

}  // namespace ptgq
