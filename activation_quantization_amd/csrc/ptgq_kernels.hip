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
// Fused SiLU.  silu(g) * u = (g / (1 + e^-g)) * u with e^-g correctly
// rounded to binary32: the double-precision exp is within about one double
// ulp, far inside the distance of e^-g from any binary32 rounding boundary
// for every 16-bit gate (checked exhaustively on the device against the
// oracle).  Each other step is one IEEE fp32 operation.
// --------------------------------------------------------------------------

__device__ __forceinline__ float silu_mul(float g, float u)
{
    const float e = (float)exp(-(double)g);
    const float d = 1.0f + e;
    const float s = g / d;
    return s * u;
}

// --------------------------------------------------------------------------
// Cluster max with DPP.  All lanes of each aligned LANES-lane cluster end
// with the cluster maximum.  Values are non-negative.
// --------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp_max(float v)
{
    const int o = __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF,
                                              0xF, false);
    return fmaxf(v, __int_as_float(o));
}

template <int LANES>
__device__ __forceinline__ float cluster_max(float v)
{
    if constexpr (LANES >= 2) v = dpp_max<0xB1>(v);    // quad_perm [1,0,3,2]
    if constexpr (LANES >= 4) v = dpp_max<0x4E>(v);    // quad_perm [2,3,0,1]
    if constexpr (LANES >= 8) v = dpp_max<0x141>(v);   // row_half_mirror
    if constexpr (LANES >= 16) v = dpp_max<0x140>(v);  // row_mirror
    return v;
}

__device__ __forceinline__ float wave_max(float v)
{
    v = cluster_max<16>(v);
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

// --------------------------------------------------------------------------
// Scale of one group: r = max(amax, eps) / qmax; fp32 multiplier 1/r (0 if
// r == 0), or UE8M0 byte e and exact multiplier 2^(127 - e).
// --------------------------------------------------------------------------

struct Scale {
    float inv;       // multiplier applied to y
    float r;         // fp32 scale
    uint32_t e;      // UE8M0 byte
};

__device__ __forceinline__ Scale group_scale(float amax, float eps, float qmax, bool ue8m0)
{
    Scale sc;
    const float a = (amax > eps) ? amax : eps;
    sc.r = a / qmax;
    if (!ue8m0) {
        sc.e = 0;
        sc.inv = (sc.r == 0.0f) ? 0.0f : 1.0f / sc.r;
    } else {
        const uint32_t b = __float_as_uint(sc.r);
        sc.e = ((b >> 23) & 0xFFu) + ((b & 0x7FFFFFu) != 0u ? 1u : 0u);
        sc.inv = __uint_as_float((254u - sc.e) << 23);
    }
    return sc;
}

// --------------------------------------------------------------------------
// Narrowing.
// --------------------------------------------------------------------------

// 4 floats -> 4 OCP e4m3 codes (byte i = code of value i).  The clamp makes
// the conversion saturating; -0 and negative values that round to zero keep
// the sign bit.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d)
{
    a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
    d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
    int p = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    p = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, p, true);
    return (uint32_t)p;
}

__device__ __forceinline__ uint32_t int8_1(float v)
{
    const float r = __builtin_amdgcn_fmed3f(__builtin_rintf(v), -128.0f, 127.0f);
    return (uint32_t)((int)r) & 0xFFu;
}

__device__ __forceinline__ uint32_t int8x4(float a, float b, float c, float d)
{
    return int8_1(a) | (int8_1(b) << 8) | (int8_1(c) << 16) | (int8_1(d) << 24);
}

template <int OUT>
__device__ __forceinline__ uint2 narrow8(const float (&v)[8])
{
    uint2 o;
    if constexpr (OUT == OUT_E4M3) {
        o.x = e4m3x4(v[0], v[1], v[2], v[3]);
        o.y = e4m3x4(v[4], v[5], v[6], v[7]);
    } else {
        o.x = int8x4(v[0], v[1], v[2], v[3]);
        o.y = int8x4(v[4], v[5], v[6], v[7]);
    }
    return o;
}

// --------------------------------------------------------------------------
// One task: slabs [j*U, min(j*U + U, spr)) of row m.
//   xe, qe, se: bases of this expert (flat: the tensors themselves).
// --------------------------------------------------------------------------

template <int IN, int G, bool FUSE, int OUT>
__device__ __forceinline__ void group_task(const GroupArgs &a, const uint16_t *__restrict__ xe,
                                           uint8_t *__restrict__ qe, uint8_t *__restrict__ se,
                                           int64_t m, int j, int lane)
{
    constexpr int LPG = G / 8;          // lanes per group
    constexpr int GPS = kSlab / G;      // groups per slab (>= 4)
    const float qmax = (OUT == OUT_E4M3) ? 448.0f : 127.0f;
    const int s_begin = j * a.U;
    const int ns = min(a.U, a.spr - s_begin);   // wave-uniform, >= 1
    const uint16_t *xr = xe + m * a.in_stride;
    uint8_t *qr = qe + m * a.K;

    uint4 rg[kMaxSlabsPerTask], ru[kMaxSlabsPerTask];
#pragma unroll
    for (int s = 0; s < kMaxSlabsPerTask; ++s) {
        rg[s] = make_uint4(0, 0, 0, 0);
        ru[s] = make_uint4(0, 0, 0, 0);
        if (s < ns) {
            const int64_t col = (int64_t)(s_begin + s) * kSlab + lane * 8;
            if (col < a.K) {
                rg[s] = *reinterpret_cast<const uint4 *>(xr + col);
                if constexpr (FUSE) ru[s] = *reinterpret_cast<const uint4 *>(xr + a.K + col);
            }
        }
    }

#pragma unroll
    for (int s = 0; s < kMaxSlabsPerTask; ++s) {
        if (s < ns) {
            const int64_t col = (int64_t)(s_begin + s) * kSlab + lane * 8;
            const bool valid = col < a.K;
            float y[8];
            widen8<IN>(rg[s], y);
            if constexpr (FUSE) {
                float u[8];
                widen8<IN>(ru[s], u);
#pragma unroll
                for (int k = 0; k < 8; ++k) y[k] = silu_mul(y[k], u[k]);
            }
            float amax = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(y[k]));
            amax = cluster_max<LPG>(amax);

            const bool ue8m0 = a.scale_fmt == SCALE_UE8M0;
            const Scale sc = group_scale(amax, a.eps, qmax, ue8m0);
            float v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = y[k] * sc.inv;
            const uint2 codes = narrow8<OUT>(v);
            if (valid) *reinterpret_cast<uint2 *>(qr + col) = codes;

            // scales
            const int lg = lane / LPG;                        // group within slab
            const int64_t gi = (int64_t)(s_begin + s) * GPS + lg;  // group within row
            const bool leader = (lane % LPG) == 0;
            if (ue8m0 && a.scale_layout == LAYOUT_COL) {
                const uint32_t byte = valid ? sc.e : 0u;
                const uint32_t b1 = (uint32_t)__shfl((int)byte, lane + LPG);
                const uint32_t b2 = (uint32_t)__shfl((int)byte, lane + 2 * LPG);
                const uint32_t b3 = (uint32_t)__shfl((int)byte, lane + 3 * LPG);
                if (leader && (lg & 3) == 0 && valid) {
                    const uint32_t word = byte | (b1 << 8) | (b2 << 16) | (b3 << 24);
                    reinterpret_cast<uint32_t *>(se)[(gi >> 2) * a.rows_pad + m] = word;
                }
            } else if (leader && valid) {
                if (ue8m0)
                    se[m * a.ng + gi] = (uint8_t)sc.e;
                else if (a.scale_layout == LAYOUT_ROW)
                    reinterpret_cast<float *>(se)[m * a.ng + gi] = sc.r;
                else
                    reinterpret_cast<float *>(se)[gi * a.rows_pad + m] = sc.r;
            }
        }
    }
}

// XCD-aware logical block id: blocks are dealt to the 8 XCDs round-robin, so
// with a grid that is a multiple of 8, XCD x gets logical ids
// [x * nb/8, (x+1) * nb/8), a contiguous range of tasks.
__device__ __forceinline__ int logical_block(int b, int nb)
{
    return (nb & 7) == 0 ? (b & 7) * (nb >> 3) + (b >> 3) : b;
}

template <int IN, int G, bool FUSE, int OUT>
__global__ __launch_bounds__(256) void ptgq_flat_kernel(GroupArgs a)
{
    const int lane = threadIdx.x & 63;
    const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wpb = blockDim.x >> 6;
    const int lb = logical_block(blockIdx.x, gridDim.x);
    const int total = gridDim.x * wpb;
    const uint16_t *x = static_cast<const uint16_t *>(a.x);
    uint8_t *s = static_cast<uint8_t *>(a.s);
    for (int t = lb * wpb + wib; t < a.n_tasks; t += total) {
        const int m = t / a.tpr;
        const int j = t - m * a.tpr;
        group_task<IN, G, FUSE, OUT>(a, x, a.q, s, m, j, lane);
    }
    // column-major pad slots (rows M .. rows_pad-1) are zero
    if (a.pad_cols > 0 && lb == 0 && wib == 0) {
        const int64_t npad = (a.rows_pad - a.rows) * (int64_t)a.pad_cols;
        for (int64_t i = lane; i < npad; i += 64) {
            const int64_t r = a.rows + i / a.pad_cols;
            const int64_t c = i % a.pad_cols;
            reinterpret_cast<uint32_t *>(s)[c * a.rows_pad + r] = 0u;
        }
    }
}

template <int IN, int G, bool FUSE, int OUT>
__global__ __launch_bounds__(256) void ptgq_masked_kernel(GroupArgs a)
{
    const int lane = threadIdx.x & 63;
    const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wpb = blockDim.x >> 6;
    const int e = blockIdx.x / a.blocks_per_expert;
    const int lb = blockIdx.x - e * a.blocks_per_expert;
    int live = a.masked_m[e];
    live = live < 0 ? 0 : (live > a.rows ? (int)a.rows : live);
    const int n = live * a.tpr;
    const uint16_t *xe = static_cast<const uint16_t *>(a.x) + e * a.x_expert_stride;
    uint8_t *qe = a.q + e * a.q_expert_stride;
    uint8_t *se = static_cast<uint8_t *>(a.s) + e * a.s_expert_stride;
    const int stride = a.blocks_per_expert * wpb;
    for (int t = lb * wpb + wib; t < n; t += stride) {
        const int m = t / a.tpr;
        const int j = t - m * a.tpr;
        group_task<IN, G, FUSE, OUT>(a, xe, qe, se, m, j, lane);
    }
}

// --------------------------------------------------------------------------
// Whole-row per-token e4m3 (sglang #34257 review page, key source snippets):
// scale = rowmax / 448 with no floor, multiplier 0 for a zero row.
// A row is read once: it stays in registers between the max and the
// quantization pass (TOKEN_WAVE: one wave per row; TOKEN_BLOCK: one 256-lane
// block per row); very long rows take the two-pass TOKEN_BLOCK_LOOP form.
// --------------------------------------------------------------------------

template <int IN, int VB>
struct TokVec {
    static constexpr int insz = (IN == IN_FP32) ? 4 : 2;
    static constexpr int EV = VB / insz;    // elements per vector
    using raw_t = typename std::conditional<VB == 16, uint4, uint2>::type;

    __device__ static __forceinline__ raw_t load(const uint8_t *p)
    {
        return *reinterpret_cast<const raw_t *>(p);
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
    __device__ static __forceinline__ void store_codes(uint8_t *p, const float (&v)[EV])
    {
        if constexpr (EV == 8) {
            uint2 o;
            o.x = e4m3x4(v[0], v[1], v[2], v[3]);
            o.y = e4m3x4(v[4], v[5], v[6], v[7]);
            *reinterpret_cast<uint2 *>(p) = o;
        } else {
            *reinterpret_cast<uint32_t *>(p) = e4m3x4(v[0], v[1], v[2], v[3]);
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
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        float f[EV];
        TV::widen(raw[k], f);
#pragma unroll
        for (int e = 0; e < EV; ++e) amax = fmaxf(amax, fabsf(f[e]));
    }
    amax = wave_max(amax);
    float r;
    const float inv = token_inv(amax, r);
    if (lane == 0) a.s[m] = r;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int i = lane + 64 * k;
        if (i < a.nv) {
            float f[EV];
            TV::widen(raw[k], f);
#pragma unroll
            for (int e = 0; e < EV; ++e) f[e] = f[e] * inv;
            TV::store_codes(qr + (int64_t)i * EV, f);
        }
    }
}

__device__ __forceinline__ float block_max(float v, float *red)
{
    v = wave_max(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float m = red[0];
    for (int i = 1; i < (int)(blockDim.x >> 6); ++i) m = fmaxf(m, red[i]);
    return m;
}

template <int IN, int VB, int NV>
__global__ __launch_bounds__(256) void ptq_block_kernel(TokenArgs a)
{
    using TV = TokVec<IN, VB>;
    constexpr int EV = TV::EV;
    __shared__ float red[4];
    const int tid = threadIdx.x;
    const int64_t m = blockIdx.x;
    const uint8_t *xr = static_cast<const uint8_t *>(a.x) + m * a.K * TV::insz;
    uint8_t *qr = a.q + m * a.K;
    typename TV::raw_t raw[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int i = tid + 256 * k;
        raw[k] = (i < a.nv) ? TV::load(xr + (int64_t)i * VB) : TV::zero();
    }
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        float f[EV];
        TV::widen(raw[k], f);
#pragma unroll
        for (int e = 0; e < EV; ++e) amax = fmaxf(amax, fabsf(f[e]));
    }
    amax = block_max(amax, red);
    float r;
    const float inv = token_inv(amax, r);
    if (tid == 0) a.s[m] = r;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int i = tid + 256 * k;
        if (i < a.nv) {
            float f[EV];
            TV::widen(raw[k], f);
#pragma unroll
            for (int e = 0; e < EV; ++e) f[e] = f[e] * inv;
            TV::store_codes(qr + (int64_t)i * EV, f);
        }
    }
}

template <int IN, int VB>
__global__ __launch_bounds__(256) void ptq_block_loop_kernel(TokenArgs a)
{
    using TV = TokVec<IN, VB>;
    constexpr int EV = TV::EV;
    __shared__ float red[4];
    const int tid = threadIdx.x;
    const int64_t m = blockIdx.x;
    const uint8_t *xr = static_cast<const uint8_t *>(a.x) + m * a.K * TV::insz;
    uint8_t *qr = a.q + m * a.K;
    float amax = 0.0f;
    for (int i = tid; i < a.nv; i += 256) {
        float f[EV];
        TV::widen(TV::load(xr + (int64_t)i * VB), f);
#pragma unroll
        for (int e = 0; e < EV; ++e) amax = fmaxf(amax, fabsf(f[e]));
    }
    amax = block_max(amax, red);
    float r;
    const float inv = token_inv(amax, r);
    if (tid == 0) a.s[m] = r;
    for (int i = tid; i < a.nv; i += 256) {
        float f[EV];
        TV::widen(TV::load(xr + (int64_t)i * VB), f);
#pragma unroll
        for (int e = 0; e < EV; ++e) f[e] = f[e] * inv;
        TV::store_codes(qr + (int64_t)i * EV, f);
    }
}

// --------------------------------------------------------------------------
// Probes: one step of the device arithmetic over arbitrary inputs.
// --------------------------------------------------------------------------

__global__ __launch_bounds__(256) void probe_e4m3_kernel(const float *__restrict__ v,
                                                         uint8_t *__restrict__ out, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = (uint8_t)(e4m3x4(v[i], 0.0f, 0.0f, 0.0f) & 0xFFu);
}

template <int IN>
__global__ __launch_bounds__(256) void probe_silu_kernel(const uint16_t *__restrict__ g,
                                                         const uint16_t *__restrict__ u,
                                                         float *__restrict__ out, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        float gf, uf;
        if constexpr (IN == IN_BF16) {
            gf = __uint_as_float((uint32_t)g[i] << 16);
            uf = __uint_as_float((uint32_t)u[i] << 16);
        } else {
            gf = fp16_to_f32(g[i]);
            uf = fp16_to_f32(u[i]);
        }
        out[i] = silu_mul(gf, uf);
    }
}

// --------------------------------------------------------------------------
// Launchers: runtime traits -> template instantiation.
// --------------------------------------------------------------------------

template <int IN, int G, bool FUSE, int OUT>
static hipError_t launch_group_t(const GroupArgs &a, bool masked, unsigned grid, unsigned block,
                                 hipStream_t st)
{
    if (masked)
        ptgq_masked_kernel<IN, G, FUSE, OUT><<<grid, block, 0, st>>>(a);
    else
        ptgq_flat_kernel<IN, G, FUSE, OUT><<<grid, block, 0, st>>>(a);
    return hipGetLastError();
}

template <int IN, int G, bool FUSE>
static hipError_t launch_group_o(const GroupArgs &a, int out, bool masked, unsigned grid,
                                 unsigned block, hipStream_t st)
{
    return out == OUT_E4M3 ? launch_group_t<IN, G, FUSE, OUT_E4M3>(a, masked, grid, block, st)
                           : launch_group_t<IN, G, FUSE, OUT_INT8>(a, masked, grid, block, st);
}

template <int IN, int G>
static hipError_t launch_group_f(const GroupArgs &a, bool fuse, int out, bool masked,
                                 unsigned grid, unsigned block, hipStream_t st)
{
    return fuse ? launch_group_o<IN, G, true>(a, out, masked, grid, block, st)
                : launch_group_o<IN, G, false>(a, out, masked, grid, block, st);
}

template <int IN>
static hipError_t launch_group_g(const GroupArgs &a, int G, bool fuse, int out, bool masked,
                                 unsigned grid, unsigned block, hipStream_t st)
{
    switch (G) {
    case 16: return launch_group_f<IN, 16>(a, fuse, out, masked, grid, block, st);
    case 32: return launch_group_f<IN, 32>(a, fuse, out, masked, grid, block, st);
    case 64: return launch_group_f<IN, 64>(a, fuse, out, masked, grid, block, st);
    case 128: return launch_group_f<IN, 128>(a, fuse, out, masked, grid, block, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_group(const GroupArgs &a, int in_dtype, int G, bool fuse, int out_dtype,
                        bool masked, unsigned grid, unsigned block, hipStream_t stream)
{
    if (in_dtype == IN_BF16)
        return launch_group_g<IN_BF16>(a, G, fuse, out_dtype, masked, grid, block, stream);
    if (in_dtype == IN_FP16)
        return launch_group_g<IN_FP16>(a, G, fuse, out_dtype, masked, grid, block, stream);
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
        else                                                                   \
            ptq_block_kernel<IN, VB, NVV><<<grid, block, 0, st>>>(a);          \
        return hipGetLastError();
    switch (nvl) {
        PTGQ_TOKEN_CASE(1)
        PTGQ_TOKEN_CASE(2)
        PTGQ_TOKEN_CASE(4)
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

hipError_t launch_probe_e4m3(const float *v, uint8_t *out, int64_t n, hipStream_t stream)
{
    const unsigned grid = (unsigned)((n + 255) / 256);
    probe_e4m3_kernel<<<grid, 256, 0, stream>>>(v, out, n);
    return hipGetLastError();
}

hipError_t launch_probe_silu(const void *g, const void *u, int in_dtype, float *out, int64_t n,
                             hipStream_t stream)
{
    const unsigned grid = (unsigned)((n + 255) / 256);
    const uint16_t *gg = static_cast<const uint16_t *>(g);
    const uint16_t *uu = static_cast<const uint16_t *>(u);
    if (in_dtype == IN_BF16)
        probe_silu_kernel<IN_BF16><<<grid, 256, 0, stream>>>(gg, uu, out, n);
    else
        probe_silu_kernel<IN_FP16><<<grid, 256, 0, stream>>>(gg, uu, out, n);
    return hipGetLastError();
}

}  // namespace ptgq
