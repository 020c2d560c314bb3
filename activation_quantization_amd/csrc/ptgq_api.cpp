// C ABI of libptgq: argument validation, launch-geometry chooser and
// dispatch to the gfx950 kernels.  Declarations and contracts: include/ptgq.h.
//
// Validation is a pure host function of the scalar arguments and pointer
// values; it runs before any HIP call, so an invalid call touches no device
// and launches nothing.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "ptgq.h"
#include "ptgq_internal.h"

using namespace ptgq;

namespace {

// ----------------------------------------------------------------- devices

constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
int g_dev_cus[kMaxDevices];            // compute units; 0 = query failed

int device_cus(int dev)
{
    if (dev < 0 || dev >= kMaxDevices) return 0;
    std::call_once(g_dev_once[dev], [dev] {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 0;
        g_dev_cus[dev] = cus;
    });
    return g_dev_cus[dev];
}

int current_cus(int *dev_out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (dev_out) *dev_out = dev;
    return device_cus(dev);
}

// ------------------------------------------------------------ tuning knobs
// Process-wide overrides of the geometry chooser (diagnostics and sweeps
// only; -1 = automatic), set through ptgq_set_tuning.
std::atomic<int64_t> g_knob[4] = {{-1}, {-1}, {-1}, {-1}};
enum { KNOB_SLABS_PER_TASK = 0, KNOB_WAVES_PER_BLOCK = 1, KNOB_BLOCKS_PER_CU = 2,
       KNOB_TOKEN_MODE = 3 };

int64_t knob(int k) { return g_knob[k].load(std::memory_order_relaxed); }

// -------------------------------------------------------------- validation

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_group_size(int G) { return G == 16 || G == 32 || G == 64 || G == 128; }

int64_t pad4(int64_t n) { return (n + 3) / 4 * 4; }

// `outer` multiplies the rows (number of experts for the masked layout, 1
// for flat calls); an empty problem needs no pointers.
int check_group_args(const void *x, int in_dtype, int64_t outer, int64_t rows, int64_t K, int G,
                     int out_dtype, int scale_fmt, int scale_layout, float eps, const void *q,
                     const void *s)
{
    if (in_dtype != PTGQ_BF16 && in_dtype != PTGQ_FP16) return PTGQ_EINVAL;
    if (out_dtype != PTGQ_E4M3 && out_dtype != PTGQ_INT8) return PTGQ_EINVAL;
    if (scale_fmt != PTGQ_SCALE_F32 && scale_fmt != PTGQ_SCALE_UE8M0) return PTGQ_EINVAL;
    if (scale_layout != PTGQ_ROW_MAJOR && scale_layout != PTGQ_COL_MAJOR) return PTGQ_EINVAL;
    if (!valid_group_size(G)) return PTGQ_EINVAL;
    if (outer < 0 || rows < 0 || K < 0 || K % G != 0) return PTGQ_EINVAL;
    if (!(std::isfinite(eps) && eps >= 0.0f)) return PTGQ_EINVAL;
    if (outer == 0 || rows == 0 || K == 0) return PTGQ_OK;
    if (!x || !q || !s) return PTGQ_EINVAL;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4)) return PTGQ_EALIGN;
    return PTGQ_OK;
}

// --------------------------------------------------------- geometry chooser

struct GroupGeom {
    int U;          // slabs per task
    int wpb;        // waves per block
    unsigned grid;  // blocks
};

// Flat schedule.  Few tasks (decode-sized M): one slab per task and one-wave
// blocks, so that the groups spread over as many CUs as possible.  Many tasks
// (prefill-sized M): up to 4 slabs per task so each lane keeps 4 x 16 B (8 x
// when fused) in flight, 4-wave blocks, and a grid capped at a few blocks per
// CU that loops over the tasks (a multiple of 8 so each XCD gets the same
// share).
GroupGeom choose_flat(int64_t rows, int32_t spr, int cus)
{
    GroupGeom g;
    const int64_t slabs = rows * spr;
    const int64_t wave_slots = (int64_t)cus * 4 * 8;   // 8 waves per SIMD
    int U = 1;
    if (slabs >= 4 * wave_slots) U = 4;
    else if (slabs >= 2 * wave_slots) U = 2;
    if (knob(KNOB_SLABS_PER_TASK) > 0) U = (int)std::min<int64_t>(knob(KNOB_SLABS_PER_TASK), 4);
    U = std::min(U, (int)spr);
    g.U = U;
    const int64_t tasks = rows * (((int64_t)spr + U - 1) / U);
    int wpb = tasks >= (int64_t)cus * 4 ? 4 : 1;
    if (knob(KNOB_WAVES_PER_BLOCK) > 0) wpb = (int)std::min<int64_t>(knob(KNOB_WAVES_PER_BLOCK), 4);
    g.wpb = wpb;
    int64_t blocks = (tasks + wpb - 1) / wpb;
    int64_t per_cu = 8;
    if (knob(KNOB_BLOCKS_PER_CU) > 0) per_cu = knob(KNOB_BLOCKS_PER_CU);
    const int64_t cap = (int64_t)cus * per_cu;
    if (blocks > cap) blocks = cap;
    if (blocks >= 64) blocks = blocks / 8 * 8;
    g.grid = (unsigned)std::max<int64_t>(blocks, 1);
    return g;
}

int launch_group_common(const void *x, int in_dtype, int64_t rows, int64_t K, int G, int fuse,
                        int out_dtype, int scale_fmt, int scale_layout, float eps, void *q,
                        void *s, const int32_t *masked_m, int64_t E, int64_t expected_m,
                        void *stream)
{
    int dev = 0;
    const int cus = current_cus(&dev);
    if (cus <= 0) return PTGQ_EDEVICE;

    GroupArgs a;
    std::memset(&a, 0, sizeof(a));
    a.x = x;
    a.q = static_cast<uint8_t *>(q);
    a.s = s;
    a.masked_m = masked_m;
    a.rows = rows;
    a.K = K;
    a.in_stride = fuse ? 2 * K : K;
    a.ng = K / G;
    a.rows_pad = pad4(rows);
    a.eps = eps;
    a.spr = (int32_t)((K + kSlab - 1) / kSlab);
    a.scale_fmt = scale_fmt;
    a.scale_layout = scale_layout;
    const bool masked = masked_m != nullptr;

    GroupGeom geo;
    if (!masked) {
        geo = choose_flat(rows, a.spr, cus);
        a.U = geo.U;
        a.tpr = (a.spr + a.U - 1) / a.U;
        const int64_t tasks = rows * (int64_t)a.tpr;
        if (tasks >= INT32_MAX) return PTGQ_EUNSUPPORTED;
        a.n_tasks = (int32_t)tasks;
        if (scale_layout == PTGQ_COL_MAJOR && a.rows_pad > rows)
            a.pad_cols = (int32_t)(scale_fmt == PTGQ_SCALE_UE8M0 ? (a.ng + 3) / 4 : a.ng);
    } else {
        // Masked schedule: each expert gets the blocks its expected live rows
        // need (all tokens_pad rows when unknown); every block reads masked_m
        // on the device and loops over the expert's live tasks.
        const int64_t hint = (expected_m > 0 && expected_m < rows) ? expected_m : rows;
        const int64_t slabs = std::max<int64_t>(hint, 1) * a.spr * E;
        int U = slabs >= (int64_t)cus * 4 * 8 * 4 ? 4 : 1;
        if (knob(KNOB_SLABS_PER_TASK) > 0) U = (int)std::min<int64_t>(knob(KNOB_SLABS_PER_TASK), 4);
        U = std::min(U, (int)a.spr);
        a.U = U;
        a.tpr = (a.spr + U - 1) / U;
        if (rows * (int64_t)a.tpr >= INT32_MAX) return PTGQ_EUNSUPPORTED;
        const int64_t tasks_hint = std::max<int64_t>(hint, 1) * a.tpr;
        int wpb = tasks_hint * E >= (int64_t)cus * 4 ? 4 : 1;
        if (knob(KNOB_WAVES_PER_BLOCK) > 0) wpb = (int)std::min<int64_t>(knob(KNOB_WAVES_PER_BLOCK), 4);
        int64_t bpe = (tasks_hint + wpb - 1) / wpb;
        int64_t per_cu = knob(KNOB_BLOCKS_PER_CU) > 0 ? knob(KNOB_BLOCKS_PER_CU) : 8;
        const int64_t cap = std::max<int64_t>(1, (int64_t)cus * per_cu / std::max<int64_t>(E, 1));
        bpe = std::max<int64_t>(1, std::min(bpe, cap));
        if (E * bpe >= INT32_MAX) return PTGQ_EUNSUPPORTED;
        a.blocks_per_expert = (int32_t)bpe;
        a.x_expert_stride = rows * a.in_stride;
        a.q_expert_stride = rows * K;
        a.s_expert_stride = (int64_t)ptgq_scale_bytes(rows, K, G, scale_fmt, scale_layout);
        geo.U = U;
        geo.wpb = wpb;
        geo.grid = (unsigned)(E * bpe);
    }
    const hipError_t err = launch_group(a, in_dtype, G, fuse != 0, out_dtype, masked, geo.grid,
                                        (unsigned)(geo.wpb * 64),
                                        static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PTGQ_OK : PTGQ_ELAUNCH;
}

int next_pow2(int64_t n)
{
    int p = 1;
    while (p < n && p < 32) p <<= 1;
    return p;
}

}  // namespace

extern "C" {

size_t ptgq_scale_bytes(int64_t rows, int64_t K, int group_size, int scale_fmt, int scale_layout)
{
    if (rows < 0 || K < 0 || !valid_group_size(group_size) || K % group_size != 0) return 0;
    if (scale_fmt != PTGQ_SCALE_F32 && scale_fmt != PTGQ_SCALE_UE8M0) return 0;
    if (scale_layout != PTGQ_ROW_MAJOR && scale_layout != PTGQ_COL_MAJOR) return 0;
    const int64_t ng = K / group_size;
    if (scale_layout == PTGQ_ROW_MAJOR)
        return (size_t)(rows * ng * (scale_fmt == PTGQ_SCALE_F32 ? 4 : 1));
    if (scale_fmt == PTGQ_SCALE_F32) return (size_t)(ng * pad4(rows) * 4);
    return (size_t)(((ng + 3) / 4) * pad4(rows) * 4);
}

const char *ptgq_status_string(int status)
{
    switch (status) {
    case PTGQ_OK: return "ok";
    case PTGQ_EINVAL: return "invalid argument (size, enum, eps or null pointer)";
    case PTGQ_EALIGN: return "misaligned pointer (x and q need 16 bytes, s needs 4)";
    case PTGQ_EUNSUPPORTED: return "unsupported argument combination or size";
    case PTGQ_ELAUNCH: return "HIP kernel launch failed";
    case PTGQ_EDEVICE: return "no usable HIP device";
    default: return "unknown status";
    }
}

int ptgq_init(int device)
{
    return device_cus(device) > 0 ? PTGQ_OK : PTGQ_EDEVICE;
}

int ptgq_quant(const void *x, int in_dtype, int64_t M, int64_t K, int group_size,
               int fuse_silu_mul, int out_dtype, int scale_fmt, int scale_layout, float eps,
               void *q, void *s, void *stream)
{
    const int rc = check_group_args(x, in_dtype, 1, M, K, group_size, out_dtype, scale_fmt,
                                    scale_layout, eps, q, s);
    if (rc != PTGQ_OK || M == 0 || K == 0) return rc;
    return launch_group_common(x, in_dtype, M, K, group_size, fuse_silu_mul, out_dtype,
                               scale_fmt, scale_layout, eps, q, s, nullptr, 1, 0, stream);
}

int ptgq_quant_masked(const void *x, int in_dtype, int64_t E, int64_t tokens_pad, int64_t K,
                      int group_size, int fuse_silu_mul, const int32_t *masked_m,
                      int64_t expected_m, int out_dtype, int scale_fmt, int scale_layout,
                      float eps, void *q, void *s, void *stream)
{
    const int rc = check_group_args(x, in_dtype, E, tokens_pad, K, group_size, out_dtype,
                                    scale_fmt, scale_layout, eps, q, s);
    if (rc != PTGQ_OK) return rc;
    if (E == 0 || tokens_pad == 0 || K == 0) return PTGQ_OK;
    if (!masked_m) return PTGQ_EINVAL;
    if (!aligned(masked_m, 4)) return PTGQ_EALIGN;
    return launch_group_common(x, in_dtype, tokens_pad, K, group_size, fuse_silu_mul, out_dtype,
                               scale_fmt, scale_layout, eps, q, s, masked_m, E, expected_m,
                               stream);
}

int ptq_quant_fp8(const void *x, int in_dtype, int64_t M, int64_t K, void *q, float *s,
                  void *stream)
{
    if (in_dtype != PTGQ_BF16 && in_dtype != PTGQ_FP16 && in_dtype != PTGQ_FP32)
        return PTGQ_EINVAL;
    if (M < 0 || K < 0 || K % 4 != 0) return PTGQ_EINVAL;
    if (M == 0 || K == 0) return PTGQ_OK;
    if (!x || !q || !s) return PTGQ_EINVAL;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4)) return PTGQ_EALIGN;
    if (M >= INT32_MAX) return PTGQ_EUNSUPPORTED;

    const int cus = current_cus(nullptr);
    if (cus <= 0) return PTGQ_EDEVICE;

    const int insz = in_dtype == PTGQ_FP32 ? 4 : 2;
    const int64_t row_bytes = K * insz;
    const int vb = (row_bytes % 16 == 0) ? 16 : 8;
    const int64_t nv = row_bytes / vb;
    if (nv >= INT32_MAX) return PTGQ_EUNSUPPORTED;

    TokenArgs a;
    a.x = x;
    a.q = static_cast<uint8_t *>(q);
    a.s = s;
    a.M = M;
    a.K = K;
    a.nv = (int32_t)nv;

    // Token-count dispatch (the analogue of the warp/CTA threshold of the
    // sglang #34257 page): with enough rows to fill the chip, one wave per row;
    // otherwise one 256-lane block per row; rows too long for registers take
    // the two-pass loop.
    const int64_t per_wave = (nv + 63) / 64;
    const int64_t per_block = (nv + 255) / 256;
    TokenMode mode;
    const int64_t forced = knob(KNOB_TOKEN_MODE);
    if (forced == TOKEN_WAVE && per_wave <= 16) mode = TOKEN_WAVE;
    else if (forced == TOKEN_BLOCK && per_block <= 16) mode = TOKEN_BLOCK;
    else if (forced == TOKEN_BLOCK_LOOP) mode = TOKEN_BLOCK_LOOP;
    else if (M >= (int64_t)cus * 8 && per_wave <= 16) mode = TOKEN_WAVE;
    else if (per_block <= 16) mode = TOKEN_BLOCK;
    else mode = TOKEN_BLOCK_LOOP;

    unsigned grid, block;
    int nvl = 0;
    if (mode == TOKEN_WAVE) {
        nvl = next_pow2(per_wave);
        block = 256;
        grid = (unsigned)((M + 3) / 4);
    } else {
        nvl = mode == TOKEN_BLOCK ? next_pow2(per_block) : 0;
        block = 256;
        grid = (unsigned)M;
    }
    const hipError_t err = launch_token(a, in_dtype, vb, mode, nvl, grid, block,
                                        static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PTGQ_OK : PTGQ_ELAUNCH;
}

int ptgq_probe_e4m3(const float *v, uint8_t *out, int64_t n, void *stream)
{
    if (n < 0) return PTGQ_EINVAL;
    if (n == 0) return PTGQ_OK;
    if (!v || !out) return PTGQ_EINVAL;
    if (n >= (int64_t)UINT32_MAX * 256) return PTGQ_EUNSUPPORTED;
    const hipError_t err = launch_probe_e4m3(v, out, n, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PTGQ_OK : PTGQ_ELAUNCH;
}

int ptgq_probe_silu_mul(const void *g, const void *u, int in_dtype, float *out, int64_t n,
                        void *stream)
{
    if (in_dtype != PTGQ_BF16 && in_dtype != PTGQ_FP16) return PTGQ_EINVAL;
    if (n < 0) return PTGQ_EINVAL;
    if (n == 0) return PTGQ_OK;
    if (!g || !u || !out) return PTGQ_EINVAL;
    if (n >= (int64_t)UINT32_MAX * 256) return PTGQ_EUNSUPPORTED;
    const hipError_t err = launch_probe_silu(g, u, in_dtype, out, n,
                                             static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PTGQ_OK : PTGQ_ELAUNCH;
}

int ptgq_set_tuning(int which, int64_t value)
{
    if (which < 0 || which > 3) return PTGQ_EINVAL;
    g_knob[which].store(value, std::memory_order_relaxed);
    return PTGQ_OK;
}

}  // extern "C"
