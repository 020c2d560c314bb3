// Internal interface between the C-ABI layer (ptgq_api.cpp) and the kernels
// (ptgq_kernels.hip).  Not installed; not part of the public header.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace ptgq {

enum : int { IN_BF16 = 0, IN_FP16 = 1, IN_FP32 = 2 };
enum : int { OUT_E4M3 = 0, OUT_INT8 = 1 };
enum : int { SCALE_F32 = 0, SCALE_UE8M0 = 1 };
enum : int { LAYOUT_ROW = 0, LAYOUT_COL = 1 };

// Elements of one "slab": 8 elements per lane across a 64-lane wave (one
// 16-byte load per lane for 16-bit inputs, two for fp32).  Every group-quant task is U = 1 or 2
// consecutive slabs of one row; the last task of a row may run past its end
// (those lanes read zeros and store nothing).
constexpr int kSlab = 512;
constexpr int kChunk = 128;   // output elements of a chunk task (fused calls of few slabs)
constexpr int kMaxSlabsPerTask = 2;
// Masked calls keep a prefix sum of E ints in LDS (2 E with flattened slabs).
constexpr int kMaxExperts = 4096;

// Exact unsigned division by a divisor fixed on the host (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994):
// with l = ceil(log2 d) and mul = floor(2^32 (2^l - d) / d) + 1,
// floor(n / d) = (mulhi(mul, n) + n) >> l for every n < 2^31 (the sum then
// fits in 32 bits).  Used for wave-uniform task indices, so the device does it
// with three scalar instructions.
struct FastDiv {
    uint32_t mul;
    uint32_t shift;
};

inline FastDiv make_fastdiv(uint32_t d)
{
    uint32_t l = 0;
    while (l < 32 && ((uint64_t)1 << l) < d) ++l;
    FastDiv f;
    f.mul = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d + 1);
    f.shift = l;
    return f;
}

__host__ __device__ inline uint32_t fastdiv(uint32_t n, FastDiv f)
{
    const uint32_t hi = (uint32_t)(((uint64_t)n * f.mul) >> 32);
    return (hi + n) >> f.shift;
}

// Arguments of the group-quantization kernels (flat and masked).  All shape
// scalars are computed on the host; the device only indexes.
struct GroupArgs {
    const void *x;            // input base (bf16 / fp16 / fp32)
    uint8_t *q;               // codes base
    void *s;                  // scale tensor base
    const int32_t *masked_m;  // masked: live rows per expert; flat: nullptr
    int64_t rows;             // flat: M; masked: tokens_pad
    int64_t K;                // output row width
    int64_t in_stride;        // input row stride in bytes (K, or 2K when fused, elements)
    int64_t ng;               // groups per row, K / G
    int64_t rows_pad;         // ceil(rows / 4) * 4 (column-major scales)
    int64_t x_expert_stride;  // masked: bytes per expert of x
    int64_t q_expert_stride;  // masked: bytes per expert of q
    int64_t s_expert_stride;  // masked: bytes per expert of s
    float eps;                // amax floor
    int32_t spr;              // slabs per row, ceil(K / kSlab)
    int32_t U;                // slabs per task: 1 or 2
    int32_t tpr;              // tasks per row, ceil(spr / U)
    int32_t n_tasks;          // flat: rows * tpr
    int32_t scale_fmt;        // SCALE_F32 / SCALE_UE8M0
    int32_t scale_layout;     // LAYOUT_ROW / LAYOUT_COL
    int32_t num_experts;      // masked: E (1..kMaxExperts)
    int32_t pad_cols;         // flat column-major: 4-byte columns whose pad rows
                              // are zeroed (ceil(ng/4) or ng); 0 = none
    int64_t q_pad_bytes;      // flat: bytes of q past row M written as zero
    int32_t xcd_chunk;        // flat: blocks per XCD chunk of the block -> task
                              // mapping; 0 = one contiguous range per XCD
    int32_t flat_slabs;       // flat, unfused: task t is slabs U*t .. U*t+U-1 of
                              // the whole [M, K] tensor taken as one sequence of
                              // slabs (tasks cross row ends).  1: K % kSlab == 0,
                              // whole-row slabs; 2: 16-bit input, K < kSlab and
                              // kSlab % K == 0, each slab kSlab / K whole rows;
                              // 3: any other K % kSlab != 0: slabs of kSlab
                              // consecutive elements of the flattened output
                              // (fused: of the flattened gate and up halves).
                              // 4 (fused, direct SiLU): chunk tasks of kChunk
                              // output elements of a row, spr = tpr = chunks
                              // per row.  Masked: 0 or 3, each expert's live
                              // rows taken as one such sequence (no task
                              // crosses experts)
    int64_t n_slabs;          // flat_slabs: slabs of the sequence
    FastDiv spr_div;          // flat_slabs: division by spr
    FastDiv tpr_div;          // row and chunk tasks: division by tpr
    int32_t fs_row;           // flat_slabs: elements per row of the slab sequence
                              // (K; kSlab for multi-row slabs)
    int32_t mr_shift;         // flat_slabs == 2: log2(ng)
    FastDiv ng_div;           // flat_slabs == 3: division by ng
    FastDiv k_div;            // flat_slabs == 3, fused: division by K
    int64_t fs_total;         // flat_slabs: elements of the tensor, M * K
    int32_t wpb;              // waves per block of the launch
};

// Arguments of the whole-row per-token kernels.
struct TokenArgs {
    const void *x;
    uint8_t *q;
    float *s;
    int64_t M;
    int64_t K;
    int32_t nv;               // vectors per row (row bytes / vector bytes)
    int32_t xcd_chunk;        // one-block-per-row kernels: blocks per XCD chunk of
                              // the block -> row mapping (0: block b takes row b)
};

enum TokenMode : int { TOKEN_WAVE = 0, TOKEN_BLOCK = 1, TOKEN_BLOCK_LOOP = 2, TOKEN_WAVE_LOOP = 3 };

// Arguments of the fp8 requantization kernel.  Expert e's live codes are the
// flat region x + e*T*K .. + live_e*K; tasks are `tcodes` contiguous codes of
// one region (1024 or 2048).
struct RequantArgs {
    const uint8_t *x;         // e4m3 codes [E, T, K]
    const float *x_scale;     // group scales, element (e, t, g) at e*se + t*st + g*sg
    const int32_t *masked_m;  // live rows per expert; nullptr: all T rows
    const float *output_scale;// device scalar
    uint8_t *out;             // e4m3 codes [E, T, K]
    int64_t T;
    int64_t K;
    int64_t se, st, sg;
    int64_t tcodes;           // codes per task
    uint32_t s_bytes;         // bytes spanned by x_scale (buffer range)
    float inv_k;              // 1 / K, for the row estimate when K < a task
    FastDiv k_div;            // division by K (code offsets within an expert, < 2^31)
    int32_t E;
    int32_t log2g;            // log2(group size)
    int32_t xcd_chunk;        // blocks per XCD chunk of the block -> task mapping (0: ranges)
};

// Arguments of the dequantization kernel.  Codes and outputs are contiguous
// [M, K]; the work is cut into flat tasks of ns sub-slabs (a sub-slab is 64
// lanes x 8 codes for 16-bit outputs, 64 x 4 for fp32), grid-strided over
// `full` rounds, then one last round of `last` codes per wave.
// fp32 scale of (row m, group g) is element m*st + g*sg; UE8M0 row-major byte
// m*ng + g; packed UE8M0 column-major byte ((g/4)*rows_pad + m)*4 + g%4.
struct DequantArgs {
    const uint8_t *q;         // codes [M, K]
    const void *s;            // scales
    void *y;                  // output [M, K]
    int64_t M;
    int64_t K;
    int64_t ng;               // groups per row
    int64_t st, sg;           // fp32 scale strides (elements)
    int64_t rows_pad;         // packed UE8M0 column-major: words per word column
    int64_t step;             // codes per round: waves * task codes
    int64_t dm;               // step / K
    int64_t full_end;         // full * step: first code of the last round
    int64_t last;             // codes per wave in the last round (whole sub-slabs)
    uint32_t dc;              // step % K
    uint32_t s_bytes;         // bytes of the scale tensor (buffer range)
    float inv_k;              // 1 / K, for the quotient estimate when K < a task
    FastDiv k_div;            // division by K, for code offsets below 2^31
    int32_t small;            // 1: every task's first code offset is below 2^31
    int32_t full;             // rounds of full tasks
    int32_t ns;               // sub-slabs per task: 1 or 4
    int32_t log2g;            // log2(G)
    int32_t xcd_chunk;        // blocks per XCD chunk (0: one contiguous range per XCD)
};

// Launchers (defined in ptgq_kernels.hip).  They return the hipError_t of the
// launch.  `grid`/`block` are chosen by the caller.
// `table`: fused kernels read g / (1 + e^-g) from their gate type's LDS-staged
// lookup table (launch with 1024-thread blocks); the tables must have been
// built on the device by launch_silu_table_init and ordered before.
hipError_t launch_group(const GroupArgs &a, int in_dtype, int G, bool fuse, int out_dtype,
                        bool table, bool masked, unsigned grid, unsigned block,
                        hipStream_t stream);
hipError_t launch_silu_table_init(hipStream_t stream);
hipError_t launch_token(const TokenArgs &a, int in_dtype, int vec_bytes, TokenMode mode,
                        int nv_per_lane, unsigned grid, unsigned block, hipStream_t stream);
hipError_t launch_requant(const RequantArgs &a, unsigned grid, unsigned block, hipStream_t stream);
hipError_t launch_dequant(const DequantArgs &a, int code_dtype, int scale_fmt, int scale_layout,
                          int out_dtype, unsigned grid, unsigned block, hipStream_t stream);
hipError_t launch_probe_e4m3(const float *v, uint8_t *out, int64_t n, hipStream_t stream);
hipError_t launch_probe_silu(const void *g, const void *u, int in_dtype, int path, float *out,
                             int64_t n, hipStream_t stream);
hipError_t launch_probe_scale(uint32_t first, int64_t n, float eps, int out_dtype, int scale_fmt,
                              void *scale_out, float *inv_out, hipStream_t stream);
hipError_t launch_probe_int8(uint32_t first, int64_t n, int8_t *out, hipStream_t stream);
hipError_t launch_probe_stream(const void *x, int64_t n, uint8_t *q, unsigned grid,
                               int32_t xcd_chunk, hipStream_t stream);

}  // namespace ptgq
