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
#include "ptgq_diag.h"
#include "ptgq_internal.h"

using namespace ptgq;

namespace {

// ----------------------------------------------------------------- devices
//
// Per-device state: the compute-unit count (queried once it succeeds; a
// failed query is not remembered) and the SiLU lookup tables of the fused
// kernels (bf16 and fp16 gates), file-scope device arrays filled by one small
// kernel ("the table" below: both are built and ordered together).  The table
// is built stream-ordered on the stream of the first call that needs it and
// an event is recorded after the build; later calls on other streams wait for
// that event on the device (hipStreamWaitEvent), and once the event has
// completed the table is ready for every stream.  No call synchronizes the
// host.  A call made while its stream is being captured into a graph never
// builds the table and never waits for a build recorded outside the capture:
// until the table is ready it takes the direct SiLU evaluation instead (same
// results, slower).

constexpr int kMaxDevices = 64;
constexpr int kPlanFields = 9;   // ptgq_plan_group's report

enum TableState : int { TABLE_NONE = 0, TABLE_PENDING = 1, TABLE_READY = 2 };

struct DeviceState {
    std::mutex mu;
    int cus = 0;                 // 0: not known yet
    int table = TABLE_NONE;
    hipEvent_t built = nullptr;  // recorded after the table kernel (PENDING, READY)
};

DeviceState g_dev[kMaxDevices];

int device_cus(int dev)
{
    if (dev < 0 || dev >= kMaxDevices) return 0;
    DeviceState &d = g_dev[dev];
    std::lock_guard<std::mutex> lock(d.mu);
    if (d.cus <= 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            cus > 0)
            d.cus = cus;
    }
    return d.cus;
}

int current_cus(int *dev_out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (dev_out) *dev_out = dev;
    return device_cus(dev);
}

// True when work enqueued on `stream` (of device `dev`, the current device)
// after this call may read the SiLU table; builds it on `stream` when no
// build exists yet and the stream is not capturing.  Never waits on the host.
bool table_usable(int dev, hipStream_t stream)
{
    if (dev < 0 || dev >= kMaxDevices) return false;
    DeviceState &d = g_dev[dev];
    std::lock_guard<std::mutex> lock(d.mu);
    if (d.table == TABLE_READY) return true;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
        return false;
    if (d.table == TABLE_PENDING) {
        const hipError_t q = hipEventQuery(d.built);
        if (q == hipSuccess) {
            d.table = TABLE_READY;
            return true;
        }
        return q == hipErrorNotReady && hipStreamWaitEvent(stream, d.built, 0) == hipSuccess;
    }
    if (!d.built && hipEventCreateWithFlags(&d.built, hipEventDisableTiming) != hipSuccess) {
        d.built = nullptr;
        return false;
    }
    if (launch_silu_table_init(stream) != hipSuccess) return false;
    // the build is only known to precede this stream's later work; without the
    // event no other stream could order itself after it, so the table stays
    // unused (a later call builds it again: the same values)
    if (hipEventRecord(d.built, stream) != hipSuccess) return false;
    d.table = TABLE_PENDING;
    return true;
}

// ------------------------------------------------------------ tuning knobs
// Process-wide overrides of the geometry chooser (diagnostics and sweeps
// only; -1 = automatic), set through ptgq_set_tuning.
constexpr int kKnobs = 8;
std::atomic<int64_t> g_knob[kKnobs] = {{-1}, {-1}, {-1}, {-1}, {-1}, {-1}, {-1}, {-1}};
enum { KNOB_SLABS_PER_TASK = 0, KNOB_WAVES_PER_BLOCK = 1, KNOB_BLOCKS_PER_CU = 2,
       KNOB_TOKEN_MODE = 3, KNOB_SILU_TABLE = 4, KNOB_XCD_CHUNK = 5, KNOB_GRID_MODE = 6,
       KNOB_FLAT_SLABS = 7 };

int64_t knob(int k) { return g_knob[k].load(std::memory_order_relaxed); }

// -------------------------------------------------------------- validation

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_group_size(int G) { return G == 16 || G == 32 || G == 64 || G == 128; }

int64_t pad4(int64_t n) { return (n + 3) / 4 * 4; }

// `outer` multiplies the rows (number of experts for the masked layout, 1
// for flat calls); an empty problem needs no pointers.
int check_group_args(const void *x, int in_dtype, int fuse, int64_t outer, int64_t rows,
                     int64_t K, int G, int out_dtype, int scale_fmt, int scale_layout, float eps,
                     const void *q, const void *s)
{
    if (in_dtype != PTGQ_BF16 && in_dtype != PTGQ_FP16 && in_dtype != PTGQ_FP32)
        return PTGQ_EINVAL;
    if (out_dtype != PTGQ_E4M3 && out_dtype != PTGQ_INT8) return PTGQ_EINVAL;
    if (scale_fmt != PTGQ_SCALE_F32 && scale_fmt != PTGQ_SCALE_UE8M0) return PTGQ_EINVAL;
    if (scale_layout != PTGQ_ROW_MAJOR && scale_layout != PTGQ_COL_MAJOR) return PTGQ_EINVAL;
    if (!valid_group_size(G)) return PTGQ_EINVAL;
    if (outer < 0 || rows < 0 || K < 0 || K % G != 0) return PTGQ_EINVAL;
    if (!(std::isfinite(eps) && eps >= 0.0f) || std::signbit(eps)) return PTGQ_EINVAL;
    if (fuse && in_dtype == PTGQ_FP32) return PTGQ_EUNSUPPORTED;   // fused: 16-bit inputs
    if (outer == 0 || rows == 0 || K == 0) return PTGQ_OK;
    if (K >= (int64_t)1 << 29) return PTGQ_EUNSUPPORTED;   // rows are 32-bit buffer ranges
    if (!x || !q || !s) return PTGQ_EINVAL;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4)) return PTGQ_EALIGN;
    return PTGQ_OK;
}

// --------------------------------------------------------- geometry chooser

struct GroupGeom {
    int U;          // slabs per task
    int wpb;        // waves per block
    bool table;     // fused 16-bit gates: LDS SiLU table (16-wave blocks)
    bool uncapped;  // one wave per task (no grid-stride loop)
    bool flat_slabs = false;  // flat-slab tasks (set before choose_blocks)
    bool fp32 = false;        // fp32 input
    int64_t per_cu; // resident blocks per CU the grid is capped at
    unsigned grid;  // blocks
};

constexpr int kTableWaves = 16;       // 1024-thread blocks stage the table once
constexpr int kTableBlocksPerCu = 1;  // one table block of 16 waves per CU
constexpr int kTable16SlabsPerCu = 32;

// Loads in flight per CU that saturate HBM for this 2:1 read/write stream
// (measured on MI355X: 48-64 KiB per CU, with every wave holding the next
// task's loads while it processes the current one).
constexpr int64_t kInflightBytesPerCu = 48 * 1024;
// Blocks per XCD chunk of the uncapped grids' block -> task mappings.
constexpr int64_t kXcdChunk = 64;
constexpr int64_t kDequantXcdChunk = 16;
constexpr int64_t kTokenXcdChunk = 32;      // per-token block mode, blocks per XCD chunk

// Slabs per task (1 or 2) and the SiLU path, for `slabs` slabs of work in
// total.  Fused work large enough to amortize staging the SiLU table in LDS
// (32 KiB for bf16 gates, 144 KiB for fp16) reads the table.  Few slabs
// (decode-sized M): one slab per task so the work spreads over as many waves
// and CUs as possible.  Many: two slabs per
// task for the plain and direct-SiLU kernels when a row has an even number of
// slabs (no task runs past a row), when the call takes flat-slab tasks, or
// for unfused 16-bit rows of at least 3 slabs; else one (measured best on
// MI355X).
// `flat_slabs`: an unfused flat call whose K is a multiple of the slab, so
// that input and codes are one contiguous sequence of whole-row slabs; its
// two-slab tasks then run over that sequence and cross row ends (no half
// task at the end of a row with an odd number of slabs).  `flat16`: other
// unfused flat calls on 16-bit input, which run two-slab row tasks also when
// a row has an odd number (>= 3) of slabs: the last task of a row holds one
// slab (measured on MI355X, fp16 rows of 3, 5 and 7 slabs: 2-10 % faster than
// capped one-slab tasks; one-slab rows stay one-slab).  `table_ok`: the SiLU
// lookup table may be read (it is built and ordered before the call).
void choose_task(GroupGeom &g, int64_t slabs, int32_t spr, bool fuse, int in_dtype, bool flat16,
                 bool flat_slabs, bool table_ok, int cus)
{
    const int64_t wave_slots = (int64_t)cus * 4 * 8;   // 8 waves per SIMD
    // The bf16 table from one slab per wave of the table grid on (16 per
    // CU): measured on MI355X, fused bf16 [M, 2 * 4096], the table against
    // the direct evaluation: M = 512 4.71 against 4.89 us, M = 1024 6.29
    // against 7.66, M = 1536 7.98 against 11.02; M = 256 (8 slabs per CU)
    // 4.30 against 3.68.  The fp16 table, 4.5 times larger, from
    // kTable16SlabsPerCu slabs per CU.
    const bool tab16 = in_dtype == PTGQ_FP16;
    const bool gate16 = in_dtype == PTGQ_BF16 || tab16;
    g.table = fuse && gate16 &&
              slabs >= (int64_t)cus * (tab16 ? kTable16SlabsPerCu : kTableWaves);
    if (fuse && gate16 && knob(KNOB_SILU_TABLE) >= 0) g.table = knob(KNOB_SILU_TABLE) > 0;
    if (!table_ok) g.table = false;
    // Table kernels (16 waves per CU) run one-slab tasks: measured 6-8 % faster
    // than two-slab tasks for the fused flat and masked workloads.
    // Two-slab tasks from half a wave per resident slot on for unfused calls
    // (flat calls then take the uncapped grid; measured on MI355X, bf16
    // [M, 7168]: M = 512 4.15 -> 3.83 us, M = 1024 6.11 -> 5.76; at M = 256,
    // 3584 slabs, one-slab tasks stay faster, 3.00 against 3.08; masked,
    // 8 experts x 128 live rows of 7168: 8.30 -> 6.89), from two waves per
    // slot for fused ones.
    const int64_t u2_min = fuse ? 2 * wave_slots : wave_slots / 2;
    int U = 1;
    if (!g.table && slabs >= u2_min && (flat_slabs || spr % 2 == 0 || (flat16 && spr >= 3)))
        U = 2;
    if (knob(KNOB_SLABS_PER_TASK) > 0) U = knob(KNOB_SLABS_PER_TASK) >= 2 ? 2 : 1;
    g.U = std::min(U, kMaxSlabsPerTask);
}

// Blocks for `tasks` tasks.  Plain and direct-SiLU kernels: 4-wave blocks
// (1-wave blocks for a handful of tasks), with the grid capped so that each
// CU holds about kInflightBytesPerCu of loads (every wave keeps two tasks of
// U slabs, 1 KiB per slab and input half, 2 KiB for fp32 input); the grid
// then loops over the tasks.
// Table kernels: one 16-wave block per CU.
// `uncapped`: one wave per task, the grid as large as the task count (no
// grid-stride loop); the hardware dispatcher then balances the short-lived
// blocks over the CUs.  Measured on MI355X for plain 16-bit inputs with
// two-slab tasks: 6.3 TB/s against 5.9 for the capped persistent grid at
// bf16 [16384, 7168] (the fused, fp32-input and masked kernels are faster
// capped).
void choose_blocks(GroupGeom &g, int64_t tasks, int cus, bool fuse, int64_t es, bool uncapped)
{
    int wpb;
    int64_t per_cu;
    if (g.table) {
        wpb = kTableWaves;   // the kernels stage the table with exactly 1024 lanes
        per_cu = kTableBlocksPerCu;
    } else {
        wpb = tasks >= (int64_t)cus * 4 ? 4 : 1;
        // Uncapped grids of flat-slab tasks run one-wave blocks, of fp32 input
        // two-wave blocks: measured on MI355X (A/B in one process) fp16 [8192,
        // 3584] -> int8 with fp32 row scales G = 128 15.93 -> 15.63 us, G = 16
        // 17.13 -> 16.38 us, -> e4m3 with UE8M0 16.0 -> 15.35 us; fp32 [8192,
        // 7168] 46.6 -> 45.7 us.  (Rows of an even number of 16-bit slabs
        // measured the same or slower with smaller blocks.)
        if (uncapped && g.flat_slabs && !g.fp32) wpb = 1;
        else if (uncapped && g.fp32) wpb = 2;
        if (knob(KNOB_WAVES_PER_BLOCK) > 0)
            wpb = (int)std::min<int64_t>(knob(KNOB_WAVES_PER_BLOCK), 4);
        const int64_t wave_bytes = 2 * (int64_t)g.U * kSlab * es * (fuse ? 2 : 1);
        const int64_t waves_per_cu = std::max<int64_t>(4, kInflightBytesPerCu / wave_bytes);
        per_cu = std::max<int64_t>(1, (waves_per_cu + wpb - 1) / wpb);   // rounded up
    }
    if (knob(KNOB_BLOCKS_PER_CU) > 0) per_cu = knob(KNOB_BLOCKS_PER_CU);
    // The capped grid loops over the tasks, so it must give every CU the same
    // number of blocks (a CU with one block more finishes last).  Its waves
    // run ceil(tasks / waves) tasks at most: when that tail costs more than 5 %
    // at per_cu blocks per CU, a third more blocks per CU is used if it
    // divides the tasks better.
    if (!g.table && knob(KNOB_BLOCKS_PER_CU) <= 0) {
        const int64_t w0 = (int64_t)cus * per_cu * wpb;
        const int64_t alt = per_cu + std::max<int64_t>(1, per_cu / 3);
        const int64_t w1 = (int64_t)cus * alt * wpb;
        const double loss0 = (double)((tasks + w0 - 1) / w0) * w0 / tasks;
        const double loss1 = (double)((tasks + w1 - 1) / w1) * w1 / tasks;
        if (tasks > w0 && loss0 > 1.05 && loss1 < loss0) per_cu = alt;
    }
    g.wpb = wpb;
    g.per_cu = per_cu;
    g.uncapped = uncapped;
    int64_t blocks = (tasks + wpb - 1) / wpb;
    const int64_t cap = uncapped && knob(KNOB_BLOCKS_PER_CU) <= 0
                            ? blocks
                            : std::max<int64_t>(1, (int64_t)cus * per_cu);
    if (blocks > cap)
        blocks = cap;                                  // a multiple of the CU count
    else if (blocks >= 64)
        blocks = (blocks + 7) / 8 * 8;                 // spare waves find no task
    g.grid = (unsigned)std::max<int64_t>(blocks, 1);
}

// The launch geometry and the geometry fields of `a` for a group call on a
// device of `cus` compute units; no HIP call (pointers, eps and the stream
// are the launcher's).  `masked`: the masked layout of E experts (rows =
// tokens_pad).  `q_rows` (flat only): rows of the q buffer, >= rows; the
// extra rows are written as zero.
int plan_group(GroupArgs &a, GroupGeom &geo, int in_dtype, int64_t rows, int64_t K, int G,
               int fuse, int scale_fmt, int scale_layout, bool masked, int64_t E,
               int64_t expected_m, int64_t q_rows, bool table_ok, int cus)
{
    std::memset(&a, 0, sizeof(a));
    a.rows = rows;
    a.K = K;
    const int64_t es = in_dtype == PTGQ_FP32 ? 4 : 2;   // input element bytes
    a.in_stride = (fuse ? 2 * K : K) * es;
    a.ng = K / G;
    a.rows_pad = pad4(rows);
    a.spr = (int32_t)((K + kSlab - 1) / kSlab);
    a.scale_fmt = scale_fmt;
    a.scale_layout = scale_layout;

    if (!masked) {
        // Flat-slab tasks for rows of an odd number of whole slabs (measured
        // on MI355X, fp16 [8192, 3584] -> int8, fp32 row scales: G = 128
        // 16.13 -> 15.92 us, G = 32 16.88 -> 16.63 us); rows of an even
        // number keep row tasks, which measured faster there (bf16 [4096,
        // 7168]: 15.35 against 15.96 us with the same tasks).
        // Rows shorter than a slab whose length divides it (16-bit input,
        // K = 16 .. 256): slabs of kSlab / K whole rows, so that no lane idles
        // past a row end (measured on MI355X, bf16 [M, K] -> e4m3, UE8M0
        // column-major, 33.5 M elements, one row per slab: K = 128 50.7 us,
        // K = 256 27.7, K = 512 17.0).
        const bool mr_ok = !fuse && es == 2 && K < kSlab && kSlab % K == 0 &&
                           knob(KNOB_FLAT_SLABS) != 0;
        // Any other K that is not a multiple of the slab (fp32 input: any
        // such K): slabs of the flattened tensor, crossing row ends anywhere
        // (groups never cross them, G dividing K), so that no lane idles on
        // a row's ragged last slab (group indices stay 32-bit).
        const bool fg_ok = !fuse && K % kSlab != 0 && !mr_ok &&
                           rows * a.ng < ((int64_t)1 << 31) && knob(KNOB_FLAT_SLABS) != 0;
        // Fused calls likewise, their lanes reading the gate and up halves
        // of their own rows (output elements < 2^31): measured on MI355X,
        // 16.8 M output elements, K = 1024 / 1536 / 2048 16.0 us, K = 1152
        // 19.9, K = 1408 18.4, K = 640 28.1 with one row per task.
        const bool fgf_ok = fuse && K % kSlab != 0 && rows * K < ((int64_t)1 << 31) &&
                            knob(KNOB_FLAT_SLABS) != 0;
        const bool fs_ok = mr_ok || fg_ok || fgf_ok ||
                           (!fuse && K % kSlab == 0 &&
                            (a.spr % 2 == 1 || knob(KNOB_FLAT_SLABS) > 0) &&
                            knob(KNOB_FLAT_SLABS) != 0);
        const int64_t seq_slabs =
            mr_ok || fg_ok || fgf_ok ? (rows * K + kSlab - 1) / kSlab : rows * (int64_t)a.spr;
        choose_task(geo, seq_slabs, a.spr, fuse != 0, in_dtype, !fuse && es == 2, fs_ok, table_ok,
                    cus);
        // Small fused calls on the direct SiLU path: chunk tasks of kChunk
        // elements, so that each wave's SiLU work, which bounds these
        // latency-bound calls, is a quarter of a slab's; up to 8 chunk tasks
        // per CU.  Measured on MI355X against one-slab tasks (A/B in one
        // process, bf16 [M, 2 K], us): K = 4096 M = 1 2.29 -> 1.91 (the
        // time without any SiLU work), M = 16 2.37 -> 2.00, M = 48 2.70 ->
        // 2.52, M = 64 2.76 -> 2.59, M = 80 (2560 chunks) 2.78 against 2.81,
        // M = 112 2.84 against 3.32; K = 1408 M = 64 2.56 -> 2.20, M = 128
        // 2.70 -> 2.49, M = 256 2.82 against 2.94; K = 7168 M = 8 2.63 ->
        // 2.21, M = 64 2.85 against 3.34.
        const int64_t chunk_tasks = rows * ((K + kChunk - 1) / kChunk);
        const bool chunks = fuse && !geo.table && knob(KNOB_FLAT_SLABS) != 0 &&
                            knob(KNOB_SLABS_PER_TASK) <= 0 && rows * a.ng < ((int64_t)1 << 31) &&
                            (knob(KNOB_FLAT_SLABS) == 2 || chunk_tasks <= (int64_t)cus * 8);
        if (chunks) geo.U = 1;
        a.U = geo.U;
        a.flat_slabs = chunks ? 4
                       : fgf_ok ? 3
                       : fs_ok && a.U == 2 ? (mr_ok ? 2 : fg_ok ? 3 : 1)
                                           : 0;
        if (a.flat_slabs == 4)
            a.spr = (int32_t)((K + kChunk - 1) / kChunk);   // chunks per row
        else if (a.flat_slabs >= 2)
            a.spr = 1;                        // the sequence's rows are its slabs
        a.tpr = (a.spr + a.U - 1) / a.U;
        a.tpr_div = make_fastdiv((uint32_t)a.tpr);
        geo.flat_slabs = a.flat_slabs != 0;
        a.n_slabs = a.flat_slabs >= 2 ? seq_slabs : rows * (int64_t)a.spr;
        if (a.n_slabs >= INT32_MAX) return PTGQ_EUNSUPPORTED;
        a.spr_div = make_fastdiv((uint32_t)a.spr);
        a.fs_row = (int32_t)(a.flat_slabs >= 2 ? kSlab : K);
        a.fs_total = rows * K;
        a.mr_shift = a.flat_slabs == 2 ? __builtin_ctzll((unsigned long long)a.ng) : -1;
        a.ng_div = make_fastdiv((uint32_t)a.ng);
        a.k_div = make_fastdiv((uint32_t)K);
        const int64_t tasks = a.flat_slabs && a.flat_slabs != 4 ? (a.n_slabs + a.U - 1) / a.U
                                                                : rows * (int64_t)a.tpr;
        if (tasks >= INT32_MAX) return PTGQ_EUNSUPPORTED;
        a.n_tasks = (int32_t)tasks;
        a.q_pad_bytes = (q_rows - rows) * K;
        // Uncapped: plain (unfused) two-slab tasks, 16-bit or fp32 input, and
        // chunk tasks.
        bool uncapped = (!fuse && geo.U == 2) || a.flat_slabs == 4;
        if (knob(KNOB_GRID_MODE) >= 0) uncapped = knob(KNOB_GRID_MODE) > 0;
        // a large zero-filled tail also needs waves: one 1 KiB wave store each
        geo.fp32 = es == 4;
        choose_blocks(geo, std::max<int64_t>(tasks, (a.q_pad_bytes + 1023) / 1024), cus,
                      fuse != 0, es, uncapped);
        // Block -> task mapping of a grid far larger than the chip: chunks of
        // 64 blocks per XCD (measured on MI355X, bf16 [M, 7168]: M = 4096
        // 16.4 -> 15.4 us, M = 16384 55.9 -> 53.4 us against one contiguous
        // range per XCD; chunks of 32..256 blocks within 1 %; fp16 [16384,
        // 3584]: 30.3 -> 28.6 us; short rows too: bf16 [16384, 2048] 17.63
        // -> 17.07 us, [32768, 1024] 17.57 -> 17.09, [16384, 3072] 24.84 ->
        // 24.25).  Grids of fewer than 4 spans (M = 256 here: 3.1 us against
        // 3.3-3.6) keep the contiguous ranges.  fp32 input: 58.7 M elements,
        // K = 1024 and 2048: capped 51.5 us, uncapped with contiguous ranges
        // 53.7, chunked 49.4; K = 7168: capped 51.4, chunked 49.1-49.4.
        // Chunks of 512 one-wave blocks for flat-slab tasks, 256 two-wave
        // blocks for fp32 input (measured with the block sizes above: fp16
        // [8192, 3584] G = 16 16.66 us with chunks of 64, 16.38 with 512; fp32
        // 45.65 us with 256; fp16 [16384, 1536] 13.95 -> 13.69-13.78 us
        // against contiguous ranges, bf16 [8192, 2560] 11.91 -> 11.70).
        const int64_t chunk = geo.wpb == 1 && geo.flat_slabs ? 512 : geo.wpb == 2 ? 256 : kXcdChunk;
        if (uncapped && geo.grid >= 4 * 8 * chunk) a.xcd_chunk = (int32_t)chunk;
        if (knob(KNOB_XCD_CHUNK) >= 0) a.xcd_chunk = (int32_t)std::min<int64_t>(knob(KNOB_XCD_CHUNK), 1 << 20);
        if (scale_layout == PTGQ_COL_MAJOR && a.rows_pad > rows)
            a.pad_cols = (int32_t)(scale_fmt == PTGQ_SCALE_UE8M0 ? (a.ng + 3) / 4 : a.ng);
    } else {
        // Masked schedule: the live rows of all experts form one task space,
        // which the kernel splits evenly over the grid after reading masked_m
        // on the device.  The grid is sized for the expected live rows (all
        // tokens_pad rows of every expert when unknown); more live rows than
        // expected only make each wave loop longer.
        if (E > kMaxExperts) return PTGQ_EUNSUPPORTED;
        // The fp16 table (144 KiB of LDS) beside the prefix sum's 2 E ints
        // (8 KiB at 1024 experts) stays inside the 160 KiB of a workgroup.
        if (in_dtype == PTGQ_FP16 && E > 1024) table_ok = false;
        const int64_t hint = std::max<int64_t>(
            (expected_m > 0 && expected_m < rows) ? expected_m : rows, 1);
        // Rows that are not whole slabs, and unfused rows of an odd number of
        // slabs: each expert's live rows as one flattened sequence of slabs,
        // cut into tasks that do not cross experts, so that no lane idles on
        // a row's ragged last slab and two-slab tasks need no half task at a
        // row end.  Measured on MI355X, 32 experts x about 8.4 M live
        // elements, bf16 -> e4m3, UE8M0 column-major, against row tasks:
        // fused K = 768 14.48 -> 11.40 us, K = 1152 15.20 -> 13.30, K = 1408
        // 14.13 -> 13.27 (128 experts, K = 768: 19.58 -> 14.11); unfused K =
        // 1408 10.68 -> 9.32, K = 1536 9.58 -> 9.24, K = 3584 9.58 -> 9.17.
        // Fused rows of whole slabs measured slower (K = 1536 12.97 -> 13.12,
        // K = 2048 12.92 -> 13.15), unfused rows of an even number the same.
        const bool mfg = rows * K < ((int64_t)1 << 31) && knob(KNOB_FLAT_SLABS) != 0 &&
                         (K % kSlab != 0 || (!fuse && a.spr % 2 == 1) ||
                          knob(KNOB_FLAT_SLABS) > 0);
        int64_t tasks;
        if (mfg) {
            choose_task(geo, (hint * K + kSlab - 1) / kSlab * E, 1, fuse != 0, in_dtype, false,
                        true, table_ok, cus);
            a.U = geo.U;
            const int64_t per = (int64_t)a.U * kSlab;
            if (E * ((rows * K + per - 1) / per) >= INT32_MAX) return PTGQ_EUNSUPPORTED;
            a.flat_slabs = 3;
            a.spr = 1;
            a.tpr = 1;
            a.ng_div = make_fastdiv((uint32_t)a.ng);
            a.k_div = make_fastdiv((uint32_t)K);
            tasks = (hint * K + per - 1) / per * E;
        } else {
            choose_task(geo, hint * a.spr * E, a.spr, fuse != 0, in_dtype, false, false, table_ok,
                        cus);
            a.U = geo.U;
            a.tpr = (a.spr + a.U - 1) / a.U;
            if (E * rows * (int64_t)a.tpr >= INT32_MAX) return PTGQ_EUNSUPPORTED;
            tasks = hint * a.tpr * E;
        }
        // Small fused calls on the direct SiLU path: chunk tasks, as for flat
        // calls, over the expected live rows.
        const int64_t cpr = (K + kChunk - 1) / kChunk;
        const bool chunks = fuse && !geo.table && knob(KNOB_FLAT_SLABS) != 0 &&
                            knob(KNOB_SLABS_PER_TASK) <= 0 && rows * a.ng < ((int64_t)1 << 31) &&
                            (knob(KNOB_FLAT_SLABS) == 2 || hint * E * cpr <= (int64_t)cus * 8);
        if (chunks) {
            if (E * rows * cpr >= INT32_MAX) return PTGQ_EUNSUPPORTED;
            geo.U = a.U = 1;
            a.flat_slabs = 4;
            a.spr = a.tpr = (int32_t)cpr;
            a.spr_div = make_fastdiv((uint32_t)cpr);
            a.ng_div = make_fastdiv((uint32_t)a.ng);
            tasks = hint * cpr * E;
        }
        a.tpr_div = make_fastdiv((uint32_t)a.tpr);
        geo.flat_slabs = a.flat_slabs != 0;
        choose_blocks(geo, tasks, cus, fuse != 0, es, false);
        a.n_tasks = (int32_t)tasks;          // expected; set on the device
        a.num_experts = (int32_t)E;
        a.x_expert_stride = rows * a.in_stride;
        a.q_expert_stride = rows * K;
        a.s_expert_stride = (int64_t)ptgq_scale_bytes(rows, K, G, scale_fmt, scale_layout);
    }
    return PTGQ_OK;
}

int launch_group_common(const void *x, int in_dtype, int64_t rows, int64_t K, int G, int fuse,
                        int out_dtype, int scale_fmt, int scale_layout, float eps, void *q,
                        void *s, const int32_t *masked_m, int64_t E, int64_t expected_m,
                        int64_t q_rows, void *stream)
{
    int dev = 0;
    const int cus = current_cus(&dev);
    if (cus <= 0) return PTGQ_EDEVICE;

    GroupArgs a;
    GroupGeom geo;
    const bool masked = masked_m != nullptr;
    int rc = plan_group(a, geo, in_dtype, rows, K, G, fuse, scale_fmt, scale_layout, masked, E,
                        expected_m, q_rows, true, cus);
    if (rc != PTGQ_OK) return rc;
    if (geo.table && !table_usable(dev, static_cast<hipStream_t>(stream))) {
        // the table is not ready for this stream: the direct evaluation
        rc = plan_group(a, geo, in_dtype, rows, K, G, fuse, scale_fmt, scale_layout, masked, E,
                        expected_m, q_rows, false, cus);
        if (rc != PTGQ_OK) return rc;
    }
    a.x = x;
    a.q = static_cast<uint8_t *>(q);
    a.s = s;
    a.masked_m = masked_m;
    a.eps = eps;
    a.wpb = geo.wpb;
    const hipError_t err = launch_group(a, in_dtype, G, fuse != 0, out_dtype, geo.table, masked,
                                        geo.grid, (unsigned)(geo.wpb * 64),
                                        static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PTGQ_OK : PTGQ_ELAUNCH;
}

// Vectors per lane of the per-token kernels that keep a row in registers:
// instantiated for 1, 2, 4, 7, 8 and 16 (7: a 7 KiB row of 16-bit elements
// over one wave, or 14 KiB over two, with no idle lane); other counts round
// up to the next instantiated one.
int vectors_per_lane(int64_t n)
{
    for (const int p : {1, 2, 4, 7, 8, 16})
        if (p >= n) return p;
    return 32;
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
    if (device < 0 || device >= kMaxDevices || device_cus(device) <= 0) return PTGQ_EDEVICE;
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess || hipSetDevice(device) != hipSuccess)
        return PTGQ_EDEVICE;
    int rc = PTGQ_OK;
    if (!table_usable(device, nullptr)) {
        rc = PTGQ_EDEVICE;
    } else {
        DeviceState &d = g_dev[device];
        std::lock_guard<std::mutex> lock(d.mu);
        if (d.table == TABLE_PENDING) {
            if (hipEventSynchronize(d.built) == hipSuccess) d.table = TABLE_READY;
            else rc = PTGQ_EDEVICE;
        }
    }
    if (prev >= 0) (void)hipSetDevice(prev);
    return rc;
}

int ptgq_quant(const void *x, int in_dtype, int64_t M, int64_t K, int group_size,
               int fuse_silu_mul, int out_dtype, int scale_fmt, int scale_layout, float eps,
               void *q, void *s, void *stream)
{
    const int rc = check_group_args(x, in_dtype, fuse_silu_mul, 1, M, K, group_size, out_dtype,
                                    scale_fmt, scale_layout, eps, q, s);
    if (rc != PTGQ_OK || M == 0 || K == 0) return rc;
    return launch_group_common(x, in_dtype, M, K, group_size, fuse_silu_mul, out_dtype,
                               scale_fmt, scale_layout, eps, q, s, nullptr, 1, 0, M, stream);
}

int ptgq_quant_padded(const void *x, int in_dtype, int64_t M, int64_t K, int group_size,
                      int fuse_silu_mul, int out_dtype, int scale_fmt, int scale_layout,
                      float eps, void *q, int64_t q_rows, void *s, void *stream)
{
    if (q_rows < M) return PTGQ_EINVAL;
    const int rc = check_group_args(x, in_dtype, fuse_silu_mul, 1, M, K, group_size, out_dtype,
                                    scale_fmt, scale_layout, eps, q, s);
    if (rc != PTGQ_OK || q_rows == 0 || K == 0) return rc;
    if (M == 0) {   // only the zero fill: no input or scales are touched
        if (!q) return PTGQ_EINVAL;
        if (!aligned(q, 16)) return PTGQ_EALIGN;
        x = q;      // never read (no tasks), but a valid base for the
        s = q;      // empty-range loads every wave issues
    }
    if (q_rows >= ((int64_t)1 << 31)) return PTGQ_EUNSUPPORTED;
    return launch_group_common(x, in_dtype, M, K, group_size, fuse_silu_mul, out_dtype,
                               scale_fmt, scale_layout, eps, q, s, nullptr, 1, 0, q_rows,
                               stream);
}

int ptgq_quant_masked(const void *x, int in_dtype, int64_t E, int64_t tokens_pad, int64_t K,
                      int group_size, int fuse_silu_mul, const int32_t *masked_m,
                      int64_t expected_m, int out_dtype, int scale_fmt, int scale_layout,
                      float eps, void *q, void *s, void *stream)
{
    const int rc = check_group_args(x, in_dtype, fuse_silu_mul, E, tokens_pad, K, group_size,
                                    out_dtype, scale_fmt, scale_layout, eps, q, s);
    if (rc != PTGQ_OK) return rc;
    if (E == 0 || tokens_pad == 0 || K == 0) return PTGQ_OK;
    if (!masked_m) return PTGQ_EINVAL;
    if (!aligned(masked_m, 4)) return PTGQ_EALIGN;
    if (E > kMaxExperts) return PTGQ_EUNSUPPORTED;
    return launch_group_common(x, in_dtype, tokens_pad, K, group_size, fuse_silu_mul, out_dtype,
                               scale_fmt, scale_layout, eps, q, s, masked_m, E, expected_m,
                               tokens_pad, stream);
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
    a.xcd_chunk = 0;

    // Dispatch (the analogue of the warp/CTA threshold of the sglang #34257
    // page, by row length here): one block per row for rows that fit in
    // registers (16 vectors per lane); longer rows take the two-pass loop.
    // Measured on MI355X against one wave per row and persistent waves: equal
    // or faster for 2, 7, 8 and 14 KiB rows.  The other modes stay selectable
    // for tests.
    const int64_t per_wave = (nv + 63) / 64;
    // Waves per row: the largest power of two up to 8 that leaves each wave
    // at least 1.75 KiB of the row.  Measured on MI355X (A/B in one process,
    // waves per row 1..8): best or within 0.3 % of best for 16-bit rows of
    // 2.7, 4, 7, 8, 10, 12, 14 and 16 KiB and fp32 rows of 14 and 28 KiB
    // (fp16 [8192, 3584] 15.53 us with 4 waves, 15.65 with 2, 18.6-20.5 with
    // 5-8; bf16 [16384, 7168] 53.6 with 8, 54.7 with 4); fp32 [8192, 2048]
    // 15.1 us, against 14.5 with 3 waves.  Fewer than ~1.75 KiB per wave is
    // slower everywhere.
    int64_t tw = 1;
    while (tw < 8 && row_bytes >= tw * 2 * 1792) tw *= 2;
    if (knob(KNOB_WAVES_PER_BLOCK) > 0) tw = std::min<int64_t>(knob(KNOB_WAVES_PER_BLOCK), 8);
    const int64_t per_block = (nv + 64 * tw - 1) / (64 * tw);
    TokenMode mode;
    const int64_t forced = knob(KNOB_TOKEN_MODE);
    if (forced == TOKEN_WAVE && per_wave <= 16) mode = TOKEN_WAVE;
    else if (forced == TOKEN_WAVE_LOOP && per_wave <= 8) mode = TOKEN_WAVE_LOOP;
    else if (forced == TOKEN_BLOCK && per_block <= 16) mode = TOKEN_BLOCK;
    else if (forced == TOKEN_BLOCK_LOOP) mode = TOKEN_BLOCK_LOOP;
    else if (per_block <= 16) mode = TOKEN_BLOCK;
    else mode = TOKEN_BLOCK_LOOP;

    unsigned grid, block;
    int nvl = 0;
    if (mode == TOKEN_WAVE) {
        // one wave per row, rows_per_block rows (waves) per block
        const int64_t rpb = knob(KNOB_WAVES_PER_BLOCK) > 0 ? std::min<int64_t>(knob(KNOB_WAVES_PER_BLOCK), 4) : 4;
        nvl = vectors_per_lane(per_wave);
        block = (unsigned)(64 * rpb);
        grid = (unsigned)((M + rpb - 1) / rpb);
    } else if (mode == TOKEN_WAVE_LOOP) {
        // persistent waves, two rows in flight each: one four-wave block per
        // CU measured best (fp16 [8192, 3584]: 16.1 us against 16.7 for one
        // wave per row and 17.4 with four blocks per CU); the grid never
        // exceeds one wave per row
        nvl = vectors_per_lane(per_wave);
        block = 256;
        const int64_t per_cu = knob(KNOB_BLOCKS_PER_CU) > 0 ? knob(KNOB_BLOCKS_PER_CU) : 1;
        grid = (unsigned)std::min<int64_t>((M + 3) / 4, (int64_t)cus * per_cu);
    } else {
        nvl = mode == TOKEN_BLOCK ? vectors_per_lane(per_block) : 0;
        block = mode == TOKEN_BLOCK ? (unsigned)(64 * tw) : 256;
        grid = (unsigned)M;
        // rows dealt to the XCDs in chunks of 32 blocks rather than one
        // contiguous range per XCD: measured on MI355X, fp16 [8192, 3584]
        // 15.72 us against 15.81, bf16 [16384, 7168] 54.9 against 55.1,
        // bf16 [32768, 1024] 16.9 against 17.2 (bf16 [16384, 2048]: 17.55
        // against 17.49)
        if (mode == TOKEN_BLOCK && M >= 4 * 8 * kTokenXcdChunk) a.xcd_chunk = (int32_t)kTokenXcdChunk;
        if (mode == TOKEN_BLOCK && knob(KNOB_XCD_CHUNK) >= 0)
            a.xcd_chunk = (int32_t)std::min<int64_t>(knob(KNOB_XCD_CHUNK), 1 << 20);
    }
    const hipError_t err = launch_token(a, in_dtype, vb, mode, nvl, grid, block,
                                        static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PTGQ_OK : PTGQ_ELAUNCH;
}

int ptgq_requant_fp8(const uint8_t *x, int64_t E, int64_t T, int64_t K, int group_size,
                     const float *x_scale, int64_t scale_stride_e, int64_t scale_stride_t,
                     int64_t scale_stride_g, const int32_t *masked_m, int64_t expected_m,
                     const float *output_scale, uint8_t *out, void *stream)
{
    if (E < 0 || T < 0 || K < 0 || !valid_group_size(group_size) || K % group_size != 0)
        return PTGQ_EINVAL;
    if (scale_stride_e < 0 || scale_stride_t < 0 || scale_stride_g < 0) return PTGQ_EINVAL;
    if (E == 0 || T == 0 || K == 0) return PTGQ_OK;
    if (!x || !x_scale || !output_scale || !out || x == out) return PTGQ_EINVAL;
    if (!aligned(x, 16) || !aligned(out, 16) || !aligned(x_scale, 4) || !aligned(output_scale, 4) ||
        (masked_m && !aligned(masked_m, 4)))
        return PTGQ_EALIGN;
    if (E > kMaxExperts || K >= ((int64_t)1 << 30)) return PTGQ_EUNSUPPORTED;
    // an expert's codes are addressed with 32-bit offsets, the scales through
    // one 32-bit buffer range
    if (T * K >= ((int64_t)1 << 31)) return PTGQ_EUNSUPPORTED;
    const int64_t ng = K / group_size;
    const int64_t smax = (E - 1) * scale_stride_e + (T - 1) * scale_stride_t +
                         (ng - 1) * scale_stride_g;
    if (smax >= ((int64_t)1 << 30) - 4) return PTGQ_EUNSUPPORTED;
    const int cus = current_cus(nullptr);
    if (cus <= 0) return PTGQ_EDEVICE;

    RequantArgs a;
    a.x = x;
    a.x_scale = x_scale;
    a.masked_m = masked_m;
    a.output_scale = output_scale;
    a.out = out;
    a.T = T;
    a.K = K;
    a.se = scale_stride_e;
    a.st = scale_stride_t;
    a.sg = scale_stride_g;
    a.s_bytes = (uint32_t)((smax + 1) * 4);
    a.inv_k = 1.0f / (float)K;
    a.k_div = make_fastdiv((uint32_t)K);
    a.E = (int32_t)E;
    a.log2g = __builtin_ctz((unsigned)group_size);
    a.xcd_chunk = 0;
    // Tasks of 2048 contiguous codes unless there are too few of them to
    // spread over the CUs; the grid is sized for the expected live rows.  When
    // it is capped, the blocks per CU (2, 3, 4 or 6 four-wave blocks, every
    // wave keeping two tasks in flight) are chosen so that the expected tasks
    // fill the rounds of the grid-stride loop most evenly (measured on MI355X:
    // a partial last round costs up to 20 %; fewer blocks break ties).
    const int64_t hint = masked_m ? ((expected_m > 0 && expected_m < T) ? expected_m : T) : T;
    const int64_t live_codes = std::max<int64_t>(hint, 1) * K;
    int64_t tcodes = E * ((live_codes + 2047) / 2048) >= (int64_t)cus * 2 ? 2048 : 1024;
    if (knob(KNOB_SLABS_PER_TASK) > 0) tcodes = knob(KNOB_SLABS_PER_TASK) >= 2 ? 2048 : 1024;
    a.tcodes = tcodes;
    if (E * ((T * K + tcodes - 1) / tcodes) >= INT32_MAX) return PTGQ_EUNSUPPORTED;
    const int64_t tasks = E * ((live_codes + tcodes - 1) / tcodes);
    int wpb = tasks >= (int64_t)cus * 4 ? 4 : 1;
    if (knob(KNOB_WAVES_PER_BLOCK) > 0) wpb = (int)std::min<int64_t>(knob(KNOB_WAVES_PER_BLOCK), 4);
    int64_t blocks = (tasks + wpb - 1) / wpb;
    int64_t per_cu = knob(KNOB_BLOCKS_PER_CU);
    if (per_cu <= 0 && blocks > (int64_t)cus * 2) {
        double best = 0.0;
        for (const int64_t c : {2, 3, 4, 6}) {
            const int64_t waves = (int64_t)cus * c * wpb;
            const double eff = (double)tasks / (double)(((tasks + waves - 1) / waves) * waves);
            if (eff > best + 1e-9) {
                best = eff;
                per_cu = c;
            }
        }
    }
    if (per_cu <= 0) per_cu = 2;
    // Uncapped (one wave per expected task, blocks dealt to the XCDs in
    // chunks of 16) once the capped grid would loop: measured on MI355X at E
    // = 8, K = 3584, 1024 live rows per expert: 12.85 -> 12.5 us (chunks of
    // 64: 12.7; contiguous ranges: 13.3).  Only for E <= 64, where each wave
    // sums masked_m in registers: the LDS prefix sum of more experts would be
    // repeated by every short-lived block.
    bool uncapped = E <= 64 && blocks > (int64_t)cus * per_cu;
    if (knob(KNOB_GRID_MODE) >= 0) uncapped = knob(KNOB_GRID_MODE) > 0;
    const int64_t cap = uncapped ? blocks : (int64_t)cus * per_cu;
    if (blocks > cap) blocks = cap;
    else if (blocks >= 64) blocks = (blocks + 7) / 8 * 8;
    if (uncapped && blocks >= 4 * 8 * kDequantXcdChunk) a.xcd_chunk = (int32_t)kDequantXcdChunk;
    if (knob(KNOB_XCD_CHUNK) >= 0)
        a.xcd_chunk = (int32_t)std::min<int64_t>(knob(KNOB_XCD_CHUNK), 1 << 20);
    const hipError_t err = launch_requant(a, (unsigned)std::max<int64_t>(blocks, 1),
                                          (unsigned)(wpb * 64), static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PTGQ_OK : PTGQ_ELAUNCH;
}

int ptgq_dequant(const uint8_t *q, int code_dtype, int64_t M, int64_t K, int group_size,
                 const void *s, int scale_fmt, int scale_layout, int out_dtype, void *y,
                 void *stream)
{
    if (code_dtype != PTGQ_E4M3 && code_dtype != PTGQ_INT8) return PTGQ_EINVAL;
    if (scale_fmt != PTGQ_SCALE_F32 && scale_fmt != PTGQ_SCALE_UE8M0) return PTGQ_EINVAL;
    if (scale_layout != PTGQ_ROW_MAJOR && scale_layout != PTGQ_COL_MAJOR) return PTGQ_EINVAL;
    if (out_dtype != PTGQ_BF16 && out_dtype != PTGQ_FP16 && out_dtype != PTGQ_FP32)
        return PTGQ_EINVAL;
    if (!valid_group_size(group_size) || M < 0 || K < 0 || K % group_size != 0)
        return PTGQ_EINVAL;
    if (M == 0 || K == 0) return PTGQ_OK;
    if (!q || !s || !y) return PTGQ_EINVAL;
    if (static_cast<const void *>(q) == y || s == y) return PTGQ_EINVAL;
    if (!aligned(q, 16) || !aligned(y, 16) || (scale_fmt == PTGQ_SCALE_F32 && !aligned(s, 4)))
        return PTGQ_EALIGN;
    if (K >= (int64_t)1 << 29 || M >= ((int64_t)1 << 31)) return PTGQ_EUNSUPPORTED;
    const int64_t ng = K / group_size;
    const size_t s_bytes = ptgq_scale_bytes(M, K, group_size, scale_fmt, scale_layout);
    if (s_bytes == 0 || s_bytes >= ((size_t)1 << 32) - (1 << 20)) return PTGQ_EUNSUPPORTED;
    const int cus = current_cus(nullptr);
    if (cus <= 0) return PTGQ_EDEVICE;
    // Tasks of ns sub-slabs (a sub-slab is 512 codes for 16-bit outputs, 256
    // for fp32), contiguous so that a wave's loads in flight stay within a few
    // pages, grid-strided over the waves for as many full rounds as fit; the
    // remainder is one last round in which every wave takes an equal share
    // (whole sub-slabs).  Problems of fewer than 16 sub-slabs per CU use one
    // sub-slab per task (measured on MI355X, e4m3 [M, 7168] -> bf16, capped
    // grid: four sub-slabs per task from M = 512 on, 4.01 -> 3.59 us; M =
    // 1024 7.68 -> 5.61, M = 2048 12.56 -> 9.44; -> fp32 M = 1024 11.77 ->
    // 6.95; M = 256 3.08 either way).  With at least as many tasks as the chip
    // holds waves, the grid is uncapped (one task per wave) and its blocks are
    // dealt to the XCDs in chunks of 16 (measured on MI355X, e4m3 [M, 7168] ->
    // bf16: M = 16384 63.7 -> 57.0 us, M = 4096 17.4 -> 16.6 us; fp32 out
    // [8192, 7168] 52.5 -> 48.3 us; chunks of 2..32 blocks within 1 %, one
    // contiguous range per XCD 62.6 us).  Fewer tasks: four four-wave blocks
    // per CU (two for fp32 outputs, whose stores are twice as wide), which
    // measured best there (M = 1024: 5.61 us against 6.28 uncapped).
    const int64_t total = M * K;
    const int64_t sub = out_dtype == PTGQ_FP32 ? 256 : 512;
    const int64_t subs = (total + sub - 1) / sub;
    if (subs >= INT32_MAX) return PTGQ_EUNSUPPORTED;
    int ns = subs >= (int64_t)cus * 16 ? 4 : 1;
    if (knob(KNOB_SLABS_PER_TASK) > 0) ns = knob(KNOB_SLABS_PER_TASK) >= 4 ? 4 : 1;
    const int64_t ts = ns * sub;
    const int64_t tasks = (subs + ns - 1) / ns;
    int wpb = tasks >= (int64_t)cus * 4 ? 4 : 1;
    if (knob(KNOB_WAVES_PER_BLOCK) > 0) wpb = (int)std::min<int64_t>(knob(KNOB_WAVES_PER_BLOCK), 4);
    int64_t blocks = (tasks + wpb - 1) / wpb;
    int64_t per_cu = out_dtype == PTGQ_FP32 ? 2 : 4;
    bool uncapped = tasks >= (int64_t)cus * 32 && knob(KNOB_BLOCKS_PER_CU) <= 0;
    if (knob(KNOB_GRID_MODE) >= 0) uncapped = knob(KNOB_GRID_MODE) > 0;
    if (knob(KNOB_BLOCKS_PER_CU) > 0) per_cu = knob(KNOB_BLOCKS_PER_CU);
    if (!uncapped && blocks > (int64_t)cus * per_cu) blocks = (int64_t)cus * per_cu;
    else if (blocks >= 64) blocks = (blocks + 7) / 8 * 8;
    if (blocks >= INT32_MAX) return PTGQ_EUNSUPPORTED;
    const int64_t waves = blocks * wpb;
    DequantArgs a;
    a.step = waves * ts;
    a.full = (int32_t)(total / a.step);
    a.full_end = a.full * a.step;
    const int64_t rem = total - a.full_end;
    a.last = (rem + waves * sub - 1) / (waves * sub) * sub;
    a.q = q;
    a.s = s;
    a.y = y;
    a.M = M;
    a.K = K;
    a.ng = ng;
    a.rows_pad = pad4(M);
    a.st = scale_layout == PTGQ_ROW_MAJOR ? ng : 1;
    a.sg = scale_layout == PTGQ_ROW_MAJOR ? 1 : a.rows_pad;
    a.dm = a.step / K;
    a.dc = (uint32_t)(a.step % K);
    a.s_bytes = (uint32_t)s_bytes;
    a.inv_k = 1.0f / (float)K;
    // every task's first code lies below total + 2 steps (the last round's
    // offsets included): 32-bit offsets divide by a multiply-high
    a.small = total + 2 * a.step < ((int64_t)1 << 31) ? 1 : 0;
    a.k_div = make_fastdiv((uint32_t)K);
    a.ns = ns;
    a.log2g = __builtin_ctz((unsigned)group_size);
    // fp32 outputs (tasks of half as many codes) in chunks of 64 blocks:
    // measured on MI355X, e4m3 [8192, 7168] -> fp32 44.2 -> 41.7 us, [16384,
    // 7168] 85.0 -> 80.7, [16384, 2048] 26.1 -> 24.8 (16-bit outputs: 16
    // stays best, fp16 [8192, 7168] 30.0 against 31.3 with 64)
    const int64_t dq_chunk = out_dtype == PTGQ_FP32 ? 4 * kDequantXcdChunk : kDequantXcdChunk;
    a.xcd_chunk = uncapped ? (int32_t)dq_chunk : 0;
    if (knob(KNOB_XCD_CHUNK) >= 0)
        a.xcd_chunk = (int32_t)std::min<int64_t>(knob(KNOB_XCD_CHUNK), 1 << 20);
    const hipError_t err = launch_dequant(a, code_dtype, scale_fmt, scale_layout, out_dtype,
                                          (unsigned)blocks, (unsigned)(wpb * 64),
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

int ptgq_probe_silu_mul(const void *g, const void *u, int in_dtype, int path, float *out,
                        int64_t n, void *stream)
{
    if (in_dtype != PTGQ_BF16 && in_dtype != PTGQ_FP16) return PTGQ_EINVAL;
    if (path != 0 && path != 1) return PTGQ_EINVAL;
    if (n < 0) return PTGQ_EINVAL;
    if (n == 0) return PTGQ_OK;
    if (!g || !u || !out) return PTGQ_EINVAL;
    if (n >= (int64_t)UINT32_MAX * 256) return PTGQ_EUNSUPPORTED;
    int dev = 0;
    if (current_cus(&dev) <= 0) return PTGQ_EDEVICE;
    // path 1 reads the lookup table: built (or ordered) on this stream first
    if (path == 1 && !table_usable(dev, static_cast<hipStream_t>(stream))) return PTGQ_EDEVICE;
    const hipError_t err = launch_probe_silu(g, u, in_dtype, path, out, n,
                                             static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PTGQ_OK : PTGQ_ELAUNCH;
}

int ptgq_probe_scale(uint32_t first_bits, int64_t n, float eps, int out_dtype, int scale_fmt,
                     void *scale_out, float *inv_out, void *stream)
{
    if (out_dtype != PTGQ_E4M3 && out_dtype != PTGQ_INT8) return PTGQ_EINVAL;
    if (scale_fmt != PTGQ_SCALE_F32 && scale_fmt != PTGQ_SCALE_UE8M0) return PTGQ_EINVAL;
    if (!(std::isfinite(eps) && eps >= 0.0f) || std::signbit(eps)) return PTGQ_EINVAL;
    if (n < 0) return PTGQ_EINVAL;
    if (n == 0) return PTGQ_OK;
    // every amax must be a non-negative finite fp32: bit patterns below +inf
    if ((int64_t)first_bits + n > (int64_t)0x7F800000) return PTGQ_EINVAL;
    if (!scale_out) return PTGQ_EINVAL;
    if (scale_fmt == PTGQ_SCALE_F32 && !aligned(scale_out, 4)) return PTGQ_EALIGN;
    if (inv_out && !aligned(inv_out, 4)) return PTGQ_EALIGN;
    if (current_cus(nullptr) <= 0) return PTGQ_EDEVICE;
    const hipError_t err = launch_probe_scale(first_bits, n, eps, out_dtype, scale_fmt, scale_out,
                                              inv_out, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PTGQ_OK : PTGQ_ELAUNCH;
}

int ptgq_probe_int8(uint32_t first_bits, int64_t n, int8_t *out, void *stream)
{
    if (n < 0 || n > ((int64_t)1 << 32)) return PTGQ_EINVAL;
    if (n == 0) return PTGQ_OK;
    if (!out) return PTGQ_EINVAL;
    if (current_cus(nullptr) <= 0) return PTGQ_EDEVICE;
    const hipError_t err = launch_probe_int8(first_bits, n, out, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PTGQ_OK : PTGQ_ELAUNCH;
}

int ptgq_probe_stream(const void *x, int64_t n, uint8_t *q, void *stream)
{
    constexpr int64_t kTask = 2 * kSlab;   // elements per wave
    if (n < 0 || n % kTask != 0) return PTGQ_EINVAL;
    if (n == 0) return PTGQ_OK;
    if (!x || !q) return PTGQ_EINVAL;
    if (!aligned(x, 16) || !aligned(q, 16)) return PTGQ_EALIGN;
    const int64_t tasks = n / kTask;
    if (tasks >= INT32_MAX) return PTGQ_EUNSUPPORTED;
    if (current_cus(nullptr) <= 0) return PTGQ_EDEVICE;
    // the plain quantization kernel's uncapped geometry: four-wave blocks,
    // one wave per task, XCD chunks of 64 blocks for large grids
    const int64_t blocks = (tasks + 3) / 4;
    const int32_t chunk = blocks >= 4 * 8 * kXcdChunk ? (int32_t)kXcdChunk : 0;
    const hipError_t err = launch_probe_stream(x, n, q, (unsigned)blocks, chunk,
                                               static_cast<hipStream_t>(stream));
    return err == hipSuccess ? PTGQ_OK : PTGQ_ELAUNCH;
}

int ptgq_diag_fastdiv(uint32_t d, const uint32_t *n, uint32_t *q, int64_t count)
{
    if (d == 0 || count < 0 || (count > 0 && (!n || !q))) return PTGQ_EINVAL;
    const FastDiv f = make_fastdiv(d);
    for (int64_t i = 0; i < count; ++i) {
        if (n[i] >= (1u << 31)) return PTGQ_EINVAL;
        q[i] = fastdiv(n[i], f);
    }
    return PTGQ_OK;
}

int ptgq_plan_group(int in_dtype, int64_t E, int64_t rows, int64_t K, int group_size,
                    int fuse_silu_mul, int64_t expected_m, int64_t q_rows, int cus, int64_t *out)
{
    if (!out || cus < 1) return PTGQ_EINVAL;
    for (int i = 0; i < kPlanFields; ++i) out[i] = 0;
    if (in_dtype != PTGQ_BF16 && in_dtype != PTGQ_FP16 && in_dtype != PTGQ_FP32)
        return PTGQ_EINVAL;
    if (!valid_group_size(group_size) || E < 0 || rows < 0 || K < 0 || K % group_size != 0)
        return PTGQ_EINVAL;
    const bool masked = E > 0;
    if (!masked && q_rows < rows) return PTGQ_EINVAL;
    if (fuse_silu_mul && in_dtype == PTGQ_FP32) return PTGQ_EUNSUPPORTED;
    if (K >= (int64_t)1 << 29 || q_rows >= ((int64_t)1 << 31)) return PTGQ_EUNSUPPORTED;
    if (K == 0 || (masked ? rows == 0 : q_rows == 0)) return PTGQ_OK;   // nothing is launched
    GroupArgs a;
    GroupGeom geo;
    const int rc = plan_group(a, geo, in_dtype, rows, K, group_size, fuse_silu_mul,
                              PTGQ_SCALE_UE8M0, PTGQ_COL_MAJOR, masked, E, expected_m,
                              masked ? rows : q_rows, true, cus);
    if (rc != PTGQ_OK) return rc;
    out[0] = geo.grid;
    out[1] = (int64_t)geo.wpb * 64;
    out[2] = a.U;
    out[3] = a.tpr;
    out[4] = a.n_tasks;
    out[5] = a.xcd_chunk;
    out[6] = geo.table ? 1 : 0;
    out[7] = geo.uncapped ? 1 : 0;
    out[8] = a.flat_slabs;
    return PTGQ_OK;
}

int ptgq_set_tuning(int which, int64_t value)
{
    if (which < 0 || which >= kKnobs) return PTGQ_EINVAL;
    g_knob[which].store(value, std::memory_order_relaxed);
    return PTGQ_OK;
}

}  // extern "C"
