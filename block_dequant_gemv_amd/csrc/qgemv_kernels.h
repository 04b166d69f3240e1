// qgemv_kernels.h -- internal interface between the C ABI (qgemv_api.hip) and
// the kernels (qgemv_kernels.hip). Not installed; not part of the public ABI.
#pragma once

#include <atomic>

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace qgk {

constexpr int kEpiPlain = 0;
constexpr int kEpiGateUp = 1;
constexpr int kEpiAffine = 2;   // M = 1: y = ((W x) + bias) + residual, fp32 or fp16 output
constexpr int kPackRows = 0;
constexpr int kPackGateUp = 1;

// Kernel arguments of the quantised GEMV (passed by value).
struct QArgs {
    qgl::Geometry geo;   // packed-weight geometry (geo.N = packed rows)
    int64_t n_out;       // outputs per activation row (N, or N_ff for gate|up)
    int64_t x_stride;    // floats between activation rows (K)
    int64_t y_stride;    // floats between output rows (N)
    int64_t tpg;         // row tiles walked by one group of W wavefronts (tstride == 0)
    int64_t tstride;     // > 0: group g walks tiles g, g + tstride, g + 2*tstride, ... (tstride = groups)
    // persistent form only
    int64_t n_wg;        // workgroups; workgroup b owns halves_base half-tiles (4 rows), one more for
                         // b < halves_extra (halves_base = 2 n_tiles / n_wg, halves_extra = 2 n_tiles % n_wg),
                         // contiguous
    int64_t halves_base;
    int64_t halves_extra;
    int64_t ranges;      // K ranges per tile (divides nseg); item = (tile, range)
    int64_t range_segs;  // segments per range (nseg / ranges)
    int64_t phases;      // divides ranges: the ranges are walked in phases of ranges/phases, each with
                         // only its segments' activations staged in LDS (1: all at once)
    // kEpiAffine only (M = 1): fp32 addends (either may be null) and the output type
    const float *bias;
    const float *residual;
    int out_f16;         // 1: y holds fp16 values (round to nearest even), 0: fp32
    // RMSNorm prologue only: the staged activations become (x * r) * gamma,
    // r = 1 / sqrt(sum(x^2) / K + eps)
    const float *gamma;
    float eps;
};

// How one quantised call is split. W depends only on (qtype, rows, K) so that
// the decode GEMV and the verify GEMV of the same weight add in the same order.
struct QPlan {
    bool persist;        // persistent form: one workgroup per CU, (tile, K range) items
    int ranges;          // persistent form: K ranges per tile (divides nseg)
    int phases;          // persistent form: phases of ranges/phases ranges (divides ranges), each
                         // staging only its segments' activations
    int64_t max_tiles;   // persistent form: most tiles any workgroup's half-tiles touch
    int W;               // classic form: wavefronts splitting one row tile along K (1, 2, 3, 4, 8)
    int64_t tpg;         // tiles per group (contiguous order)
    int64_t tstride;     // > 0: grid-stride tile order over this many groups (tpg unused)
    int64_t grid;        // workgroups
    int block;           // threads per workgroup (64 * wavefronts)
    int depth;           // units in flight ahead of the one being computed (1 or 2; 2 only for M = 1)
    bool x_in_lds;       // activations staged in LDS
    size_t lds_bytes;    // dynamic LDS per workgroup
    bool norm;           // RMSNorm prologue on the staged activations (M = 1, x_in_lds)
    int row_groups = 1;  // tile form, plain store: gridDim.y groups of the kernel's M activation rows each
    bool one_unit = false;   // persistent form with one segment per K range (every item is one unit)
};

struct F16Plan {
    int R;               // lane-split form: rows per workgroup (register-blocked)
    int waves;           // lane-split and split-K row forms: wavefronts splitting K;
                         // row form: rows (wavefronts) per workgroup
    bool vec;            // 16-byte path (K % 8 == 0 and aligned pointers)
    int L;               // 1..kF16RowMaxL: row form for K = 512 * L
    int cpl;             // 1, 2, 4: split-K row form with cpl chunks per lane (L == 0)
    int64_t grid;
};

// The fp16 row form takes rows of K = 512 * L weights, L <= 16: each lane holds
// L 16-byte chunks of its row at once (4 L registers).
constexpr int kF16RowMaxL = 16;

// Two timing events bound to the next GEMV kernel this thread launches: they
// receive that kernel's own start and end timestamps. The launch takes them
// and clears the setting; (nullptr, nullptr) clears it too.
void set_launch_events(hipEvent_t start, hipEvent_t stop);
void take_launch_events(hipEvent_t &start, hipEvent_t &stop);

// Launch `kern` on `stream`: with timing events bound, through hipExtLaunchKernel
// (the events take the dispatch's start and end times); otherwise as a plain
// launch, which a caller may also record into a HIP graph.
template <typename Kern, typename... Args>
inline void launch_timed(Kern kern, dim3 grid, dim3 block, uint32_t lds, hipStream_t stream, Args... args)
{
    hipEvent_t e0, e1;
    take_launch_events(e0, e1);
    if (e0 != nullptr)
        hipExtLaunchKernelGGL(kern, grid, block, lds, stream, e0, e1, 0u, args...);
    else
        hipLaunchKernelGGL(kern, grid, block, lds, stream, args...);
}

// Launch bound of the one-wavefront-per-tile form (qgemv_kernel). A split
// workgroup (W > 1) has exactly W wavefronts. The k-quant kernels with 5 or 6
// activation rows declare a bound of at most 256 threads (one wavefront per
// SIMD), which lets them use the accumulation registers instead of spilling to
// scratch (measured, split kernels: M = 6 on 8000 x 2048, Q6_K 23.4 -> 17.5 us,
// Q4_K 20.8 -> 18.1 us; M = 5 with W = 2 about 10% faster); the planner keeps
// their workgroups within it. With fewer rows they spill little or nothing,
// and the wider register budget only lowers their occupancy (Q6_K M = 4 on the
// same matrix 11.1 -> 13.2 us), so every other instantiation keeps the
// 512-thread bound. Unsplit Q6_K rows fit 256 VGPRs at M = 5, 6 and keep it too.
constexpr int qgemv_max_threads(int QT, int M, int W)
{
    if (M >= 5 && (QT == qgl::kQ4_K || QT == qgl::kQ6_K)) {
        if (W > 1) return 64 * W;
        if (QT == qgl::kQ4_K) return 256;
    }
    return 512;
}

// Threads per workgroup of the persistent form (its launch bound): as many
// wavefronts as one CU holds at the kernel's register count. Single-row
// kernels, and Q4_0 with 2 or 3 rows, fit 128 VGPRs (16 wavefronts; Q4_0
// 17408 x 5120 at M = 3: 22.2 -> 21.5 us against 12 wavefronts, M = 2
// unchanged); the other multi-row kernels up to 168 (12 wavefronts) where they
// fit without spilling, else 256 (8); Q4_K with 5 or 6 rows 4 wavefronts (512
// registers each, no scratch). one: every item is one unit (one segment per K
// range), so no accumulator lives from one unit to the next (Q4_0 at M = 6
// with staged activations: 149 -> 111 VGPRs): Q4_0 fits 128 VGPRs at every M
// (with activations from L2, or staged in phases, up to 4 rows), Q8_0 with staged activations up to 4
// rows, 168 above; Q6_K fits 168 up to 3 rows (4, and 5 unphased, with staged
// activations; Q6_K 17408 x 5120 at M = 5: 32.1-32.9 -> 30.9-31.4 us against 8
// wavefronts) and 256 without scratch at 5 and 6 (the general form spills there); Q4_K with 5
// rows and staged activations (whose block sums it reads instead of adding
// them up) fits 256 at 8 wavefronts (Q4_K 17408 x 5120 at M = 5: 34.5 -> 29.3 us
// against 4 wavefronts, the same bits).
constexpr int persist_threads(int qt, int M, bool xlds, bool one = false, bool phased = false)
{
    if (M == 1) return 1024;
    if (one) {
        if (qt == qgl::kQ4_0) return ((xlds && !(phased && M >= 5)) || M <= 4) ? 1024 : 768;
        if (qt == qgl::kQ8_0 && xlds) return M <= 4 ? 1024 : 768;
        if (qt == qgl::kQ6_K) return (M <= 3 || ((M == 4 || (M == 5 && !phased)) && xlds)) ? 768 : 512;
        if (qt == qgl::kQ4_K && M == 5 && xlds) return 512;
    }
    if (qt == qgl::kQ4_0) return M <= 3 ? 1024 : ((M <= 4 || xlds) ? 768 : 512);
    if (qt == qgl::kQ4_K) return M <= 2 ? 768 : (M <= 4 ? 512 : 256);
    if (qt == qgl::kQ6_K) return M <= 2 ? 768 : 512;
    return (M <= 3 || xlds) ? 768 : 512;
}

// Q4_K kernels with staged activations and no RMSNorm prologue follow the
// staged copy with its block sums (one float per activation row and 32-weight
// block, written once per workgroup after staging), so that every wavefront
// reads a block's sum of x instead of adding it up. The RMSNorm kernels add
// them up per unit as before, which keeps their activation limit that of the
// other types. Bytes of LDS per staged 1024-weight segment of one activation
// row, the sums included.
constexpr bool x_sums_staged(int qt, bool xlds, bool norm) { return qt == qgl::kQ4_K && xlds && !norm; }
constexpr size_t staged_seg_bytes(int qt, bool norm)
{
    return (size_t)qgl::kSegWeights * sizeof(float) + (x_sums_staged(qt, true, norm) ? 32 * sizeof(float) : 0);
}

// Static LDS of the quantised GEMV kernels. The kernels declare their arrays
// with these sizes and the launch planner adds them to the dynamic activation
// copy, so that a plan never asks for more than a CU's LDS:
//   qgemv_kernel: `red`, the split-K partials [W][M][slot][row] for W > 1, one
//     float per wavefront (at most 8) for the RMSNorm prologue, else one float;
//   qgemv_persist: `nred`, one float per wavefront (at most 16) for the RMSNorm
//     prologue, else one float.
constexpr int tile_red_floats(int M, int W, bool norm)
{
    return W > 1 ? W * M * qgl::kSlots * qgl::kRowsPerLane : (norm ? 8 : 1);
}
constexpr int persist_red_floats(bool norm) { return norm ? 16 : 1; }
// Bytes that a static array of `floats` floats occupies ahead of the dynamic
// array, which is 16-byte aligned (f32x4).
constexpr size_t static_lds_bytes(int floats) { return ((size_t)floats * sizeof(float) + 15) / 16 * 16; }
// LDS of one workgroup on gfx950 (static plus dynamic).
constexpr size_t kLdsPerWorkgroup = 160 * 1024;

// Raise a kernel's dynamic-LDS limit to `bytes` (needed above 64 KiB) unless it is
// already that high on the current device. `set` is the caller's record for that
// one kernel (one per template instantiation), so a decode loop pays for the
// attribute call once per kernel and device, not once per launch.
inline hipError_t ensure_lds_limit(const void *kern, size_t bytes, std::atomic<int> (&set)[16])
{
    if (bytes <= 64 * 1024) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::atomic<int> *rec = (dev >= 0 && dev < 16) ? &set[dev] : nullptr;
    if (rec && rec->load(std::memory_order_relaxed) >= (int)bytes) return hipSuccess;
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return e;
    if (rec) {
        int cur = rec->load(std::memory_order_relaxed);
        while (cur < (int)bytes && !rec->compare_exchange_weak(cur, (int)bytes)) {
        }
    }
    return hipSuccess;
}

hipError_t launch_qgemv(int qt, int M, int epi, const QPlan &p, const uint8_t *wp, const float *x, float *y,
                        const QArgs &a, hipStream_t s);
hipError_t launch_rmsnorm(const float *x, const float *gamma, float eps, float *out, int64_t K, hipStream_t s);
hipError_t launch_f16(const F16Plan &p, const uint16_t *w, const float *x, float *y, int64_t N, int64_t K,
                      hipStream_t s);
hipError_t launch_probe_stream(const void *buf, uint64_t bytes, uint32_t *sink, uint32_t magic, hipStream_t s);
hipError_t launch_probe_empty(hipStream_t s);
hipError_t launch_pack(const qgl::Geometry &g, const uint8_t *canon, const uint8_t *canon_up, uint8_t *packed,
                       int mode, int64_t row0, int64_t nrows, int64_t rows_to_write, bool zero_gaps,
                       hipStream_t s);

}  // namespace qgk
