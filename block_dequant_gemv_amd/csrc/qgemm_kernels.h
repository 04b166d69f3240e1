// qgemm_kernels.h -- internal interface of the small-M GEMM kernels
// (qgemm_kernels.hip) for the C ABI. Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"
#include "qgemv_kernels.h"

namespace qgk {

// Kernel arguments of the GEMM (passed by value).
struct GemmArgs {
    qgl::Geometry geo;   // packed-weight geometry
    int64_t N;           // weight rows = outputs per activation row
    int64_t M;           // activation rows
    int64_t n_mg;        // groups of MT 16-row activation tiles (workgroup index = row block * n_mg + group)
    int64_t y_stride;    // floats between output rows (N)
    int64_t ksplit;      // K ranges (gridDim.y); range ky covers chunks [n_chunks*ky/ksplit, n_chunks*(ky+1)/ksplit)
    float *part;         // ksplit > 1: partial sums [ky][M][N] (summed in ky order by the reduce kernel)
};

// Rows of activations per matrix-core tile, activation tiles per workgroup (at
// most), blocks of 32 weights per staged chunk of K, chunks loaded ahead of the
// one being computed, and the ring of staging buffers that this takes.
constexpr int kGemmTileM = 16;
constexpr int kGemmMaxMT = 4;
constexpr int kGemmChunk = 4;
constexpr int kGemmDepth = 2;
constexpr int kGemmRing = kGemmDepth + 1;

// s_waitcnt vmcnt(n) for n < 64 (expcnt and lgkmcnt left free): the encoding of
// gfx9-family parts (vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Words of one staged chunk's scales per wavefront copy (one 64-lane copy per
// wavefront: a workgroup's 2 RG G row tiles x 2 slots x kGemmChunk blocks x 8 B
// fit in G x 64 words for RG <= 2).
constexpr int kGemmScaleWordsPerWave = 64;

// 16-byte weight loads per wavefront, chunk and row group: one per load group of
// 4 (Q4_0) or 2 (Q8_0) blocks.
constexpr int gemm_weight_loads(int qt) { return kGemmChunk / (qt == qgl::kQ8_0 ? 2 : 4); }

// LDS of one GEMM workgroup of G wavefronts with RG row groups each:
// kGemmRing buffers (two chunks in flight while a third is read), each the
// chunk's split activations (MT tiles x kGemmChunk blocks x 2 KiB), the scales
// of the workgroup's rows (one 64-word copy per wavefront) and its weights (one
// KiB per wavefront, load group and row group).
constexpr size_t gemm_lds_bytes(int qt, int MT, int RG, int G)
{
    return (size_t)kGemmRing * ((size_t)MT * kGemmChunk * 2048 + (size_t)G * kGemmScaleWordsPerWave * 4 +
                                (size_t)G * gemm_weight_loads(qt) * RG * 1024);
}

// Y[m][n] = sum over ky (in order) of part[ky][m][n], m < M, n < N.
hipError_t launch_ksum(const float *part, float *Y, int64_t ksplit, int64_t M, int64_t N, hipStream_t s);

// Split X fp32 [M][K] into the per-row scaled fp16 hi/lo parts the GEMM reads
// (xs: M_pad * K * 2 halves, unscale: M_pad floats; M_pad = M rounded up to 16).
hipError_t launch_split_x(int qt, const float *X, _Float16 *xs, float *unscale, int64_t M, int64_t M_pad, int64_t K,
                          hipStream_t s);

// The GEMM over every activation tile group at once: gridDim.x = row blocks x
// a.n_mg, gridDim.y = a.ksplit; MT in 1..4 activation tiles per workgroup, G
// wavefronts per workgroup (1, 2, 4 or 8) of RG 16-row groups each (1 or 2).
hipError_t launch_qgemm(int qt, int MT, int RG, int G, int64_t row_blocks, const uint8_t *wp, const _Float16 *xs,
                        const float *unscale, float *Y, const GemmArgs &a, hipStream_t s);

}  // namespace qgk
