// qgemm_kernels.h -- internal interface of the small-M GEMM kernels
// (qgemm_kernels.hip) for the C ABI. Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"
#include "qgemv_kernels.h"

namespace qgk {

// Kernel arguments of one GEMM pass (passed by value).
struct GemmArgs {
    qgl::Geometry geo;   // packed-weight geometry
    int64_t N;           // weight rows = outputs per activation row
    int64_t M;           // activation rows
    int64_t mt0;         // first 16-row activation tile of this pass
    int64_t y_stride;    // floats between output rows (N)
    int64_t ksplit;      // K ranges (gridDim.y); range ky covers segments [nseg*ky/ksplit, nseg*(ky+1)/ksplit)
    float *part;         // ksplit > 1: partial sums [ky][M][N] (summed in ky order by the reduce kernel)
};

// Rows of activations per matrix-core tile, activation tiles per GEMM pass (at
// most), blocks of 32 weights per staged chunk of K.
constexpr int kGemmTileM = 16;
constexpr int kGemmMaxMT = 4;
constexpr int kGemmChunk = 4;
// Blocks per staged chunk for MT activation tiles per pass: one tile stages
// 8 blocks at a time (fewer waits per K, twice the weights in flight).
constexpr int gemm_chunk(int MT) { return MT == 1 ? 2 * kGemmChunk : kGemmChunk; }

// s_waitcnt vmcnt(n) for n < 16 (expcnt and lgkmcnt left free): the encoding of
// gfx9-family parts (vmcnt bits 3:0, expcnt 6:4, lgkmcnt 11:8).
constexpr int vmcnt_imm(int n) { return 0x0F70 | n; }

// 4-byte words of one staged chunk's scales (wg_tiles x 2 slots x CB blocks x
// 8 B), rounded up to whole 64-lane copies.
constexpr int gemm_scale_words(int wg_tiles, int CB)
{
    return (wg_tiles * 2 * CB * 2 + 63) / 64 * 64;
}

// LDS of one GEMM workgroup, two buffers (one chunk staged while the other is
// read) of: the chunk's split activations (MT tiles x 2 KiB per block) and the
// scales of its row tiles (2 slots x 4 rows x fp16 per block).
constexpr size_t gemm_lds_bytes(int MT, int wg_tiles)
{
    return 2 * ((size_t)MT * gemm_chunk(MT) * 128 * 16 + (size_t)gemm_scale_words(wg_tiles, gemm_chunk(MT)) * 4);
}

// Y[m][n] = sum over ky (in order) of part[ky][m][n], m < M, n < N.
hipError_t launch_ksum(const float *part, float *Y, int64_t ksplit, int64_t M, int64_t N, hipStream_t s);

// Split X fp32 [M][K] into the per-row scaled fp16 hi/lo parts the GEMM reads
// (xs: M_pad * K * 2 halves, unscale: M_pad floats; M_pad = M rounded up to 16).
hipError_t launch_split_x(int qt, const float *X, _Float16 *xs, float *unscale, int64_t M, int64_t M_pad, int64_t K,
                          hipStream_t s);

// One GEMM pass over activation tiles [a.mt0, a.mt0 + MT), MT in 1..4, with G
// wavefronts per workgroup (1..4) of RG 16-row groups each (1, 2 or 4; a pass
// of 3 tiles runs with one row group, of 4 tiles with at most two).
hipError_t launch_qgemm(int qt, int MT, int RG, int G, const uint8_t *wp, const _Float16 *xs, const float *unscale,
                        float *Y, const GemmArgs &a, hipStream_t s);

}  // namespace qgk
