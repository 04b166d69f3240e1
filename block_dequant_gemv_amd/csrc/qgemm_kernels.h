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
};

// Rows of activations per matrix-core tile, and activation tiles per GEMM pass.
constexpr int kGemmTileM = 16;
constexpr int kGemmMaxMT = 2;

// Split X fp32 [M][K] into the per-row scaled fp16 hi/lo parts the GEMM reads
// (xs: M_pad * K * 2 halves, unscale: M_pad floats; M_pad = M rounded up to 16).
hipError_t launch_split_x(int qt, const float *X, _Float16 *xs, float *unscale, int64_t M, int64_t M_pad, int64_t K,
                          hipStream_t s);

// One GEMM pass over activation tiles [a.mt0, a.mt0 + MT), MT in {1, 2}.
hipError_t launch_qgemm(int qt, int MT, const uint8_t *wp, const _Float16 *xs, const float *unscale, float *Y,
                        const GemmArgs &a, int64_t grid, int block, hipStream_t s);

}  // namespace qgk
