// qgemv_kernels.hip -- gfx950 kernels of libqgemv other than the quantised
// GEMV itself (qgemv_device.h, instantiated in qgemv_inst.hip): the fp16 GEMV in
// its two forms, the standalone RMSNorm, the load-time packer, and the host-side
// launch entry points of every kernel.
#include "qgemv_device.h"

namespace qgk {

// ---------------------------------------------------------------------------
// fp16 split-K GEMV: a workgroup of nw wavefronts owns R rows; its 64*nw lanes
// split K in 8-element chunks (16 bytes of weights per lane per row); partials
// are summed per wavefront (butterfly) and then over wavefronts in order in LDS.
template <int R, bool VEC>
__global__ void __launch_bounds__(1024)
gemv_f16_kernel(const uint16_t *__restrict__ w, const float *__restrict__ x, float *__restrict__ y, int64_t N,
                int64_t K)
{
    __shared__ float red[16 * R];
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int wave = tid >> 6, lane = tid & 63, nwave = nthr >> 6;
    const int64_t row0 = (int64_t)blockIdx.x * R;

    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0f;

    if (VEC) {
        const int64_t nch = K >> 3;
        for (int64_t c = tid; c < nch; c += nthr) {
            const f32x4 xa = *(const f32x4 *)(x + c * 8);
            const f32x4 xb = *(const f32x4 *)(x + c * 8 + 4);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if (row0 + r < N) {
                    const u32x4 wv = *(const u32x4 *)(w + (row0 + r) * K + c * 8);
                    const h2 p0 = as_h2(wv.x), p1 = as_h2(wv.y), p2 = as_h2(wv.z), p3 = as_h2(wv.w);
                    float s_ = acc[r];
                    s_ = __builtin_fmaf((float)p0.x, xa.x, s_);
                    s_ = __builtin_fmaf((float)p0.y, xa.y, s_);
                    s_ = __builtin_fmaf((float)p1.x, xa.z, s_);
                    s_ = __builtin_fmaf((float)p1.y, xa.w, s_);
                    s_ = __builtin_fmaf((float)p2.x, xb.x, s_);
                    s_ = __builtin_fmaf((float)p2.y, xb.y, s_);
                    s_ = __builtin_fmaf((float)p3.x, xb.z, s_);
                    s_ = __builtin_fmaf((float)p3.y, xb.w, s_);
                    acc[r] = s_;
                }
            }
        }
    } else {
        const _Float16 *wh = (const _Float16 *)w;
        for (int64_t k = tid; k < K; k += nthr) {
            const float xk = x[k];
#pragma unroll
            for (int r = 0; r < R; ++r)
                if (row0 + r < N) acc[r] = __builtin_fmaf((float)wh[(row0 + r) * K + k], xk, acc[r]);
        }
    }

#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float h = half_wave_sum(acc[r]);
        const float tot = as_f(__builtin_amdgcn_readlane(as_i(h), 0)) + as_f(__builtin_amdgcn_readlane(as_i(h), 32));
        if (lane == 0) red[wave * R + r] = tot;
    }
    __syncthreads();
    if (tid < R && row0 + tid < N) {
        float v = red[tid];
        for (int wv = 1; wv < nwave; ++wv) v += red[wv * R + tid];
        y[row0 + tid] = v;
    }
}

// ---------------------------------------------------------------------------
// fp16 GEMV, row form, for K = 512 * L: wavefront g of a workgroup of G owns
// row blockIdx * G + g. Every thread first issues its share of x (K / 4
// float4, at most XN per thread), then the wavefront issues all L of its row's
// 1 KiB loads (lane l takes the 16-byte chunks l, l + 64, ..., l + 64 (L - 1));
// loads complete in issue order, so writing x to LDS waits for x alone and the
// barrier passes while the weights are still in flight. x goes to LDS as two
// planes: float4 c of plane 0 holds x[8c .. 8c + 3], of plane 1
// x[8c + 4 .. 8c + 7], so each lane reads 16 contiguous bytes from each plane
// for its chunk c. A lane's sum is one fma chain over its chunks in order (8
// products each), then the wavefront butterfly: at most 8 L + 6 = 134
// roundings deep. Wavefronts past the last row load row N - 1 and store
// nothing.
template <int L, int G>
__global__ void __launch_bounds__(64 * G)
gemv_f16_row_kernel(const uint16_t *__restrict__ w, const float *__restrict__ x, float *__restrict__ y, int64_t N,
                    int64_t K)
{
    constexpr uint32_t kChunks = 64 * L;                     // 16-byte chunks per row
    constexpr uint32_t kX4 = 2 * kChunks;                    // float4 of x
    constexpr uint32_t XN = (kX4 + 64 * G - 1) / (64 * G);   // x float4 per thread
    extern __shared__ f32x4 xp[];                            // [2][kChunks]
    const uint32_t tid = threadIdx.x, lane = tid & 63;
    const int64_t row_raw = (int64_t)blockIdx.x * G + (tid >> 6);
    const bool live = row_raw < N;
    const int64_t row = live ? row_raw : N - 1;
    const u32x4 *wr = (const u32x4 *)(w + row * K);
    const f32x4 *x4 = (const f32x4 *)x;

    f32x4 xv[XN];
#pragma unroll
    for (uint32_t r = 0; r < XN; ++r) {
        const uint32_t q = tid + r * 64 * G;
        xv[r] = x4[q < kX4 ? q : 0u];
    }
    u32x4 v[L];
#pragma unroll
    for (int i = 0; i < L; ++i) v[i] = __builtin_nontemporal_load(wr + lane + 64 * i);
#pragma unroll
    for (uint32_t r = 0; r < XN; ++r) {
        const uint32_t q = tid + r * 64 * G;
        if (q < kX4) xp[(q & 1) * kChunks + (q >> 1)] = xv[r];
    }
    __syncthreads();

    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const uint32_t c = lane + 64 * i;
        const f32x4 xa = xp[c], xb = xp[kChunks + c];
        const h2 p0 = as_h2(v[i].x), p1 = as_h2(v[i].y), p2 = as_h2(v[i].z), p3 = as_h2(v[i].w);
        acc = __builtin_fmaf((float)p0.x, xa.x, acc);
        acc = __builtin_fmaf((float)p0.y, xa.y, acc);
        acc = __builtin_fmaf((float)p1.x, xa.z, acc);
        acc = __builtin_fmaf((float)p1.y, xa.w, acc);
        acc = __builtin_fmaf((float)p2.x, xb.x, acc);
        acc = __builtin_fmaf((float)p2.y, xb.y, acc);
        acc = __builtin_fmaf((float)p3.x, xb.z, acc);
        acc = __builtin_fmaf((float)p3.y, xb.w, acc);
    }
    const float h = half_wave_sum(acc);
    const float tot = as_f(__builtin_amdgcn_readlane(as_i(h), 0)) + as_f(__builtin_amdgcn_readlane(as_i(h), 32));
    if (live && lane == 0) y[row] = tot;
}

// ---------------------------------------------------------------------------
// fp16 GEMV, split-K row form, for short matrices (few rows, long K): one
// workgroup per row, whose W = blockDim / 64 wavefronts own consecutive K
// ranges of 64 CPL 16-byte chunks (8 weights) each: lane l of wavefront v takes
// chunks 64 CPL v + 64 i + l, i < CPL, and chunks at or past K / 8 count as
// nothing. Every lane issues all its weight and activation loads at once (the
// activations straight from L2: each wavefront reads only its range), then one
// fma chain over its chunks in order (8 products each), the wavefront
// butterfly, and the W partial sums are added in wavefront order through LDS:
// at most 8 CPL + 6 + W roundings. Needs K % 8 == 0 and 16-byte aligned w, x.
template <int CPL>
__global__ void __launch_bounds__(1024)
gemv_f16_wsplit_kernel(const uint16_t *__restrict__ w, const float *__restrict__ x, float *__restrict__ y,
                       int64_t N, int64_t K)
{
    __shared__ float red[16];
    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwave = blockDim.x >> 6;
    const int64_t row = blockIdx.x;
    const uint32_t nch = (uint32_t)(K >> 3);
    const u32x4 *wr = (const u32x4 *)(w + row * K);
    const f32x4 *x4 = (const f32x4 *)x;
    u32x4 v[CPL];
    f32x4 xa[CPL], xb[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const uint32_t c = wave * (64u * CPL) + 64u * i + lane;
        const uint32_t cc = c < nch ? c : 0u;
        v[i] = __builtin_nontemporal_load(wr + cc);
        xa[i] = x4[2 * cc];
        xb[i] = x4[2 * cc + 1];
    }
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const h2 p0 = as_h2(v[i].x), p1 = as_h2(v[i].y), p2 = as_h2(v[i].z), p3 = as_h2(v[i].w);
        float t = acc;
        t = __builtin_fmaf((float)p0.x, xa[i].x, t);
        t = __builtin_fmaf((float)p0.y, xa[i].y, t);
        t = __builtin_fmaf((float)p1.x, xa[i].z, t);
        t = __builtin_fmaf((float)p1.y, xa[i].w, t);
        t = __builtin_fmaf((float)p2.x, xb[i].x, t);
        t = __builtin_fmaf((float)p2.y, xb[i].y, t);
        t = __builtin_fmaf((float)p3.x, xb[i].z, t);
        t = __builtin_fmaf((float)p3.y, xb[i].w, t);
        acc = (wave * (64u * CPL) + 64u * i + lane < nch) ? t : acc;
    }
    const float h = half_wave_sum(acc);
    const float tot = as_f(__builtin_amdgcn_readlane(as_i(h), 0)) + as_f(__builtin_amdgcn_readlane(as_i(h), 32));
    if (lane == 0) red[wave] = tot;
    __syncthreads();
    if (tid == 0) {
        float sum = red[0];
        for (uint32_t u = 1; u < nwave; ++u) sum += red[u];
        y[row] = sum;
    }
}

// ---------------------------------------------------------------------------
// Standalone RMSNorm of one activation vector (one workgroup): out[k] =
// (x[k] * r) * gamma[k], r = 1 / sqrt(sum(x^2) / K + eps), with the same
// reduction scheme as the GEMV prologue.
__global__ void __launch_bounds__(1024)
rmsnorm_kernel(const float *__restrict__ x, const float *__restrict__ gamma, float eps, float *__restrict__ out,
               int64_t K)
{
    __shared__ float red[16];
    const int64_t tid = threadIdx.x, nthr = blockDim.x;
    float s = 0.0f;
    for (int64_t k = tid; k < K; k += nthr) s = __builtin_fmaf(x[k], x[k], s);
    const float r = rms_scale(block_sum(s, red), K, eps);
    for (int64_t k = tid; k < K; k += nthr) out[k] = (x[k] * r) * gamma[k];
}

// ---------------------------------------------------------------------------
// Load-time packing: one thread per (packed row, block).
//   mode kPackRows:   packed rows [row0, row0 + nrows) <- canonical rows 0..nrows-1,
//                     plus zero padding rows [N, n_tiles*8) when row0 + nrows == N
//   mode kPackGateUp: virtual row v <- gate row v/2 (v even) / up row v/2 (v odd)
__global__ void pack_kernel(Geometry g, const uint8_t *__restrict__ canon, const uint8_t *__restrict__ canon_up,
                            uint8_t *__restrict__ packed, int mode, int64_t row0, int64_t nrows, int64_t nthreads)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nthreads) return;
    const int64_t r = i / g.KB, blk = i - r * g.KB;
    const int64_t rb = canon_row_bytes(g.qt, g.K);
    if (mode == kPackRows) {
        const int64_t row = row0 + r;
        const uint8_t *src = (r < nrows) ? canon + r * rb : nullptr;
        pack_block(g, src, packed, row, blk);
    } else {
        const int64_t v = r;
        const int64_t n = v >> 1;
        const uint8_t *base = (v & 1) ? canon_up : canon;
        const uint8_t *src = (v < g.N) ? base + n * rb : nullptr;
        pack_block(g, src, packed, v, blk);
    }
}

// Zero the alignment gaps after the packed planes (so that a packed buffer is
// fully determined by its canonical input): [gap[2k], gap[2k+1]) for k < 3.
struct Gaps {
    int64_t b[6];
};

__global__ void zero_gaps_kernel(uint8_t *__restrict__ packed, Gaps gp)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
#pragma unroll
    for (int k = 0; k < 3; ++k)
        if (gp.b[2 * k] + i < gp.b[2 * k + 1]) packed[gp.b[2 * k] + i] = 0;
}

// ---------------------------------------------------------------------------
// launch entry points (host side)

namespace {
thread_local hipEvent_t t_ev_start = nullptr, t_ev_stop = nullptr;
}  // namespace

void take_launch_events(hipEvent_t &start, hipEvent_t &stop)
{
    start = t_ev_start;
    stop = t_ev_stop;
    t_ev_start = t_ev_stop = nullptr;
}

void set_launch_events(hipEvent_t start, hipEvent_t stop)
{
    t_ev_start = start;
    t_ev_stop = stop;
}

// The quantised GEMV instantiations live in their own translation units.
extern template hipError_t launch_qgemv_m1<kQ8_0>(int, const QPlan &, const uint8_t *, const float *, float *,
                                                      const QArgs &, hipStream_t);
extern template hipError_t launch_qgemv_rows<kQ8_0, 2>(const QPlan &, const uint8_t *, const float *, float *,
                                                           const QArgs &, hipStream_t);
extern template hipError_t launch_qgemv_rows<kQ8_0, 3>(const QPlan &, const uint8_t *, const float *, float *,
                                                           const QArgs &, hipStream_t);
extern template hipError_t launch_qgemv_rows<kQ8_0, 4>(const QPlan &, const uint8_t *, const float *, float *,
                                                           const QArgs &, hipStream_t);
extern template hipError_t launch_qgemv_rows<kQ8_0, 5>(const QPlan &, const uint8_t *, const float *, float *,
                                                           const QArgs &, hipStream_t);
extern template hipError_t launch_qgemv_rows<kQ8_0, 6>(const QPlan &, const uint8_t *, const float *, float *,
                                                           const QArgs &, hipStream_t);
extern template hipError_t launch_qgemv_m1<kQ4_0>(int, const QPlan &, const uint8_t *, const float *, float *,
                                                      const QArgs &, hipStream_t);
extern template hipError_t launch_qgemv_rows<kQ4_0, 2>(const QPlan &, const uint8_t *, const float *, float *,
                                                           const QArgs &, hipStream_t);
extern template hipError_t launch_qgemv_rows<kQ4_0, 3>(const QPlan &, const uint8_t *, const float *, float *,
                                                           const QArgs &, hipStream_t);
extern template hipError_t launch_qgemv_rows<kQ4_0, 4>(const QPlan &, const uint8_t *, const float *, float *,
                                                           const QArgs &, hipStream_t);
extern template hipError_t launch_qgemv_rows<kQ4_0, 5>(const QPlan &, const uint8_t *, const float *, float *,
                                                           const QArgs &, hipStream_t);
extern template hipError_t launch_qgemv_rows<kQ4_0, 6>(const QPlan &, const uint8_t *, const float *, float *,
                                                           const QArgs &, hipStream_t);
extern template hipError_t launch_qgemv_m1<kQ4_K>(int, const QPlan &, const uint8_t *, const float *, float *,
                                                      const QArgs &, hipStream_t);
extern template hipError_t launch_qgemv_rows<kQ4_K, 2>(const QPlan &, const uint8_t *, const float *, float *,
                                                           const QArgs &, hipStream_t);
extern template hipError_t launch_qgemv_rows<kQ4_K, 3>(const QPlan &, const uint8_t *, const float *, float *,
                                                           const QArgs &, hipStream_t);
extern template hipError_t launch_qgemv_rows<kQ4_K, 4>(const QPlan &, const uint8_t *, const float *, float *,
                                                           const QArgs &, hipStream_t);
extern template hipError_t launch_qgemv_rows<kQ4_K, 5>(const QPlan &, const uint8_t *, const float *, float *,
                                                           const QArgs &, hipStream_t);
extern template hipError_t launch_qgemv_rows<kQ4_K, 6>(const QPlan &, const uint8_t *, const float *, float *,
                                                           const QArgs &, hipStream_t);
extern template hipError_t launch_qgemv_m1<kQ6_K>(int, const QPlan &, const uint8_t *, const float *, float *,
                                                      const QArgs &, hipStream_t);
extern template hipError_t launch_qgemv_rows<kQ6_K, 2>(const QPlan &, const uint8_t *, const float *, float *,
                                                           const QArgs &, hipStream_t);
extern template hipError_t launch_qgemv_rows<kQ6_K, 3>(const QPlan &, const uint8_t *, const float *, float *,
                                                           const QArgs &, hipStream_t);
extern template hipError_t launch_qgemv_rows<kQ6_K, 4>(const QPlan &, const uint8_t *, const float *, float *,
                                                           const QArgs &, hipStream_t);
extern template hipError_t launch_qgemv_rows<kQ6_K, 5>(const QPlan &, const uint8_t *, const float *, float *,
                                                           const QArgs &, hipStream_t);
extern template hipError_t launch_qgemv_rows<kQ6_K, 6>(const QPlan &, const uint8_t *, const float *, float *,
                                                           const QArgs &, hipStream_t);

template <int QT>
static hipError_t launch_type(int M, int epi, const QPlan &p, const uint8_t *wp, const float *x, float *y,
                              const QArgs &a, hipStream_t s)
{
    if (epi != kEpiPlain || M <= 1) return launch_qgemv_m1<QT>(epi, p, wp, x, y, a, s);
    switch (M) {
    case 2: return launch_qgemv_rows<QT, 2>(p, wp, x, y, a, s);
    case 3: return launch_qgemv_rows<QT, 3>(p, wp, x, y, a, s);
    case 4: return launch_qgemv_rows<QT, 4>(p, wp, x, y, a, s);
    case 5: return launch_qgemv_rows<QT, 5>(p, wp, x, y, a, s);
    default: return launch_qgemv_rows<QT, 6>(p, wp, x, y, a, s);
    }
}

hipError_t launch_qgemv(int qt, int M, int epi, const QPlan &p, const uint8_t *wp, const float *x, float *y,
                        const QArgs &a, hipStream_t s)
{
    if (qt == kQ8_0) return launch_type<kQ8_0>(M, epi, p, wp, x, y, a, s);
    if (qt == kQ4_K) return launch_type<kQ4_K>(M, epi, p, wp, x, y, a, s);
    if (qt == kQ6_K) return launch_type<kQ6_K>(M, epi, p, wp, x, y, a, s);
    return launch_type<kQ4_0>(M, epi, p, wp, x, y, a, s);
}

hipError_t launch_rmsnorm(const float *x, const float *gamma, float eps, float *out, int64_t K, hipStream_t s)
{
    launch(rmsnorm_kernel, dim3(1), dim3(1024), 0u, s, x, gamma, eps, out, K);
    return hipGetLastError();
}

hipError_t launch_f16(const F16Plan &p, const uint16_t *w, const float *x, float *y, int64_t N, int64_t K,
                      hipStream_t s)
{
    const dim3 grid((unsigned)p.grid), block(p.waves * 64);
    auto go = [&](auto kern) { launch(kern, grid, block, 0u, s, w, x, y, N, K); };
    if (p.cpl > 0) {
        // split-K row form: one row per workgroup, every chunk of the row covered
        if (!p.vec || p.grid != N || p.waves < 1 || p.waves > 16 ||
            (K / 8) > (int64_t)p.waves * 64 * p.cpl || (K / 8) <= (int64_t)(p.waves - 1) * 64 * p.cpl)
            return hipErrorInvalidConfiguration;
        switch (p.cpl) {
        case 1: go(gemv_f16_wsplit_kernel<1>); break;
        case 2: go(gemv_f16_wsplit_kernel<2>); break;
        case 4: go(gemv_f16_wsplit_kernel<4>); break;
        default: return hipErrorInvalidConfiguration;
        }
        return hipGetLastError();
    }
    if (p.L > 0) {
        // row form: K = 512 L, x staged in K * 4 bytes of LDS (at most 32 KiB)
        if (!p.vec || p.L > kF16RowMaxL || K != 512 * (int64_t)p.L || (p.waves != 2 && p.waves != 4 && p.waves != 8))
            return hipErrorInvalidConfiguration;
        auto row = [&](auto kern) { launch(kern, grid, block, (uint32_t)(K * 4), s, w, x, y, N, K); };
        auto rows = [&](auto lc) {
            constexpr int Lc = decltype(lc)::value;
            switch (p.waves) {
            case 4: row(gemv_f16_row_kernel<Lc, 4>); break;
            case 8: row(gemv_f16_row_kernel<Lc, 8>); break;
            default: row(gemv_f16_row_kernel<Lc, 2>); break;
            }
        };
        switch (p.L) {
        case 1: rows(std::integral_constant<int, 1>{}); break;
        case 2: rows(std::integral_constant<int, 2>{}); break;
        case 3: rows(std::integral_constant<int, 3>{}); break;
        case 4: rows(std::integral_constant<int, 4>{}); break;
        case 5: rows(std::integral_constant<int, 5>{}); break;
        case 6: rows(std::integral_constant<int, 6>{}); break;
        case 7: rows(std::integral_constant<int, 7>{}); break;
        case 8: rows(std::integral_constant<int, 8>{}); break;
        case 9: rows(std::integral_constant<int, 9>{}); break;
        case 10: rows(std::integral_constant<int, 10>{}); break;
        case 11: rows(std::integral_constant<int, 11>{}); break;
        case 12: rows(std::integral_constant<int, 12>{}); break;
        case 13: rows(std::integral_constant<int, 13>{}); break;
        case 14: rows(std::integral_constant<int, 14>{}); break;
        case 15: rows(std::integral_constant<int, 15>{}); break;
        default: rows(std::integral_constant<int, 16>{}); break;
        }
        return hipGetLastError();
    }
    if (p.vec) {
        switch (p.R) {
        case 1: go(gemv_f16_kernel<1, true>); break;
        case 2: go(gemv_f16_kernel<2, true>); break;
        default: go(gemv_f16_kernel<4, true>); break;
        }
    } else {
        switch (p.R) {
        case 1: go(gemv_f16_kernel<1, false>); break;
        case 2: go(gemv_f16_kernel<2, false>); break;
        default: go(gemv_f16_kernel<4, false>); break;
        }
    }
    return hipGetLastError();
}

hipError_t launch_pack(const Geometry &g, const uint8_t *canon, const uint8_t *canon_up, uint8_t *packed, int mode,
                       int64_t row0, int64_t nrows, int64_t rows_to_write, bool zero_gaps, hipStream_t s)
{
    const int64_t nthreads = rows_to_write * g.KB;
    const int block = 256;
    if (nthreads > 0) {
        const int64_t grid = (nthreads + block - 1) / block;
        hipLaunchKernelGGL(pack_kernel, dim3((unsigned)grid), dim3(block), 0, s, g, canon, canon_up, packed, mode,
                           row0, nrows, nthreads);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (zero_gaps) {
        Gaps gp;
        gp.b[0] = g.n_tiles * g.tile_q;
        gp.b[1] = g.scale_off;
        gp.b[2] = g.scale_off + g.n_tiles * g.tile_s;
        gp.b[3] = g.sup_off;
        gp.b[4] = g.sup_off + g.n_tiles * g.tile_u;
        gp.b[5] = g.total;
        // each gap is under 256 bytes (plane alignment)
        if (gp.b[1] > gp.b[0] || gp.b[3] > gp.b[2] || gp.b[5] > gp.b[4]) {
            hipLaunchKernelGGL(zero_gaps_kernel, dim3(1), dim3(256), 0, s, packed, gp);
            return hipGetLastError();
        }
    }
    return hipSuccess;
}

}  // namespace qgk
