// qgemm_kernels.hip -- small-M GEMM over the packed Q8_0 / Q4_0 weights on the
// matrix cores (v_mfma_f32_16x16x32_f16), for prefill chunks of M activation rows.
//
//   Y[m][n] = sum_k W[n][k] X[m][k] = sum_b d[n][b] * S[n][b][m],
//   S[n][b][m] = sum_{e<32} v[n][32b+e] * X[m][32b+e]        (one block b)
//
// One MFMA computes S for 16 weight rows x 16 activation rows and one block:
// A = the 16 rows' quants as fp16 (exact: |v| <= 128), B = the block's
// activations. The activations go to the matrix cores as two fp16 parts,
// x*2^e = hi + lo (hi = fp16(x*2^e), lo = fp16(x*2^e - hi)), with one power of
// two 2^e per activation row chosen so that the row's largest |x| lands in
// [2^14, 2^15): hi + lo keeps 22 significant bits, the products q*hi and q*lo
// are exact in the fp32 accumulator, and the row's result is multiplied by
// 2^-e at the end (exact). The block scale is applied on the VALU,
// acc = fma(d, S, acc), per block; blocks are summed per 1024-weight segment,
// then the segment sums in order. The longest rounding chain per output is
// the MFMA's 64 products + 32 blocks + the segments, within the 1e-5 relative
// bound of the product's magnitude.
//
// Operand layouts (v_mfma_f32_16x16x32_f16, measured on gfx950):
//   A: lane l holds A[l % 16][8 (l / 16) + j], j = 0..7
//   B: lane l holds B[8 (l / 16) + j][l % 16]
//   D: lane l holds D[4 (l / 16) + r][l % 16], r = 0..3
// Only the pairing of A's and B's K indices matters, so within a block the
// K order follows the packed weights: each lane of a wavefront loads one whole
// 16-byte packed unit (four K-chunks), and a 4 x 4 transpose across the four
// 16-lane groups (v_permlane32_swap, v_permlane16_swap) hands every lane its
// chunk. Q4_0: chunk c of a block is packed dword c, elements 8c..8c+7. Q8_0:
// chunk c is dword c of the block's first and second 16-byte halves, elements
// 4c..4c+3 and 16+4c..16+4c+3. The split pre-pass writes the activations in
// the same order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dequant.h"
#include "layout.h"
#include "qgemm_kernels.h"

namespace qgk {

using namespace qgl;

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// Activation split: one workgroup per activation row m (rows M..M_pad-1 of
// the last 16-row tile are written as zeros). Writes unscale[m] = 2^-e and the
// fp16 parts in B-operand order: xs[((mt * KB + b) * 2 + h) * 512 + lane * 8 + e]
// with mt = m / 16, lane = 16 c + m % 16, h = 0 (hi) / 1 (lo), where (c, e)
// is the position of the block's element in its lane (see above).
template <int QT>
__global__ void __launch_bounds__(256)
split_x_kernel(const float *__restrict__ X, _Float16 *__restrict__ xs, float *__restrict__ unscale, int64_t M,
               int64_t K)
{
    __shared__ float red[4];
    const int64_t m = blockIdx.x;
    const int tid = threadIdx.x;
    const bool live = m < M;
    const float *xr = X + m * K;
    float mx = 0.0f;
    if (live)
        for (int64_t k = tid; k < K; k += 256) mx = __builtin_fmaxf(mx, __builtin_fabsf(xr[k]));
    // workgroup maximum (max is exact, so the order does not matter)
    for (int o = 32; o >= 1; o >>= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, o));
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    mx = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
    // 2^e with max|x| * 2^e in [2^14, 2^15); 1 for a zero or non-finite maximum
    int e = 0;
    if (mx > 0.0f && mx <= 3.4028234663852886e38f) {
        int E;
        (void)__builtin_frexpf(mx, &E);   // mx = f * 2^E, f in [0.5, 1)
        e = 15 - E;
        e = e < -126 ? -126 : (e > 127 ? 127 : e);
    }
    const float sc = __builtin_ldexpf(1.0f, e);
    if (tid == 0) unscale[m] = __builtin_ldexpf(1.0f, -e);
    const int64_t KB = K / 32;
    const int64_t mt = m >> 4;
    const int mi = (int)(m & 15);
    for (int64_t k = tid; k < K; k += 256) {
        const float v = live ? xr[k] * sc : 0.0f;
        const _Float16 hi = (_Float16)v;
        const _Float16 lo = (_Float16)(v - (float)hi);
        const int64_t b = k >> 5;
        const int p = (int)(k & 31);
        int c, el;
        if (QT == kQ4_0) {
            c = p >> 3;
            el = p & 7;
        } else {
            c = (p & 15) >> 2;
            el = (p & 3) + (p >= 16 ? 4 : 0);
        }
        const int64_t at = ((mt * KB + b) * 2) * 512 + (int64_t)(c * 16 + mi) * 8 + el;
        xs[at] = hi;
        xs[at + 512] = lo;
    }
}

// 4 x 4 transpose of (16-lane group, register): afterwards register r of lane
// (i, g) holds what register g of lane (i, r) held (i = lane % 16, g = lane / 16).
__device__ __forceinline__ void group_transpose(uint32_t (&v)[4])
{
    auto a = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
    auto b = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
    auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
    auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    v[0] = c[0];
    v[1] = c[1];
    v[2] = d[0];
    v[3] = d[1];
}

// ---------------------------------------------------------------------------
// The GEMM. A workgroup of G wavefronts owns 16 G weight rows (wavefront w:
// row tiles 2 (blockIdx.x G + w) and + 1, i.e. 16 rows) and MT 16-row tiles of
// activations starting at tile a.mt0. Per 1024-weight segment the workgroup
// copies the segment's split activations into LDS (MT x 64 KiB), then every
// wavefront walks the segment's blocks in groups of 4 (Q4_0) or 2 (Q8_0): one
// 16-byte load per lane, the group transpose, the dequant, two MFMAs (hi, lo)
// per activation tile and block, and acc = fma(d, S, acc).
template <int QT, int MT>
__global__ void __launch_bounds__(512)
qgemm_kernel(const uint8_t *__restrict__ wp, const _Float16 *__restrict__ xs, const float *__restrict__ unscale,
             float *__restrict__ Y, GemmArgs a)
{
    constexpr int NH = (QT == kQ8_0) ? 2 : 1;
    constexpr int BPG = (QT == kQ8_0) ? 2 : 4;   // blocks per load group
    extern __shared__ u32x4 lx[];                // [mt][block in segment][h][lane] x 16 B

    const Geometry &g = a.geo;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int G = blockDim.x >> 6;
    const int i = lane & 15, c = lane >> 4;
    const int64_t t_first = ((int64_t)blockIdx.x * G + wave) * 2;
    const int64_t t_last = g.n_tiles - 1;
    // A operand: this lane loads the units of weight row t_first*8 + i
    const int64_t tA = t_first + (i >> 3) < t_last ? t_first + (i >> 3) : t_last;
    const int slotA = (i & 7) >> 2, browA = i & 3;
    // D layout: this lane's outputs are rows t_first*8 + 4c + r, r = 0..3
    const int64_t tD = t_first + (c >> 1) < t_last ? t_first + (c >> 1) : t_last;
    const int slotD = c & 1;
    const Consts k = make_consts();
    constexpr int64_t seg_q = (int64_t)kTileRows * kSegBlocks * NH * kUnit;
    constexpr int64_t seg_s = (int64_t)kTileRows * kSegBlocks * 2;

    f32x4 tot[MT], seg[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) tot[mt] = seg[mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    for (int64_t s = 0; s < g.nseg; ++s) {
        const int nb = (int)seg_blocks(g, s);
        __syncthreads();   // the previous segment's activations are no longer read
        {
            const uint32_t per_mt = (uint32_t)nb * 128;   // 16-byte chunks per activation tile
            for (uint32_t u = threadIdx.x; u < MT * per_mt; u += blockDim.x) {
                const uint32_t mt = u / per_mt, r = u - mt * per_mt;
                const u32x4 *src = (const u32x4 *)xs + ((a.mt0 + mt) * g.KB + s * kSegBlocks) * 128 + r;
                lx[mt * (kSegBlocks * 128) + r] = *src;
            }
        }
        __syncthreads();
        const uint8_t *qa = wp + tA * g.tile_q + s * seg_q;
        const uint8_t *sd = wp + g.scale_off + tD * g.tile_s + s * seg_s;
        const int ngroups = (nb + BPG - 1) / BPG;
        for (int q = 0; q < ngroups; ++q) {
            int jb, hh;
            if (QT == kQ4_0) {
                jb = 4 * q + c;
                hh = 0;
            } else {
                jb = 2 * q + (c >> 1);
                hh = c & 1;
            }
            jb = jb < nb ? jb : nb - 1;   // past a ragged segment's end: a valid unit, never used
            const u32x4 raw = __builtin_nontemporal_load(
                (const u32x4 *)(qa + (int64_t)(((browA * NH + hh) * kSlots + slotA) * nb + jb) * kUnit));
            uint32_t v[4] = {raw.x, raw.y, raw.z, raw.w};
            group_transpose(v);
#pragma unroll
            for (int bb = 0; bb < BPG; ++bb) {
                const int j = BPG * q + bb;
                if (j >= nb) break;   // wave-uniform
                h8 A;
                if (QT == kQ4_0) {
                    h2 p[4];
                    q4_pairs(v[bb], k, p);
                    A = h8{p[0].x, p[0].y, p[1].x, p[1].y, p[2].x, p[2].y, p[3].x, p[3].y};
                } else {
                    h2 p0[2], p1[2];
                    q8_pairs(v[2 * bb], p0);
                    q8_pairs(v[2 * bb + 1], p1);
                    A = h8{p0[0].x, p0[0].y, p0[1].x, p0[1].y, p1[0].x, p1[0].y, p1[1].x, p1[1].y};
                }
                const u32x2 dd = *(const u32x2 *)(sd + (int64_t)(slotD * nb + j) * (kRowsPerLane * 2));
                const h2 d01 = as_h2(dd.x), d23 = as_h2(dd.y);
                const float d[4] = {(float)d01.x, (float)d01.y, (float)d23.x, (float)d23.y};
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const u32x4 bh = lx[(mt * kSegBlocks + j) * 128 + lane];
                    const u32x4 bl = lx[(mt * kSegBlocks + j) * 128 + 64 + lane];
                    f32x4 S = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, __builtin_bit_cast(h8, bh),
                                                                     f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                    S = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, __builtin_bit_cast(h8, bl), S, 0, 0, 0);
                    seg[mt].x = __builtin_fmaf(d[0], S.x, seg[mt].x);
                    seg[mt].y = __builtin_fmaf(d[1], S.y, seg[mt].y);
                    seg[mt].z = __builtin_fmaf(d[2], S.z, seg[mt].z);
                    seg[mt].w = __builtin_fmaf(d[3], S.w, seg[mt].w);
                }
            }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            tot[mt].x += seg[mt].x;
            tot[mt].y += seg[mt].y;
            tot[mt].z += seg[mt].z;
            tot[mt].w += seg[mt].w;
            seg[mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    }

    const int64_t n0 = t_first * kTileRows + 4 * c;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int64_t m = (a.mt0 + mt) * 16 + i;
        if (m >= a.M) continue;
        const float us = unscale[m];
        float *yr = Y + m * a.y_stride;
        const float o[4] = {tot[mt].x, tot[mt].y, tot[mt].z, tot[mt].w};
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (n0 + r < a.N) yr[n0 + r] = o[r] * us;
    }
}

// ---------------------------------------------------------------------------
// host side

hipError_t launch_split_x(int qt, const float *X, _Float16 *xs, float *unscale, int64_t M, int64_t M_pad, int64_t K,
                          hipStream_t s)
{
    if (qt == kQ8_0)
        hipLaunchKernelGGL(split_x_kernel<kQ8_0>, dim3((unsigned)M_pad), dim3(256), 0, s, X, xs, unscale, M, K);
    else
        hipLaunchKernelGGL(split_x_kernel<kQ4_0>, dim3((unsigned)M_pad), dim3(256), 0, s, X, xs, unscale, M, K);
    return hipGetLastError();
}

template <int QT, int MT>
static hipError_t launch_one(const uint8_t *wp, const _Float16 *xs, const float *unscale, float *Y,
                             const GemmArgs &a, int64_t grid, int block, hipStream_t s)
{
    auto kern = qgemm_kernel<QT, MT>;
    const size_t lds = (size_t)MT * kSegBlocks * 128 * 16;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    launch_timed(kern, dim3((unsigned)grid), dim3(block), (uint32_t)lds, s, wp, xs, unscale, Y, a);
    return hipGetLastError();
}

hipError_t launch_qgemm(int qt, int MT, const uint8_t *wp, const _Float16 *xs, const float *unscale, float *Y,
                        const GemmArgs &a, int64_t grid, int block, hipStream_t s)
{
    if (qt == kQ8_0)
        return MT == 1 ? launch_one<kQ8_0, 1>(wp, xs, unscale, Y, a, grid, block, s)
                       : launch_one<kQ8_0, 2>(wp, xs, unscale, Y, a, grid, block, s);
    return MT == 1 ? launch_one<kQ4_0, 1>(wp, xs, unscale, Y, a, grid, block, s)
                   : launch_one<kQ4_0, 2>(wp, xs, unscale, Y, a, grid, block, s);
}

}  // namespace qgk
