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
#include "qgemv_kernels.h"

namespace qgk {

using namespace qgl;

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// Activation split: one workgroup per activation row m (rows M..M_pad-1 of
// the last 16-row tile are written as zeros). Writes unscale[m] = 2^-e and the
// fp16 parts in B-operand order: xs[((mt * KB + b) * 2 + h) * 512 + lane * 8 + e]
// with mt = m / 16, lane = 16 c + m % 16, h = 0 (hi) / 1 (lo), where (c, e)
// is the position of the block's element in its lane (see above).
constexpr int kSplitThreads = 1024;   // one workgroup per activation row

template <int QT>
__global__ void __launch_bounds__(kSplitThreads)
split_x_kernel(const float *__restrict__ X, _Float16 *__restrict__ xs, float *__restrict__ unscale, int64_t M,
               int64_t K)
{
    __shared__ float red[kSplitThreads / 64];
    const int64_t m = blockIdx.x;
    const int tid = threadIdx.x;
    const bool live = m < M;
    const float *xr = X + m * K;
    float mx = 0.0f;
    if (live)
        for (int64_t k = tid; k < K; k += kSplitThreads) mx = __builtin_fmaxf(mx, __builtin_fabsf(xr[k]));
    // workgroup maximum (max is exact, so the order does not matter)
    for (int o = 32; o >= 1; o >>= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, o));
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    mx = red[0];
    for (int w = 1; w < kSplitThreads / 64; ++w) mx = __builtin_fmaxf(mx, red[w]);
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
    for (int64_t k = tid; k < K; k += kSplitThreads) {
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
// The GEMM. A workgroup of G wavefronts owns 16 RG G weight rows: wavefront w
// covers RG groups of 16 rows (row tiles 2 RG (blockIdx.x G + w) + 2 rg and
// + 1 for group rg), for the MT 16-row activation tiles [a.mt0, a.mt0 + MT).
// K is walked in chunks of CB = gemm_chunk(MT) blocks, staged into two LDS buffers in
// turn: the chunk's split activations (MT x 2 KiB per block) and the scales of
// the workgroup's rows are copied with LDS-direct loads (global_load_lds, no
// registers) one chunk ahead, so the copy of chunk c + 1 runs under the
// matrix-core work of chunk c; one vmcnt wait and one barrier per chunk. The
// weights of a chunk are loaded one chunk ahead too: load groups of 4 (Q4_0) or
// 2 (Q8_0) blocks, one 16-byte load per lane and row group. Each wavefront
// walks a chunk's groups: the group transpose, the dequant, and per block and
// activation tile two MFMAs (hi, lo) per row group, each B operand read once
// from LDS and used by the RG row groups; then acc = fma(d, S, acc).
// Block sums are added per segment of 32 blocks and the segment sums in order.
// With a.ksplit > 1, workgroup column blockIdx.y takes one range of segments
// and writes its sums to a.part; launch_ksum then adds the ranges in order.
template <int QT, int MT, int RG>
__global__ void __launch_bounds__(256)
qgemm_kernel(const uint8_t *__restrict__ wp, const _Float16 *__restrict__ xs, const float *__restrict__ unscale,
             float *__restrict__ Y, GemmArgs a)
{
    constexpr int NH = (QT == kQ8_0) ? 2 : 1;
    constexpr int BPG = (QT == kQ8_0) ? 2 : 4;   // blocks per load group
    constexpr int CB = gemm_chunk(MT);           // blocks per staged chunk (a multiple of BPG)
    extern __shared__ u32x4 lds[];
    u32x4 *lx = lds;   // 2 buffers x [mt][CB][h][64 lanes] x 16 B
    // 2 buffers x [tile of the workgroup][slot][CB] x 4 fp16, in 4-byte words, padded to whole wavefront copies
    uint32_t *lsc_base = (uint32_t *)(lds + 2 * MT * CB * 128);

    const Geometry &g = a.geo;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: its arithmetic stays scalar
    const int G = blockDim.x >> 6;
    const int i = lane & 15, c = lane >> 4;
    const int64_t wg_tile0 = (int64_t)blockIdx.x * G * 2 * RG;   // first row tile of the workgroup
    const int wg_tiles = G * 2 * RG;
    const int lsc_words = gemm_scale_words(wg_tiles, CB);
    const int64_t t_first = wg_tile0 + (int64_t)wave * 2 * RG;    // first row tile of this wavefront
    const int64_t t_last = g.n_tiles - 1;
    const int slotA = (i & 7) >> 2, browA = i & 3;
    int64_t qoffA[RG];   // byte offset of this lane's A row in its tile (row group rg)
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        int64_t t = t_first + 2 * rg + (i >> 3);
        t = t < t_last ? t : t_last;
        qoffA[rg] = t * g.tile_q;
    }
    const Consts k = make_consts();
    constexpr int64_t seg_q = (int64_t)kTileRows * kSegBlocks * NH * kUnit;
    constexpr int64_t seg_s = (int64_t)kTileRows * kSegBlocks * 2;

    f32x4 tot[RG][MT], seg[RG][MT];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) tot[rg][mt] = seg[rg][mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // Load group q of segment s (nb blocks): lane (i, c) loads the 16-byte unit
    // of row i of each row group for block 4q + c (Q4_0) or block 2q + c/2, half
    // c%2 (Q8_0); past a ragged segment's end it loads a valid unit, never used.
    auto load_group = [&](u32x4 (&raw)[RG], int64_t s, int nb, int q) {
        int jb = (QT == kQ4_0) ? 4 * q + c : 2 * q + (c >> 1);
        const int hh = (QT == kQ4_0) ? 0 : (c & 1);
        jb = jb < nb ? jb : nb - 1;
        const int64_t off = s * seg_q + (int64_t)(((browA * NH + hh) * kSlots + slotA) * nb + jb) * kUnit;
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) raw[rg] = __builtin_nontemporal_load((const u32x4 *)(wp + qoffA[rg] + off));
    };

    const int64_t KB = g.KB;
    const int64_t ky = blockIdx.y;
    const int64_t s_begin = g.nseg * ky / a.ksplit, s_end = g.nseg * (ky + 1) / a.ksplit;
    // The K range as a flat sequence of chunks of CB blocks: every segment but the
    // matrix's last holds 32 / CB of them.
    constexpr int CPS = kSegBlocks / CB;
    struct ChunkPos {
        int64_t s;
        int j0, nb, nbc;
    };
    auto chunk_at = [&](int64_t c) {
        ChunkPos p;
        p.s = s_begin + c / CPS;
        p.j0 = (int)(c % CPS) * CB;
        p.nb = (int)seg_blocks(g, p.s);
        p.nbc = p.nb - p.j0 < CB ? p.nb - p.j0 : CB;
        return p;
    };
    const int64_t n_chunks =
        s_end > s_begin ? (s_end - s_begin - 1) * CPS + (seg_blocks(g, s_end - 1) + CB - 1) / CB : 0;

    // Stage chunk c into buffer `buf` with LDS-direct loads (no registers; they
    // complete under vmcnt): wavefront w copies 1 KiB pieces w, w + G, ... of the
    // activations (MT tiles x nbc blocks x 2 KiB, each tile's run contiguous in
    // the workspace and in LDS), then its share of the scales as 4-byte words
    // (run (tile, slot) = CB entries of 8 B; words past the chunk's blocks or
    // past the runs re-read a valid word and land in the padding).
    auto stage = [&](int buf, int64_t c) {
        const ChunkPos p = chunk_at(c);
        u32x4 *lxd = lx + buf * (MT * CB * 128);
        const int nkib = MT * p.nbc * 2;
        for (int q = wave; q < nkib; q += G) {
            // a full chunk's run per tile is 2 CB pieces (a power of two)
            const int mt = MT == 1 ? 0 : (p.nbc == CB ? q / (2 * CB) : q / (p.nbc * 2));
            const int r = q - mt * (p.nbc * 2);
            const u32x4 *src =
                (const u32x4 *)xs + ((a.mt0 + mt) * KB + p.s * kSegBlocks + p.j0) * 128 + r * 64 + lane;
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                             (__attribute__((address_space(3))) void *)(lxd + mt * CB * 128 + r * 64),
                                             16, 0, 0);
        }
        uint32_t *lsd = (uint32_t *)(lsc_base + buf * lsc_words);
        const int nwords = wg_tiles * 2 * CB * 2;
        // the workgroup's first tile and this segment (uniform), then per lane its
        // tile (clamped to the matrix's last) and its place in the segment
        const uint8_t *sbase = wp + g.scale_off + wg_tile0 * g.tile_s + p.s * seg_s;
        const int tl_last = (int)(t_last - wg_tile0);
        for (int q = wave; q * 64 < lsc_words; q += G) {
            int wi = q * 64 + lane;
            wi = wi < nwords ? wi : 0;
            const int run = wi / (2 * CB), within = wi - run * (2 * CB);
            int tl = run >> 1;
            tl = tl < tl_last ? tl : tl_last;
            const int sl = run & 1;
            int jj = within >> 1;
            jj = jj < p.nbc ? jj : p.nbc - 1;
            const uint8_t *src = sbase + (uint64_t)(uint32_t)tl * (uint64_t)g.tile_s +
                                 (uint32_t)((sl * p.nb + p.j0 + jj) * (kRowsPerLane * 2) + (within & 1) * 4);
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                             (__attribute__((address_space(3))) void *)(lsd + q * 64), 4, 0, 0);
        }
    };

    // All NG load groups of a chunk, loaded one chunk ahead (a ragged last chunk's
    // extra groups load valid units that are never used).
    constexpr int NG = CB / BPG;
    auto load_chunk = [&](u32x4 (&raw)[NG][RG], int64_t c) {
        const ChunkPos p = chunk_at(c);
#pragma unroll
        for (int q = 0; q < NG; ++q) load_group(raw[q], p.s, p.nb, p.j0 / BPG + q);
    };
    // Two register sets take turns: chunk ci computes from one while chunk
    // ci + 1's weights load into the other (the loop is unrolled by two).
    u32x4 rawA[NG][RG], rawB[NG][RG];
    if (n_chunks > 0) {
        stage(0, 0);
        load_chunk(rawA, 0);
    }
    auto chunk_step = [&](u32x4 (&cur)[NG][RG], u32x4 (&nxt)[NG][RG], int64_t ci) {
        // Everything this wavefront issued is chunk ci's: its copies into buffer
        // ci & 1 and its weight groups, both issued one chunk earlier. After the
        // barrier every wavefront's copies are in LDS and every wavefront is past
        // chunk ci - 1, whose buffer the next copies take. Nothing issued after a
        // load comes between that load and its use, so no wait below covers the
        // next chunk's loads.
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        uint32_t v[NG][RG][4];
#pragma unroll
        for (int q = 0; q < NG; ++q)
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
                v[q][rg][0] = cur[q][rg].x;
                v[q][rg][1] = cur[q][rg].y;
                v[q][rg][2] = cur[q][rg].z;
                v[q][rg][3] = cur[q][rg].w;
            }
        __syncthreads();
        if (ci + 1 < n_chunks) {
            stage((int)((ci + 1) & 1), ci + 1);
            load_chunk(nxt, ci + 1);
        }
        const ChunkPos cp = chunk_at(ci);
        const int nb = cp.nb, nbc = cp.nbc, j0 = cp.j0;
        const u32x4 *lxb = lx + (ci & 1) * (MT * CB * 128);
        const u32x2 *lscb = (const u32x2 *)(lsc_base + (ci & 1) * lsc_words);
#pragma unroll
        for (int qq = 0; qq < NG; ++qq) {
            if (qq * BPG >= nbc) break;   // wave-uniform
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) group_transpose(v[qq][rg]);
#pragma unroll
            for (int bb = 0; bb < BPG; ++bb) {
                const int jj = qq * BPG + bb;   // block within the chunk
                if (jj >= nbc) break;           // wave-uniform
                h8 A[RG];
                h2 d01[RG], d23[RG];
#pragma unroll
                for (int rg = 0; rg < RG; ++rg) {
                    if (QT == kQ4_0) {
                        h2 p[4];
                        q4_pairs(v[qq][rg][bb], k, p);
                        A[rg] = h8{p[0].x, p[0].y, p[1].x, p[1].y, p[2].x, p[2].y, p[3].x, p[3].y};
                    } else {
                        h2 p0[2], p1[2];
                        q8_pairs(v[qq][rg][2 * bb], p0);
                        q8_pairs(v[qq][rg][2 * bb + 1], p1);
                        A[rg] = h8{p0[0].x, p0[0].y, p0[1].x, p0[1].y, p1[0].x, p1[0].y, p1[1].x, p1[1].y};
                    }
                    // rows 4c + r of row group rg: tile (wave*RG + rg)*2 + c/2 of the workgroup, slot c%2
                    const u32x2 dd = lscb[(((wave * RG + rg) * 2 + (c >> 1)) * 2 + (c & 1)) * CB + jj];
                    d01[rg] = as_h2(dd.x);
                    d23[rg] = as_h2(dd.y);
                }
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const h8 bh = __builtin_bit_cast(h8, lxb[(mt * CB + jj) * 128 + lane]);
                    const h8 bl = __builtin_bit_cast(h8, lxb[(mt * CB + jj) * 128 + 64 + lane]);
                    f32x4 S[RG];
#pragma unroll
                    for (int rg = 0; rg < RG; ++rg)
                        S[rg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[rg], bh, f32x4{0.0f, 0.0f, 0.0f, 0.0f},
                                                                       0, 0, 0);
#pragma unroll
                    for (int rg = 0; rg < RG; ++rg)
                        S[rg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[rg], bl, S[rg], 0, 0, 0);
#pragma unroll
                    for (int rg = 0; rg < RG; ++rg) {
                        f32x4 &acc = seg[rg][mt];
                        acc.x = __builtin_fmaf((float)d01[rg].x, S[rg].x, acc.x);
                        acc.y = __builtin_fmaf((float)d01[rg].y, S[rg].y, acc.y);
                        acc.z = __builtin_fmaf((float)d23[rg].x, S[rg].z, acc.z);
                        acc.w = __builtin_fmaf((float)d23[rg].y, S[rg].w, acc.w);
                    }
                }
            }
        }
        if (j0 + nbc == nb) {   // the segment's last chunk: add its sum, in segment order
#pragma unroll
            for (int rg = 0; rg < RG; ++rg)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    tot[rg][mt].x += seg[rg][mt].x;
                    tot[rg][mt].y += seg[rg][mt].y;
                    tot[rg][mt].z += seg[rg][mt].z;
                    tot[rg][mt].w += seg[rg][mt].w;
                    seg[rg][mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                }
        }
    };
    int64_t ci = 0;
    for (; ci + 1 < n_chunks; ci += 2) {
        chunk_step(rawA, rawB, ci);
        chunk_step(rawB, rawA, ci + 1);
    }
    if (ci < n_chunks) chunk_step(rawA, rawB, ci);

#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int64_t m = (a.mt0 + mt) * 16 + i;
        if (m >= a.M) continue;
        const float us = unscale[m];
        // with K ranges, each range's sum goes to its own partial buffer (the
        // unscale is exact, so it may be applied before the ranges are added)
        float *yr = (a.ksplit > 1 ? a.part + (ky * a.M + m) * a.N : Y + m * a.y_stride);
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            const int64_t n0 = (t_first + 2 * rg) * kTileRows + 4 * c;
            const float o[4] = {tot[rg][mt].x, tot[rg][mt].y, tot[rg][mt].z, tot[rg][mt].w};
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (n0 + r < a.N) yr[n0 + r] = o[r] * us;
        }
    }
}

// Sum of the K-range partials in range order: one thread per output.
__global__ void __launch_bounds__(256)
ksum_kernel(const float *__restrict__ part, float *__restrict__ Y, int64_t ksplit, int64_t MN)
{
    const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (o >= MN) return;
    float v = part[o];
    for (int64_t r = 1; r < ksplit; ++r) v += part[r * MN + o];
    Y[o] = v;
}

// ---------------------------------------------------------------------------
// host side

hipError_t launch_ksum(const float *part, float *Y, int64_t ksplit, int64_t M, int64_t N, hipStream_t s)
{
    const int64_t MN = M * N;
    hipLaunchKernelGGL(ksum_kernel, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, s, part, Y, ksplit, MN);
    return hipGetLastError();
}

hipError_t launch_split_x(int qt, const float *X, _Float16 *xs, float *unscale, int64_t M, int64_t M_pad, int64_t K,
                          hipStream_t s)
{
    if (qt == kQ8_0)
        hipLaunchKernelGGL(split_x_kernel<kQ8_0>, dim3((unsigned)M_pad), dim3(kSplitThreads), 0, s, X, xs, unscale,
                           M, K);
    else
        hipLaunchKernelGGL(split_x_kernel<kQ4_0>, dim3((unsigned)M_pad), dim3(kSplitThreads), 0, s, X, xs, unscale,
                           M, K);
    return hipGetLastError();
}

template <int QT, int MT, int RG>
static hipError_t launch_one(const uint8_t *wp, const _Float16 *xs, const float *unscale, float *Y,
                             const GemmArgs &a, int G, hipStream_t s)
{
    auto kern = qgemm_kernel<QT, MT, RG>;
    const int64_t grid = (a.geo.n_tiles + 2 * RG * G - 1) / (2 * RG * G);
    const dim3 grid3((unsigned)grid, (unsigned)a.ksplit);
    const size_t lds = gemm_lds_bytes(MT, G * 2 * RG);
    static std::atomic<int> lds_set[16];
    hipError_t e = ensure_lds_limit((const void *)kern, lds, lds_set);
    if (e != hipSuccess) return e;
    launch_timed(kern, grid3, dim3(64 * G), (uint32_t)lds, s, wp, xs, unscale, Y, a);
    return hipGetLastError();
}

template <int QT, int MT>
static hipError_t launch_rg(const uint8_t *wp, const _Float16 *xs, const float *unscale, float *Y, const GemmArgs &a,
                            int RG, int G, hipStream_t s)
{
    switch (RG) {
    case 1: return launch_one<QT, MT, 1>(wp, xs, unscale, Y, a, G, s);
    case 2: return launch_one<QT, MT, 2>(wp, xs, unscale, Y, a, G, s);
    default: return launch_one<QT, MT, 4>(wp, xs, unscale, Y, a, G, s);
    }
}

template <int QT>
static hipError_t launch_mt(const uint8_t *wp, const _Float16 *xs, const float *unscale, float *Y, const GemmArgs &a,
                            int MT, int RG, int G, hipStream_t s)
{
    switch (MT) {
    case 1: return launch_rg<QT, 1>(wp, xs, unscale, Y, a, RG, G, s);
    case 2: return launch_rg<QT, 2>(wp, xs, unscale, Y, a, RG, G, s);
    case 3: return launch_one<QT, 3, 1>(wp, xs, unscale, Y, a, G, s);   // the tail pass of a 4-tile plan
    default:
        // four activation tiles: one or two row groups per wavefront (registers)
        return RG == 1 ? launch_one<QT, 4, 1>(wp, xs, unscale, Y, a, G, s)
                       : launch_one<QT, 4, 2>(wp, xs, unscale, Y, a, G, s);
    }
}

hipError_t launch_qgemm(int qt, int MT, int RG, int G, const uint8_t *wp, const _Float16 *xs, const float *unscale,
                        float *Y, const GemmArgs &a, hipStream_t s)
{
    if (qt == kQ8_0) return launch_mt<kQ8_0>(wp, xs, unscale, Y, a, MT, RG, G, s);
    return launch_mt<kQ4_0>(wp, xs, unscale, Y, a, MT, RG, G, s);
}

}  // namespace qgk
