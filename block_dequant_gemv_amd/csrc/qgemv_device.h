// qgemv_device.h -- the quantised GEMV kernels of libqgemv (gfx950) and their
// launch templates. Each (qtype, activation rows) pair is instantiated in a
// translation unit of its own (qgemv_inst.hip), so they build in parallel.
//
// Quantised GEMV (Q8_0 / Q4_0), its fused gate|up SiLU epilogue and the
// multi-row verify all come from ONE kernel template, so that a row's
// floating-point operations are the same whatever M is:
//
//   per lane, per block of 32 weights, per activation row m:
//     s = 0;  s = fma(v_e, x_e, s) for e = 0..31      (v_e = q or nibble-8, exact in fp16)
//     acc = fma(d, s, acc)                             (d = the block's fp16 scale)
//   acc of the 32 lanes that share a row: one fixed tree of pairings
//     (permlane16 swap and DPP; tile_sums)
//   split-K wavefronts (if any): partials added in wavefront order in LDS
//
// Nothing in that sequence depends on M, on which wavefront or workgroup
// handles the row, or on how many tiles a wavefront walks, so row m of the
// verify output equals the M=1 output bit for bit. The build uses
// -ffp-contract=off and every multiply-add is an explicit fma.
//
// Memory: each lane loads 16-byte units of the packed planes (layout.h); a
// wavefront load instruction reads 1 KiB contiguous. Activations are staged
// once per workgroup into LDS in a lane-swizzled order (chunk c of block j at
// float4 slot c*32 + j), so the 32 lanes of a row read consecutive 16-byte
// LDS words (no bank conflicts) and the two row slots of a wavefront read the
// same words (broadcast).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "dequant.h"
#include "layout.h"
#include "qgemv_kernels.h"

namespace qgk {

using namespace qgl;

// Sum over the 32 lanes of one wavefront half (lanes 0-31 and 32-63 separately).
// Butterfly: xor 1, xor 2 (quad_perm), mirror within 8, mirror within 16 (DPP),
// xor 16 (ds_swizzle). Every lane of the half ends with the same bits. Used for
// single values (the RMSNorm sum of squares, the fp16 GEMV); the quantised row
// tiles use tile_sums below.
__device__ __forceinline__ float half_wave_sum(float v)
{
    v += as_f(__builtin_amdgcn_update_dpp(0, as_i(v), 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
    v += as_f(__builtin_amdgcn_update_dpp(0, as_i(v), 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
    v += as_f(__builtin_amdgcn_update_dpp(0, as_i(v), 0x141, 0xF, 0xF, false)); // row_half_mirror
    v += as_f(__builtin_amdgcn_update_dpp(0, as_i(v), 0x140, 0xF, 0xF, false)); // row_mirror
    v += as_f(__builtin_amdgcn_ds_swizzle(as_i(v), 0x401F));                     // lane ^ 16 within 32
    return v;
}

__device__ __forceinline__ float silu_mul(float g, float u)
{
    return g / (1.0f + expf(-g)) * u;
}

// ---------------------------------------------------------------------------
// The sums of a row tile: each of the V = 4 M values a lane holds (activation
// row m, weight row b of its slot; value index i = 4 m + b) is added over the
// 32 lanes of the slot (lanes slot*32 + j, j = 0..31) through one fixed tree of
// five pairing levels, in this order:
//   L1 j ^ 16, L2 j ^ 8, L3 j ^ 7 (mirror within groups of 8), L4 j ^ 1, L5 j ^ 2.
// Each level adds the partial sums of two disjoint halves of the final lane set
// (lane sets {j, j^16}, then j ^ {0, 8, 16, 24}, then j ^ {0, 7, 8, 15, 16, 23,
// 24, 31}, ...). A level is done either as a butterfly (both lanes of a pair
// get every sum: one DPP add per value) or as a reduce-scatter: the two lanes
// split a pair of values, each adding the partner's copy of the value it keeps,
// so later levels have half as many values to add. The additions, and so the
// bits of every sum, are the same either way (a + b == b + a); only which lanes
// end up holding which sums differs. RS levels are reduce-scatter:
//   L1 (v_permlane16_swap, one swap and one add per pair of values), then, for
//   RS >= 2, L2 and for RS = 3 L3 (a select of the kept and the sent value and
//   one DPP add per pair); the rest are butterflies.
// After L1 the lanes with j bit 4 clear hold values i < 2M, the others i + 2M;
// L2 splits each half by j bit 3 and L3 by j bit 2 (tile_sum_index).
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane 7 - l within 8 (l ^ 7)
constexpr int kDppRor8 = 0x128;       // row_ror:8, lane l ^ 8 within 16

template <int CTRL>
__device__ __forceinline__ float dpp_bfly(float v)
{
    return v + as_f(__builtin_amdgcn_update_dpp(0, as_i(v), CTRL, 0xF, 0xF, false));
}

// Lanes with hi clear keep p, the others q; each adds its partner's copy.
template <int CTRL>
__device__ __forceinline__ float dpp_split(float p, float q, bool hi)
{
    const float keep = hi ? q : p, send = hi ? p : q;
    return keep + as_f(__builtin_amdgcn_update_dpp(0, as_i(send), CTRL, 0xF, 0xF, false));
}

// Registers a lane holds after the reduction.
constexpr int tile_sum_regs(int M, int RS) { return RS == 1 ? 2 * M : (RS == 2 ? M : M / 2 + (M & 1)); }

template <int M, int RS>
__device__ __forceinline__ void tile_sums(const float (&acc)[M][kRowsPerLane], float (&out)[tile_sum_regs(M, RS)],
                                          int j)
{
    constexpr int B = kRowsPerLane, H1 = 2 * M;
    static_assert(RS >= 1 && RS <= 3, "one to three reduce-scatter levels");
    float v1[H1];
#pragma unroll
    for (int i = 0; i < H1; ++i) {
        const int i2 = i + H1;
        const auto pr = __builtin_amdgcn_permlane16_swap(as_i(acc[i / B][i % B]), as_i(acc[i2 / B][i2 % B]), false,
                                                         false);
        v1[i] = as_f(pr[0]) + as_f(pr[1]);
    }
    if constexpr (RS == 1) {
#pragma unroll
        for (int i = 0; i < H1; ++i) {
            float v = dpp_bfly<kDppRor8>(v1[i]);
            v = dpp_bfly<kDppHalfMirror>(v);
            v = dpp_bfly<kDppXor1>(v);
            out[i] = dpp_bfly<kDppXor2>(v);
        }
    } else {
        const bool h3 = (j & 8) != 0;
        float v2[M];
#pragma unroll
        for (int i = 0; i < M; ++i) v2[i] = dpp_split<kDppRor8>(v1[i], v1[i + M], h3);
        if constexpr (RS == 2) {
#pragma unroll
            for (int i = 0; i < M; ++i) {
                float v = dpp_bfly<kDppHalfMirror>(v2[i]);
                v = dpp_bfly<kDppXor1>(v);
                out[i] = dpp_bfly<kDppXor2>(v);
            }
        } else {
            constexpr int H3 = M / 2;
            const bool h2 = (j & 4) != 0;
#pragma unroll
            for (int i = 0; i < H3; ++i) out[i] = dpp_split<kDppHalfMirror>(v2[i], v2[i + H3], h2);
            if constexpr (M & 1) out[H3] = dpp_bfly<kDppHalfMirror>(v2[M - 1]);
#pragma unroll
            for (int i = 0; i < tile_sum_regs(M, RS); ++i) out[i] = dpp_bfly<kDppXor2>(dpp_bfly<kDppXor1>(out[i]));
        }
    }
}

// Value index i = 4 m + b that register r of lane j holds after tile_sums, and
// whether lane j is the one lane of its slot that writes it (the lowest j
// holding it).
template <int M, int RS>
__device__ __forceinline__ int tile_sum_index(int r, int j)
{
    const int b4 = (j >> 4) & 1, b3 = (j >> 3) & 1, b2 = (j >> 2) & 1;
    if (RS == 1) return r + 2 * M * b4;
    if (RS == 2) return r + M * b3 + 2 * M * b4;
    constexpr int H3 = M / 2;
    return (r < H3 ? r + H3 * b2 : M - 1) + M * b3 + 2 * M * b4;
}
template <int M, int RS>
__device__ __forceinline__ bool tile_sum_owner(int r, int j)
{
    if (RS == 1) return (j & 15) == 0;
    if (RS == 2) return (j & 7) == 0;
    return (j & 3) == 0 && (r < M / 2 || (j & 4) == 0);
}

// Reduce-scatter depth of each epilogue: gate|up keeps a gate row and its up
// row (values 2p, 2p + 1) in one lane, so it splits at L1 only.
template <int EPI>
constexpr int tile_rs() { return EPI == kEpiGateUp ? 1 : 3; }

// One lane's packed data for one (row tile, segment): 16 bytes per row and
// half-block, plus the fp16 scales of its 4 rows (Q4_K: their 6-bit scales and
// mins, and in `sup` the d and dmin of their super-blocks; Q6_K: their two int8
// scales, in `hq` the high 2-bit parts of rows 0-1 and 2-3, and in `sup` d).
template <int QT>
struct Unit {
    static constexpr int NH = (QT == kQ8_0) ? 2 : 1;
    using Sup = typename std::conditional<QT == kQ6_K, u32x2, u32x4>::type;
    u32x4 q[kRowsPerLane][NH];
    u32x2 sc;
    Sup sup;
    u32x4 hq[2];
};

// A lane's place in a segment: the byte offset of its first 16-byte quant
// unit and the block whose activations it reads, for full segments and for a
// ragged last segment of nb_last < 32 blocks. In the ragged segment lanes
// j >= nb_last read block nb_last - 1 again (in bounds) and count as dead:
// their scales are zeroed, so they add nothing.
struct LanePlace {
    uint32_t off_full, off_last;   // (slot * nb + jc) * 16 for nb = 32 / nb_last
    uint32_t str_last;             // bytes between the b/h units of the last segment (wave-uniform)
    uint32_t sup_full, sup_last;   // Q4_K / Q6_K: slot * nb/8 + jc/8, the super-block scales of the 4 rows
    int j_last;                    // jc in the last segment
    bool live_last;
};

__device__ __forceinline__ LanePlace lane_place(const Geometry &g, int slot, int j)
{
    LanePlace p;
    const int nb_last = (int)seg_blocks(g, g.nseg - 1);
    p.j_last = j < nb_last ? j : nb_last - 1;
    p.live_last = j < nb_last;
    p.off_full = (uint32_t)(slot * kSegBlocks + j) * kUnit;
    p.off_last = (uint32_t)(slot * nb_last + p.j_last) * kUnit;
    p.str_last = (uint32_t)(kSlots * nb_last * kUnit);
    p.sup_full = (uint32_t)(slot * (kSegBlocks / kSuperBlocks) + j / kSuperBlocks);
    p.sup_last = (uint32_t)(slot * (nb_last / kSuperBlocks) + p.j_last / kSuperBlocks);
    return p;
}

// Buffer descriptors: word 3 of a raw (untyped) buffer resource on gfx9, and
// the cache policy of the weight loads (nontemporal: each byte is read once).
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kLoadNT = 2;

// A raw buffer descriptor for `base` with `bytes` bytes in range: all (-1) or
// none (0, for a unit past the end: its loads return zeros and read nothing).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t plane_rsrc(const uint8_t *base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, bytes, kRsrcWord3);
}

// Issue the loads of tile t, segment s (t, s wave-uniform) as buffer loads: a
// descriptor per plane based at the unit (scalar registers), the lane's 32-bit
// offset, and the wave-uniform offset of row b / half h in the scalar offset,
// so that no address arithmetic runs on the vector ALU. With `real` false (no
// unit left) the descriptors cover no bytes: every load returns zeros without a
// memory access. The loop body thus always issues the same loads with no
// branch around them, so the compiler's wait counts keep the next unit in
// flight while the current one is computed.
template <int QT>
__device__ __forceinline__ void load_unit(Unit<QT> &u, const uint8_t *__restrict__ wp, const Geometry &g, int64_t t,
                                          int64_t s, const LanePlace &lp, bool real)
{
    constexpr int NH = Unit<QT>::NH;
    constexpr int64_t seg_q = (int64_t)kTileRows * kSegBlocks * packed_quant_bytes(QT);   // bytes per segment
    constexpr uint32_t str_full = (uint32_t)(kSlots * kSegBlocks * kUnit);
    const bool last = s == g.nseg - 1;
    const uint32_t off = last ? lp.off_last : lp.off_full;
    const uint32_t ustride = last ? lp.str_last : str_full;
    // wave-uniform by construction (the unit counters are); readfirstlane tells
    // the compiler so, which keeps the descriptors in scalar registers
    const int in_range = __builtin_amdgcn_readfirstlane(real ? -1 : 0);
    const __amdgpu_buffer_rsrc_t rq = plane_rsrc(wp + t * g.tile_q + s * seg_q, in_range);
#pragma unroll
    for (int b = 0; b < kRowsPerLane; ++b)
#pragma unroll
        for (int h = 0; h < NH; ++h)
            u.q[b][h] = __builtin_amdgcn_raw_buffer_load_b128(rq, (int)off, (int)((uint32_t)(b * NH + h) * ustride),
                                                              kLoadNT);
    // scales: (slot * nb + jc) * 8 bytes = half the quant offset
    const __amdgpu_buffer_rsrc_t rs =
        plane_rsrc(wp + g.scale_off + t * g.tile_s + s * (int64_t)(kTileRows * kSegBlocks * 2), in_range);
    u.sc = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)(off >> 1), 0, kLoadNT);
    if constexpr (QT == kQ4_K || QT == kQ6_K) {
        constexpr uint32_t ub = (QT == kQ4_K) ? 4 : 2;   // super-plane bytes per row
        const uint32_t so = (last ? lp.sup_last : lp.sup_full) * (kRowsPerLane * ub);
        const __amdgpu_buffer_rsrc_t ru = plane_rsrc(
            wp + g.sup_off + t * g.tile_u + s * (int64_t)(kTileRows * (kSegBlocks / kSuperBlocks) * ub), in_range);
        if constexpr (QT == kQ4_K)
            u.sup = __builtin_amdgcn_raw_buffer_load_b128(ru, (int)so, 0, kLoadNT);
        else
            u.sup = __builtin_amdgcn_raw_buffer_load_b64(ru, (int)so, 0, kLoadNT);
    }
    if constexpr (QT == kQ6_K) {
#pragma unroll
        for (int bp = 0; bp < 2; ++bp)
            u.hq[bp] = __builtin_amdgcn_raw_buffer_load_b128(rq, (int)off,
                                                             (int)((uint32_t)(kRowsPerLane + bp) * ustride), kLoadNT);
    }
}

// Per-lane form of load_unit for the persistent kernel, whose two wavefront
// halves may work on different row tiles and segments: every plane's
// descriptor is based at the workgroup's first tile T0 and covers the `span`
// tiles it touches, and each lane's whole offset (tile, segment, slot, block,
// row) is in its VGPR (24-bit multiplies: the host keeps a tile's planes below
// 2^24 bytes and span * tile bytes below 2^31). No branch: a branch around the
// loads makes the compiler wait for every load in flight. A lane with `alive`
// false gets an offset past the descriptor's range, so its loads return zeros
// without a memory access.
constexpr uint32_t kDeadOffset = 0x80000000u;
template <int QT>
__device__ __forceinline__ void load_unit_lane(Unit<QT> &u, const uint8_t *__restrict__ wp, const Geometry &g,
                                               int64_t T0, uint32_t span, uint32_t t_rel, uint32_t s,
                                               uint32_t slot, int j, bool alive)
{
    constexpr int NH = Unit<QT>::NH;
    constexpr uint32_t seg_q = (uint32_t)(kTileRows * kSegBlocks * packed_quant_bytes(QT));
    constexpr uint32_t seg_s = (uint32_t)(kTileRows * kSegBlocks * 2);
    const uint32_t tq = (uint32_t)g.tile_q, ts = (uint32_t)g.tile_s;
    const uint32_t nb_last = (uint32_t)seg_blocks(g, g.nseg - 1);
    const bool last = s == (uint32_t)(g.nseg - 1);
    const uint32_t nb = last ? nb_last : (uint32_t)kSegBlocks;
    const uint32_t jc = last && (uint32_t)j >= nb_last ? nb_last - 1 : (uint32_t)j;
    const uint32_t ustride = (uint32_t)kSlots * nb * kUnit;
    const uint32_t lane_u = (slot * nb + jc) * kUnit;
    const uint32_t off = alive ? __umul24(t_rel, tq) + s * seg_q + lane_u : kDeadOffset;
    const __amdgpu_buffer_rsrc_t rq = plane_rsrc(wp + T0 * g.tile_q, (int)(span * tq));
#pragma unroll
    for (int b = 0; b < kRowsPerLane; ++b)
#pragma unroll
        for (int h = 0; h < NH; ++h)
            u.q[b][h] = __builtin_amdgcn_raw_buffer_load_b128(rq, (int)(off + (uint32_t)(b * NH + h) * ustride), 0,
                                                              kLoadNT);
    const __amdgpu_buffer_rsrc_t rs = plane_rsrc(wp + g.scale_off + T0 * g.tile_s, (int)(span * ts));
    const uint32_t off_s = alive ? __umul24(t_rel, ts) + s * seg_s + (lane_u >> 1) : kDeadOffset;
    u.sc = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)off_s, 0, kLoadNT);
    if constexpr (QT == kQ4_K || QT == kQ6_K) {
        constexpr uint32_t ub = (QT == kQ4_K) ? 4 : 2;   // super-plane bytes per row
        const uint32_t tu = (uint32_t)g.tile_u;
        const uint32_t sup = slot * (nb / kSuperBlocks) + jc / kSuperBlocks;
        const uint32_t off_u = alive ? __umul24(t_rel, tu) +
                                           s * (uint32_t)(kTileRows * (kSegBlocks / kSuperBlocks) * ub) +
                                           sup * (kRowsPerLane * ub)
                                     : kDeadOffset;
        const __amdgpu_buffer_rsrc_t ru = plane_rsrc(wp + g.sup_off + T0 * g.tile_u, (int)(span * tu));
        if constexpr (QT == kQ4_K)
            u.sup = __builtin_amdgcn_raw_buffer_load_b128(ru, (int)off_u, 0, kLoadNT);
        else
            u.sup = __builtin_amdgcn_raw_buffer_load_b64(ru, (int)off_u, 0, kLoadNT);
    }
    if constexpr (QT == kQ6_K) {
#pragma unroll
        for (int bp = 0; bp < 2; ++bp)
            u.hq[bp] = __builtin_amdgcn_raw_buffer_load_b128(
                rq, (int)(off + (uint32_t)(kRowsPerLane + bp) * ustride), 0, kLoadNT);
    }
}

// acc[m][b] += d_b * sum_e v_e * x_m[e] over the lane's block of segment s.
// j is the block whose activations the lane reads; live is false only for
// lanes past the end of a ragged last segment.
// Q4_K: acc[m][b] += d*sc * sum_e (q_e - c) x_e + (d*sc*c - dmin*mn) * sum_e x_e
// over the lane's sub-block, c the sub-block's centre from the packed scale
// word (layout.h): one fma per weight and row, and each row's sum of x shared
// by the 4 weight rows. With the centre, both terms are bounded by 3 |w| per
// weight (w = d*sc*q - dmin*mn), so the rounding scales with sum |w x| even
// where d*sc*q and dmin*mn cancel. The centred quants arrive as exact fp16
// subnormals (q - c) * 2^-24 and are summed in one fp32 fma chain of 32 per
// row; the 2^24 goes into d*sc. d*sc and dmin*mn are exact (11-bit by 6-bit
// products) and d*sc*c - dmin*mn is one fma. Dead lanes of a ragged segment
// get zero terms: they add 0. Every activation row goes through the same
// operations for any M. PRE: the block's sum of x comes from the workgroup's
// staged sums (block_x_sums, the same additions in the same order) instead of
// being added up here by every wavefront.
template <int M, bool XLDS, bool PRE = false>
__device__ __forceinline__ void compute_unit_q4k(const Unit<kQ4_K> &u, float (&acc)[M][kRowsPerLane],
                                                 const Consts &k, const f32x4 *xs4, const float *__restrict__ x,
                                                 int64_t x_stride, int64_t nseg, int64_t s, int j, bool live)
{
    constexpr int B = kRowsPerLane;
    float sq[M][B], sx[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        sx[m] = 0.0f;
#pragma unroll
        for (int b = 0; b < B; ++b) sq[m][b] = 0.0f;
    }
    const uint32_t x_row = (uint32_t)nseg << 8;
    const f32x4 *xl = xs4 + ((uint32_t)s << 8) + (uint32_t)j;
    const float *xg = x + s * kSegWeights + j * 32;
    // each row's scale word: bits 0-3 the centre c, 4-9 sc, 10-15 mn; the centre
    // as the fp16 subnormal pair (c * 2^-24, c * 2^-24)
    auto word = [&](int b) { return ((b < 2) ? u.sc.x : u.sc.y) >> (16 * (b & 1)); };
    uint32_t c_lo[B];
#pragma unroll
    for (int b = 0; b < B; ++b) c_lo[b] = (word(b) & 15u) * 0x00010001u;
    auto row_fma = [&](const h2 (&p)[4], const f32x4 (&xv)[2], int m, int b) {
        float t = sq[m][b];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            t = __builtin_fmaf((float)p[2 * cc].x, xv[cc].x, t);
            t = __builtin_fmaf((float)p[2 * cc].y, xv[cc].y, t);
            t = __builtin_fmaf((float)p[2 * cc + 1].x, xv[cc].z, t);
            t = __builtin_fmaf((float)p[2 * cc + 1].y, xv[cc].w, t);
        }
        sq[m][b] = t;
    };
    // Per dword of 8 elements. One activation row: its 2 float4 of x, then the 4
    // weight rows one at a time. Several: the 4 weight rows' pairs once, then the
    // activation rows one at a time (2 float4 of x live, not 2 M). Each
    // accumulator sees the same operations in the same order either way.
#pragma unroll
    for (int c = 0; c < 8; c += 2) {
        auto load_x = [&](f32x4 (&xv)[2], int m) {
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
                xv[cc] = XLDS ? xl[m * x_row + (c + cc) * 32] : *(const f32x4 *)(xg + m * x_stride + (c + cc) * 4);
            if (!PRE)
                sx[m] = sx[m] + (((xv[0].x + xv[0].y) + (xv[0].z + xv[0].w)) + ((xv[1].x + xv[1].y) + (xv[1].z + xv[1].w)));
        };
        if constexpr (M == 1) {
            f32x4 xv[2];
            load_x(xv, 0);
#pragma unroll
            for (int b = 0; b < B; ++b) {
                h2 p[4];
                q4k_pairs(u.q[b][0][c >> 1], k, c_lo[b], p);
                row_fma(p, xv, 0, b);
            }
        } else {
            h2 p[B][4];
#pragma unroll
            for (int b = 0; b < B; ++b) q4k_pairs(u.q[b][0][c >> 1], k, c_lo[b], p[b]);
#pragma unroll
            for (int m = 0; m < M; ++m) {
                f32x4 xv[2];
                load_x(xv, m);
#pragma unroll
                for (int b = 0; b < B; ++b) row_fma(p[b], xv, m, b);
            }
        }
    }
    if (PRE) {
        // row m's sums follow the staged copy: float m * nseg * 32 + s * 32 + j
        const float *xsl = (const float *)(xs4 + (uint32_t)M * x_row) + ((uint32_t)s << 5) + (uint32_t)j;
#pragma unroll
        for (int m = 0; m < M; ++m) sx[m] = xsl[(uint32_t)m * ((uint32_t)nseg << 5)];
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const uint32_t sw = word(b);
        const h2 dd = as_h2(u.sup[b]);                                        // (d, dmin)
        const float a = (float)dd.x * (float)((sw >> 4) & 63u);                // d*sc, exact
        const float scl = live ? a * 16777216.0f : 0.0f;
        const float ct = live ? __builtin_fmaf(a, (float)(sw & 15u), -((float)dd.y * (float)((sw >> 10) & 63u)))
                              : 0.0f;                                          // d*sc*c - dmin*mn
#pragma unroll
        for (int m = 0; m < M; ++m) acc[m][b] = acc[m][b] + __builtin_fmaf(scl, sq[m][b], ct * sx[m]);
    }
}

// Q6_K: acc[m][b] += d * (sc_lo * sum_{e<16} v_e x_e + sc_hi * sum_{e>=16} v_e x_e)
// with v = q - 32 exact in fp16: the low nibble goes into a magic-number fp16
// (1024 + q or 1024 + 16 q) as in Q4_0 and the high 2 bits are OR-ed in above it
// from the row's dword of high parts (a shift by 0 / 2 for the first 16 elements'
// dword halves, a rotation by 24 and a shift by 2 for the second), then -1056 or
// (/16 - 96). One fp32 fma per weight and row, as for Q4_0; the int8 scales are
// exact in fp32. Dead lanes of a ragged segment get d = 0. Every activation row
// goes through the same operations for any M.
template <int M, bool XLDS>
__device__ __forceinline__ void compute_unit_q6k(const Unit<kQ6_K> &u, float (&acc)[M][kRowsPerLane],
                                                 const Consts &k, const f32x4 *xs4, const float *__restrict__ x,
                                                 int64_t x_stride, int64_t nseg, int64_t s, int j, bool live)
{
    constexpr int B = kRowsPerLane;
    float s16[M][B][2];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int b = 0; b < B; ++b) s16[m][b][0] = s16[m][b][1] = 0.0f;
    const uint32_t x_row = (uint32_t)nseg << 8;
    const f32x4 *xl = xs4 + ((uint32_t)s << 8) + (uint32_t)j;
    const float *xg = x + s * kSegWeights + j * 32;
    // Per dword of 8 elements, in the same two loop orders as Q4_K above.
#pragma unroll
    for (int c = 0; c < 8; c += 2) {
        const int dw = c >> 1;   // dword of 8 elements: 8 dw .. 8 dw + 7
        auto pairs = [&](h2 (&p)[4], int b) {
            const u32x4 &hv = u.hq[b >> 1];
            q6k_pairs(u.q[b][0][dw], hv[2 * (b & 1) + (dw >> 1)], (dw & 1) != 0, k, p);
        };
        auto load_x = [&](f32x4 (&xv)[2], int m) {
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
                xv[cc] = XLDS ? xl[m * x_row + (c + cc) * 32] : *(const f32x4 *)(xg + m * x_stride + (c + cc) * 4);
        };
        auto row_fma = [&](const h2 (&p)[4], const f32x4 (&xv)[2], int m, int b) {
            float s_ = s16[m][b][dw >> 1];
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                s_ = __builtin_fmaf((float)p[2 * cc].x, xv[cc].x, s_);
                s_ = __builtin_fmaf((float)p[2 * cc].y, xv[cc].y, s_);
                s_ = __builtin_fmaf((float)p[2 * cc + 1].x, xv[cc].z, s_);
                s_ = __builtin_fmaf((float)p[2 * cc + 1].y, xv[cc].w, s_);
            }
            s16[m][b][dw >> 1] = s_;
        };
        if constexpr (M == 1) {
            f32x4 xv[2];
            load_x(xv, 0);
#pragma unroll
            for (int b = 0; b < B; ++b) {
                h2 p[4];
                pairs(p, b);
                row_fma(p, xv, 0, b);
            }
        } else {
            h2 p[B][4];
#pragma unroll
            for (int b = 0; b < B; ++b) pairs(p[b], b);
#pragma unroll
            for (int m = 0; m < M; ++m) {
                f32x4 xv[2];
                load_x(xv, m);
#pragma unroll
                for (int b = 0; b < B; ++b) row_fma(p[b], xv, m, b);
            }
        }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
        const uint32_t sw = ((b < 2) ? u.sc.x : u.sc.y) >> (16 * (b & 1));   // byte 0: sc_lo, byte 1: sc_hi
        const float sc_lo = (float)(int8_t)(sw & 0xFFu);
        const float sc_hi = (float)(int8_t)((sw >> 8) & 0xFFu);
        const uint32_t dw = ((b < 2) ? u.sup.x : u.sup.y) >> (16 * (b & 1));
        const float d = live ? (float)as_h2(dw).x : 0.0f;
#pragma unroll
        for (int m = 0; m < M; ++m)
            acc[m][b] = __builtin_fmaf(d, __builtin_fmaf(sc_hi, s16[m][b][1], sc_lo * s16[m][b][0]), acc[m][b]);
    }
}

// s[b] += the 8 products of weight row b's fp16 pairs p[b] (elements 0..7 of a
// dword) with the activations xv, one fma each in element order, for the B rows
// of a lane. The rows' chains are interleaved instruction by instruction: each
// fma depends on the one B instructions back, not on the one before it (which
// would cost a wait state per fma), and each accumulator still sees its 8 fmas
// in element order.
template <int B>
__device__ __forceinline__ void rows_fma(const h2 (&p)[B][4], const f32x4 (&xv)[2], float (&s)[B])
{
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
        for (int b = 0; b < B; ++b) s[b] = __builtin_fmaf((float)p[b][2 * cc].x, xv[cc].x, s[b]);
#pragma unroll
        for (int b = 0; b < B; ++b) s[b] = __builtin_fmaf((float)p[b][2 * cc].y, xv[cc].y, s[b]);
#pragma unroll
        for (int b = 0; b < B; ++b) s[b] = __builtin_fmaf((float)p[b][2 * cc + 1].x, xv[cc].z, s[b]);
#pragma unroll
        for (int b = 0; b < B; ++b) s[b] = __builtin_fmaf((float)p[b][2 * cc + 1].y, xv[cc].w, s[b]);
    }
}

template <int QT, int M, bool XLDS, bool NORM = false>
__device__ __forceinline__ void compute_unit(const Unit<QT> &u, float (&acc)[M][kRowsPerLane], const Consts &k,
                                             const f32x4 *xs4, const float *__restrict__ x, int64_t x_stride,
                                             int64_t nseg, int64_t s, int j, bool live)
{
    if constexpr (QT == kQ4_K) {
        compute_unit_q4k<M, XLDS, x_sums_staged(QT, XLDS, NORM)>(u, acc, k, xs4, x, x_stride, nseg, s, j, live);
        return;
    }
    if constexpr (QT == kQ6_K) {
        compute_unit_q6k<M, XLDS>(u, acc, k, xs4, x, x_stride, nseg, s, j, live);
        return;
    }
    constexpr int B = kRowsPerLane;
    float sb[M][B];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int b = 0; b < B; ++b) sb[m][b] = 0.0f;
    // LDS: row m, segment s, chunk c of block j at float4 m*nseg*256 + s*256 + c*32 + j
    const uint32_t x_row = (uint32_t)nseg << 8;
    const f32x4 *xl = xs4 + ((uint32_t)s << 8) + (uint32_t)j;
    const float *xg = x + s * kSegWeights + j * 32;

    // 8 float4 chunks of x per block; Q4_0 consumes 2 chunks per dword, Q8_0 one.
    // Per dword of 8 elements, one activation row: its 2 float4 of x, then the 4
    // weight rows one at a time. Several: the 4 weight rows' fp16 pairs once, then
    // the activation rows one at a time (2 float4 of x live, not 2 M). Each
    // accumulator sees the same 8 fmas in the same order either way.
    auto pairs = [&](int b, int c, h2 (&p)[4]) {
        if (QT == kQ4_0) {
            q4_pairs(u.q[b][0][c >> 1], k, p);
        } else {
            h2 p01[2], p23[2];
            q8_pairs(u.q[b][c >> 2][c & 3], p01);
            q8_pairs(u.q[b][c >> 2][(c & 3) + 1], p23);
            p[0] = p01[0];
            p[1] = p01[1];
            p[2] = p23[0];
            p[3] = p23[1];
        }
    };
    auto load_x = [&](f32x4 (&xv)[2], int m, int c) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
            xv[cc] = XLDS ? xl[m * x_row + (c + cc) * 32] : *(const f32x4 *)(xg + m * x_stride + (c + cc) * 4);
    };
#pragma unroll
    for (int c = 0; c < 8; c += 2) {
        h2 p[B][4];
#pragma unroll
        for (int b = 0; b < B; ++b) pairs(b, c, p[b]);
#pragma unroll
        for (int m = 0; m < M; ++m) {
            f32x4 xv[2];
            load_x(xv, m, c);
            rows_fma<B>(p, xv, sb[m]);
        }
    }
    const h2 d01 = as_h2(live ? u.sc.x : 0u), d23 = as_h2(live ? u.sc.y : 0u);
    const _Float16 d[4] = {d01.x, d01.y, d23.x, d23.y};
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[m][b] = __builtin_fmaf((float)d[b], sb[m][b], acc[m][b]);
}

// Stage rows 0..M-1 of X as xs4[m*nseg*256 + seg*256 + c*32 + jj], where
// float4 chunk i = seg*256 + jj*8 + c of a row holds x[4i .. 4i+3] (zero past
// K; K % 32 == 0, so a chunk is wholly inside K or wholly past it). The staged
// area is taken as one flat sequence of chunks f = m*nseg*256 + i over all M
// rows; each thread loads a batch of NB chunks f = tid + q*nthreads before
// writing any, so that an area of up to NB chunks per thread costs one memory
// round trip, not one per row or per batch of 4 (every single-row
// configuration needs at most 5 per thread: K = 5120 over 256 threads, K =
// 17408 over 1024). The batch is sized to stay inside the kernels' register
// budgets (x_batch). Reads are coalesced (consecutive threads, consecutive 16-byte
// chunks); the LDS stores scatter into the lane-swizzled order. Each thread
// walks its chunks incrementally (XWalk) and computes a chunk's row, offset and
// LDS slot once, when its load is issued. Indexing is 32-bit (the staged area
// is at most LDS-sized).
//
// The first batch is split off (stage_x_issue): a kernel issues it before its
// first weight loads, so that the activation lines reach the memory queues
// ahead of the weight stream instead of behind it, and writes it
// (stage_x_finish, which also stages anything past the first batch) after
// them. The caller synchronises the workgroup afterwards.
// Chunks per thread and batch: 5 for one row; for several rows in the
// persistent form (launched at 2 or 3 wavefronts per SIMD, which its registers
// allow) 8, and 10 for 5 or 6 rows (K = 5120 at 768 threads: one batch); 4 in
// the tile form, whose occupancy more registers would lower.
constexpr int x_batch(int M, bool persistent) { return M == 1 ? 5 : (persistent ? (M >= 5 ? 10 : 8) : 4); }

__device__ __forceinline__ uint32_t x_slot(uint32_t i) { return (i & ~255u) | ((i & 7u) << 5) | ((i >> 3) & 31u); }

// Chunk walk of one thread: chunks f = tid, tid + nthr, tid + 2 nthr, ... of
// the staged area as (row m, chunk i of the row). The stride nthr is dm rows
// and di chunks, so a step is two adds and at most one wrap; only the first
// position takes a division. m >= M means past the staged area.
struct XWalk {
    uint32_t m, i, dm, di, per_m;
    __device__ __forceinline__ void step()
    {
        i += di;
        m += dm;
        if (i >= per_m) {
            i -= per_m;
            ++m;
        }
    }
};

__device__ __forceinline__ XWalk x_walk(int64_t nseg)
{
    XWalk w;
    w.per_m = (uint32_t)nseg << 8;
    const uint32_t nthr = blockDim.x, tid = threadIdx.x;
    w.dm = nthr / w.per_m;
    w.di = nthr - w.dm * w.per_m;
    w.m = tid / w.per_m;
    w.i = tid - w.m * w.per_m;
    return w;
}

// One batch of NB chunks in flight: the values and the LDS float4 slot each one
// goes to (kNoSlot past the staged area).
constexpr uint32_t kNoSlot = ~0u;
template <int NB>
struct XFirst {
    f32x4 v[NB];
    uint32_t at[NB];
    XWalk w;
};

template <int M, int NB>
__device__ __forceinline__ void x_batch_load(f32x4 (&v)[NB], uint32_t (&at)[NB], XWalk &w,
                                             const float *__restrict__ x, int64_t x_stride, uint32_t k4)
{
#pragma unroll
    for (int q = 0; q < NB; ++q) {
        const bool in = w.m < (uint32_t)M;
        v[q] = in && w.i < k4 ? *(const f32x4 *)(x + (uint64_t)w.m * (uint64_t)x_stride + 4 * (size_t)w.i)
                              : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        at[q] = in ? w.m * w.per_m + x_slot(w.i) : kNoSlot;
        w.step();
    }
}

template <int M, int NB>
__device__ __forceinline__ void stage_x_issue(XFirst<NB> &xf, const float *__restrict__ x, int64_t x_stride,
                                              int64_t nseg, int64_t K)
{
    xf.w = x_walk(nseg);
    x_batch_load<M, NB>(xf.v, xf.at, xf.w, x, x_stride, (uint32_t)(K >> 2));
}

template <int M, int NB>
__device__ __forceinline__ void stage_x_finish(XFirst<NB> &xf, f32x4 *xs4, const float *__restrict__ x,
                                               int64_t x_stride, int64_t nseg, int64_t K)
{
    const uint32_t per_m = (uint32_t)nseg << 8;
    const uint32_t total = (uint32_t)M * per_m;
    const uint32_t nthr = blockDim.x;
#pragma unroll
    for (int q = 0; q < NB; ++q)
        if (xf.at[q] != kNoSlot) xs4[xf.at[q]] = xf.v[q];
    for (uint32_t base = NB * nthr; base < total; base += NB * nthr) {   // uniform: batches after the first
        f32x4 v[NB];
        uint32_t at[NB];
        x_batch_load<M, NB>(v, at, xf.w, x, x_stride, (uint32_t)(K >> 2));
#pragma unroll
        for (int q = 0; q < NB; ++q)
            if (at[q] != kNoSlot) xs4[at[q]] = v[q];
    }
}

// Sum of squares of one thread's values, then of the workgroup: a per-thread fma
// chain, the wavefront butterfly (both halves), then the wavefront partials added
// in wavefront order through `red` (one float per wavefront). Every thread gets
// the same bits. The caller's threads must all arrive; `red` is reused after a
// barrier.
__device__ __forceinline__ float block_sum(float s, float *red)
{
    const uint32_t nthr = blockDim.x, tid = threadIdx.x;
    const float h = half_wave_sum(s);
    const float w = as_f(__builtin_amdgcn_readlane(as_i(h), 0)) + as_f(__builtin_amdgcn_readlane(as_i(h), 32));
    if ((tid & 63) == 0) red[tid >> 6] = w;
    __syncthreads();
    float t = red[0];
    for (uint32_t i = 1; i < (nthr >> 6); ++i) t += red[i];
    __syncthreads();
    return t;
}

// 1 / sqrt(mean + eps), correctly rounded square root and division.
__device__ __forceinline__ float rms_scale(float ss, int64_t K, float eps)
{
    return 1.0f / __builtin_sqrtf(ss / (float)K + eps);
}

// RMSNorm prologue: the staged activations (row 0, float4 chunk i at
// xs4[x_slot(i)], zero past K) become (x * r) * gamma in place, with
// r = 1 / sqrt(sum(x^2) / K + eps). Every thread of the workgroup must call it.
__device__ __forceinline__ void norm_staged_x(f32x4 *xs4, float *red, const float *__restrict__ gamma, float eps,
                                              int64_t K)
{
    const uint32_t k4 = (uint32_t)(K >> 2);
    const uint32_t nthr = blockDim.x, tid = threadIdx.x;
    float s = 0.0f;
    for (uint32_t i = tid; i < k4; i += nthr) {
        const f32x4 v = xs4[x_slot(i)];
        s = __builtin_fmaf(v.x, v.x, s);
        s = __builtin_fmaf(v.y, v.y, s);
        s = __builtin_fmaf(v.z, v.z, s);
        s = __builtin_fmaf(v.w, v.w, s);
    }
    const float r = rms_scale(block_sum(s, red), K, eps);
    for (uint32_t i = tid; i < k4; i += nthr) {
        const uint32_t sl = x_slot(i);
        const f32x4 gm = *(const f32x4 *)(gamma + 4 * (size_t)i);
        const f32x4 v = xs4[sl];
        xs4[sl] = f32x4{(v.x * r) * gm.x, (v.y * r) * gm.y, (v.z * r) * gm.z, (v.w * r) * gm.w};
    }
    __syncthreads();
}

// Block sums of the staged activations (Q4_K): for each row m, segment s and
// block j of the staged copy, the sum of its 32 values in the order a wavefront
// adds them (pairs of float4 chunks, ((x0 + x1) + (x2 + x3)) + ((x4 + x5) +
// (x6 + x7)), added in chunk order), written after the copy at float
// m * nseg * 32 + s * 32 + j. One thread per block, then a barrier. Every
// thread of the workgroup must call it.
template <int M>
__device__ __forceinline__ void block_x_sums(f32x4 *xs4, uint32_t nseg)
{
    float *xsum = (float *)(xs4 + (uint32_t)M * (nseg << 8));
    const uint32_t nb = (uint32_t)M * (nseg << 5);
    for (uint32_t i = threadIdx.x; i < nb; i += blockDim.x) {
        const f32x4 *xb = xs4 + ((i >> 5) << 8) + (i & 31u);   // chunk c of the block at xb[32 c]
        float sx = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; c += 2) {
            const f32x4 v0 = xb[c * 32], v1 = xb[(c + 1) * 32];
            sx = sx + (((v0.x + v0.y) + (v0.z + v0.w)) + ((v1.x + v1.y) + (v1.z + v1.w)));
        }
        xsum[i] = sx;
    }
    __syncthreads();
}

// Store output n of activation row m (n < n_out). The affine epilogue adds the
// bias and then the residual to the finished product, one fp32 addition each,
// and writes fp32 or fp16 (v_cvt_f16_f32, round to nearest even). The residual
// is read before y[n] is written, so residual == y updates y in place.
template <int M, int EPI>
__device__ __forceinline__ void store_out(float *__restrict__ y, const QArgs &a, int m, int64_t n, float v)
{
    if (EPI == kEpiAffine) {
        if (a.bias != nullptr) v = v + a.bias[n];
        if (a.residual != nullptr) v = v + a.residual[n];
        if (a.out_f16) {
            ((_Float16 *)y)[n] = (_Float16)v;
            return;
        }
        y[n] = v;
    } else {
        y[m * a.y_stride + n] = v;
    }
}

// The sums a lane holds after tile_sums for epilogue EPI.
template <int M, int EPI>
using TileSums = float[tile_sum_regs(M, tile_rs<EPI>())];

// Write the finished rows of tile t from the sums of one slot (tile_sums).
//   plain, affine: the owner lane of value i = 4 m + b stores row b of
//                  activation row m
//   gate|up (M = 1, one split level): registers 0 and 1 of lane j hold gate row
//                  2p and up row 2p + 1, p = j bit 4; lane j = 16 p stores
//                  output n = row0/2 + p
template <int M, int EPI>
__device__ __forceinline__ void store_tile(const TileSums<M, EPI> &sums, float *__restrict__ y, const QArgs &a,
                                           int64_t t, int slot, int j)
{
    constexpr int B = kRowsPerLane, RS = tile_rs<EPI>();
    const int64_t n_out = a.n_out;
    const int64_t row0 = t * kTileRows + slot * kRowsPerLane;
    if (EPI != kEpiGateUp) {
#pragma unroll
        for (int r = 0; r < tile_sum_regs(M, RS); ++r) {
            if (tile_sum_owner<M, RS>(r, j)) {
                const int i = tile_sum_index<M, RS>(r, j), m = i / B, b = i % B;
                if (row0 + b < n_out) store_out<M, EPI>(y, a, m, row0 + b, sums[r]);
            }
        }
    } else {
        if ((j & 15) == 0) {
            const int64_t n = row0 / 2 + (j >> 4);
            if (n < n_out) y[n] = silu_mul(sums[0], sums[1]);
        }
    }
}

// Park the sums of one slot at dst[m * kTileRows + b] (dst already offset by
// the slot's first row): each value is written once, by its owner lane.
template <int M, int EPI>
__device__ __forceinline__ void park_tile(const TileSums<M, EPI> &sums, float *dst, int j)
{
    constexpr int B = kRowsPerLane, RS = tile_rs<EPI>();
#pragma unroll
    for (int r = 0; r < tile_sum_regs(M, RS); ++r) {
        if (tile_sum_owner<M, RS>(r, j)) {
            const int i = tile_sum_index<M, RS>(r, j);
            dst[(i / B) * kTileRows + i % B] = sums[r];
        }
    }
}

// ---------------------------------------------------------------------------
// Quantised GEMV. Template parameters:
//   QT   kQ8_0 / kQ4_0
//   M    activation rows (1 = decode GEMV, 2..6 = verify)
//   EPI  kEpiPlain (y = W x), kEpiGateUp (y = silu(gate) * up, M = 1) or
//        kEpiAffine (y = ((W x) + bias) + residual, fp32 or fp16, M = 1)
//   W    wavefronts that split one row tile along K (1, 2, 3, 4 or 8)
//   XLDS activations staged in LDS (true) or read from global memory
// W == 1: a workgroup holds blockDim/64 independent wavefronts; wavefront g of
//         workgroup b is group b*G + g.
// W  > 1: a workgroup is one group of W wavefronts; wavefront w adds segments
//         [nseg*w/W, nseg*(w+1)/W) of every tile of the group and the W partial
//         sums are combined in LDS in wavefront order.
// Group q walks the tiles [q * tpg, q * tpg + tpg) (contiguous order) or, with
// tstride > 0, the tiles q, q + tstride, q + 2*tstride, ... (grid-stride order:
// the groups resident at any moment read one contiguous window of the weights).
// Which group handles a tile changes none of its rows' operations.
// Each wavefront walks its (tile, segment) sequence with the loads of the next
// D units in flight while the current one is computed (a ring of D+1 units).
// gridDim.y > 1 (plain store only): row group blockIdx.y takes activation rows
// [blockIdx.y M, blockIdx.y M + M) of a call with gridDim.y M rows, so a small
// matrix's verify spreads over more wavefronts; each row still goes through
// the M = 1 operations.
// The launch bound is qgemv_max_threads (qgemv_kernels.h).
template <int QT, int M, int EPI, int W, bool XLDS, int D, bool NORM>
__global__ void __launch_bounds__(qgemv_max_threads(QT, M, W))
qgemv_kernel(const uint8_t *__restrict__ wp, const float *__restrict__ x, float *__restrict__ y, QArgs a)
{
    if (EPI == kEpiPlain) {
        x += (int64_t)blockIdx.y * M * a.x_stride;
        y += (int64_t)blockIdx.y * M * a.y_stride;
    }
    static_assert(!NORM || (XLDS && M == 1), "the RMSNorm prologue works on staged single-row activations");
    constexpr int B = kRowsPerLane;
    constexpr int S = D + 1;   // ring size
    extern __shared__ f32x4 xs4[];
    __shared__ float red[tile_red_floats(M, W, NORM)];  // [W][M][slot][b]; norm: [wavefront]

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int slot = lane >> 5, j = lane & 31;
    const int wk = (W > 1) ? wave : 0;
    const int64_t group = (W > 1) ? (int64_t)blockIdx.x : (int64_t)blockIdx.x * (blockDim.x >> 6) + wave;

    const Geometry &g = a.geo;
    const int64_t K = g.K, nseg = g.nseg;
    int64_t t_begin, t_step, my_tiles;
    if (a.tstride > 0) {
        t_begin = group;
        t_step = a.tstride;
        my_tiles = group < g.n_tiles ? (g.n_tiles - group + t_step - 1) / t_step : 0;
    } else {
        t_begin = group * a.tpg;
        t_step = 1;
        const int64_t t_end = (t_begin + a.tpg < g.n_tiles) ? t_begin + a.tpg : g.n_tiles;
        my_tiles = t_end > t_begin ? t_end - t_begin : 0;
    }
    const int64_t s_begin = nseg * wk / W, s_end = nseg * (wk + 1) / W;

    const Consts k = make_consts();
    const LanePlace lp = lane_place(g, slot, j);
    // This wavefront's units, in order: (t, s) for its tiles t, s in [s_begin, s_end).
    const int64_t n_units = my_tiles * (s_end - s_begin);

    // Load cursor: the unit whose loads are issued next (D units ahead of the compute cursor).
    int64_t t_ld = t_begin, s_ld = s_begin, u_ld = 0;
    auto advance = [&](int64_t &tt, int64_t &ss) {
        if (++ss == s_end) {
            ss = s_begin;
            tt += t_step;
        }
    };
    XFirst<x_batch(M, false)> xf;
    if (XLDS) stage_x_issue<M>(xf, x, a.x_stride, nseg, K);
    Unit<QT> ring[S];
#pragma unroll
    for (int r = 0; r < D; ++r) {
        load_unit<QT>(ring[r], wp, g, t_ld, s_ld, lp, u_ld < n_units);
        advance(t_ld, s_ld);
        ++u_ld;
    }

    if (XLDS) {
        stage_x_finish<M>(xf, xs4, x, a.x_stride, nseg, K);
        __syncthreads();
    }
    if (NORM) norm_staged_x(xs4, red, a.gamma, a.eps, K);
    if (x_sums_staged(QT, XLDS, NORM)) block_x_sums<M>(xs4, (uint32_t)nseg);
    if (n_units == 0) return;   // uniform across the workgroup when W > 1

    float acc[M][B];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[m][b] = 0.0f;

    int64_t t = t_begin, s = s_begin;   // compute cursor: the unit being computed

    // Issue the loads of unit u+D into `nxt` (a dummy one-line load past the
    // last unit), then compute unit u from `cur` and finish the tile after its
    // last segment.
    auto step = [&](Unit<QT> &cur, Unit<QT> &nxt) {
        load_unit<QT>(nxt, wp, g, t_ld, s_ld, lp, u_ld < n_units);
        advance(t_ld, s_ld);
        ++u_ld;
        // keep the scheduler from sinking these loads into the compute below
        __builtin_amdgcn_sched_barrier(0);
        const bool last = s == nseg - 1;
        compute_unit<QT, M, XLDS, NORM>(cur, acc, k, xs4, x, a.x_stride, nseg, s, last ? lp.j_last : j,
                                        !last || lp.live_last);
        if (s + 1 == s_end) {
            TileSums<M, EPI> sums;
            tile_sums<M, tile_rs<EPI>()>(acc, sums, j);
            if (W == 1) {
                store_tile<M, EPI>(sums, y, a, t, slot, j);
            } else {
                // fixed-order combine of the split-K partials: ((p0 + p1) + p2) + p3,
                // red[w][m][slot][b]; lane j of wavefront 0 finishes value j
                park_tile<M, EPI>(sums, red + wk * M * kTileRows + slot * B, j);
                __syncthreads();
                if (wk == 0) {
                    const int64_t row0 = t * kTileRows + slot * B;
                    if (EPI != kEpiGateUp) {
                        if (j < M * B) {
                            const int m = j / B, b = j % B;
                            float v = red[m * kTileRows + slot * B + b];
#pragma unroll
                            for (int w = 1; w < W; ++w) v += red[(w * M + m) * kTileRows + slot * B + b];
                            if (row0 + b < a.n_out) store_out<M, EPI>(y, a, m, row0 + b, v);
                        }
                    } else if (j < B / 2) {
                        float gv = red[slot * B + 2 * j], uv = red[slot * B + 2 * j + 1];
#pragma unroll
                        for (int w = 1; w < W; ++w) {
                            gv += red[w * kTileRows + slot * B + 2 * j];
                            uv += red[w * kTileRows + slot * B + 2 * j + 1];
                        }
                        const int64_t n = row0 / 2 + j;
                        if (n < a.n_out) y[n] = silu_mul(gv, uv);
                    }
                }
                __syncthreads();
            }
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int b = 0; b < B; ++b) acc[m][b] = 0.0f;
        }
        advance(t, s);
    };

    // A counted loop over groups of S units with no early exit, so that the only
    // way back to the loop head is through every step; unit u lives in ring[u % S].
    const int64_t n_groups = n_units / S;
    for (int64_t gi = 0; gi < n_groups; ++gi) {
#pragma unroll
        for (int r = 0; r < S; ++r) step(ring[r], ring[(r + D) % S]);
    }
    const int64_t rem = n_units - n_groups * S;
#pragma unroll
    for (int r = 0; r < S - 1; ++r)
        if (r < rem) step(ring[r], ring[(r + D) % S]);
}


// ---------------------------------------------------------------------------
// Persistent form of the quantised GEMV, for matrices with too few row tiles
// to balance the CUs one tile per wavefront. One workgroup per CU, and the work
// is split in half-tiles: the 4 rows of one slot of a row tile are outputs of
// their own, so workgroup b owns a contiguous run of 2 n_tiles / n_wg
// half-tiles, one more for the first 2 n_tiles % n_wg workgroups (the same
// number to within one: 17408 x 5120 gives every CU 17, where whole tiles gave
// half of them 9 and half 8), and stages the activations once. Each half-tile
// splits along K into R = a.ranges equal ranges of nseg/R segments; each half
// of a wavefront takes one (half-tile, range) item, the two halves usually the
// same range of neighbouring half-tiles, so a wavefront-unit still reads two
// 512-byte runs per load and shares its activation reads. A wavefront walks
// its units with the next unit's loads in flight; after an item's last unit
// each half reduces its 32 lanes (tile_sums, the same tree as above) and, for
// R > 1, parks its 4-row partial in LDS. When every wavefront is done, the
// partials of each row are added in range order, ((p0 + p1) + p2) + ..., and
// stored (with the SiLU epilogue for gate|up). For any M a row goes through
// the same operations, so the verify rows still equal the M=1 rows bit for
// bit. PHASED (several activation rows that do not fit in LDS at once): the
// ranges are walked in phases, each staging only its segments' activations
// (see the phase loop below).
template <int QT, int M, int EPI, bool XLDS, bool NORM, bool PHASED = false, bool ONE = false>
__global__ void __launch_bounds__(persist_threads(QT, M, XLDS, ONE, PHASED))
qgemv_persist(const uint8_t *__restrict__ wp, const float *__restrict__ x, float *__restrict__ y, QArgs a)
{
    static_assert(!NORM || (XLDS && M == 1), "the RMSNorm prologue works on staged single-row activations");
    static_assert(!PHASED || (XLDS && !NORM), "phases stage windows of the activations");
    constexpr int B = kRowsPerLane;
    constexpr int S = 2;   // ring: one unit in flight ahead of the one being computed
    extern __shared__ f32x4 xs4[];
    __shared__ float nred[persist_red_floats(NORM)];

    const int tid = threadIdx.x;
    constexpr int G = persist_threads(QT, M, XLDS, ONE, PHASED) >> 6;   // the launch's wavefronts (checked by the host)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const uint32_t hw = (uint32_t)lane >> 5;   // wavefront half: its own (half-tile, K range) item
    const int j = lane & 31;

    const Geometry &g = a.geo;
    const int64_t K = g.K, nseg = g.nseg;
    const uint32_t R = (uint32_t)a.ranges;
    const uint32_t L = ONE ? 1u : (uint32_t)a.range_segs;   // segments per range (1 for single-unit items)
    // Half-tiles h = 2 tile + slot (4 weight rows each). Workgroup b owns the
    // half-tiles [H0, H0 + nh); it touches the tiles T0 = H0 / 2 .. T0 + span - 1
    // (the first and the last may be shared with a neighbour, each owning its half).
    const uint32_t bx = blockIdx.x, hextra = (uint32_t)a.halves_extra;
    const int64_t H0 = (int64_t)bx * a.halves_base + (bx < hextra ? bx : hextra);
    const uint32_t nh = (uint32_t)a.halves_base + (bx < hextra ? 1u : 0u);
    const int64_t T0 = H0 >> 1;
    const uint32_t h0 = (uint32_t)(H0 & 1);   // half-tile index of H0 within its tile
    const uint32_t span = (h0 + nh + 1) >> 1;
    // Phases: the ranges are walked in P phases; phase ph takes the ranges
    // [r0, r1) = [R ph / P, R (ph + 1) / P), stages only the activations of
    // their segments [r0 L, r1 L) (a window of nsegw segments; all of them when
    // P = 1) and lists its items range by range: i = rl nh + hl (range r0 + rl,
    // half-tile H0 + hl). Wavefront-unit u is the item pair (2u, 2u + 1), one
    // per wavefront half, and wavefront w takes the units w, w + G, ...; so a
    // workgroup's load is its half-tiles' share whatever the split into tiles.
    // The partials follow the largest window.
    const uint32_t P = PHASED ? (uint32_t)a.phases : 1u;
    const uint32_t nsegw_max = PHASED ? (R + P - 1) / P * L : (uint32_t)nseg;
    // the partials [tile][range][m][8] follow the largest window (and its block
    // sums where x_sums_staged)
    float *part = (float *)(xs4 + (XLDS ? (uint32_t)M * (nsegw_max << 8) : 0u)) +
                  (x_sums_staged(QT, XLDS, NORM) ? (uint32_t)M * (nsegw_max << 5) : 0u);

    const Consts k = make_consts();

    // A cursor over this wavefront's units of the phase whose first range is r0:
    // wavefront-unit (pair) u, whose even item is 2u = rl nh + hl, and unit kk < L
    // of the items; wave-uniform (scalar registers). The wavefront's pairs are
    // u = wave, wave + G, ...: with 2 G = qH nh + rH a step to the next pair is
    // two adds and at most one wrap. A half's own item is the pair's even item
    // moved by hw (half): one add and at most one wrap, in `where`.
    struct Cur {
        uint32_t rl, hl, kk;
    };
    uint32_t r0 = 0, RP = R, qH = 0, rH = 0;
    auto advance = [&](Cur &c) {
        if (++c.kk == L) {
            c.kk = 0;
            c.hl += rH;
            c.rl += qH;
            if (c.hl >= nh) {
                c.hl -= nh;
                ++c.rl;
            }
        }
    };
    float acc[M][B];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int b = 0; b < B; ++b) acc[m][b] = 0.0f;

    for (uint32_t ph = 0; ph < P; ++ph) {
        r0 = PHASED ? R * ph / P : 0u;
        RP = PHASED ? R * (ph + 1) / P - r0 : R;
        const uint32_t nsegw = PHASED ? RP * L : (uint32_t)nseg;
        const uint32_t n_pairs = (nh * RP + 1) >> 1;
        const uint32_t my_pairs = n_pairs > (uint32_t)wave ? (n_pairs - (uint32_t)wave + G - 1) / G : 0u;
        const int64_t n_units = (int64_t)my_pairs * L;
        const int64_t s0 = PHASED ? (int64_t)r0 * L : 0;
        const float *xw = x + s0 * kSegWeights;   // the window's first activation of row 0
        const int64_t Kw = K - s0 * kSegWeights;  // activations of a row from the window on
        if (PHASED && ph > 0) __syncthreads();    // every wavefront done with the previous window
        qH = (uint32_t)(2 * G) / nh;
        rH = (uint32_t)(2 * G) - qH * nh;
        Cur ld, cu;
        {
            const uint32_t i0 = 2u * (uint32_t)wave;
            ld.rl = i0 / nh;
            ld.hl = i0 - ld.rl * nh;
            ld.kk = 0;
        }
        cu = ld;
        int64_t u_ld = 0;
        // the unit of the pair cursor c for this lane's half: its tile (relative
        // to T0), slot and segment, and whether the half has an item (the last
        // pair of a phase may have one only); a dead half reads the window's
        // first segment (in bounds; it loads zeros, and its sums are neither
        // parked nor stored)
        auto where = [&](const Cur &c, uint32_t &t_rel, uint32_t &slot, uint32_t &seg, uint32_t &r, bool &dead) {
            uint32_t hl = c.hl + hw, rl = c.rl;
            if (hl >= nh) {
                hl -= nh;
                ++rl;
            }
            dead = rl >= RP;
            const uint32_t h = h0 + hl;
            t_rel = h >> 1;
            slot = h & 1u;
            r = r0 + rl;
            seg = dead ? r0 * L : r * L + c.kk;
        };
        auto load = [&](Unit<QT> &u) {
            uint32_t t_rel, slot, seg, r;
            bool dead;
            where(ld, t_rel, slot, seg, r, dead);
            load_unit_lane<QT>(u, wp, g, T0, span, t_rel, seg, slot, j, u_ld < n_units && !dead);
            advance(ld);
            ++u_ld;
        };

        // phased windows are staged in batches of 4 (the registers of the phased
        // kernels are at their limit)
        XFirst<PHASED ? 4 : x_batch(M, true)> xf;
        if (XLDS) stage_x_issue<M>(xf, xw, a.x_stride, nsegw, Kw);
        Unit<QT> ring[S];
        load(ring[0]);

        if (XLDS) {
            stage_x_finish<M>(xf, xs4, xw, a.x_stride, nsegw, Kw);
            __syncthreads();
        }
        if (NORM) norm_staged_x(xs4, nred, a.gamma, a.eps, K);
        if (x_sums_staged(QT, XLDS, NORM)) block_x_sums<M>(xs4, nsegw);

        const uint32_t nb_last = (uint32_t)seg_blocks(g, g.nseg - 1);
        auto step = [&](Unit<QT> &cur, Unit<QT> &nxt) {
            load(nxt);
            __builtin_amdgcn_sched_barrier(0);
            uint32_t t_rel, slot, seg, r;
            bool dead;
            where(cu, t_rel, slot, seg, r, dead);
            const bool last = seg == (uint32_t)(nseg - 1);
            const int jc = last && (uint32_t)j >= nb_last ? (int)nb_last - 1 : j;
            const bool live = !last || (uint32_t)j < nb_last;
            if (ONE) {
                // every item is this one unit: its sums start from zero here, and no
                // accumulator lives from one unit to the next (the same operations:
                // the general form zeroes acc after each item)
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int b = 0; b < B; ++b) acc[m][b] = 0.0f;
            }
            compute_unit<QT, M, XLDS, NORM>(cur, acc, k, xs4, x, a.x_stride, nsegw, (int64_t)seg - s0, jc, live);
            if (ONE || cu.kk + 1 == L) {
                TileSums<M, EPI> sums;
                tile_sums<M, tile_rs<EPI>()>(acc, sums, j);
                if (!dead) {
                    if (R == 1)
                        store_tile<M, EPI>(sums, y, a, T0 + t_rel, (int)slot, j);
                    else
                        park_tile<M, EPI>(sums, part + ((size_t)t_rel * R + r) * (M * kTileRows) + slot * B, j);
                }
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int b = 0; b < B; ++b) acc[m][b] = 0.0f;
            }
            advance(cu);
        };

        const int64_t n_groups = n_units / S;
        for (int64_t gi = 0; gi < n_groups; ++gi) {
            step(ring[0], ring[1]);
            step(ring[1], ring[0]);
        }
        if (n_units - n_groups * S) step(ring[0], ring[1]);
    }

    if (R > 1) {
        // every wavefront reaches this barrier (no early exit above); each row of
        // the workgroup's own half-tiles adds its partials in range order
        __syncthreads();
        if (EPI != kEpiGateUp) {
            for (uint32_t o = tid; o < nh * (M * B); o += blockDim.x) {
                const uint32_t hl = o / (M * B), rem = o - hl * (M * B);
                const uint32_t m = rem / B, b = rem - m * B;
                const uint32_t h = h0 + hl, t_rel = h >> 1, row = (h & 1u) * B + b;
                const float *pp = part + (size_t)t_rel * R * (M * kTileRows) + m * kTileRows + row;
                float v = pp[0];
                for (uint32_t r = 1; r < R; ++r) v += pp[(size_t)r * (M * kTileRows)];
                const int64_t n = (T0 + t_rel) * kTileRows + row;
                if (n < a.n_out) store_out<M, EPI>(y, a, (int)m, n, v);
            }
        } else {
            for (uint32_t o = tid; o < nh * (B / 2); o += blockDim.x) {
                const uint32_t hl = o / (B / 2), q = o - hl * (B / 2);
                const uint32_t h = h0 + hl, t_rel = h >> 1, pr = (h & 1u) * (B / 2) + q;   // pair in the tile
                const float *pp = part + (size_t)t_rel * R * kTileRows + 2 * pr;
                float gv = pp[0], uv = pp[1];
                for (uint32_t r = 1; r < R; ++r) {
                    gv += pp[(size_t)r * kTileRows];
                    uv += pp[(size_t)r * kTileRows + 1];
                }
                const int64_t n = (T0 + t_rel) * (kTileRows / 2) + pr;
                if (n < a.n_out) y[n] = silu_mul(gv, uv);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// launch templates (host side)

template <typename Kern, typename... Args>
static void launch(Kern kern, dim3 grid, dim3 block, uint32_t lds, hipStream_t stream, Args... args)
{
    launch_timed(kern, grid, block, lds, stream, args...);
}

template <int QT, int M, int EPI, int W, bool XLDS, int D, bool NORM = false>
static hipError_t launch_q(const uint8_t *wp, const float *x, float *y, const QArgs &a, dim3 grid, int block,
                           size_t lds, hipStream_t stream)
{
    auto kern = qgemv_kernel<QT, M, EPI, W, XLDS, D, NORM>;
    static std::atomic<int> lds_set[16];
    hipError_t e = ensure_lds_limit((const void *)kern, lds, lds_set);
    if (e != hipSuccess) return e;
    launch(kern, grid, dim3(block), (uint32_t)lds, stream, wp, x, y, a);
    return hipGetLastError();
}

template <int QT, int M, int EPI, int W>
static hipError_t dispatch_x(const uint8_t *wp, const float *x, float *y, const QArgs &a, dim3 grid, int block,
                             size_t lds, bool xlds, int depth, bool norm, hipStream_t s)
{
    // the RMSNorm prologue: single-row plain and gate|up kernels, staged activations, depth 1
    if constexpr (M == 1 && EPI != kEpiAffine) {
        if (norm) {
            if (!xlds) return hipErrorInvalidConfiguration;
            return launch_q<QT, M, EPI, W, true, 1, true>(wp, x, y, a, grid, block, lds, s);
        }
    }
    if (norm) return hipErrorInvalidConfiguration;
    // prefetch depth 2 is instantiated for the single-row kernels without the
    // affine epilogue only (elsewhere a request for it runs depth 1)
    if constexpr (M == 1 && EPI != kEpiAffine) {
        if (depth >= 2)
            return xlds ? launch_q<QT, M, EPI, W, true, 2>(wp, x, y, a, grid, block, lds, s)
                        : launch_q<QT, M, EPI, W, false, 2>(wp, x, y, a, grid, block, 0, s);
    }
    return xlds ? launch_q<QT, M, EPI, W, true, 1>(wp, x, y, a, grid, block, lds, s)
                : launch_q<QT, M, EPI, W, false, 1>(wp, x, y, a, grid, block, 0, s);
}

template <int QT, int M, int EPI>
static hipError_t dispatch_w(const uint8_t *wp, const float *x, float *y, const QArgs &a, int W, dim3 grid,
                             int block, size_t lds, bool xlds, int depth, bool norm, hipStream_t s)
{
    switch (W) {
    case 1: return dispatch_x<QT, M, EPI, 1>(wp, x, y, a, grid, block, lds, xlds, depth, norm, s);
    case 2: return dispatch_x<QT, M, EPI, 2>(wp, x, y, a, grid, block, lds, xlds, depth, norm, s);
    case 3: return dispatch_x<QT, M, EPI, 3>(wp, x, y, a, grid, block, lds, xlds, depth, norm, s);
    case 4: return dispatch_x<QT, M, EPI, 4>(wp, x, y, a, grid, block, lds, xlds, depth, norm, s);
    default: return dispatch_x<QT, M, EPI, 8>(wp, x, y, a, grid, block, lds, xlds, depth, norm, s);
    }
}

template <int QT, int M, int EPI>
static hipError_t launch_persist(const uint8_t *wp, const float *x, float *y, const QArgs &a, const QPlan &p,
                                 hipStream_t stream)
{
    // ONE: every item is one unit (one segment per K range)
    auto pick = [&](auto one) -> std::pair<decltype(&qgemv_persist<QT, M, EPI, true, false>), int> {
        constexpr bool ONE = decltype(one)::value;
        if (p.phases > 1) {
            // several activation rows walked in phases (staged windows), plain store only
            if constexpr (M > 1 && EPI == kEpiPlain) {
                if (!p.x_in_lds || p.norm) return {nullptr, 0};
                return {qgemv_persist<QT, M, EPI, true, false, true, ONE>, 3};
            } else {
                return {nullptr, 0};
            }
        }
        if (p.norm) {
            // the RMSNorm prologue: single-row plain and gate|up kernels with staged activations
            if constexpr (M == 1 && EPI != kEpiAffine) {
                if (!p.x_in_lds) return {nullptr, 0};
                return {qgemv_persist<QT, M, EPI, true, true, false, ONE>, 2};
            } else {
                return {nullptr, 0};
            }
        }
        return p.x_in_lds ? std::make_pair(qgemv_persist<QT, M, EPI, true, false, false, ONE>, 0)
                          : std::make_pair(qgemv_persist<QT, M, EPI, false, false, false, ONE>, 1);
    };
    const auto kw = p.one_unit ? pick(std::true_type{}) : pick(std::false_type{});
    const auto kern = kw.first;
    const int which = kw.second + (p.one_unit ? 4 : 0);
    if (kern == nullptr) return hipErrorInvalidConfiguration;
    if (p.block != persist_threads(QT, M, p.x_in_lds, p.one_unit, p.phases > 1)) return hipErrorInvalidConfiguration;
    static std::atomic<int> lds_set[8][16];   // one record per kernel chosen above
    hipError_t e = ensure_lds_limit((const void *)kern, p.lds_bytes, lds_set[which]);
    if (e != hipSuccess) return e;
    launch(kern, dim3((unsigned)p.grid), dim3(p.block), (uint32_t)p.lds_bytes, stream, wp, x, y, a);
    return hipGetLastError();
}

template <int QT, int M, int EPI>
static hipError_t dispatch_form(const uint8_t *wp, const float *x, float *y, const QArgs &a, const QPlan &p,
                                hipStream_t s)
{
    if (p.persist) {
        if (p.row_groups != 1) return hipErrorInvalidConfiguration;
        return launch_persist<QT, M, EPI>(wp, x, y, a, p, s);
    }
    if (p.row_groups < 1 || (p.row_groups > 1 && EPI != kEpiPlain)) return hipErrorInvalidConfiguration;
    return dispatch_w<QT, M, EPI>(wp, x, y, a, p.W, dim3((unsigned)p.grid, (unsigned)p.row_groups), p.block,
                                  p.lds_bytes, p.x_in_lds, p.depth, p.norm, s);
}

// The single-row calls of type QT: plain, gate|up and affine epilogues, with or
// without the RMSNorm prologue.
template <int QT>
hipError_t launch_qgemv_m1(int epi, const QPlan &p, const uint8_t *wp, const float *x, float *y, const QArgs &a,
                           hipStream_t s)
{
    if (epi == kEpiGateUp) return dispatch_form<QT, 1, kEpiGateUp>(wp, x, y, a, p, s);
    if (epi == kEpiAffine) return dispatch_form<QT, 1, kEpiAffine>(wp, x, y, a, p, s);
    return dispatch_form<QT, 1, kEpiPlain>(wp, x, y, a, p, s);
}

// The verify calls of type QT with M activation rows (plain store).
template <int QT, int M>
hipError_t launch_qgemv_rows(const QPlan &p, const uint8_t *wp, const float *x, float *y, const QArgs &a,
                             hipStream_t s)
{
    return dispatch_form<QT, M, kEpiPlain>(wp, x, y, a, p, s);
}

}  // namespace qgk
