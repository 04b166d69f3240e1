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

#include <algorithm>
#include <type_traits>

#include "dequant.h"
#include "layout.h"
#include "qgemm_kernels.h"
#include "qgemv_kernels.h"

namespace qgk {

using namespace qgl;

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// Activation split: gridDim.y workgroups per activation row m = blockIdx.x
// (rows M..M_pad-1 of the last 16-row tile are written as zeros). Writes
// unscale[m] = 2^-e and the fp16 parts in B-operand order:
// xs[((mt * KB + b) * 2 + h) * 512 + lane * 8 + e] with mt = m / 16,
// lane = 16 c + m % 16, h = 0 (hi) / 1 (lo), where (c, e) is the position of the
// block's element in its lane (see above). Every workgroup of a row finds the
// row's maximum itself (the same value), then splits its share of the row's
// lane runs (block b, chunk c: the 8 elements one MFMA lane holds), writing
// their hi and lo parts as two 16-byte stores. Loads are issued four at a time
// per thread. VEC: the row is 16-byte aligned and read with 16-byte loads.
constexpr int kSplitThreads = 256;

// The 8 activations of lane run u of row xr: Q4_0 elements 8c..8c+7 of block
// b = u / 4 (c = u % 4), Q8_0 elements 4c..4c+3 and 16+4c..16+4c+3.
template <int QT, bool VEC>
__device__ inline void split_load_run(const float *__restrict__ xr, int64_t u, float (&v)[8])
{
    const int64_t b = u >> 2;
    const int c = (int)(u & 3);
    const int64_t k0 = b * 32 + (QT == kQ4_0 ? 8 * c : 4 * c);
    const int64_t k1 = QT == kQ4_0 ? k0 + 4 : k0 + 16;
    if (VEC) {
        const f32x4 a0 = *(const f32x4 *)(xr + k0);
        const f32x4 a1 = *(const f32x4 *)(xr + k1);
        v[0] = a0.x; v[1] = a0.y; v[2] = a0.z; v[3] = a0.w;
        v[4] = a1.x; v[5] = a1.y; v[6] = a1.z; v[7] = a1.w;
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[j] = xr[k0 + j];
            v[4 + j] = xr[k1 + j];
        }
    }
}

// 2^e with max|x| * 2^e in [2^14, 2^15); 1 for a zero or non-finite maximum.
__device__ inline int split_exponent(float mx)
{
    int e = 0;
    if (mx > 0.0f && mx <= 3.4028234663852886e38f) {
        int E;
        (void)__builtin_frexpf(mx, &E);   // mx = f * 2^E, f in [0.5, 1)
        e = 15 - E;
        e = e < -126 ? -126 : (e > 127 ? 127 : e);
    }
    return e;
}

// The hi and lo parts of lane run u of activation row m (scaled by sc), as two
// 16-byte stores at the run's B-operand position.
__device__ inline void split_store_run(_Float16 *__restrict__ xs, int64_t m, int64_t KB, int64_t u,
                                       const float (&v)[8], float sc)
{
    const int64_t b = u >> 2;
    const int c = (int)(u & 3);
    h8 hi, lo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float t = v[j] * sc;
        const _Float16 h = (_Float16)t;
        hi[j] = h;
        lo[j] = (_Float16)(t - (float)h);
    }
    _Float16 *dst = xs + (((m >> 4) * KB + b) * 2) * 512 + (int64_t)(c * 16 + (int)(m & 15)) * 8;
    *(h8 *)dst = hi;
    *(h8 *)(dst + 512) = lo;
}

template <int QT, bool VEC>
__global__ void __launch_bounds__(kSplitThreads)
split_x_kernel(const float *__restrict__ X, _Float16 *__restrict__ xs, float *__restrict__ unscale, int64_t M,
               int64_t K)
{
    constexpr int T = kSplitThreads;
    __shared__ float red[T / 64];
    const int64_t m = blockIdx.x;
    const int tid = threadIdx.x;
    const bool live = m < M;
    const float *xr = X + m * K;
    float mx = 0.0f;
    if (live) {
        if (VEC) {
            const f32x4 *x4 = (const f32x4 *)xr;
            const int64_t K4 = K / 4;
            for (int64_t k = tid; k < K4; k += 4 * T) {
                f32x4 v[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) v[j] = k + j * T < K4 ? x4[k + j * T] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    mx = __builtin_fmaxf(mx, __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(v[j].x), __builtin_fabsf(v[j].y)),
                                                             __builtin_fmaxf(__builtin_fabsf(v[j].z), __builtin_fabsf(v[j].w))));
            }
        } else {
            for (int64_t k = tid; k < K; k += 4 * T) {
                float v[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) v[j] = k + j * T < K ? xr[k + j * T] : 0.0f;
#pragma unroll
                for (int j = 0; j < 4; ++j) mx = __builtin_fmaxf(mx, __builtin_fabsf(v[j]));
            }
        }
    }
    // workgroup maximum (max is exact, so the order does not matter)
    for (int o = 32; o >= 1; o >>= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, o));
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    mx = red[0];
    for (int w = 1; w < T / 64; ++w) mx = __builtin_fmaxf(mx, red[w]);
    const int e = split_exponent(mx);
    const float sc = __builtin_ldexpf(1.0f, e);
    if (tid == 0 && blockIdx.y == 0) unscale[m] = __builtin_ldexpf(1.0f, -e);
    const int64_t KB = K / 32;
    // this workgroup's lane runs u in [u0, u1)
    const int64_t U = KB * 4;
    const int64_t u0 = U * blockIdx.y / gridDim.y, u1 = U * (blockIdx.y + 1) / gridDim.y;
    auto run = [&](int64_t u) {
        float v[8];
        if (live) {
            split_load_run<QT, VEC>(xr, u, v);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = 0.0f;
        }
        split_store_run(xs, m, KB, u, v, sc);
    };
    int64_t u = u0 + tid;
    for (; u + T < u1; u += 2 * T) {   // two runs per thread in flight
        run(u);
        run(u + T);
    }
    if (u < u1) run(u);
}

// Activation split in one pass: one workgroup per activation row, thread t
// holding the lane runs t, t + T, ..., t + (R - 1) T of the row (T = blockDim)
// in registers. The row is read once; its maximum is taken from the registers
// and the hi and lo parts are written from them, so the pass costs one memory
// round trip where split_x_kernel takes two or more (a maximum pass and a
// split pass). The parts are the same values as split_x_kernel's.
template <int QT, bool VEC, int R>
__global__ void __launch_bounds__(1024)
split_x_row_kernel(const float *__restrict__ X, _Float16 *__restrict__ xs, float *__restrict__ unscale,
                   int64_t M, int64_t K)
{
    __shared__ float red[16];
    const int64_t m = blockIdx.x;
    const int tid = threadIdx.x, T = blockDim.x;
    const bool live = m < M;
    const float *xr = X + m * K;
    const int64_t KB = K / 32, U = KB * 4;
    float v[R][8];
    float mx = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t u = tid + (int64_t)r * T;
        if (live && u < U) {
            split_load_run<QT, VEC>(xr, u, v[r]);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[r][j] = 0.0f;
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < 8; ++j) mx = __builtin_fmaxf(mx, __builtin_fabsf(v[r][j]));
    // workgroup maximum (max is exact, so the order does not matter)
    for (int o = 32; o >= 1; o >>= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, o));
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    mx = red[0];
    for (int w = 1; w < T / 64; ++w) mx = __builtin_fmaxf(mx, red[w]);
    const int e = split_exponent(mx);
    const float sc = __builtin_ldexpf(1.0f, e);
    if (tid == 0) unscale[m] = __builtin_ldexpf(1.0f, -e);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t u = tid + (int64_t)r * T;
        if (u < U) split_store_run(xs, m, KB, u, v[r], sc);
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
// The GEMM. Workgroup (row block rb, activation group mg) of G wavefronts owns
// the 16 RG G weight rows of row block rb (wavefront w: row tiles 2 RG (rb G + w)
// + 2 rg and + 1 for row group rg) and the MT 16-row activation tiles
// [mg MT, mg MT + MT); blockIdx.x = rb * n_mg + mg, so the groups that read the
// same weights are launched next to each other. K is walked in chunks of
// kGemmChunk blocks through a ring of kGemmRing staging buffers: while chunk c is
// computed, the loads of chunks c + 1 and c + 2 are in flight (the time of two
// chunks of matrix-core work covers the memory latency). Per chunk every
// wavefront issues the same number of loads:
//   * its share of the chunk's split activations, 1 KiB pieces copied with
//     LDS-direct loads (global_load_lds, no registers), MT x kGemmChunk x 2 pieces
//     over the G wavefronts;
//   * one 64-lane copy of the scales of the workgroup's rows (LDS-direct);
//   * its weights: load groups of 4 (Q4_0) or 2 (Q8_0) blocks, one 16-byte load
//     per lane and row group (LDS-direct as well: no load has a register
//     destination, so nothing but the one wait per chunk waits for them).
// A ragged chunk (the end of a ragged K segment) re-reads valid pieces into
// slots nobody reads, so the counts, and with them the one vmcnt wait per chunk,
// stay fixed; one barrier per chunk then hands the staged data to every
// wavefront and frees the buffer the next loads take. Per block and activation
// tile each wavefront runs two MFMAs (hi, lo) per row group, each B operand read
// once from LDS and used by the RG row groups, then acc = fma(d, S, acc). Block
// sums are added per segment of 32 blocks and the segment sums in order; with
// a.ksplit > 1, workgroup row blockIdx.y takes one range of chunks and writes its
// sums to a.part, which launch_ksum adds in range order.
//
// Addressing: the chunk loop is unrolled over the three ring buffers, so every
// LDS address is a per-lane base plus a constant. In a full segment of 32
// blocks each load is a wave-uniform base (advanced per chunk on the scalar
// unit) plus a 32-bit per-lane offset fixed for the whole walk; only the chunks
// of a ragged last segment take the general address arithmetic.
template <int V>
using IntC = std::integral_constant<int, V>;

typedef const __attribute__((address_space(1))) void *gvoid;
typedef __attribute__((address_space(3))) void *lvoid;

template <int QT, int MT, int RG, int G>
__global__ void __launch_bounds__(64 * G)
qgemm_kernel(const uint8_t *__restrict__ wp, const _Float16 *__restrict__ xs, const float *__restrict__ unscale,
             float *__restrict__ Y, GemmArgs a)
{
    constexpr int NH = (QT == kQ8_0) ? 2 : 1;
    constexpr int BPG = (QT == kQ8_0) ? 2 : 4;   // blocks per load group
    constexpr int CB = kGemmChunk;               // blocks per staged chunk
    constexpr int NG = CB / BPG;                 // load groups per chunk
    constexpr int PIECES = MT * CB * 2;          // 1 KiB activation pieces per chunk
    static_assert(PIECES % G == 0, "every wavefront copies the same number of pieces");
    constexpr int PPW = PIECES / G;
    constexpr int XBUF = MT * CB * 128;          // u32x4 per activation buffer
    constexpr int SBUF = G * kGemmScaleWordsPerWave;
    constexpr int WBUF = G * NG * RG * 64;       // u32x4 per weight buffer
    constexpr int WG_TILES = 2 * RG * G;         // 8-row tiles per workgroup
    constexpr int SWORDS = WG_TILES * 2 * CB * 2;   // scale words of a chunk: tile x slot x block x 8 B
    static_assert(SWORDS <= SBUF, "one scale copy per wavefront");
    constexpr int LOADS = PPW + 1 + NG * RG;     // vector-memory loads per chunk and wavefront
    static_assert((kGemmDepth - 1) * LOADS < 64, "vmcnt range");
    static_assert(kGemmDepth == 2 && kGemmRing == 3, "the chunk loop below is unrolled for a ring of three");
    constexpr int CPS = kSegBlocks / CB;
    static_assert(CPS == 8, "chunk positions below use shifts by 3");
    // LDS: kGemmRing activation buffers of XBUF u32x4, then kGemmRing weight
    // buffers of WBUF u32x4, then kGemmRing scale buffers of SBUF words
    extern __shared__ u32x4 lds[];

    const Geometry &g = a.geo;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: its arithmetic stays scalar
    const int i = lane & 15, c = lane >> 4;
    const int64_t mg = (int64_t)blockIdx.x % a.n_mg;
    const int64_t rb = (int64_t)blockIdx.x / a.n_mg;
    const int64_t mt0 = mg * MT;
    const int64_t wg_tile0 = rb * WG_TILES;                       // first row tile of the workgroup
    const int64_t t_first = wg_tile0 + (int64_t)wave * 2 * RG;    // first row tile of this wavefront
    const int64_t t_last = g.n_tiles - 1;
    const int slotA = (i & 7) >> 2, browA = i & 3;
    // every lane's A-row tile lies at or after tb (tiles past the end are clamped to the last)
    const int64_t tb = t_first < t_last ? t_first : t_last;
    uint32_t w_tile[RG];   // byte offset of this lane's A-row tile (row group rg) from tile tb
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        int64_t t = t_first + 2 * rg + (i >> 3);
        t = t < t_last ? t : t_last;
        w_tile[rg] = (uint32_t)((t - tb) * g.tile_q);
    }
    const uint8_t *w_wave = wp + tb * g.tile_q;
    const Consts k = make_consts();
    constexpr int64_t seg_q = (int64_t)kTileRows * kSegBlocks * NH * kUnit;
    constexpr int64_t seg_s = (int64_t)kTileRows * kSegBlocks * 2;

    f32x4 tot[RG][MT], seg[RG][MT];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) tot[rg][mt] = seg[rg][mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // K as a flat sequence of chunks: every segment but the matrix's last holds
    // 32 / CB of them, and chunk ch covers blocks [ch CB, ch CB + CB) of the whole
    // K (the split activations are laid out block after block); workgroup row ky
    // takes chunks [c_begin, c_end).
    const int64_t nseg_last = g.nseg - 1;
    const int nb_last = (int)seg_blocks(g, nseg_last);
    const bool ragged = nb_last < kSegBlocks;   // the last segment takes the general path
    const int64_t n_all = nseg_last * CPS + (nb_last + CB - 1) / CB;
    const int64_t ky = blockIdx.y;
    const int64_t c_begin = n_all * ky / a.ksplit, c_end = n_all * (ky + 1) / a.ksplit;
    const int n = (int)(c_end - c_begin);
    const int64_t KB = g.KB;

    // Activations: this wavefront's pieces q = wave + G t of a full chunk are
    // (tile q / 2CB, 1 KiB piece q % 2CB); byte offsets from the chunk's start
    // (global) and from the buffer's start (LDS).
    const uint8_t *x_wg = (const uint8_t *)xs + mt0 * KB * 2048;
    const uint32_t lane16 = (uint32_t)lane * 16;
    int64_t x_off[PPW];
    int l_off[PPW];
#pragma unroll
    for (int t = 0; t < PPW; ++t) {
        const int q = wave + G * t, mt = q / (2 * CB), r = q % (2 * CB);
        x_off[t] = (int64_t)mt * KB * 2048 + r * 1024;
        l_off[t] = (mt * CB * 128 + r * 64) * 16;
    }
    // Weights: lane (i, c) loads row i's unit of block jq = 4q + c (Q4_0) or
    // 2q + c/2, half c%2 (Q8_0) of the load group; unit (b, h, slot, j) of a
    // segment with nb blocks sits at ((b NH + h) kSlots + slot) nb + j.
    const int hh = (QT == kQ4_0) ? 0 : (c & 1);
    const int lane_unit = (browA * NH + hh) * kSlots + slotA;
    auto jq = [&](int q) { return (QT == kQ4_0) ? 4 * q + c : 2 * q + (c >> 1); };
    uint32_t w_lane[NG][RG];   // in a full segment: the lane's byte offset from the chunk's base
#pragma unroll
    for (int q = 0; q < NG; ++q)
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) w_lane[q][rg] = w_tile[rg] + (uint32_t)((lane_unit * kSegBlocks + jq(q)) * kUnit);
    // Scales: word wi = wave 64 + lane of a chunk = (run = tile x 2 + slot, block jj, half).
    int sc_tl, sc_sl, sc_jj, sc_half;
    {
        int wi = wave * kGemmScaleWordsPerWave + lane;
        wi = wi < SWORDS ? wi : 0;
        const int srun = wi / (2 * CB), within = wi - srun * (2 * CB);
        const int tl_last = (int)(t_last - wg_tile0);
        sc_tl = (srun >> 1) < tl_last ? (srun >> 1) : tl_last;
        sc_sl = srun & 1;
        sc_jj = within >> 1;
        sc_half = within & 1;
    }
    const uint8_t *s_wg = wp + g.scale_off + wg_tile0 * g.tile_s;
    const uint32_t s_tile = (uint32_t)(sc_tl * g.tile_s + sc_half * 4);
    const uint32_t s_lane = s_tile + (uint32_t)((sc_sl * kSegBlocks + sc_jj) * (kRowsPerLane * 2));

    // LDS byte addresses this lane reads (buffer 0; the others at constant distances)
    const int lx_lane = lane * 16;
    const int lw_lane = (kGemmRing * XBUF + wave * NG * RG * 64 + lane) * 16;
    const int ls_lane = kGemmRing * (XBUF + WBUF) * 16 + (((wave * RG * 2 + (c >> 1)) * 2 + (c & 1)) * CB) * 8;
    const uint8_t *lds_b = (const uint8_t *)lds;

    // The LOADS loads of a chunk ch of a full segment into ring buffer BUF, as
    // one list (the weights, then the scales, then the activation pieces), of
    // which entries [lo, hi) are issued.
    auto issue_full = [&](auto BUF, int64_t ch, int lo, int hi) {
        const int B = BUF;
        const int64_t s = ch >> 3;
        const int j0 = (int)(ch & 7) * CB;
        uint8_t *lb = (uint8_t *)lds;
        const uint8_t *wu = w_wave + (s * seg_q + j0 * kUnit);
        const uint8_t *xu = x_wg + ch * (CB * 2048);
#pragma unroll
        for (int l = 0; l < LOADS; ++l) {
            if (l < lo || l >= hi) continue;
            if (l < NG * RG) {
                const int q = l / RG, rg = l % RG;
                __builtin_amdgcn_global_load_lds(
                    (gvoid)(wu + w_lane[q][rg]),
                    (lvoid)(lb + (kGemmRing * XBUF + B * WBUF + ((wave * NG + q) * RG + rg) * 64) * 16), 16, 0, 0);
            } else if (l == NG * RG) {
                __builtin_amdgcn_global_load_lds(
                    (gvoid)(s_wg + (s * seg_s + j0 * (kRowsPerLane * 2)) + s_lane),
                    (lvoid)(lb + kGemmRing * (XBUF + WBUF) * 16 + (B * SBUF + wave * kGemmScaleWordsPerWave) * 4), 4,
                    0, 0);
            } else {
                const int t = l - NG * RG - 1;
                __builtin_amdgcn_global_load_lds((gvoid)(xu + x_off[t] + lane16),
                                                 (lvoid)(lb + B * XBUF * 16 + l_off[t]), 16, 0, 0);
            }
        }
    };

    // The loads of any chunk ch into ring buffer BUF, all at once.
    auto issue = [&](auto BUF, int64_t ch) {
        const int B = BUF;
        const int64_t s = ch >> 3;
        const int j0 = (int)(ch & 7) * CB;
        const uint8_t *xu = x_wg + ch * (CB * 2048);
        uint8_t *lb = (uint8_t *)lds;
        if (!(ragged && s == nseg_last)) {
            issue_full(BUF, ch, 0, LOADS);
            return;
        }
        // a chunk of the ragged last segment (nb_last blocks)
        const int nb = nb_last;
        const int nbc = nb - j0 < CB ? nb - j0 : CB;
        if (nbc == CB) {
#pragma unroll
            for (int t = 0; t < PPW; ++t)
                __builtin_amdgcn_global_load_lds((gvoid)(xu + x_off[t] + lane16),
                                                 (lvoid)(lb + B * XBUF * 16 + l_off[t]), 16, 0, 0);
        } else {
            // tile runs of nbc x 2 KiB; spare copies re-read piece 0
            const int run = nbc * 2;
#pragma unroll
            for (int t = 0; t < PPW; ++t) {
                int q = wave + G * t;
                q = q < MT * run ? q : 0;
                const int mt = q / run, r = q - mt * run;
                __builtin_amdgcn_global_load_lds((gvoid)(xu + (int64_t)mt * KB * 2048 + r * 1024 + lane16),
                                                 (lvoid)(lb + B * XBUF * 16 + (mt * CB * 128 + r * 64) * 16), 16, 0,
                                                 0);
            }
        }
        {
            const int jj = sc_jj < nbc ? sc_jj : nbc - 1;
            const uint8_t *src = s_wg + s * seg_s + s_tile + (uint32_t)((sc_sl * nb + j0 + jj) * (kRowsPerLane * 2));
            __builtin_amdgcn_global_load_lds(
                (gvoid)src, (lvoid)(lb + kGemmRing * (XBUF + WBUF) * 16 + (B * SBUF + wave * kGemmScaleWordsPerWave) * 4),
                4, 0, 0);
        }
        const uint8_t *wu = w_wave + s * seg_q;
#pragma unroll
        for (int q = 0; q < NG; ++q) {
            int jb = j0 + jq(q);
            jb = jb < nb ? jb : nb - 1;   // past a ragged segment's end: a valid unit, never used
#pragma unroll
            for (int rg = 0; rg < RG; ++rg)
                __builtin_amdgcn_global_load_lds(
                    (gvoid)(wu + w_tile[rg] + (uint32_t)((lane_unit * nb + jb) * kUnit)),
                    (lvoid)(lb + (kGemmRing * XBUF + B * WBUF + ((wave * NG + q) * RG + rg) * 64) * 16), 16, 0, 0);
        }
    };

    // Chunk computation from ring buffer BUF: nbc valid blocks (CB in a full
    // segment, a compile-time constant there).
    auto compute = [&](auto BUF, auto NBC, auto hook) {
        const int B = BUF;
        const int nbc = NBC;
        uint32_t v[NG][RG][4];
#pragma unroll
        for (int q = 0; q < NG; ++q)
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
                const u32x4 w = *(const u32x4 *)(lds_b + lw_lane + (B * WBUF + (q * RG + rg) * 64) * 16);
                v[q][rg][0] = w.x;
                v[q][rg][1] = w.y;
                v[q][rg][2] = w.z;
                v[q][rg][3] = w.w;
            }
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
                    const u32x2 dd = *(const u32x2 *)(lds_b + ls_lane + B * SBUF * 4 + (rg * 4 * CB + jj) * 8);
                    d01[rg] = as_h2(dd.x);
                    d23[rg] = as_h2(dd.y);
                }
                // every MFMA of the block first, then the scale fmas: an fma never
                // waits right behind the MFMA that feeds it
                f32x4 S[MT][RG];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const uint8_t *xb = lds_b + lx_lane + (B * XBUF + (mt * CB + jj) * 128) * 16;
                    const h8 bh = *(const h8 *)xb;
                    const h8 bl = *(const h8 *)(xb + 1024);
#pragma unroll
                    for (int rg = 0; rg < RG; ++rg)
                        S[mt][rg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[rg], bh, f32x4{0.0f, 0.0f, 0.0f, 0.0f},
                                                                           0, 0, 0);
#pragma unroll
                    for (int rg = 0; rg < RG; ++rg)
                        S[mt][rg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[rg], bl, S[mt][rg], 0, 0, 0);
                }
                hook(jj);   // loads of a later chunk, issued while the matrix cores work
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int rg = 0; rg < RG; ++rg) {
                        f32x4 &acc = seg[rg][mt];
                        acc.x = __builtin_fmaf((float)d01[rg].x, S[mt][rg].x, acc.x);
                        acc.y = __builtin_fmaf((float)d01[rg].y, S[mt][rg].y, acc.y);
                        acc.z = __builtin_fmaf((float)d23[rg].x, S[mt][rg].z, acc.z);
                        acc.w = __builtin_fmaf((float)d23[rg].y, S[mt][rg].w, acc.w);
                    }
            }
        }
    };

    // the segment's last chunk: add its sum, in segment order
    auto end_segment = [&]() {
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
    };

    // Step ci (ring buffer BUF = ci % 3): wait for chunk ci's loads (the LOADS
    // of chunk ci + 1 may stay in flight), synchronise, then compute chunk ci
    // and issue chunk ci + 2 into the buffers chunk ci - 1 used. FULL: chunks ci
    // and ci + 2 lie in full segments or ci + 2 is past the range, BUF is a
    // compile-time buffer, and the loads are spread over the chunk's blocks (past
    // the range they re-read the range's first chunk into the free buffer, so
    // every step issues the same loads).
    auto step = [&](auto BUF, auto FULL, int ci) {
        const int B = BUF;
        if (ci + 1 < n)
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(LOADS));
        else
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        // Every wavefront's chunk-ci copies are in LDS once it passes its wait, and
        // every wavefront is done reading chunk ci - 1's buffers (its reads fed the
        // matrix cores in the previous step). A plain s_barrier: a fenced one
        // would wait for the loads of chunk ci + 1 as well (they write LDS). The
        // memory clobber keeps the compiler from moving LDS accesses across it.
        asm volatile("s_barrier" ::: "memory");
        if constexpr (decltype(FULL)::value) {
            constexpr int BC = decltype(BUF)::value;
            const int64_t ch2 = ci + kGemmDepth < n ? c_begin + ci + kGemmDepth : c_begin;
            compute(BUF, IntC<CB>{}, [&](int jj) {
                issue_full(IntC<(BC + kGemmDepth) % kGemmRing>{}, ch2, jj * LOADS / CB, (jj + 1) * LOADS / CB);
            });
            if (((c_begin + ci) & 7) == CPS - 1) end_segment();
        } else {
            if (ci + kGemmDepth < n) {
                const int nb2 = B + kGemmDepth < kGemmRing ? B + kGemmDepth : B + kGemmDepth - kGemmRing;
                issue(nb2, c_begin + ci + kGemmDepth);
            }
            const int64_t cc = c_begin + ci;
            const int cj0 = (int)(cc & 7) * CB;
            const int cnb = (cc >> 3) == nseg_last ? nb_last : kSegBlocks;
            const int nbc = cnb - cj0 < CB ? cnb - cj0 : CB;
            compute(B, nbc, [](int) {});
            if (cj0 + nbc == cnb) end_segment();
        }
    };

    // Chunks [0, n_full) of the range lie in full segments. The unrolled walk
    // takes three steps at a time while the chunks it computes are full and the
    // chunks it loads are full or past the range; the rest (a ragged last
    // segment and the steps before it that load its chunks, one or two steps
    // at the end) take the general step.
    int n_full = n;
    if (ragged) {
        const int64_t f = nseg_last * CPS - c_begin;
        n_full = f < 0 ? 0 : (f < n ? (int)f : n);
    }
    const int n_fast = n_full == n ? n : n_full - kGemmDepth;
    if (n > 0) issue(IntC<0>{}, c_begin);
    if (n > 1) issue(IntC<1>{}, c_begin + 1);
    int ci = 0;
    for (; ci + kGemmRing <= n_fast; ci += kGemmRing) {
        step(IntC<0>{}, std::true_type{}, ci);
        step(IntC<1>{}, std::true_type{}, ci + 1);
        step(IntC<2>{}, std::true_type{}, ci + 2);
    }
    for (; ci < n; ++ci) step(ci % kGemmRing, std::false_type{}, ci);
    // the unrolled walk's last steps may leave re-reads in flight: they write LDS
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

    // a range that ends inside a segment (K split) adds the segment's part
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            tot[rg][mt].x += seg[rg][mt].x;
            tot[rg][mt].y += seg[rg][mt].y;
            tot[rg][mt].z += seg[rg][mt].z;
            tot[rg][mt].w += seg[rg][mt].w;
        }

#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int64_t m = (mt0 + mt) * 16 + i;
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
    const bool vec = ((uintptr_t)X & 15) == 0;   // rows are K * 4 bytes, a multiple of 128
    const int64_t U = K / 32 * 4;                 // lane runs per row
    if (U <= 4 * 1024) {
        // one pass: one workgroup per row, at most 4 runs per thread
        const int R = U <= 1024 ? 1 : (U <= 2048 ? 2 : 4);
        const int64_t T = std::min<int64_t>(1024, (U + 63) / 64 * 64);
        const dim3 grid((unsigned)M_pad), block((unsigned)T);
        auto go = [&](auto q, auto v) {
            constexpr int Q = decltype(q)::value;
            constexpr bool V = decltype(v)::value;
            switch (R) {
            case 1: hipLaunchKernelGGL((split_x_row_kernel<Q, V, 1>), grid, block, 0, s, X, xs, unscale, M, K); break;
            case 2: hipLaunchKernelGGL((split_x_row_kernel<Q, V, 2>), grid, block, 0, s, X, xs, unscale, M, K); break;
            default: hipLaunchKernelGGL((split_x_row_kernel<Q, V, 4>), grid, block, 0, s, X, xs, unscale, M, K); break;
            }
        };
        using Q8 = std::integral_constant<int, kQ8_0>;
        using Q4 = std::integral_constant<int, kQ4_0>;
        if (qt == kQ8_0) {
            if (vec) go(Q8{}, std::true_type{}); else go(Q8{}, std::false_type{});
        } else {
            if (vec) go(Q4{}, std::true_type{}); else go(Q4{}, std::false_type{});
        }
        return hipGetLastError();
    }
    // longer rows: the two-pass form, up to four workgroups per row while fewer
    // than 256 rows fill the chip, at least 512 lane runs (4096 elements) each
    int64_t per_row = std::min<int64_t>(4, std::max<int64_t>(1, 256 / M_pad));
    per_row = std::max<int64_t>(1, std::min<int64_t>(per_row, K / 8 / 512));
    const dim3 grid((unsigned)M_pad, (unsigned)per_row), block(kSplitThreads);
    if (qt == kQ8_0) {
        if (vec)
            hipLaunchKernelGGL((split_x_kernel<kQ8_0, true>), grid, block, 0, s, X, xs, unscale, M, K);
        else
            hipLaunchKernelGGL((split_x_kernel<kQ8_0, false>), grid, block, 0, s, X, xs, unscale, M, K);
    } else {
        if (vec)
            hipLaunchKernelGGL((split_x_kernel<kQ4_0, true>), grid, block, 0, s, X, xs, unscale, M, K);
        else
            hipLaunchKernelGGL((split_x_kernel<kQ4_0, false>), grid, block, 0, s, X, xs, unscale, M, K);
    }
    return hipGetLastError();
}

template <int QT, int MT, int RG, int G>
static hipError_t launch_one(int64_t row_blocks, const uint8_t *wp, const _Float16 *xs, const float *unscale, float *Y,
                             const GemmArgs &a, hipStream_t s)
{
    auto kern = qgemm_kernel<QT, MT, RG, G>;
    const dim3 grid3((unsigned)(row_blocks * a.n_mg), (unsigned)a.ksplit);
    const size_t lds = gemm_lds_bytes(QT, MT, RG, G);
    static std::atomic<int> lds_set[16];
    hipError_t e = ensure_lds_limit((const void *)kern, lds, lds_set);
    if (e != hipSuccess) return e;
    launch_timed(kern, grid3, dim3(64 * G), (uint32_t)lds, s, wp, xs, unscale, Y, a);
    return hipGetLastError();
}

template <int QT, int MT, int RG>
static hipError_t launch_g(int G, int64_t rbs, const uint8_t *wp, const _Float16 *xs, const float *unscale, float *Y,
                           const GemmArgs &a, hipStream_t s)
{
    switch (G) {
    case 1: return launch_one<QT, MT, RG, 1>(rbs, wp, xs, unscale, Y, a, s);
    case 2: return launch_one<QT, MT, RG, 2>(rbs, wp, xs, unscale, Y, a, s);
    case 4: return launch_one<QT, MT, RG, 4>(rbs, wp, xs, unscale, Y, a, s);
    case 8: return launch_one<QT, MT, RG, 8>(rbs, wp, xs, unscale, Y, a, s);
    default: return hipErrorInvalidConfiguration;
    }
}

template <int QT, int MT>
static hipError_t launch_rg(int RG, int G, int64_t rbs, const uint8_t *wp, const _Float16 *xs, const float *unscale,
                            float *Y, const GemmArgs &a, hipStream_t s)
{
    if (RG == 1) return launch_g<QT, MT, 1>(G, rbs, wp, xs, unscale, Y, a, s);
    if (RG == 2) return launch_g<QT, MT, 2>(G, rbs, wp, xs, unscale, Y, a, s);
    return hipErrorInvalidConfiguration;
}

template <int QT>
static hipError_t launch_mt(int MT, int RG, int G, int64_t rbs, const uint8_t *wp, const _Float16 *xs,
                            const float *unscale, float *Y, const GemmArgs &a, hipStream_t s)
{
    switch (MT) {
    case 1: return launch_rg<QT, 1>(RG, G, rbs, wp, xs, unscale, Y, a, s);
    case 2: return launch_rg<QT, 2>(RG, G, rbs, wp, xs, unscale, Y, a, s);
    case 3: return launch_rg<QT, 3>(RG, G, rbs, wp, xs, unscale, Y, a, s);
    case 4: return launch_rg<QT, 4>(RG, G, rbs, wp, xs, unscale, Y, a, s);
    default: return hipErrorInvalidConfiguration;
    }
}

hipError_t launch_qgemm(int qt, int MT, int RG, int G, int64_t row_blocks, const uint8_t *wp, const _Float16 *xs,
                        const float *unscale, float *Y, const GemmArgs &a, hipStream_t s)
{
    if (qt == kQ8_0) return launch_mt<kQ8_0>(MT, RG, G, row_blocks, wp, xs, unscale, Y, a, s);
    return launch_mt<kQ4_0>(MT, RG, G, row_blocks, wp, xs, unscale, Y, a, s);
}

}  // namespace qgk
