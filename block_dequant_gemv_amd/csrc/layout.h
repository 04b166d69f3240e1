// layout.h -- the packed weight layout of libqgemv (host and device).
//
// The canonical GGUF-style blocks (34 B Q8_0 / 18 B Q4_0: fp16 scale then the
// quants) are not 16-byte aligned, so a wavefront cannot stream them with
// 16-byte-per-lane loads. At load time they are re-tiled into two planes:
//
//   quant plane: [tile][segment][b][h][slot][j] 16-byte units
//   scale plane: [tile][segment][slot][j][b]    fp16 scales
//
//   tile     8 consecutive rows (row = tile*8 + slot*4 + b)
//   segment  32 consecutive blocks of a row (1024 weights); the last segment
//            of a row holds nb = KB - 32*segment blocks when K % 1024 != 0
//   slot     which half of the wavefront (lanes 0-31 / 32-63) owns the row
//   j        lane within the slot = block within the segment
//   b        one of the 4 rows a lane works on at once (register blocking)
//   h        Q8_0 only: first or second 16 quants of the block
//
// With this order the lanes of a wavefront read one contiguous 1 KiB run per
// load instruction (64 lanes x 16 B), each lane's 16 bytes belong to one
// block, and a wavefront walks its tiles as one sequential stream. The scales
// of a lane's 4 rows sit next to each other (one 8-byte load per segment).
//
// Bytes inside a 16-byte unit are arranged for cheap conversion to fp16:
//   Q8_0, half h: byte i = q[16h + i] XOR 0x80 (offset binary, so that
//        0x6400 | byte is the fp16 number 1024 + q + 128).
//   Q4_0: dword d holds elements 8d..8d+7; element 8d+e sits in nibble
//        position p = e/2 + 4*(e%2), so that masking with 0x000F000F and
//        0x00F000F0 (before and after a shift by 8) yields element pairs
//        (e, e+1) in the two fp16 halves of a register.
// The nibble value is kept as stored (0..15); the -8 offset is applied in fp16.
//
// Q4_K (256-weight super-blocks of 8 sub-blocks of 32 weights; canonical
// block: fp16 d, fp16 dmin, 12 bytes of 6-bit sub-block scales and mins, 128
// bytes of nibbles, weight = d * sc * q - dmin * mn) is packed per 32-weight
// sub-block like Q4_0: the quant plane holds its nibbles in the Q4_0
// arrangement, the scale plane a 16-bit word per row where Q4_0 keeps the fp16
// scale, and a third plane holds the super-block's d and dmin:
//   scale word:  bits 0-3 the centre c, bits 4-9 sc, bits 10-15 mn
//   super plane: [tile][segment][slot][super-block of the segment][b] x (d, dmin) fp16
// so a lane's 16-byte load gets d and dmin of its 4 rows. 148 bytes per
// 256 weights (144 canonical). The centre c (0..15) is derived at load time
// (q4_k_centre) and is not part of the canonical block: the GEMV sums each
// sub-block as d*sc * sum((q - c) x) + (d*sc*c - dmin*mn) * sum(x), two terms
// whose magnitudes are at most 3 |w| per weight, so its rounding scales with
// sum |w x| even where d*sc*q and dmin*mn cancel.
//
// Q6_K (256-weight super-blocks; canonical block: 128 bytes of low 4-bit
// parts, 64 bytes of high 2-bit parts, 16 int8 scales (one per 16 weights),
// fp16 d; weight = d * sc * (q - 32)) is packed per 32-weight block: the low
// nibbles in the Q4_0 arrangement as units b = 0..3 of the quant plane, the
// high 2-bit parts as two more units (row pairs 0-1 and 2-3, 8 bytes a row),
// the block's two int8 scales where Q4_0 keeps its fp16 scale, and d in the
// super plane (2 bytes a row). A row's 8 bytes of high parts are two dwords,
// each covering 16 elements: element e of the first 8 sits at bit pair
// q6_hi_pos(e), the second 8 at that position rotated by 24, so that a shift
// by 0 or 2 (first 8) or a rotation by 24 and a further shift by 2 (second 8)
// lines each pair of elements up under bits 4-5 / 8-9 of the fp16 halves the
// low nibbles occupy. 210 bytes per 256 weights, as canonical.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define QG_HD __host__ __device__ __forceinline__
#else
#define QG_HD inline
#endif

namespace qgl {

constexpr int kQ8_0 = 1;
constexpr int kQ4_0 = 2;
constexpr int kQ4_K = 3;
constexpr int kQ6_K = 4;
constexpr int kSuperBlocks = 8;   // Q4_K, Q6_K: 32-weight blocks per super-block

constexpr int kSlots = 2;         // rows processed side by side per wavefront
constexpr int kLanesPerSlot = 32; // lanes sharing one row = blocks per segment
constexpr int kSegBlocks = 32;
constexpr int kRowsPerLane = 4;   // register blocking of rows per lane
constexpr int kTileRows = kSlots * kRowsPerLane;
constexpr int kUnit = 16;         // bytes per lane per load
constexpr int kSegWeights = kSegBlocks * 32;

// Canonical bytes of one row of K weights (K % 32 == 0; K % 256 == 0 for Q4_K, Q6_K).
QG_HD int64_t canon_row_bytes(int qt, int64_t K)
{
    if (qt == kQ8_0) return (K / 32) * 34;
    if (qt == kQ4_0) return (K / 32) * 18;
    return (K / 256) * (qt == kQ4_K ? 144 : 210);
}
// Quant-plane bytes per row and 32-weight block (Q6_K: 16 of low nibbles + 8 of high parts).
QG_HD constexpr int packed_quant_bytes(int qt) { return qt == kQ8_0 ? 32 : (qt == kQ6_K ? 24 : 16); }
// Super-plane bytes per row and super-block (Q4_K: d, dmin; Q6_K: d).
QG_HD int super_row_bytes(int qt) { return qt == kQ4_K ? 4 : (qt == kQ6_K ? 2 : 0); }
QG_HD int halves(int qt) { return qt == kQ8_0 ? 2 : 1; }

struct Geometry {
    int qt;
    int64_t N;        // rows (virtual rows for a fused gate|up weight)
    int64_t K;
    int64_t KB;       // blocks per row
    int64_t nseg;     // segments per row
    int64_t n_tiles;
    int64_t tile_q;   // quant bytes per tile
    int64_t tile_s;   // scale bytes per tile
    int64_t scale_off;
    int64_t tile_u;   // Q4_K / Q6_K super-scale bytes per tile (0 otherwise)
    int64_t sup_off;  // Q4_K / Q6_K super-scale plane
    int64_t total;
};

QG_HD int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

QG_HD Geometry geometry(int qt, int64_t N, int64_t K)
{
    Geometry g;
    g.qt = qt;
    g.N = N;
    g.K = K;
    g.KB = K / 32;
    g.nseg = (g.KB + kSegBlocks - 1) / kSegBlocks;
    g.n_tiles = (N + kTileRows - 1) / kTileRows;
    g.tile_q = (int64_t)kTileRows * g.KB * packed_quant_bytes(qt);
    g.tile_s = (int64_t)kTileRows * g.KB * 2;
    g.scale_off = round_up(g.n_tiles * g.tile_q, 256);
    g.tile_u = (int64_t)kTileRows * (g.KB / kSuperBlocks) * super_row_bytes(qt);
    g.sup_off = g.scale_off + round_up(g.n_tiles * g.tile_s, 256);
    g.total = g.sup_off + round_up(g.n_tiles * g.tile_u, 256);
    return g;
}

QG_HD int64_t seg_blocks(const Geometry &g, int64_t seg)
{
    int64_t r = g.KB - seg * kSegBlocks;
    return r < kSegBlocks ? r : kSegBlocks;
}

// Byte offset of 16-byte unit u of block j of row slot `slot` in segment seg of tile t.
QG_HD int64_t unit_offset(const Geometry &g, int64_t t, int64_t seg, int u, int slot, int j)
{
    int64_t nb = seg_blocks(g, seg);
    return t * g.tile_q + seg * (int64_t)kTileRows * kSegBlocks * packed_quant_bytes(g.qt) +
           (((int64_t)u * kSlots + slot) * nb + j) * kUnit;
}

// Unit (b, h): row b's quants (half h of a Q8_0 block).
QG_HD int64_t quant_offset(const Geometry &g, int64_t t, int64_t seg, int b, int h, int slot, int j)
{
    return unit_offset(g, t, seg, b * halves(g.qt) + h, slot, j);
}

// Q6_K: the unit of high 2-bit parts of rows 2bp, 2bp+1 (8 bytes each).
QG_HD int64_t q6_hi_offset(const Geometry &g, int64_t t, int64_t seg, int bp, int slot, int j)
{
    return unit_offset(g, t, seg, kRowsPerLane + bp, slot, j);
}

// Q6_K: bit position of element e (0..15) of a 16-element span in its dword of
// high parts. Elements 0..7 pair up as (0,1) (2,3) (4,5) (6,7) with the fp16
// halves of the low-nibble pairs: 4 / 20, 8 / 24, then the same two +2; the
// second 8 sit 24 bits further round.
QG_HD int q6_hi_pos(int e)
{
    const int f = e % 8;
    const int p = (f % 2) * 16 + 4 + 4 * ((f / 2) % 2) + 2 * (f / 4);
    return (p + 24 * (e / 8)) % 32;
}

// Byte offset of the 4 scales (rows b = 0..3) of block j, slot `slot`, segment seg, tile t.
QG_HD int64_t scale_offset(const Geometry &g, int64_t t, int64_t seg, int slot, int j)
{
    int64_t nb = seg_blocks(g, seg);
    return g.scale_off + t * g.tile_s + seg * (int64_t)kTileRows * kSegBlocks * 2 +
           ((int64_t)slot * nb + j) * kRowsPerLane * 2;
}

// Q4_K / Q6_K: byte offset of the super-block scales (d, dmin / d) of rows b =
// 0..3 (slot `slot`) for super-block sb of segment seg, tile t.
QG_HD int64_t super_offset(const Geometry &g, int64_t t, int64_t seg, int slot, int sb)
{
    const int ub = super_row_bytes(g.qt);
    int64_t nsb = seg_blocks(g, seg) / kSuperBlocks;
    return g.sup_off + t * g.tile_u + seg * (int64_t)kTileRows * (kSegBlocks / kSuperBlocks) * ub +
           ((int64_t)slot * nsb + sb) * kRowsPerLane * ub;
}

QG_HD int q4_nibble_pos(int e) { return e / 2 + 4 * (e % 2); }  // e in 0..7 within a dword

// Q4_K: the 6-bit scale and min of sub-block j (0..7) from a super-block's 12 bytes u.
QG_HD void q4_k_unpack_scale(const uint8_t *u, int j, uint8_t &sc, uint8_t &mn)
{
    if (j < 4) {
        sc = (uint8_t)(u[j] & 63);
        mn = (uint8_t)(u[j + 4] & 63);
    } else {
        sc = (uint8_t)((u[j + 4] & 15) | ((u[j - 4] >> 6) << 4));
        mn = (uint8_t)((u[j + 4] >> 4) | ((u[j] >> 6) << 4));
    }
}

// Q4_K: OR the bits of sub-block j's scale and min into the 12 bytes u (the inverse).
QG_HD void q4_k_pack_scale(uint8_t *u, int j, uint8_t sc, uint8_t mn)
{
    if (j < 4) {
        u[j] |= (uint8_t)(sc & 63);
        u[j + 4] |= (uint8_t)(mn & 63);
    } else {
        u[j + 4] |= (uint8_t)((sc & 15) | ((mn & 15) << 4));
        u[j - 4] |= (uint8_t)((sc >> 4) << 6);
        u[j] |= (uint8_t)((mn >> 4) << 6);
    }
}

// Exact value of an fp16 bit pattern as a double (infinities and NaN included).
QG_HD double half_bits_value(uint32_t h)
{
    const uint32_t e = (h >> 10) & 31u, m = h & 1023u;
    double v;
    if (e == 0)
        v = (double)m * (1.0 / 16777216.0);   // subnormal: m * 2^-24
    else if (e == 31)
        v = m ? __builtin_nan("") : __builtin_inf();
    else {
        v = (double)(m | 1024u);
        int s = (int)e - 25;                   // (1024 + m) * 2^(e - 25)
        for (; s > 0; --s) v *= 2.0;
        for (; s < 0; ++s) v *= 0.5;
    }
    return (h & 0x8000u) ? -v : v;
}

// Q4_K: the centre c of a sub-block with scale a = d*sc and min term b = dmin*mn
// (weight = a q - b, q in 0..15): c = b / a rounded to the nearest integer (ties
// down) and clamped to 0..15, or 0 when a is 0 or not finite. With this c every
// weight satisfies |a (q - c)| + |a c - b| <= 3 |a q - b|: when b / a lies in
// [-1/2, 15 + 1/2], |a c - b| <= |a| / 2 and a q - b is 0 only where q = c;
// outside it, a (q - c) and a c - b have the same sign. Exact comparisons of
// doubles (each product has at most 17 significant bits), so the host and the
// device packer agree bit for bit.
QG_HD uint32_t q4_k_centre(uint32_t d_bits, uint32_t dmin_bits, uint32_t sc, uint32_t mn)
{
    const double a = half_bits_value(d_bits) * (double)sc;
    const double b2 = 2.0 * half_bits_value(dmin_bits) * (double)mn;
    if (!(a != 0.0) || a - a != 0.0 || b2 - b2 != 0.0) return 0;
    uint32_t c = 0;
    for (int k = 0; k < 15; ++k)   // b / a > k + 1/2  <=>  2b > (2k + 1) a for a > 0, < for a < 0
        c += (a > 0.0) ? (b2 > (2 * k + 1) * a) : (b2 < (2 * k + 1) * a);
    return c;
}

// Q4_K scale word of a sub-block (see the layout above) and its fields.
QG_HD uint32_t q4_k_scale_word(uint32_t centre, uint32_t sc, uint32_t mn) { return centre | (sc << 4) | (mn << 10); }

// Nibble of element e (0..31) of 32-weight block blk of a canonical row: Q4_0
// byte e / e-16 of the block; Q4_K sub-block j = blk % 8 of super-block blk / 8,
// the low (j even) or high (j odd) nibbles of bytes 32 (j / 2) .. + 31.
QG_HD uint32_t canon_nibble(int qt, const uint8_t *canon_row, int64_t blk, int e)
{
    if (qt == kQ4_0) {
        const uint8_t *qs = canon_row + blk * 18 + 2;
        return (e < 16) ? (qs[e] & 0x0Fu) : (uint32_t)(qs[e - 16] >> 4);
    }
    const int j = (int)(blk % kSuperBlocks);
    const uint8_t *qs = canon_row + (blk / kSuperBlocks) * 144 + 16 + 32 * (j / 2);
    return (j % 2 == 0) ? (qs[e] & 0x0Fu) : (uint32_t)(qs[e] >> 4);
}

// Q6_K: low 4 bits and high 2 bits of element e (0..31) of 32-weight block blk
// of a canonical row (super-block blk / 8; group jj = blk % 8 of it, in half jj / 4
// with g = jj % 4: low bits in the low (g < 2) or high nibble of ql[64h + 32(g%2)
// + e], high bits at bits 2g of qh[32h + e]).
QG_HD uint32_t q6_canon_lo(const uint8_t *canon_row, int64_t blk, int e)
{
    const uint8_t *sb = canon_row + (blk / kSuperBlocks) * 210;
    const int jj = (int)(blk % kSuperBlocks), h = jj / 4, g = jj % 4;
    const uint8_t v = sb[64 * h + 32 * (g % 2) + e];
    return g < 2 ? (v & 0x0Fu) : (uint32_t)(v >> 4);
}
QG_HD uint32_t q6_canon_hi(const uint8_t *canon_row, int64_t blk, int e)
{
    const uint8_t *sb = canon_row + (blk / kSuperBlocks) * 210;
    const int jj = (int)(blk % kSuperBlocks), h = jj / 4, g = jj % 4;
    return (uint32_t)(sb[128 + 32 * h + e] >> (2 * g)) & 3u;
}

// Write block `blk` (32 weights) of row `row` from the row's canonical bytes
// `canon_row` into the packed buffer. A null `canon_row` writes a zero block
// (padding rows).
QG_HD void pack_block(const Geometry &g, const uint8_t *canon_row, uint8_t *packed, int64_t row, int64_t blk)
{
    int64_t t = row / kTileRows;
    int rt = (int)(row % kTileRows);
    int slot = rt / kRowsPerLane, b = rt % kRowsPerLane;
    int64_t seg = blk / kSegBlocks;
    int j = (int)(blk % kSegBlocks);
    uint8_t *sp = packed + scale_offset(g, t, seg, slot, j) + b * 2;
    if (g.qt == kQ8_0) {
        const uint8_t *c = canon_row ? canon_row + blk * 34 : nullptr;
        sp[0] = c ? c[0] : 0;
        sp[1] = c ? c[1] : 0;
        for (int h = 0; h < 2; ++h) {
            uint8_t *qp = packed + quant_offset(g, t, seg, b, h, slot, j);
            for (int i = 0; i < 16; ++i) qp[i] = c ? (uint8_t)(c[2 + 16 * h + i] ^ 0x80) : 0;
        }
        return;
    }
    if (g.qt == kQ6_K) {
        const uint8_t *sb = canon_row ? canon_row + (blk / kSuperBlocks) * 210 : nullptr;
        const int jj = (int)(blk % kSuperBlocks);
        sp[0] = sb ? sb[192 + 2 * jj] : 0;       // scale of elements 0..15
        sp[1] = sb ? sb[192 + 2 * jj + 1] : 0;   // scale of elements 16..31
        if (jj == 0) {
            uint8_t *up = packed + super_offset(g, t, seg, slot, j / kSuperBlocks) + b * 2;
            up[0] = sb ? sb[208] : 0;
            up[1] = sb ? sb[209] : 0;
        }
        uint8_t *qp = packed + quant_offset(g, t, seg, b, 0, slot, j);
        uint8_t *hp = packed + q6_hi_offset(g, t, seg, b / 2, slot, j) + (b % 2) * 8;
        uint32_t dw[4] = {0, 0, 0, 0}, hw[2] = {0, 0};
        if (canon_row)
            for (int e = 0; e < 32; ++e) {
                dw[e / 8] |= q6_canon_lo(canon_row, blk, e) << (4 * q4_nibble_pos(e % 8));
                hw[e / 16] |= q6_canon_hi(canon_row, blk, e) << q6_hi_pos(e % 16);
            }
        for (int d = 0; d < 4; ++d)
            for (int i = 0; i < 4; ++i) qp[4 * d + i] = (uint8_t)(dw[d] >> (8 * i));
        for (int d = 0; d < 2; ++d)
            for (int i = 0; i < 4; ++i) hp[4 * d + i] = (uint8_t)(hw[d] >> (8 * i));
        return;
    }
    if (g.qt == kQ4_0) {
        const uint8_t *c = canon_row ? canon_row + blk * 18 : nullptr;
        sp[0] = c ? c[0] : 0;
        sp[1] = c ? c[1] : 0;
    } else {
        const uint8_t *sb = canon_row ? canon_row + (blk / kSuperBlocks) * 144 : nullptr;
        uint8_t sc = 0, mn = 0;
        uint32_t centre = 0;
        if (sb) {
            q4_k_unpack_scale(sb + 4, (int)(blk % kSuperBlocks), sc, mn);
            centre = q4_k_centre(sb[0] | ((uint32_t)sb[1] << 8), sb[2] | ((uint32_t)sb[3] << 8), sc, mn);
        }
        const uint32_t word = q4_k_scale_word(centre, sc, mn);
        sp[0] = (uint8_t)word;
        sp[1] = (uint8_t)(word >> 8);
        if (blk % kSuperBlocks == 0) {
            uint8_t *up = packed + super_offset(g, t, seg, slot, j / kSuperBlocks) + b * 4;
            for (int i = 0; i < 4; ++i) up[i] = sb ? sb[i] : 0;
        }
    }
    uint8_t *qp = packed + quant_offset(g, t, seg, b, 0, slot, j);
    uint32_t dw[4] = {0, 0, 0, 0};
    if (canon_row)
        for (int e = 0; e < 32; ++e) dw[e / 8] |= canon_nibble(g.qt, canon_row, blk, e) << (4 * q4_nibble_pos(e % 8));
    for (int d = 0; d < 4; ++d)
        for (int i = 0; i < 4; ++i) qp[4 * d + i] = (uint8_t)(dw[d] >> (8 * i));
}

// Inverse of pack_block: rebuild block `blk` of the row's canonical bytes. For
// Q4_K the block's bits are OR-ed into the super-block (whose bytes must start
// at zero) and d, dmin are written with its first sub-block.
QG_HD void unpack_block(const Geometry &g, const uint8_t *packed, uint8_t *canon_row, int64_t row, int64_t blk)
{
    int64_t t = row / kTileRows;
    int rt = (int)(row % kTileRows);
    int slot = rt / kRowsPerLane, b = rt % kRowsPerLane;
    int64_t seg = blk / kSegBlocks;
    int j = (int)(blk % kSegBlocks);
    const uint8_t *sp = packed + scale_offset(g, t, seg, slot, j) + b * 2;
    if (g.qt == kQ8_0) {
        uint8_t *c = canon_row + blk * 34;
        c[0] = sp[0];
        c[1] = sp[1];
        for (int h = 0; h < 2; ++h) {
            const uint8_t *qp = packed + quant_offset(g, t, seg, b, h, slot, j);
            for (int i = 0; i < 16; ++i) c[2 + 16 * h + i] = (uint8_t)(qp[i] ^ 0x80);
        }
        return;
    }
    if (g.qt == kQ6_K) {
        const int jj = (int)(blk % kSuperBlocks), h = jj / 4, gg = jj % 4;
        uint8_t *sb = canon_row + (blk / kSuperBlocks) * 210;
        sb[192 + 2 * jj] = sp[0];
        sb[192 + 2 * jj + 1] = sp[1];
        if (jj == 0) {
            const uint8_t *up = packed + super_offset(g, t, seg, slot, j / kSuperBlocks) + b * 2;
            sb[208] = up[0];
            sb[209] = up[1];
        }
        const uint8_t *qp = packed + quant_offset(g, t, seg, b, 0, slot, j);
        const uint8_t *hp = packed + q6_hi_offset(g, t, seg, b / 2, slot, j) + (b % 2) * 8;
        for (int e = 0; e < 32; ++e) {
            const int d = e / 8, hd = e / 16;
            uint32_t dw = (uint32_t)qp[4 * d] | ((uint32_t)qp[4 * d + 1] << 8) | ((uint32_t)qp[4 * d + 2] << 16) |
                          ((uint32_t)qp[4 * d + 3] << 24);
            uint32_t hw = (uint32_t)hp[4 * hd] | ((uint32_t)hp[4 * hd + 1] << 8) |
                          ((uint32_t)hp[4 * hd + 2] << 16) | ((uint32_t)hp[4 * hd + 3] << 24);
            const uint32_t lo = (dw >> (4 * q4_nibble_pos(e % 8))) & 0xFu;
            const uint32_t hi = (hw >> q6_hi_pos(e % 16)) & 3u;
            sb[64 * h + 32 * (gg % 2) + e] |= (uint8_t)(gg < 2 ? lo : lo << 4);
            sb[128 + 32 * h + e] |= (uint8_t)(hi << (2 * gg));
        }
        return;
    }
    const uint8_t *qp = packed + quant_offset(g, t, seg, b, 0, slot, j);
    uint8_t nib[32];
    for (int e = 0; e < 32; ++e) {
        int d = e / 8, p = q4_nibble_pos(e % 8);
        uint32_t dw = (uint32_t)qp[4 * d] | ((uint32_t)qp[4 * d + 1] << 8) | ((uint32_t)qp[4 * d + 2] << 16) |
                      ((uint32_t)qp[4 * d + 3] << 24);
        nib[e] = (uint8_t)((dw >> (4 * p)) & 0xF);
    }
    if (g.qt == kQ4_0) {
        uint8_t *c = canon_row + blk * 18;
        c[0] = sp[0];
        c[1] = sp[1];
        for (int i = 0; i < 16; ++i) c[2 + i] = (uint8_t)(nib[i] | (nib[i + 16] << 4));
        return;
    }
    const int js = (int)(blk % kSuperBlocks);
    uint8_t *sb = canon_row + (blk / kSuperBlocks) * 144;
    const uint32_t word = sp[0] | ((uint32_t)sp[1] << 8);   // the centre (bits 0-3) is derived, not stored
    q4_k_pack_scale(sb + 4, js, (uint8_t)((word >> 4) & 63u), (uint8_t)(word >> 10));
    if (js == 0) {
        const uint8_t *up = packed + super_offset(g, t, seg, slot, j / kSuperBlocks) + b * 4;
        for (int i = 0; i < 4; ++i) sb[i] = up[i];
    }
    uint8_t *qs = sb + 16 + 32 * (js / 2);
    for (int e = 0; e < 32; ++e) qs[e] |= (uint8_t)(js % 2 == 0 ? nib[e] : nib[e] << 4);
}

}  // namespace qgl
