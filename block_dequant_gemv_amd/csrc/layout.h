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

constexpr int kSlots = 2;         // rows processed side by side per wavefront
constexpr int kLanesPerSlot = 32; // lanes sharing one row = blocks per segment
constexpr int kSegBlocks = 32;
constexpr int kRowsPerLane = 4;   // register blocking of rows per lane
constexpr int kTileRows = kSlots * kRowsPerLane;
constexpr int kUnit = 16;         // bytes per lane per load
constexpr int kSegWeights = kSegBlocks * 32;

QG_HD int canon_block_bytes(int qt) { return qt == kQ8_0 ? 34 : 18; }
QG_HD int packed_quant_bytes(int qt) { return qt == kQ8_0 ? 32 : 16; }
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
    g.total = g.scale_off + round_up(g.n_tiles * g.tile_s, 256);
    return g;
}

QG_HD int64_t seg_blocks(const Geometry &g, int64_t seg)
{
    int64_t r = g.KB - seg * kSegBlocks;
    return r < kSegBlocks ? r : kSegBlocks;
}

// Byte offset of 16-byte unit (b, h) of block j of row slot `slot` in segment seg of tile t.
QG_HD int64_t quant_offset(const Geometry &g, int64_t t, int64_t seg, int b, int h, int slot, int j)
{
    int64_t nb = seg_blocks(g, seg);
    return t * g.tile_q + seg * (int64_t)kTileRows * kSegBlocks * packed_quant_bytes(g.qt) +
           (((int64_t)(b * halves(g.qt) + h) * kSlots + slot) * nb + j) * kUnit;
}

// Byte offset of the 4 scales (rows b = 0..3) of block j, slot `slot`, segment seg, tile t.
QG_HD int64_t scale_offset(const Geometry &g, int64_t t, int64_t seg, int slot, int j)
{
    int64_t nb = seg_blocks(g, seg);
    return g.scale_off + t * g.tile_s + seg * (int64_t)kTileRows * kSegBlocks * 2 +
           ((int64_t)slot * nb + j) * kRowsPerLane * 2;
}

QG_HD int q4_nibble_pos(int e) { return e / 2 + 4 * (e % 2); }  // e in 0..7 within a dword

// Write one canonical block (scale + quants) of row `row`, block `blk` into the packed buffer.
// A null `canon` writes a zero block (padding rows).
QG_HD void pack_block(const Geometry &g, const uint8_t *canon, uint8_t *packed, int64_t row, int64_t blk)
{
    int64_t t = row / kTileRows;
    int rt = (int)(row % kTileRows);
    int slot = rt / kRowsPerLane, b = rt % kRowsPerLane;
    int64_t seg = blk / kSegBlocks;
    int j = (int)(blk % kSegBlocks);
    uint8_t *sp = packed + scale_offset(g, t, seg, slot, j) + b * 2;
    sp[0] = canon ? canon[0] : 0;
    sp[1] = canon ? canon[1] : 0;
    if (g.qt == kQ8_0) {
        for (int h = 0; h < 2; ++h) {
            uint8_t *qp = packed + quant_offset(g, t, seg, b, h, slot, j);
            for (int i = 0; i < 16; ++i) qp[i] = canon ? (uint8_t)(canon[2 + 16 * h + i] ^ 0x80) : 0;
        }
    } else {
        uint8_t *qp = packed + quant_offset(g, t, seg, b, 0, slot, j);
        uint32_t dw[4] = {0, 0, 0, 0};
        if (canon) {
            for (int e = 0; e < 32; ++e) {
                uint32_t nib = (e < 16) ? (canon[2 + e] & 0x0Fu) : (uint32_t)(canon[2 + e - 16] >> 4);
                dw[e / 8] |= nib << (4 * q4_nibble_pos(e % 8));
            }
        }
        for (int d = 0; d < 4; ++d)
            for (int i = 0; i < 4; ++i) qp[4 * d + i] = (uint8_t)(dw[d] >> (8 * i));
    }
}

// Inverse of pack_block: rebuild the canonical block bytes.
QG_HD void unpack_block(const Geometry &g, const uint8_t *packed, uint8_t *canon, int64_t row, int64_t blk)
{
    int64_t t = row / kTileRows;
    int rt = (int)(row % kTileRows);
    int slot = rt / kRowsPerLane, b = rt % kRowsPerLane;
    int64_t seg = blk / kSegBlocks;
    int j = (int)(blk % kSegBlocks);
    const uint8_t *sp = packed + scale_offset(g, t, seg, slot, j) + b * 2;
    canon[0] = sp[0];
    canon[1] = sp[1];
    if (g.qt == kQ8_0) {
        for (int h = 0; h < 2; ++h) {
            const uint8_t *qp = packed + quant_offset(g, t, seg, b, h, slot, j);
            for (int i = 0; i < 16; ++i) canon[2 + 16 * h + i] = (uint8_t)(qp[i] ^ 0x80);
        }
    } else {
        const uint8_t *qp = packed + quant_offset(g, t, seg, b, 0, slot, j);
        for (int i = 0; i < 16; ++i) canon[2 + i] = 0;
        for (int e = 0; e < 32; ++e) {
            int d = e / 8, p = q4_nibble_pos(e % 8);
            uint32_t dw = (uint32_t)qp[4 * d] | ((uint32_t)qp[4 * d + 1] << 8) | ((uint32_t)qp[4 * d + 2] << 16) |
                          ((uint32_t)qp[4 * d + 3] << 24);
            uint8_t nib = (uint8_t)((dw >> (4 * p)) & 0xF);
            if (e < 16) canon[2 + e] |= nib;
            else canon[2 + e - 16] |= (uint8_t)(nib << 4);
        }
    }
}

}  // namespace qgl
