// dequant.h -- device helpers shared by the GEMV and GEMM kernels of libqgemv:
// exact conversion of packed Q8_0 / Q4_0 quants to fp16 pairs (layout.h gives
// the byte arrangement they rely on).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qgk {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }
__device__ __forceinline__ float as_f(int v) { return __builtin_bit_cast(float, v); }
__device__ __forceinline__ int as_i(float v) { return __builtin_bit_cast(int, v); }

// fp16 magic: 0x6400 | m is the fp16 number 1024 + m for m < 1024.
// Registers that hold the conversion constants for the whole kernel. gfx9 VOP3
// instructions take no literal operand and read at most one SGPR, so the mask
// of v_and_or_b32 lives in an SGPR and the fp16 magic in a VGPR; the opaque
// moves keep the compiler from re-materialising them before every use.
struct Consts {
    uint32_t magic;    // VGPR 0x64006400
    uint32_t m_lo;     // SGPR 0x000F000F
    uint32_t m_hi;     // SGPR 0x00F000F0
};

__device__ __forceinline__ Consts make_consts()
{
    Consts c;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(c.magic));
    asm volatile("s_mov_b32 %0, 0xf000f" : "=s"(c.m_lo));
    asm volatile("s_mov_b32 %0, 0xf000f0" : "=s"(c.m_hi));
    return c;
}

// (a & mask) | c in one instruction.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t c)
{
    uint32_t d;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(mask), "v"(c));
    return d;
}

// Q4_0 dword -> the 8 weights (nibble - 8) as 4 fp16 pairs, elements (0,1) (2,3) (4,5) (6,7).
// Nibbles at bits 0-3 / 16-19 give 1024 + q; nibbles at bits 4-7 / 20-23 give
// 1024 + 16 q, which (x/16 - 72) maps to q - 8 exactly.
__device__ __forceinline__ void q4_pairs(uint32_t w, const Consts &k, h2 (&p)[4])
{
    const h2 off = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2 off16 = {(_Float16)-72.0f, (_Float16)-72.0f};
    const uint32_t w8 = w >> 8;
    p[0] = as_h2(and_or(w, k.m_lo, k.magic)) + off;
    p[1] = __builtin_elementwise_fma(as_h2(and_or(w, k.m_hi, k.magic)), sixteenth, off16);
    p[2] = as_h2(and_or(w8, k.m_lo, k.magic)) + off;
    p[3] = __builtin_elementwise_fma(as_h2(and_or(w8, k.m_hi, k.magic)), sixteenth, off16);
}

// Q4_K dword -> the 8 centred quants (q - c) * 2^-24 (q 0..15, c the
// sub-block's centre, 0..15) as 4 fp16 pairs, in the order of q4_pairs. Each
// pair of nibbles is masked out in place and read as fp16 subnormals: q * 2^-24
// (mantissa bits 0..3: pairs 0 and 2), from which the centre pair c_lo =
// c * 0x00010001 (= c * 2^-24 twice) is subtracted, or q * 2^-20 (bits 4..7:
// pairs 1 and 3), scaled by 1/16 and the centre subtracted in one fma. Every
// value involved is a multiple of 2^-24 below 2^-14 in magnitude, so each
// result is exact.
__device__ __forceinline__ void q4k_pairs(uint32_t w, const Consts &k, uint32_t c_lo, h2 (&p)[4])
{
    const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2 c = as_h2(c_lo);
    const uint32_t w8 = w >> 8;
    p[0] = as_h2(w & k.m_lo) - c;
    p[1] = __builtin_elementwise_fma(as_h2(w & k.m_hi), sixteenth, -c);
    p[2] = as_h2(w8 & k.m_lo) - c;
    p[3] = __builtin_elementwise_fma(as_h2(w8 & k.m_hi), sixteenth, -c);
}

// Q6_K: the low-nibble dword w (Q4_0 arrangement) and the row's dword h of high
// 2-bit parts for these 8 elements -> 4 fp16 pairs of q - 32, exact. For the
// second dword of a 16-element span (odd) the high parts sit 24 bits further
// round; after the rotation both cases read pairs 0/1 from bits 4-5 / 8-9 of
// the fp16 halves and pairs 2/3 from the same bits 2 higher.
__device__ __forceinline__ void q6k_pairs(uint32_t w, uint32_t h, bool odd, const Consts &k, h2 (&p)[4])
{
    const h2 off = {(_Float16)-1056.0f, (_Float16)-1056.0f};
    const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2 off16 = {(_Float16)-96.0f, (_Float16)-96.0f};
    const uint32_t a = odd ? __builtin_amdgcn_alignbit(h, h, 24) : h;
    const uint32_t b2 = a >> 2;
    const uint32_t w8 = w >> 8;
    p[0] = as_h2(and_or(a, 0x00300030u, and_or(w, k.m_lo, k.magic))) + off;
    p[1] = __builtin_elementwise_fma(as_h2(and_or(a, 0x03000300u, and_or(w, k.m_hi, k.magic))), sixteenth, off16);
    p[2] = as_h2(and_or(b2, 0x00300030u, and_or(w8, k.m_lo, k.magic))) + off;
    p[3] = __builtin_elementwise_fma(as_h2(and_or(b2, 0x03000300u, and_or(w8, k.m_hi, k.magic))), sixteenth, off16);
}

// Q8_0 dword (bytes q XOR 0x80) -> the 4 int8 weights as 2 fp16 pairs, elements (0,1) (2,3).
// v_perm_b32 builds [byte, 0x64, byte, 0x64] = fp16 (1024 + q + 128) twice.
__device__ __forceinline__ void q8_pairs(uint32_t w, h2 (&p)[2])
{
    const h2 off = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    p[0] = as_h2(__builtin_amdgcn_perm(0x64646464u, w, 0x04010400u)) + off;
    p[1] = as_h2(__builtin_amdgcn_perm(0x64646464u, w, 0x04030402u)) + off;
}

}  // namespace qgk
