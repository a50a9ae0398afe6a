// wq_decode.h -- in-register unpack of packed int4 / int5 / int8 codes to exact binary16.
//
// A code c (two's complement) is first turned into offset form c + 8 (int4) or
// c + 128 (int8) by flipping its top bit; ORing that field into the mantissa of
// binary16 1024.0 (0x6400) gives 1024 + (c + offset), and one packed fp16
// subtract recovers c exactly. The flip and the OR are one 3-input bit
// operation: out = K ^ (d & mask), where K holds the flip bits inside the mask
// and 0x6400 outside it. The mask/constant pairs are pinned to VGPRs so gfx950
// can use v_bitop3_b32 (a VOP3 instruction cannot take two literal constants).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wq {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t vgpr(uint32_t c)
{
    asm volatile("" : "+v"(c));   // keep the constant in a VGPR
    return c;
}

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }

struct DecodeConsts {
    uint32_t m_lo;     // nibbles 0 and 4 of a dword
    uint32_t m_hi;     // nibbles 1 and 5
    uint32_t k_lo;     // 0x6400 magic with the int4 sign flip (bit 3) inside m_lo
    uint32_t k_hi;     // same for m_hi (bit 7)
    uint32_t m_b;      // bytes 0 and 2
    uint32_t k_b;      // 0x6400 magic with the int8 sign flip (bit 7) inside m_b
    __device__ __forceinline__ static DecodeConsts make()
    {
        DecodeConsts c;
        c.m_lo = vgpr(0x000F000Fu);
        c.m_hi = vgpr(0x00F000F0u);
        c.k_lo = vgpr(0x64086408u);
        c.k_hi = vgpr(0x64806480u);
        c.m_b = vgpr(0x00FF00FFu);
        c.k_b = vgpr(0x64806480u);
        return c;
    }
};

// int4 dword holding codes k0..k7 (nibble i = code k_i) -> exact fp16 pairs
// (k0,k4), (k1,k5), (k2,k6), (k3,k7).
__device__ __forceinline__ void decode_int4(uint32_t d, const DecodeConsts &c, h2 &p04, h2 &p15,
                                            h2 &p26, h2 &p37)
{
    const uint32_t v = d >> 8;
    const h2 a = as_h2(c.k_lo ^ (d & c.m_lo));   // 1024 + (k + 8)
    const h2 b = as_h2(c.k_hi ^ (d & c.m_hi));   // 1024 + 16 (k + 8)
    const h2 e = as_h2(c.k_lo ^ (v & c.m_lo));
    const h2 f = as_h2(c.k_hi ^ (v & c.m_hi));
    const h2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
    const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2 off16 = {(_Float16)72.0f, (_Float16)72.0f};
    p04 = a - off;                               // exact small integers
    p15 = b * sixteenth - off16;
    p26 = e - off;
    p37 = f * sixteenth - off16;
}

// int8 dword holding codes k0..k3 -> exact fp16 pairs (k0,k2), (k1,k3).
__device__ __forceinline__ void decode_int8(uint32_t d, const DecodeConsts &c, h2 &p02, h2 &p13)
{
    const uint32_t v = d >> 8;
    const h2 a = as_h2(c.k_b ^ (d & c.m_b));     // 1024 + (k + 128)
    const h2 b = as_h2(c.k_b ^ (v & c.m_b));
    const h2 off = {(_Float16)1152.0f, (_Float16)1152.0f};
    p02 = a - off;
    p13 = b - off;
}

// Eight consecutive codes as one h8 in the order used for matrix-core operands:
// int4 dword -> {k0,k4,k1,k5,k2,k6,k3,k7}; int8 dwords -> {k0,k2,k1,k3,k4,k6,k5,k7}.
__device__ __forceinline__ h8 unpack8_int4(uint32_t d, const DecodeConsts &c)
{
    h2 a, b, e, f;
    decode_int4(d, c, a, b, e, f);
    h8 r;
    r[0] = a.x; r[1] = a.y; r[2] = b.x; r[3] = b.y;
    r[4] = e.x; r[5] = e.y; r[6] = f.x; r[7] = f.y;
    return r;
}

__device__ __forceinline__ h8 unpack8_int8(uint32_t d0, uint32_t d1, const DecodeConsts &c)
{
    h2 a, b, e, f;
    decode_int8(d0, c, a, b);
    decode_int8(d1, c, e, f);
    h8 r;
    r[0] = a.x; r[1] = a.y; r[2] = b.x; r[3] = b.y;
    r[4] = e.x; r[5] = e.y; r[6] = f.x; r[7] = f.y;
    return r;
}

// int5 (codes in [-16, 15]): a dword of low nibbles as in int4 (unsigned low 4
// bits of codes k0..k7) and a byte whose bit i is bit 4 of code k_i. The nibble
// is taken as is and NOT(bit 4) goes into the mantissa bit above it, so each
// half holds 1024 + (k + 16) (or 1024 + 16 (k + 16) for the odd nibbles), and
// one packed fp16 subtract (or FMA) recovers k exactly.
struct Decode5Consts {
    uint32_t m_lo, m_hi;   // nibbles 0 and 4, 1 and 5
    uint32_t k;            // 0x6400 magic in both halves
    uint32_t b0, b1, b2, b3;
    __device__ __forceinline__ static Decode5Consts make()
    {
        Decode5Consts c;
        c.m_lo = vgpr(0x000F000Fu);
        c.m_hi = vgpr(0x00F000F0u);
        c.k = vgpr(0x64006400u);
        c.b0 = vgpr(0x00010001u);
        c.b1 = vgpr(0x00020002u);
        c.b2 = vgpr(0x00040004u);
        c.b3 = vgpr(0x00080008u);
        return c;
    }
};

// -> exact fp16 pairs (k0,k4), (k1,k5), (k2,k6), (k3,k7), as decode_int4.
__device__ __forceinline__ void decode_int5(uint32_t d, uint32_t hbyte, const Decode5Consts &c, h2 &p04,
                                            h2 &p15, h2 &p26, h2 &p37)
{
    const uint32_t nh = ~hbyte;
    const uint32_t t = (nh & 0xFu) | ((nh & 0xF0u) << 12);   // NOT bit 4 of k0..k3 in bits 0-3, k4..k7 in 16-19
    const uint32_t v = d >> 8;
    const h2 a = as_h2((d & c.m_lo) | ((t & c.b0) << 4) | c.k);   // 1024 + (k + 16)
    const h2 b = as_h2((d & c.m_hi) | ((t & c.b1) << 7) | c.k);   // 1024 + 16 (k + 16)
    const h2 e = as_h2((v & c.m_lo) | ((t & c.b2) << 2) | c.k);
    const h2 f = as_h2((v & c.m_hi) | ((t & c.b3) << 5) | c.k);
    const h2 off = {(_Float16)1040.0f, (_Float16)1040.0f};
    const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2 off16 = {(_Float16)80.0f, (_Float16)80.0f};
    p04 = a - off;
    p15 = b * sixteenth - off16;
    p26 = e - off;
    p37 = f * sixteenth - off16;
}

__device__ __forceinline__ h8 unpack8_int5(uint32_t d, uint32_t hbyte, const Decode5Consts &c)
{
    h2 a, b, e, f;
    decode_int5(d, hbyte, c, a, b, e, f);
    h8 r;
    r[0] = a.x; r[1] = a.y; r[2] = b.x; r[3] = b.y;
    r[4] = e.x; r[5] = e.y; r[6] = f.x; r[7] = f.y;
    return r;
}

// Codes straight to exact fp32 values with full-rate bit operations (no
// binary16 step, no conversion): a code field c in offset form (c + 8 or
// c + 128, by flipping its top bit) is placed in the mantissa of 2^23, which
// gives the float 2^23 + (c + offset) * 2^p for a field at bit p, and one fp32
// subtract of 2^23 + offset * 2^p leaves c * 2^p exactly. Fields at bit 0
// ("lo") give the code itself; fields at bit 4 (int4) or 8 (int8) ("hi") give
// 16 or 256 times the code, which the caller accumulates separately and
// scales back by the same power of two.
struct DecodeF32Consts {
    uint32_t m4lo, m4hi, k4lo, k4hi;   // int4: nibble masks at bits 0 and 4, 2^23 magic with the sign flip
    uint32_t m8lo, m8hi, k8lo, k8hi;   // int8: byte masks at bits 0 and 8
    __device__ __forceinline__ static DecodeF32Consts make()
    {
        DecodeF32Consts c;
        c.m4lo = vgpr(0x0000000Fu);
        c.m4hi = vgpr(0x000000F0u);
        c.k4lo = vgpr(0x4B000008u);
        c.k4hi = vgpr(0x4B000080u);
        c.m8lo = vgpr(0x000000FFu);
        c.m8hi = vgpr(0x0000FF00u);
        c.k8lo = vgpr(0x4B000080u);
        c.k8hi = vgpr(0x4B008000u);
        return c;
    }
};

__device__ __forceinline__ float as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }

// int4 dword holding codes k0..k7: lo[i] = k(2i), hi[i] = 16 * k(2i+1), exact.
__device__ __forceinline__ void decode_int4_f32(uint32_t d, const DecodeF32Consts &c, float (&lo)[4], float (&hi)[4])
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t e = d >> (8 * i);
        lo[i] = as_f32(c.k4lo ^ (e & c.m4lo)) - 8388616.0f;   // 2^23 + 8
        hi[i] = as_f32(c.k4hi ^ (e & c.m4hi)) - 8388736.0f;   // 2^23 + 128
    }
}

// int8 dword holding codes k0..k3: lo[i] = k(2i), hi[i] = 256 * k(2i+1), exact.
__device__ __forceinline__ void decode_int8_f32(uint32_t d, const DecodeF32Consts &c, float (&lo)[2], float (&hi)[2])
{
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t e = d >> (16 * i);
        lo[i] = as_f32(c.k8lo ^ (e & c.m8lo)) - 8388736.0f;   // 2^23 + 128
        hi[i] = as_f32(c.k8hi ^ (e & c.m8hi)) - 8421376.0f;   // 2^23 + 32768
    }
}

// Position of k (0..7) within an 8-group in the operand order above.
template <int BITS>
__device__ __forceinline__ constexpr int operand_slot(int k)
{
    // int4 and int5: k0->0 k4->1 k1->2 k5->3 k2->4 k6->5 k3->6 k7->7
    // int8:          k0->0 k2->1 k1->2 k3->3 k4->4 k6->5 k5->6 k7->7
    return BITS != 8 ? ((k & 3) * 2 + (k >> 2)) : ((k & 4) + (k & 1) * 2 + ((k >> 1) & 1));
}

}  // namespace wq
