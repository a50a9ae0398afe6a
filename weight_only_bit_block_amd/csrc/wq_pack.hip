// wq_pack.hip -- quantize + pack, and unpack, for block-32 int4 / int5 / int8 codes.
//
// The block-32 symmetric scheme is the one the pages describe for the MOSS
// decoder (moss-transcribe-diarize-litert card, "v2 decoder": int4 block-32;
// soniqo MOSS guide RU, implementation notes: symmetric linear INT8 block-32);
// int5 is the MLX default of the soniqo MOSS guide ("INT5 vs INT8"), for which
// the pages give no rule, so the same one is read with Q = 15.
// Scale rule and rounding (this library's reading of those pages):
//   amax = max |w| over the 32 values;  s = binary16_rne(amax / Q), Q = 7, 15
//   or 127, fp32 division;  s == 0 -> all codes 0;  else
//   q = clamp(rne(w / s), -Q-1, Q) with fp32 division by the stored binary16 scale.
// int5 row layout: K/2 bytes of the low 4 bits of every code (as int4), then
// K/8 bytes of bit 4 of every code (code k in bit k%8 of byte k/8).
// The library is built with correctly rounded fp32 division and without
// denormal flushing, so the result is bit-exact.
#include "wq_internal.h"
#include "wq_device.h"

namespace wq {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// One thread per (row, block). Offline path: clarity over bandwidth.
template <int BITS>
__global__ __launch_bounds__(256) void pack_kernel(const float *__restrict__ w, int64_t N,
                                                   int64_t K, uint8_t *__restrict__ q,
                                                   uint16_t *__restrict__ scales)
{
    constexpr float kQ = BITS == 4 ? 7.0f : BITS == 5 ? 15.0f : 127.0f;
    constexpr float kLo = -kQ - 1.0f;
    constexpr float kHi = kQ;
    const int64_t nb = K / kBlock;
    const int64_t total = N * nb;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t n = i / nb;
        const int64_t b = i - n * nb;
        const f4 *src = reinterpret_cast<const f4 *>(w + n * K + b * kBlock);
        float v[kBlock];
#pragma unroll
        for (int j = 0; j < kBlock / 4; ++j) {
            const f4 t = src[j];
            v[4 * j + 0] = t.x;
            v[4 * j + 1] = t.y;
            v[4 * j + 2] = t.z;
            v[4 * j + 3] = t.w;
        }
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < kBlock; ++j) amax = fmaxf(amax, fabsf(v[j]));

        const float s32 = amax / kQ;                    // correctly rounded
        const _Float16 s16 = (_Float16)s32;             // round to nearest even
        const float sf = (float)s16;                    // exact
        uint16_t sbits = __builtin_bit_cast(uint16_t, s16);

        int code[kBlock];
        if (sf == 0.0f) {
            sbits = 0;
#pragma unroll
            for (int j = 0; j < kBlock; ++j) code[j] = 0;
        } else {
#pragma unroll
            for (int j = 0; j < kBlock; ++j) {
                float t = rintf(v[j] / sf);             // fp32 division, ties to even
                t = fminf(fmaxf(t, kLo), kHi);
                code[j] = (int)t;
            }
        }
        scales[i] = sbits;

        if (BITS == 4 || BITS == 5) {
            // byte j holds code 2j (low nibble) and 2j+1 (high nibble); dword d
            // holds codes 8d..8d+7 at nibble positions 0..7 (int5: their low
            // 4 bits, and bit 4 of code j in bit j of the block's high-bit dword)
            const int64_t row = BITS == 4 ? K / 2 : K / 2 + K / 8;
            u4 out;
            uint32_t dw[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                uint32_t acc = 0;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc |= ((uint32_t)code[8 * d + e] & 0xFu) << (4 * e);
                dw[d] = acc;
            }
            out.x = dw[0]; out.y = dw[1]; out.z = dw[2]; out.w = dw[3];
            *reinterpret_cast<u4 *>(q + n * row + b * 16) = out;
            if (BITS == 5) {
                uint32_t hb = 0;
#pragma unroll
                for (int j = 0; j < kBlock; ++j) hb |= (((uint32_t)code[j] >> 4) & 1u) << j;
                *reinterpret_cast<uint32_t *>(q + n * row + K / 2 + b * 4) = hb;
            }
        } else {
            uint32_t dw[8];
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                uint32_t acc = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) acc |= ((uint32_t)code[4 * d + e] & 0xFFu) << (8 * e);
                dw[d] = acc;
            }
            u4 *dst = reinterpret_cast<u4 *>(q + n * K + b * kBlock);
            u4 lo, hi;
            lo.x = dw[0]; lo.y = dw[1]; lo.z = dw[2]; lo.w = dw[3];
            hi.x = dw[4]; hi.y = dw[5]; hi.z = dw[6]; hi.w = dw[7];
            dst[0] = lo;
            dst[1] = hi;
        }
    }
}

// One thread per (row, block): codes back to one int8 per value.
template <int BITS>
__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t *__restrict__ q, int64_t N,
                                                     int64_t K, int8_t *__restrict__ codes)
{
    const int64_t nb = K / kBlock;
    const int64_t total = N * nb;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t n = i / nb;
        const int64_t b = i - n * nb;
        uint32_t out[8];
        if (BITS == 5) {
            const int64_t row = K / 2 + K / 8;
            const u4 in = *reinterpret_cast<const u4 *>(q + n * row + b * 16);
            const uint32_t hb = *reinterpret_cast<const uint32_t *>(q + n * row + K / 2 + b * 4);
            const uint32_t dw[4] = {in.x, in.y, in.z, in.w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                uint32_t lo = 0, hi = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // 5-bit field: nibble e (and e+4) of dword d with its bit 4, sign-extended
                    const uint32_t fa = ((dw[d] >> (4 * e)) & 0xFu) | (((hb >> (8 * d + e)) & 1u) << 4);
                    const uint32_t fc = ((dw[d] >> (4 * e + 16)) & 0xFu) | (((hb >> (8 * d + e + 4)) & 1u) << 4);
                    const int32_t a = (int32_t)(fa << 27) >> 27;
                    const int32_t c = (int32_t)(fc << 27) >> 27;
                    lo |= ((uint32_t)a & 0xFFu) << (8 * e);
                    hi |= ((uint32_t)c & 0xFFu) << (8 * e);
                }
                out[2 * d] = lo;
                out[2 * d + 1] = hi;
            }
        } else if (BITS == 4) {
            const u4 in = *reinterpret_cast<const u4 *>(q + n * (K / 2) + b * 16);
            const uint32_t dw[4] = {in.x, in.y, in.z, in.w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                uint32_t lo = 0, hi = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // sign-extend nibble e (and e+4) of dword d to a byte
                    const int32_t a = (int32_t)(dw[d] << (28 - 4 * e)) >> 28;
                    const int32_t c = (int32_t)(dw[d] << (12 - 4 * e)) >> 28;
                    lo |= ((uint32_t)a & 0xFFu) << (8 * e);
                    hi |= ((uint32_t)c & 0xFFu) << (8 * e);
                }
                out[2 * d] = lo;
                out[2 * d + 1] = hi;
            }
        } else {
            const u4 *in = reinterpret_cast<const u4 *>(q + n * K + b * kBlock);
            const u4 a = in[0], c = in[1];
            out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
            out[4] = c.x; out[5] = c.y; out[6] = c.z; out[7] = c.w;
        }
        u4 *dst = reinterpret_cast<u4 *>(codes + n * K + b * kBlock);
        u4 lo, hi;
        lo.x = out[0]; lo.y = out[1]; lo.z = out[2]; lo.w = out[3];
        hi.x = out[4]; hi.y = out[5]; hi.z = out[6]; hi.w = out[7];
        dst[0] = lo;
        dst[1] = hi;
    }
}

inline unsigned grid_for(int64_t items)
{
    int64_t g = (items + 255) / 256;
    if (g > 65536) g = 65536;          // grid-stride loop covers the rest
    if (g < 1) g = 1;
    return (unsigned)g;
}

}  // namespace

hipError_t launch_pack(const float *w, int64_t N, int64_t K, int bits, void *q,
                       uint16_t *scales, hipStream_t stream)
{
    const unsigned grid = grid_for(N * (K / kBlock));
    if (bits == 4)
        pack_kernel<4><<<grid, 256, 0, stream>>>(w, N, K, (uint8_t *)q, scales);
    else if (bits == 5)
        pack_kernel<5><<<grid, 256, 0, stream>>>(w, N, K, (uint8_t *)q, scales);
    else
        pack_kernel<8><<<grid, 256, 0, stream>>>(w, N, K, (uint8_t *)q, scales);
    return hipGetLastError();
}

hipError_t launch_unpack(const void *q, int64_t N, int64_t K, int bits, int8_t *codes,
                         hipStream_t stream)
{
    const unsigned grid = grid_for(N * (K / kBlock));
    if (bits == 4)
        unpack_kernel<4><<<grid, 256, 0, stream>>>((const uint8_t *)q, N, K, codes);
    else if (bits == 5)
        unpack_kernel<5><<<grid, 256, 0, stream>>>((const uint8_t *)q, N, K, codes);
    else
        unpack_kernel<8><<<grid, 256, 0, stream>>>((const uint8_t *)q, N, K, codes);
    return hipGetLastError();
}

}  // namespace wq
