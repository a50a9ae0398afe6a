// wq_embed.hip -- tied token embedding: rows of the packed lm_head table,
// dequantized on the fly.
//
// The MOSS-Transcribe-Diarize LiteRT card ("Files") keeps the token embedding
// and the lm_head as one tied table in the embedder file, next to its `logits`
// signature, with `embed_1` and `embed_128` signatures that look up one or 128
// tokens. Here that table is the packed block-32 lm_head itself: row ids[i] is
// decoded and scaled into out[i] in fp32 and no dequantized table is ever stored.
// code * scale is exact in fp32 (a binary16 scale has 11 significant bits, a
// code at most 8), so every output is the exact dequantized weight. int4, int5
// and int8 tables are accepted (int5: a row's low-nibble plane, then its bit-4
// plane).
//
// One thread per 8 consecutive values of an output row: consecutive threads
// read consecutive code bytes of a row and write consecutive 32-byte pieces of
// out, so both sides are coalesced; all 8 values share one block scale.
// Rows whose id is outside [0, N) are filled with quiet NaN and never read.
#include "wq_internal.h"
#include "wq_device.h"

namespace wq {
namespace {

constexpr int kEmbedThreads = 256;

typedef float f4 __attribute__((ext_vector_type(4)));

template <int BITS>
__global__ __launch_bounds__(kEmbedThreads) void embed_kernel(const int32_t *__restrict__ ids, int K, int64_t N,
                                                              const uint8_t *__restrict__ q,
                                                              const uint16_t *__restrict__ s,
                                                              float *__restrict__ out, int64_t groups)
{
    const int64_t gi = (int64_t)blockIdx.x * kEmbedThreads + threadIdx.x;
    if (gi >= groups) return;
    const int per_row = K >> 3;                  // 8-value groups per row
    const int64_t i = gi / per_row;
    const int k0 = (int)(gi - i * per_row) * 8;
    const int64_t id = ids[i];
    f4 *dst = reinterpret_cast<f4 *>(out + i * (int64_t)K + k0);
    if (id < 0 || id >= N) {
        const float nan = __builtin_nanf("");
        dst[0] = f4{nan, nan, nan, nan};
        dst[1] = f4{nan, nan, nan, nan};
        return;
    }
    const float sc = (float)__builtin_bit_cast(_Float16, s[id * (K >> 5) + (k0 >> 5)]);
    int c[8];
    if constexpr (BITS == 8) {
        const uint2 v = *reinterpret_cast<const uint2 *>(q + id * (int64_t)K + k0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            c[j] = (int)(int8_t)(v.x >> (8 * j));
            c[4 + j] = (int)(int8_t)(v.y >> (8 * j));
        }
    } else if constexpr (BITS == 5) {
        // the row's low-nibble plane, then its bit-4 plane
        const uint8_t *row = q + id * (int64_t)(K / 2 + K / 8);
        const uint32_t v = *reinterpret_cast<const uint32_t *>(row + (k0 >> 1));
        const uint32_t hb = row[(K >> 1) + (k0 >> 3)];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t f = ((v >> (4 * j)) & 0xFu) | (((hb >> j) & 1u) << 4);
            c[j] = (int)(f << 27) >> 27;                                       // 5-bit field, sign-extended
        }
    } else {
        const uint32_t v = *reinterpret_cast<const uint32_t *>(q + id * (int64_t)(K >> 1) + (k0 >> 1));
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = (int)(v << (28 - 4 * j)) >> 28;   // nibble j, sign-extended
    }
    dst[0] = f4{(float)c[0] * sc, (float)c[1] * sc, (float)c[2] * sc, (float)c[3] * sc};
    dst[1] = f4{(float)c[4] * sc, (float)c[5] * sc, (float)c[6] * sc, (float)c[7] * sc};
}

}  // namespace

hipError_t launch_embed(const int32_t *ids, int64_t n_ids, int64_t K, int64_t N, int bits, const void *q,
                        const uint16_t *scales, float *out, hipStream_t stream)
{
    const int64_t groups = n_ids * (K / 8);
    const unsigned grid = (unsigned)((groups + kEmbedThreads - 1) / kEmbedThreads);
    if (bits == 4)
        embed_kernel<4><<<grid, kEmbedThreads, 0, stream>>>(ids, (int)K, N, (const uint8_t *)q, scales, out, groups);
    else if (bits == 5)
        embed_kernel<5><<<grid, kEmbedThreads, 0, stream>>>(ids, (int)K, N, (const uint8_t *)q, scales, out, groups);
    else
        embed_kernel<8><<<grid, kEmbedThreads, 0, stream>>>(ids, (int)K, N, (const uint8_t *)q, scales, out, groups);
    return hipGetLastError();
}

}  // namespace wq
