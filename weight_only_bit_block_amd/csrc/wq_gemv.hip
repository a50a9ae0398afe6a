// wq_gemv.hip -- decode GEMV for block-32 int4 / int8 weights, 1 <= M <= 16.
//
// The devpost page for TinyMOSS-Diarize ("How we built it") describes a
// separate GEMV path for decode that multiplies straight out of the packed
// weights, activations in FP32, dequantization fused, nothing materialized.
// This is that path designed for gfx950:
//
//  * HBM-bound weight stream: each lane owns whole 32-value blocks of a row
//    (16 B of int4 or 32 B of int8 codes, loaded with 128-bit loads); G lanes
//    share a row so a wavefront's loads are contiguous; each lane keeps J rows
//    in flight.
//  * x is staged once per workgroup in LDS (padded so the 128-bit reads of 64
//    lanes hit distinct banks) and reused across the J rows.
//  * Unpack in registers without int->float conversions: a nibble (byte) ORed
//    into the mantissa of binary16 1024.0 gives 1024 + code offset, and one
//    packed fp16 subtract recovers the exact integer code. The fp32 FMA takes
//    the binary16 code directly as an operand (mixed-precision FMA), so every
//    product q*x is formed exactly and accumulated in fp32.
//  * Per block: partial sums over the block's 32 values (two chains of 16),
//    then acc += scale * partial in fp32; lanes of a row are reduced with a
//    butterfly, so every lane of the group holds the same bits.
//
// Error: summation depth per output is 16 + 2 + (K/32)/G + log2(G), below the
// depth of ~160 at which fp32 rounding could reach 1e-5 * sum |x||w|.
#include "wq_internal.h"

namespace wq {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }

// int4: one dword of eight codes k0..k7 (nibble i = code k_i) to four fp16
// pairs holding the exact codes: (k0,k4), (k1,k5), (k2,k6), (k3,k7).
__device__ __forceinline__ void decode_int4(uint32_t d, h2 &p04, h2 &p15, h2 &p26, h2 &p37)
{
    const uint32_t u = d ^ 0x88888888u;        // two's complement -> code + 8
    const uint32_t v = u >> 8;
    const uint32_t magic = 0x64006400u;        // binary16 1024.0 in both halves
    const h2 a = as_h2((u & 0x000F000Fu) | magic);   // 1024 + (c + 8)
    const h2 b = as_h2((u & 0x00F000F0u) | magic);   // 1024 + 16 (c + 8)
    const h2 c = as_h2((v & 0x000F000Fu) | magic);
    const h2 e = as_h2((v & 0x00F000F0u) | magic);
    const h2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
    const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2 off16 = {(_Float16)72.0f, (_Float16)72.0f};
    p04 = a - off;                             // exact small integers
    p15 = b * sixteenth - off16;
    p26 = c - off;
    p37 = e * sixteenth - off16;
}

// int8: one dword of four codes k0..k3 to two fp16 pairs (k0,k1), (k2,k3).
__device__ __forceinline__ void decode_int8(uint32_t d, h2 &p01, h2 &p23)
{
    const uint32_t u = d ^ 0x80808080u;        // two's complement -> code + 128
    // bytes {u.b0, 0x64, u.b1, 0x64} and {u.b2, 0x64, u.b3, 0x64}
    const h2 a = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u));
    const h2 b = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u));
    const h2 off = {(_Float16)1152.0f, (_Float16)1152.0f};
    p01 = a - off;
    p23 = b - off;
}

__device__ __forceinline__ float fmix(_Float16 w, float x, float acc)
{
    return __builtin_fmaf((float)w, x, acc);   // one v_fma_mix_f32: exact product, one rounding
}

// One workgroup tile of the GEMV: rows [row0, row0 + 4 * (64/G) * J).
template <int BITS, int MT, int J>
__device__ __forceinline__ void gemv_tile(const float *__restrict__ x, int M, int K, int64_t N,
                                          const uint8_t *__restrict__ q,
                                          const uint16_t *__restrict__ s, float *__restrict__ y,
                                          int64_t row0, float *__restrict__ xs, int lds_floats)
{
    constexpr int CB = BITS * 4;               // bytes of codes per 32-value block
    constexpr int NV = CB / 16;                // 128-bit loads per block
    const int C = K >> 5;                      // blocks per row
    const int G = gemv_group(K);
    const int lg = __builtin_ctz(G);
    const int RW = kWave >> lg;                // rows per wavefront pass
    const int CPL = C >> lg;                   // blocks per lane per row
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int slot = lane >> lg;
    const int li = lane & (G - 1);
    const int64_t wrow0 = row0 + (int64_t)wave * RW * J;
    const size_t qrow = (size_t)C * CB;

    const uint8_t *qp[J];
    const uint16_t *sp[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        int64_t r = wrow0 + (int64_t)j * RW + slot;
        r = r < N ? r : N - 1;                 // clamp: loads stay in bounds, stores are masked
        qp[j] = q + (size_t)r * qrow;
        sp[j] = s + (size_t)r * C;
    }

    // Staged segment: rounds of G consecutive blocks; x rows mg..mg+MT-1.
    int seg_rounds = lds_floats / (MT * G * kGemvChunkPad);
    if (seg_rounds > CPL) seg_rounds = CPL;

    for (int mg = 0; mg < M; mg += MT) {
        const int mc = (M - mg) < MT ? (M - mg) : MT;
        float acc[J][MT];
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[j][m] = 0.0f;

        for (int r0 = 0; r0 < CPL; r0 += seg_rounds) {
            const int nr = (CPL - r0) < seg_rounds ? (CPL - r0) : seg_rounds;
            const int nchunks = nr * G;
            const int c0 = r0 * G;
            __syncthreads();                   // previous readers of xs are done
            const int items = MT * nchunks * 8;   // float4 items
            for (int i = threadIdx.x; i < items; i += kGemvThreads) {
                const int m = i / (nchunks * 8);
                const int rem = i - m * nchunks * 8;
                const int c = rem >> 3;
                const int f = rem & 7;
                f4 v = {0.0f, 0.0f, 0.0f, 0.0f};
                if (m < mc)
                    v = *reinterpret_cast<const f4 *>(x + (size_t)(mg + m) * K + (size_t)(c0 + c) * kBlock + f * 4);
                *reinterpret_cast<f4 *>(xs + (m * nchunks + c) * kGemvChunkPad + f * 4) = v;
            }
            __syncthreads();

            for (int rr = 0; rr < nr; ++rr) {
                const int chunk = c0 + rr * G + li;
                u4 wv[J][NV];
                float sc[J];
#pragma unroll
                for (int j = 0; j < J; ++j) {
#pragma unroll
                    for (int h = 0; h < NV; ++h)
                        wv[j][h] = *reinterpret_cast<const u4 *>(qp[j] + (size_t)chunk * CB + 16 * h);
                    sc[j] = (float)__builtin_bit_cast(_Float16, sp[j][chunk]);
                }
                const float *xc = xs + (rr * G + li) * kGemvChunkPad;
                float p0[J][MT], p1[J][MT];
#pragma unroll
                for (int j = 0; j < J; ++j)
#pragma unroll
                    for (int m = 0; m < MT; ++m) { p0[j][m] = 0.0f; p1[j][m] = 0.0f; }

#pragma unroll
                for (int sub = 0; sub < 4; ++sub) {
                    float xv[MT][8];
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        const f4 a = *reinterpret_cast<const f4 *>(xc + m * nchunks * kGemvChunkPad + sub * 8);
                        const f4 b = *reinterpret_cast<const f4 *>(xc + m * nchunks * kGemvChunkPad + sub * 8 + 4);
                        xv[m][0] = a.x; xv[m][1] = a.y; xv[m][2] = a.z; xv[m][3] = a.w;
                        xv[m][4] = b.x; xv[m][5] = b.y; xv[m][6] = b.z; xv[m][7] = b.w;
                    }
#pragma unroll
                    for (int j = 0; j < J; ++j) {
                        if (BITS == 4) {
                            const uint32_t d = wv[j][0][sub];
                            h2 t04, t15, t26, t37;
                            decode_int4(d, t04, t15, t26, t37);
#pragma unroll
                            for (int m = 0; m < MT; ++m) {
                                p0[j][m] = fmix(t04.x, xv[m][0], p0[j][m]);
                                p1[j][m] = fmix(t04.y, xv[m][4], p1[j][m]);
                                p0[j][m] = fmix(t15.x, xv[m][1], p0[j][m]);
                                p1[j][m] = fmix(t15.y, xv[m][5], p1[j][m]);
                                p0[j][m] = fmix(t26.x, xv[m][2], p0[j][m]);
                                p1[j][m] = fmix(t26.y, xv[m][6], p1[j][m]);
                                p0[j][m] = fmix(t37.x, xv[m][3], p0[j][m]);
                                p1[j][m] = fmix(t37.y, xv[m][7], p1[j][m]);
                            }
                        } else {
                            const uint32_t d0 = wv[j][sub >> 1][(sub & 1) * 2];
                            const uint32_t d1 = wv[j][sub >> 1][(sub & 1) * 2 + 1];
                            h2 t01, t23, t45, t67;
                            decode_int8(d0, t01, t23);
                            decode_int8(d1, t45, t67);
#pragma unroll
                            for (int m = 0; m < MT; ++m) {
                                p0[j][m] = fmix(t01.x, xv[m][0], p0[j][m]);
                                p1[j][m] = fmix(t01.y, xv[m][1], p1[j][m]);
                                p0[j][m] = fmix(t23.x, xv[m][2], p0[j][m]);
                                p1[j][m] = fmix(t23.y, xv[m][3], p1[j][m]);
                                p0[j][m] = fmix(t45.x, xv[m][4], p0[j][m]);
                                p1[j][m] = fmix(t45.y, xv[m][5], p1[j][m]);
                                p0[j][m] = fmix(t67.x, xv[m][6], p0[j][m]);
                                p1[j][m] = fmix(t67.y, xv[m][7], p1[j][m]);
                            }
                        }
                    }
                }
#pragma unroll
                for (int j = 0; j < J; ++j)
#pragma unroll
                    for (int m = 0; m < MT; ++m)
                        acc[j][m] = __builtin_fmaf(sc[j], p0[j][m] + p1[j][m], acc[j][m]);
            }
        }

        // butterfly over the G lanes of a row: every lane ends with the same sum
        for (int off = G >> 1; off > 0; off >>= 1) {
#pragma unroll
            for (int j = 0; j < J; ++j)
#pragma unroll
                for (int m = 0; m < MT; ++m) acc[j][m] += __shfl_xor(acc[j][m], off, kWave);
        }
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int64_t r = wrow0 + (int64_t)j * RW + slot;
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const int idx = j * MT + m;
                if ((idx & (G - 1)) == li && m < mc && r < N)
                    y[(size_t)(mg + m) * N + r] = acc[j][m];
            }
        }
    }
}

template <int BITS, int MT, int J>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(const float *__restrict__ x, int M, int K,
                                                            int64_t N, const uint8_t *__restrict__ q,
                                                            const uint16_t *__restrict__ s,
                                                            float *__restrict__ y, int lds_floats)
{
    extern __shared__ float xs[];
    const int64_t row0 = (int64_t)blockIdx.x * gemv_rows_per_tile(K, J);
    gemv_tile<BITS, MT, J>(x, M, K, N, q, s, y, row0, xs, lds_floats);
}

// Grouped launch: one workgroup per tile of any tensor of the table.
template <int MT, int J>
__global__ __launch_bounds__(kGemvThreads) void gemv_grouped_kernel(const uint8_t *__restrict__ base,
                                                                    const wq_desc *__restrict__ table,
                                                                    int count, int M, int lds_floats)
{
    extern __shared__ float xs[];
    const int64_t tile = blockIdx.x;
    int lo = 0, hi = count - 1;                // last entry with tile_begin <= tile
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (table[mid].tile_begin <= tile) lo = mid; else hi = mid - 1;
    }
    const wq_desc d = table[lo];
    const int64_t row0 = (tile - d.tile_begin) * gemv_rows_per_tile(d.K, J);
    const uint8_t *q = base + d.q_off;
    const uint16_t *s = reinterpret_cast<const uint16_t *>(base + d.s_off);
    if (d.bits == 4)
        gemv_tile<4, MT, J>(d.x, M, (int)d.K, d.N, q, s, d.y, row0, xs, lds_floats);
    else
        gemv_tile<8, MT, J>(d.x, M, (int)d.K, d.N, q, s, d.y, row0, xs, lds_floats);
}

// LDS budget per workgroup for the staged x: MT * 16 KiB.
inline int lds_floats_for(int MT) { return MT * 4096; }

template <int BITS, int MT>
hipError_t launch_gemv_mt(const float *x, int64_t M, int64_t K, int64_t N, const void *q,
                          const uint16_t *s, float *y, hipStream_t stream)
{
    // Pick J so that the launch has enough workgroups to cover the chip.
    int J = 8;
    while (J > 1 && (N + gemv_rows_per_tile(K, J) - 1) / gemv_rows_per_tile(K, J) < 512) J >>= 1;
    const int64_t rows = gemv_rows_per_tile(K, J);
    const unsigned grid = (unsigned)((N + rows - 1) / rows);
    const int G = gemv_group(K);
    int lds_floats = lds_floats_for(MT);
    const int need = (int)(MT * (K / kBlock) * kGemvChunkPad);   // whole row staged at once
    if (need < lds_floats) lds_floats = need;
    if (lds_floats < MT * G * kGemvChunkPad) lds_floats = MT * G * kGemvChunkPad;
    const size_t lds = (size_t)lds_floats * sizeof(float);
    const uint8_t *qb = (const uint8_t *)q;
    switch (J) {
    case 8: gemv_kernel<BITS, MT, 8><<<grid, kGemvThreads, lds, stream>>>(x, (int)M, (int)K, N, qb, s, y, lds_floats); break;
    case 4: gemv_kernel<BITS, MT, 4><<<grid, kGemvThreads, lds, stream>>>(x, (int)M, (int)K, N, qb, s, y, lds_floats); break;
    case 2: gemv_kernel<BITS, MT, 2><<<grid, kGemvThreads, lds, stream>>>(x, (int)M, (int)K, N, qb, s, y, lds_floats); break;
    default: gemv_kernel<BITS, MT, 1><<<grid, kGemvThreads, lds, stream>>>(x, (int)M, (int)K, N, qb, s, y, lds_floats); break;
    }
    return hipGetLastError();
}

template <int BITS>
hipError_t launch_gemv_bits(const float *x, int64_t M, int64_t K, int64_t N, const void *q,
                            const uint16_t *s, float *y, hipStream_t stream)
{
    switch (gemv_mt(M)) {
    case 1: return launch_gemv_mt<BITS, 1>(x, M, K, N, q, s, y, stream);
    case 2: return launch_gemv_mt<BITS, 2>(x, M, K, N, q, s, y, stream);
    case 3: return launch_gemv_mt<BITS, 3>(x, M, K, N, q, s, y, stream);
    default: return launch_gemv_mt<BITS, 4>(x, M, K, N, q, s, y, stream);
    }
}

template <int MT>
hipError_t launch_grouped_mt(const void *base, const wq_desc *table, int count, int64_t total_tiles,
                             int64_t M, hipStream_t stream)
{
    constexpr int J = MT <= 2 ? 8 : 4;
    static_assert(J == (MT <= 2 ? 8 : 4), "grouped J must match gemv_grouped_j");
    const int lds_floats = lds_floats_for(MT);
    gemv_grouped_kernel<MT, J><<<(unsigned)total_tiles, kGemvThreads, (size_t)lds_floats * sizeof(float), stream>>>(
        (const uint8_t *)base, table, count, (int)M, lds_floats);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const float *x, int64_t M, int64_t K, int64_t N, int bits, const void *q,
                       const uint16_t *scales, float *y, hipStream_t stream)
{
    if (bits == 4) return launch_gemv_bits<4>(x, M, K, N, q, scales, y, stream);
    return launch_gemv_bits<8>(x, M, K, N, q, scales, y, stream);
}

hipError_t launch_gemv_grouped(const void *base, const wq_desc *table_dev, int count,
                               int64_t total_tiles, int64_t M, hipStream_t stream)
{
    switch (gemv_mt(M)) {
    case 1: return launch_grouped_mt<1>(base, table_dev, count, total_tiles, M, stream);
    case 2: return launch_grouped_mt<2>(base, table_dev, count, total_tiles, M, stream);
    case 3: return launch_grouped_mt<3>(base, table_dev, count, total_tiles, M, stream);
    default: return launch_grouped_mt<4>(base, table_dev, count, total_tiles, M, stream);
    }
}

}  // namespace wq
