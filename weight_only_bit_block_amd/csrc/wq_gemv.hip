// wq_gemv.hip -- decode GEMV for block-32 int4 / int8 weights, 1 <= M <= 16.
//
// The devpost page for TinyMOSS-Diarize ("How we built it") describes a
// separate GEMV path for decode that multiplies straight out of the packed
// weights, activations in FP32, dequantization fused, nothing materialized.
// This is that path designed for gfx950:
//
//  * HBM-bound weight stream: each lane owns whole 32-value blocks of a row
//    (16 B of int4 or 32 B of int8 codes, non-temporal 128-bit loads); G lanes
//    share a row so a wavefront's loads are contiguous; each lane keeps J rows
//    in flight; a workgroup walks several consecutive tiles of one tensor, and
//    the wavefronts resident on a CU keep the memory system busy.
//  * x is staged in LDS (padded so the 128-bit reads of 64 lanes hit distinct
//    banks) once per workgroup when it fits, and reused across all rows.
//  * Unpack in registers without int->float conversions (wq_decode.h); the fp32
//    FMA takes the binary16 code directly as an operand (v_fma_mix_f32), so each
//    product q*x is exact and is accumulated in fp32.
//  * Per block: partial sums over the block's 32 values (two chains of 16),
//    then acc += scale * partial in fp32; lanes of a row are reduced with a
//    butterfly, so every lane of the group holds the same bits. The arithmetic of
//    an output does not depend on the tile shape, so every launch shape (and
//    the grouped launch) gives bitwise identical results.
//
// Error: summation depth per output is 16 + 2 + (K/32)/G + log2(G), below the
// depth of ~160 at which fp32 rounding could reach 1e-5 * sum |x||w|.
#include "wq_internal.h"
#include "wq_decode.h"

namespace wq {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float fmix(_Float16 w, float x, float acc)
{
    return __builtin_fmaf((float)w, x, acc);   // one v_fma_mix_f32: exact product, one rounding
}

template <int BITS, int J>
struct RoundBuf {
    static constexpr int NV = BITS / 4;        // 128-bit loads per block (1 for int4, 2 for int8)
    u4 w[J][NV];
    uint16_t s[J];
};

// Weights are streamed once: non-temporal 128-bit loads.
template <int BITS, int J>
__device__ __forceinline__ void load_round(RoundBuf<BITS, J> &b, const uint8_t *const (&qp)[J],
                                           const uint16_t *const (&sp)[J], int chunk)
{
    constexpr int CB = BITS * 4;
#pragma unroll
    for (int j = 0; j < J; ++j) {
#pragma unroll
        for (int h = 0; h < RoundBuf<BITS, J>::NV; ++h)
            b.w[j][h] = __builtin_nontemporal_load(reinterpret_cast<const u4 *>(qp[j] + (size_t)chunk * CB) + h);
        b.s[j] = sp[j][chunk];
    }
}

// One round: every lane multiplies its block of J rows by the staged x chunk.
template <int BITS, int MT, int J>
__device__ __forceinline__ void compute_round(const RoundBuf<BITS, J> &b, const float *__restrict__ xc,
                                              int mstride, const DecodeConsts &dc, float (&acc)[J][MT])
{
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
            const f4 a = *reinterpret_cast<const f4 *>(xc + m * mstride + sub * 8);
            const f4 c = *reinterpret_cast<const f4 *>(xc + m * mstride + sub * 8 + 4);
            xv[m][0] = a.x; xv[m][1] = a.y; xv[m][2] = a.z; xv[m][3] = a.w;
            xv[m][4] = c.x; xv[m][5] = c.y; xv[m][6] = c.z; xv[m][7] = c.w;
        }
#pragma unroll
        for (int j = 0; j < J; ++j) {
            if (BITS == 4) {
                h2 t04, t15, t26, t37;
                decode_int4(b.w[j][0][sub], dc, t04, t15, t26, t37);
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
                h2 t02, t13, t46, t57;
                decode_int8(b.w[j][sub >> 1][(sub & 1) * 2], dc, t02, t13);
                decode_int8(b.w[j][sub >> 1][(sub & 1) * 2 + 1], dc, t46, t57);
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    p0[j][m] = fmix(t02.x, xv[m][0], p0[j][m]);
                    p1[j][m] = fmix(t02.y, xv[m][2], p1[j][m]);
                    p0[j][m] = fmix(t13.x, xv[m][1], p0[j][m]);
                    p1[j][m] = fmix(t13.y, xv[m][3], p1[j][m]);
                    p0[j][m] = fmix(t46.x, xv[m][4], p0[j][m]);
                    p1[j][m] = fmix(t46.y, xv[m][6], p1[j][m]);
                    p0[j][m] = fmix(t57.x, xv[m][5], p0[j][m]);
                    p1[j][m] = fmix(t57.y, xv[m][7], p1[j][m]);
                }
            }
        }
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const float sc = (float)__builtin_bit_cast(_Float16, b.s[j]);
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[j][m] = __builtin_fmaf(sc, p0[j][m] + p1[j][m], acc[j][m]);
    }
}

// Stage x rows [mg, mg+mc) and blocks [c0, c0+nchunks) into LDS, padded rows.
template <int MT>
__device__ __forceinline__ void stage_x(const float *__restrict__ x, int K, int mg, int mc, int c0,
                                        int nchunks, float *__restrict__ xs)
{
    const int items = MT * nchunks * 8;        // float4 items
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
}

// A workgroup computes `ntiles` consecutive tiles starting at row `row0` for all
// M activation rows. Steps are (tile, m-group, round); the weights of step s+1
// are loaded before step s is computed.
template <int BITS, int MT, int J>
__device__ __forceinline__ void gemv_tiles(const float *__restrict__ x, int M, int K, int64_t N,
                                           const uint8_t *__restrict__ q,
                                           const uint16_t *__restrict__ s, float *__restrict__ y,
                                           int64_t row0, int ntiles, float *__restrict__ xs,
                                           int lds_floats)
{
    constexpr int CB = BITS * 4;
    const int C = K >> 5;                      // blocks per row
    const int G = gemv_group(K);
    const int lg = __builtin_ctz(G);
    const int RW = kWave >> lg;                // rows per wavefront pass
    const int CPL = C >> lg;                   // rounds per tile
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int slot = lane >> lg;
    const int li = lane & (G - 1);
    const size_t qrow = (size_t)C * CB;
    const int64_t tile_rows = (int64_t)kGemvWaves * RW * J;
    const DecodeConsts dc = DecodeConsts::make();

    int seg = lds_floats / (MT * G * kGemvChunkPad);   // rounds staged at once
    if (seg > CPL) seg = CPL;
    const int n_mg = (M + MT - 1) / MT;
    // x stays resident for the whole workgroup when one m-group and one segment cover it
    const bool resident = (n_mg == 1) && (seg == CPL);
    const int steps_per_tile = n_mg * CPL;
    const int steps = ntiles * steps_per_tile;

    const uint8_t *qp[J];
    const uint16_t *sp[J];
    auto set_rows = [&](int tile) {
        const int64_t wrow0 = row0 + (int64_t)tile * tile_rows + (int64_t)wave * RW * J;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            int64_t r = wrow0 + (int64_t)j * RW + slot;
            r = r < N ? r : N - 1;             // clamp: loads stay in bounds, stores are masked
            qp[j] = q + (size_t)r * qrow;
            sp[j] = s + (size_t)r * C;
        }
    };

    // One step of the (tile, m-group, round) sequence: issue this step's J
    // weight loads, then compute. Loads are not carried across iterations (the
    // compiler would otherwise wait on all of them at the loop back-edge);
    // latency is hidden by the other wavefronts resident on the CU.
    float acc[J][MT];
    for (int st = 0; st < steps; ++st) {
        const int tile = st / steps_per_tile;
        const int rem = st - tile * steps_per_tile;
        const int mgi = rem / CPL;
        const int rnd = rem - mgi * CPL;
        const int mg = mgi * MT;
        const int mc = (M - mg) < MT ? (M - mg) : MT;
        const int sidx = rnd / seg;            // segment of this round
        const int c0 = sidx * seg * G;
        const int nr = (CPL - sidx * seg) < seg ? (CPL - sidx * seg) : seg;
        const int nchunks = nr * G;

        if (rnd == 0 && mgi == 0) set_rows(tile);
        RoundBuf<BITS, J> cur;
        load_round<BITS, J>(cur, qp, sp, rnd * G + li);
        if (rnd % seg == 0 && (!resident || st == 0)) {
            lds_barrier();                     // earlier readers of xs are done
            stage_x<MT>(x, K, mg, mc, c0, nchunks, xs);
            lds_barrier();
        }
        if (rnd == 0) {
#pragma unroll
            for (int j = 0; j < J; ++j)
#pragma unroll
                for (int m = 0; m < MT; ++m) acc[j][m] = 0.0f;
        }
        const float *xc = xs + ((rnd - sidx * seg) * G + li) * kGemvChunkPad;
        compute_round<BITS, MT, J>(cur, xc, nchunks * kGemvChunkPad, dc, acc);

        if (rnd == CPL - 1) {
            // butterfly over the G lanes of a row: every lane ends with the same sum
            for (int off = G >> 1; off > 0; off >>= 1) {
#pragma unroll
                for (int j = 0; j < J; ++j)
#pragma unroll
                    for (int m = 0; m < MT; ++m) acc[j][m] += __shfl_xor(acc[j][m], off, kWave);
            }
            const int64_t wrow0 = row0 + (int64_t)tile * tile_rows + (int64_t)wave * RW * J;
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
}

template <int BITS, int MT, int J>
__global__ __launch_bounds__(kGemvThreads, 2) void gemv_kernel(const float *__restrict__ x, int M, int K,
                                                               int64_t N, const uint8_t *__restrict__ q,
                                                               const uint16_t *__restrict__ s,
                                                               float *__restrict__ y, int tiles_per_wg,
                                                               int64_t total_tiles, int lds_floats)
{
    extern __shared__ float xs[];
    const int64_t t0 = (int64_t)blockIdx.x * tiles_per_wg;
    const int64_t left = total_tiles - t0;
    const int nt = left < tiles_per_wg ? (int)left : tiles_per_wg;
    gemv_tiles<BITS, MT, J>(x, M, K, N, q, s, y, t0 * gemv_rows_per_tile(K, J), nt, xs, lds_floats);
}

// Grouped launch: each workgroup takes up to kGroupedTilesPerWg consecutive
// tiles of one tensor of the table.
template <int MT>
__global__ __launch_bounds__(kGemvThreads, 2) void gemv_grouped_kernel(const uint8_t *__restrict__ base,
                                                                       const wq_desc *__restrict__ table,
                                                                       int count, int M, int lds_floats)
{
    extern __shared__ float xs[];
    const int64_t item = blockIdx.x;
    int lo = 0, hi = count - 1;                // last entry with tile_begin <= item
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (table[mid].tile_begin <= item) lo = mid; else hi = mid - 1;
    }
    const wq_desc d = table[lo];
    const uint8_t *q = base + d.q_off;
    const uint16_t *s = reinterpret_cast<const uint16_t *>(base + d.s_off);
    const int64_t t0 = (item - d.tile_begin) * kGroupedTilesPerWg;
    if (d.bits == 4) {
        constexpr int J = MT <= 2 ? 8 : 4;
        const int64_t rows = gemv_rows_per_tile(d.K, J);
        const int64_t tiles = (d.N + rows - 1) / rows;
        const int nt = (tiles - t0) < kGroupedTilesPerWg ? (int)(tiles - t0) : kGroupedTilesPerWg;
        gemv_tiles<4, MT, J>(d.x, M, (int)d.K, d.N, q, s, d.y, t0 * rows, nt, xs, lds_floats);
    } else {
        constexpr int J = MT <= 2 ? 4 : 2;
        const int64_t rows = gemv_rows_per_tile(d.K, J);
        const int64_t tiles = (d.N + rows - 1) / rows;
        const int nt = (tiles - t0) < kGroupedTilesPerWg ? (int)(tiles - t0) : kGroupedTilesPerWg;
        gemv_tiles<8, MT, J>(d.x, M, (int)d.K, d.N, q, s, d.y, t0 * rows, nt, xs, lds_floats);
    }
}

// LDS floats for staging: the whole (padded) x of an m-group if it fits the
// budget, else as many rounds as fit (at least one).
inline int lds_floats_for(int MT, int64_t K)
{
    const int G = gemv_group(K);
    int f = MT * kGemvLdsFloatsPerMT;
    const int64_t whole = (int64_t)MT * (K / kBlock) * kGemvChunkPad;
    if (whole < f) f = (int)whole;
    if (f < MT * G * kGemvChunkPad) f = MT * G * kGemvChunkPad;
    return f;
}

template <int BITS, int MT, int J>
hipError_t launch_j(const float *x, int64_t M, int64_t K, int64_t N, const void *q, const uint16_t *s,
                    float *y, hipStream_t stream)
{
    const int64_t rows = gemv_rows_per_tile(K, J);
    const int64_t tiles = (N + rows - 1) / rows;
    // consecutive tiles per workgroup: keep at least ~1024 workgroups when possible
    int tpw = (int)(tiles / 1024);
    if (tpw < 1) tpw = 1;
    if (tpw > 8) tpw = 8;
    const int64_t grid = (tiles + tpw - 1) / tpw;
    const int lds_floats = lds_floats_for(MT, K);
    gemv_kernel<BITS, MT, J><<<(unsigned)grid, kGemvThreads, (size_t)lds_floats * sizeof(float), stream>>>(
        x, (int)M, (int)K, N, (const uint8_t *)q, s, y, tpw, tiles, lds_floats);
    return hipGetLastError();
}

template <int BITS, int MT>
hipError_t launch_gemv_mt(const float *x, int64_t M, int64_t K, int64_t N, const void *q,
                          const uint16_t *s, float *y, hipStream_t stream)
{
    // The grouped depth J when the launch still has >= 512 workgroups, else
    // shallower tiles so small GEMVs spread over the chip.
    constexpr int JG = BITS == 4 ? (MT <= 2 ? 8 : 4) : (MT <= 2 ? 4 : 2);
    int J = JG;
    while (J > 1 && (N + gemv_rows_per_tile(K, J) - 1) / gemv_rows_per_tile(K, J) < 512) J >>= 1;
    switch (J) {
    case JG: return launch_j<BITS, MT, JG>(x, M, K, N, q, s, y, stream);
    case (JG >= 2 ? JG / 2 : 1): return launch_j<BITS, MT, (JG >= 2 ? JG / 2 : 1)>(x, M, K, N, q, s, y, stream);
    default: return launch_j<BITS, MT, 1>(x, M, K, N, q, s, y, stream);
    }
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
hipError_t launch_grouped_mt(const void *base, const wq_desc *table, int count, int64_t items,
                             int64_t M, hipStream_t stream)
{
    const int lds_floats = MT * kGemvLdsFloatsPerMT;
    gemv_grouped_kernel<MT><<<(unsigned)items, kGemvThreads, (size_t)lds_floats * sizeof(float), stream>>>(
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
                               int64_t total_items, int64_t M, hipStream_t stream)
{
    switch (gemv_mt(M)) {
    case 1: return launch_grouped_mt<1>(base, table_dev, count, total_items, M, stream);
    case 2: return launch_grouped_mt<2>(base, table_dev, count, total_items, M, stream);
    case 3: return launch_grouped_mt<3>(base, table_dev, count, total_items, M, stream);
    default: return launch_grouped_mt<4>(base, table_dev, count, total_items, M, stream);
    }
}

}  // namespace wq
