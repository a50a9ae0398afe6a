// wq_gemm.hip -- prefill GEMM for block-32 int4 / int8 weights (any M, tuned for M >= 128).
//
// The TinyMOSS-Diarize devpost page ("How we built it") describes a blocked
// prefill GEMM that unpacks each weight group once into a fast tile and reuses
// it across all activation rows. On gfx950 the tile lives in LDS and the inner
// product runs on the matrix cores:
//
//  * A workgroup computes a 128 x 128 tile of y with 4 wavefronts (2 x 2, each
//    64 x 64 = 4 x 4 fragments of 16 x 16).
//  * Each K step is exactly one quantization block (32 values): the weight
//    codes of the tile are unpacked once into LDS as binary16 (exact integers),
//    x is rounded to binary16 (nearest even) into LDS, and one
//    v_mfma_f32_16x16x32_f16 per fragment forms the block's fp32 partial from a
//    zero accumulator; the partial is then scaled by that row's block scale and
//    added to the fp32 accumulator.
//  * Two LDS buffers: the global loads of step k+1 are issued before the
//    matrix work of step k; one barrier per step.
//  * Within a block the order of the 32 values is permuted identically for x
//    and the weights (the int4 unpack yields pairs (k0,k4), (k1,k5), ...), which
//    leaves every dot product unchanged.
#include "wq_internal.h"

namespace wq {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int LDH = 40;            // halfs per LDS row: 32 + 8 padding (80 B; 128-bit reads conflict-free)
constexpr int kThreads = 256;

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }

// int4 dword (codes k0..k7) -> h8 {k0,k4,k1,k5,k2,k6,k3,k7}, exact.
__device__ __forceinline__ h8 unpack8_int4(uint32_t d)
{
    const uint32_t u = d ^ 0x88888888u;
    const uint32_t v = u >> 8;
    const uint32_t magic = 0x64006400u;
    const h2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
    const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2 off16 = {(_Float16)72.0f, (_Float16)72.0f};
    const h2 a = as_h2((u & 0x000F000Fu) | magic) - off;
    const h2 b = as_h2((u & 0x00F000F0u) | magic) * sixteenth - off16;
    const h2 c = as_h2((v & 0x000F000Fu) | magic) - off;
    const h2 e = as_h2((v & 0x00F000F0u) | magic) * sixteenth - off16;
    h8 r;
    r[0] = a.x; r[1] = a.y; r[2] = b.x; r[3] = b.y;
    r[4] = c.x; r[5] = c.y; r[6] = e.x; r[7] = e.y;
    return r;
}

// int8 dwords (codes k0..k3, k4..k7) -> h8 {k0..k7}, exact.
__device__ __forceinline__ h8 unpack8_int8(uint32_t d0, uint32_t d1)
{
    const h2 off = {(_Float16)1152.0f, (_Float16)1152.0f};
    const uint32_t u0 = d0 ^ 0x80808080u, u1 = d1 ^ 0x80808080u;
    const h2 a = as_h2(__builtin_amdgcn_perm(0x64646464u, u0, 0x04010400u)) - off;
    const h2 b = as_h2(__builtin_amdgcn_perm(0x64646464u, u0, 0x04030402u)) - off;
    const h2 c = as_h2(__builtin_amdgcn_perm(0x64646464u, u1, 0x04010400u)) - off;
    const h2 e = as_h2(__builtin_amdgcn_perm(0x64646464u, u1, 0x04030402u)) - off;
    h8 r;
    r[0] = a.x; r[1] = a.y; r[2] = b.x; r[3] = b.y;
    r[4] = c.x; r[5] = c.y; r[6] = e.x; r[7] = e.y;
    return r;
}

// 8 fp32 x values -> binary16 (nearest even) in the same order as the weights.
template <int BITS>
__device__ __forceinline__ h8 pack8_x(const f4 &lo, const f4 &hi)
{
    h8 r;
    if (BITS == 4) {
        r[0] = (_Float16)lo.x; r[1] = (_Float16)hi.x;
        r[2] = (_Float16)lo.y; r[3] = (_Float16)hi.y;
        r[4] = (_Float16)lo.z; r[5] = (_Float16)hi.z;
        r[6] = (_Float16)lo.w; r[7] = (_Float16)hi.w;
    } else {
        r[0] = (_Float16)lo.x; r[1] = (_Float16)lo.y;
        r[2] = (_Float16)lo.z; r[3] = (_Float16)lo.w;
        r[4] = (_Float16)hi.x; r[5] = (_Float16)hi.y;
        r[6] = (_Float16)hi.z; r[7] = (_Float16)hi.w;
    }
    return r;
}

template <int BITS>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const float *__restrict__ x, int M, int K,
                                                        int N, const uint8_t *__restrict__ q,
                                                        const uint16_t *__restrict__ s,
                                                        float *__restrict__ y, int tiles_n)
{
    __shared__ _Float16 As[2][BM * LDH];
    __shared__ _Float16 Bs[2][BN * LDH];
    __shared__ float Ss[2][BN];

    const int tm = blockIdx.x / tiles_n;
    const int tn = blockIdx.x - tm * tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int C = K >> 5;

    // staging role: row r of the tile, half h of the block (16 values)
    const int r = t >> 1, h = t & 1;
    const int xr = (m0 + r) < M ? (m0 + r) : (M - 1);
    const int wr = (n0 + r) < N ? (n0 + r) : (N - 1);
    const float *xrow = x + (size_t)xr * K + 16 * h;
    const uint8_t *qrow = q + (size_t)wr * (K * BITS / 8) + h * (BITS * 2);
    const int sr = (n0 + t) < N ? (n0 + t) : (N - 1);
    const uint16_t *srow = s + (size_t)sr * C;

    f4 xg[4];
    u4 wg;
    uint16_t sg = 0;

    auto load = [&](int kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) xg[i] = *reinterpret_cast<const f4 *>(xrow + (size_t)kb * kBlock + 4 * i);
        if (BITS == 4) {
            const u2 v = *reinterpret_cast<const u2 *>(qrow + (size_t)kb * 16);
            wg.x = v.x; wg.y = v.y;
        } else {
            wg = *reinterpret_cast<const u4 *>(qrow + (size_t)kb * 32);
        }
        if (t < BN) sg = srow[kb];
    };
    auto store = [&](int buf) {
        h8 xa = pack8_x<BITS>(xg[0], xg[1]);
        h8 xb = pack8_x<BITS>(xg[2], xg[3]);
        *reinterpret_cast<h8 *>(&As[buf][r * LDH + 16 * h]) = xa;
        *reinterpret_cast<h8 *>(&As[buf][r * LDH + 16 * h + 8]) = xb;
        h8 wa, wb;
        if (BITS == 4) {
            wa = unpack8_int4(wg.x);
            wb = unpack8_int4(wg.y);
        } else {
            wa = unpack8_int8(wg.x, wg.y);
            wb = unpack8_int8(wg.z, wg.w);
        }
        *reinterpret_cast<h8 *>(&Bs[buf][r * LDH + 16 * h]) = wa;
        *reinterpret_cast<h8 *>(&Bs[buf][r * LDH + 16 * h + 8]) = wb;
        if (t < BN) Ss[buf][t] = (float)__builtin_bit_cast(_Float16, sg);
    };

    f4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f4{0.0f, 0.0f, 0.0f, 0.0f};

    load(0);
    store(0);
    __syncthreads();

    const int frow = lane & 15, fk = (lane >> 4) * 8;
    for (int kb = 0; kb < C; ++kb) {
        const int cur = kb & 1;
        if (kb + 1 < C) load(kb + 1);

        h8 a[4], b[4];
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a[i] = *reinterpret_cast<const h8 *>(&As[cur][(wm * 64 + i * 16 + frow) * LDH + fk]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            b[j] = *reinterpret_cast<const h8 *>(&Bs[cur][(wn * 64 + j * 16 + frow) * LDH + fk]);
            sc[j] = Ss[cur][wn * 64 + j * 16 + frow];
        }
        const f4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f4 p = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], zero, 0, 0, 0);
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[i][j][v] = __builtin_fmaf(sc[j], p[v], acc[i][j][v]);
            }

        if (kb + 1 < C) store(cur ^ 1);
        __syncthreads();
    }

    // D fragment layout: lane holds column (lane & 15), rows 4*(lane >> 4) + v.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + wn * 64 + j * 16 + (lane & 15);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = m0 + wm * 64 + i * 16 + 4 * (lane >> 4) + v;
                if (m < M && n < N) y[(size_t)m * N + n] = acc[i][j][v];
            }
        }
}

}  // namespace

hipError_t launch_gemm(const float *x, int64_t M, int64_t K, int64_t N, int bits, const void *q,
                       const uint16_t *scales, float *y, hipStream_t stream)
{
    const int tiles_m = (int)((M + BM - 1) / BM);
    const int tiles_n = (int)((N + BN - 1) / BN);
    const unsigned grid = (unsigned)tiles_m * (unsigned)tiles_n;
    if (bits == 4)
        gemm_kernel<4><<<grid, kThreads, 0, stream>>>(x, (int)M, (int)K, (int)N, (const uint8_t *)q, scales, y, tiles_n);
    else
        gemm_kernel<8><<<grid, kThreads, 0, stream>>>(x, (int)M, (int)K, (int)N, (const uint8_t *)q, scales, y, tiles_n);
    return hipGetLastError();
}

}  // namespace wq
