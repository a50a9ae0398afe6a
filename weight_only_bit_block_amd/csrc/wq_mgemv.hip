// wq_mgemv.hip -- decode GEMV for 3 <= M <= 16 activation rows on the matrix cores.
//
// The decode path of the TinyMOSS-Diarize devpost page ("How we built it")
// multiplies straight out of the packed weights with FP32 activations. With one
// activation row that is the fp32 FMA kernel of wq_gemv.hip. With several, an
// fp32 FMA design re-reads x from LDS for every weight row a lane owns (8*M bytes
// of LDS reads per byte of codes), which makes it LDS-bound on gfx950 well
// before HBM. Here the M rows of x go through the fp16 matrix cores instead,
// with fp32 accuracy kept:
//
//  * Exact split of x. Per activation row m and quantization block b the
//    values are scaled by a power of two 2^e (the block's largest magnitude
//    lands in [2^14, 2^15)), then split into three binary16 parts
//    h1 = rne(x'), h2 = rne(x' - h1), h3 = rne(x' - h1 - h2) (each difference
//    exact in fp32), so h1 + h2 + h3 == x' for every value within 2^16 of the
//    block's largest (smaller ones keep an absolute error below 2^-25 of the
//    scaled unit). A 32-row matrix operand holds 8 activation rows: h1 of row
//    m in operand row m, h2 in row 8+m, h3 in row 16+m (rows 24..31 unused);
//    M > 8 takes a second operand. Codes are exact binary16 integers, every
//    product is exact and the matrix core sums in fp32.
//  * Per block and operand, two chained v_mfma_f32_32x32x16_f16 from a zero
//    accumulator give P[32 x 32]; operand rows m, 8+m and 16+m land in one lane
//    (values v, v+4, v+8), so row m's block partial is P[v] + P[v+4] + P[v+8],
//    and acc[m] += (s[n,b] * 2^-e[m,b]) * partial in fp32 (the product of a
//    binary16 scale and a power of two is exact). The summation depth per
//    output is about 8 + K/32, far below the ~160 at which fp32 rounding could
//    reach 1e-5 * sum |x||w|.
//  * A workgroup of 4 wavefronts owns 128 consecutive weight rows (32 per
//    wavefront, one matrix column each) for all K. Lane (n, g) of a wavefront
//    loads codes 16g..16g+15 of every block of its row straight from HBM into
//    registers (one segment of 8 blocks ahead, cached: the 8 loads of a segment
//    share each row's cache lines); x of the next segment is loaded
//    into registers while the current one is computed, then split into the
//    other of two LDS buffers. The operand order of the 8 values of a k-group is
//    the order the unpack produces, identical for x and the codes.
//  * The operand rows are stored with a row-dependent XOR swizzle of their
//    16-byte slots, so the 16 lanes of each 128-bit LDS read hit distinct banks.
// x blocks whose largest magnitude is below 2^-112 lose relative precision (the
// factor 2^e is capped at 2^126 so that 2^-e stays a normal fp32 number); any
// other finite fp32 x is split exactly as above.
#include "wq_internal.h"
#include "wq_decode.h"

namespace wq {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int kSB = 8;                           // blocks per segment
constexpr int kRowBytes = kSB * 32 * 2;          // one operand row of a segment, binary16
constexpr int kOpBytes = 32 * kRowBytes;         // one 32-row operand (8 activation rows, 3 parts)
constexpr int kEBytes = 16 * kSB * 4;            // 2^-e per (block, x row): [kSB][16] floats

template <int MF>
struct Buf {
    static constexpr int A_BYTES = MF * kOpBytes;
    static constexpr int BYTES = A_BYTES + kEBytes;
};

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// 16-byte slot s of operand row r (32 slots per row in a segment)
__device__ __forceinline__ int aoff(int r, int s) { return r * kRowBytes + ((s ^ r) & 31) * 16; }

// Lane (n, g) codes of one block as two groups of 8 in unpack order, (int5) the
// two bytes of their bit 4, and the block's scale.
template <int BITS>
struct LaneCodes {
    uint32_t v[BITS == 8 ? 4 : 2];
    uint32_t h;
    uint32_t sc;
};

template <int BITS>
__device__ __forceinline__ LaneCodes<BITS> load_codes(__amdgpu_buffer_rsrc_t qr, __amdgpu_buffer_rsrc_t sr,
                                                      uint32_t rowq, uint32_t hrow, uint32_t rows, int b, int g)
{
    LaneCodes<BITS> c;
    c.sc = __builtin_amdgcn_raw_buffer_load_b16(sr, rows + (uint32_t)b * 2, 0, 0);
    if constexpr (BITS == 8) {
        const u4 v = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(qr, rowq + (uint32_t)b * 32 + g * 16, 0, 0));
        c.v[0] = v.x; c.v[1] = v.y; c.v[2] = v.z; c.v[3] = v.w;
        c.h = 0;
    } else {
        const u2 v = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(qr, rowq + (uint32_t)b * 16 + g * 8, 0, 0));
        c.v[0] = v.x; c.v[1] = v.y;
        c.h = 0;
        if constexpr (BITS == 5)
            c.h = __builtin_amdgcn_raw_buffer_load_b16(qr, hrow + (uint32_t)b * 4 + g * 2, 0, 0);
    }
    return c;
}

template <int BITS>
__device__ __forceinline__ void unpack_codes(const LaneCodes<BITS> &c, const DecodeConsts &dc,
                                             const Decode5Consts &dc5, h8 (&b)[2])
{
    if constexpr (BITS == 4) {
        b[0] = unpack8_int4(c.v[0], dc);
        b[1] = unpack8_int4(c.v[1], dc);
    } else if constexpr (BITS == 5) {
        b[0] = unpack8_int5(c.v[0], c.h & 0xFF, dc5);
        b[1] = unpack8_int5(c.v[1], c.h >> 8, dc5);
    } else {
        b[0] = unpack8_int8(c.v[0], c.v[1], dc);
        b[1] = unpack8_int8(c.v[2], c.v[3], dc);
    }
}

// x of one segment: group i (8 values) of the segment is row m, block blk,
// k-group q (i = (m * kSB + blk) * 4 + q); a thread holds XG groups.
constexpr int kXG = 16 * kSB * 4 / 256;          // groups per thread (M <= 16): 2

struct XStage {
    f4 v[kXG][2];
};

__device__ __forceinline__ void load_x(XStage &xs, const float *__restrict__ x, int M, int K, int b0, int t)
{
    const int C = K >> 5;
#pragma unroll
    for (int i = 0; i < kXG; ++i) {
        const int idx = t + i * 256;
        int m = idx / (kSB * 4);
        const int blk = (idx / 4) % kSB, q = idx & 3;
        int b = b0 + blk;
        m = m < M ? m : M - 1;                   // rows past M and blocks past K load valid data, unused
        b = b < C ? b : C - 1;
        const f4 *p = reinterpret_cast<const f4 *>(x + (size_t)m * K + b * 32 + q * 8);
        xs.v[i][0] = p[0];
        xs.v[i][1] = p[1];
    }
}

// Split the staged x into the operand rows and the per-(row, block) factors.
template <int BITS, int MF>
__device__ __forceinline__ void store_x(const XStage &xs, int M, uint8_t *buf, int t)
{
    float *E = reinterpret_cast<float *>(buf + Buf<MF>::A_BYTES);
#pragma unroll
    for (int i = 0; i < kXG; ++i) {
        const int idx = t + i * 256;
        const int m = idx / (kSB * 4);
        const int blk = (idx / 4) % kSB, q = idx & 3;
        const float v[8] = {xs.v[i][0].x, xs.v[i][0].y, xs.v[i][0].z, xs.v[i][0].w,
                            xs.v[i][1].x, xs.v[i][1].y, xs.v[i][1].z, xs.v[i][1].w};
        float mx = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) mx = fmaxf(mx, fabsf(v[k]));
        // the 4 groups of a (row, block) are lanes 4j..4j+3: block maximum
        mx = fmaxf(mx, dpp<0xB1>(mx));
        mx = fmaxf(mx, dpp<0x4E>(mx));
        int e = 0;
        if (mx > 0.0f) {
            const int E2 = (int)((__builtin_bit_cast(uint32_t, mx) >> 23) & 0xFF) - 127;   // floor(log2) for normals
            e = 14 - E2;
            e = e > 126 ? 126 : e;
        }
        h8 p1, p2, p3;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float xv = __builtin_ldexpf(v[k], e);
            const _Float16 h1 = (_Float16)xv;                 // nearest even
            const float r1 = xv - (float)h1;                  // exact in fp32
            const _Float16 h2 = (_Float16)r1;
            const _Float16 h3 = (_Float16)(r1 - (float)h2);   // exact difference, then nearest even
            p1[operand_slot<BITS>(k)] = h1;
            p2[operand_slot<BITS>(k)] = h2;
            p3[operand_slot<BITS>(k)] = h3;
        }
        if (m < M) {
            const int s = blk * 4 + q;
            uint8_t *op = buf + (m >> 3) * kOpBytes;
            const int mm = m & 7;
            *reinterpret_cast<h8 *>(op + aoff(mm, s)) = p1;
            *reinterpret_cast<h8 *>(op + aoff(8 + mm, s)) = p2;
            *reinterpret_cast<h8 *>(op + aoff(16 + mm, s)) = p3;
            if (q == 0) E[blk * 16 + m] = __builtin_ldexpf(1.0f, -e);
        }
    }
}

// One item: weight rows row0 .. row0+127 of one tensor, all M activation rows
// (M <= 8 * MF).
template <int BITS, int MF>
__device__ __forceinline__ void mgemv_item(const float *__restrict__ x, int M, int K, int64_t N,
                                           const uint8_t *__restrict__ q, const uint16_t *__restrict__ s,
                                           float *__restrict__ y, int64_t row0, uint8_t *__restrict__ lds)
{
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int r = lane & 31, g = lane >> 5;
    const int C = K >> 5;
    const int nseg = (C + kSB - 1) / kSB;
    const uint32_t qrow = (uint32_t)K * BITS / 8;
    const DecodeConsts dc = DecodeConsts::make();
    Decode5Consts dc5;
    if constexpr (BITS == 5) dc5 = Decode5Consts::make();
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(q, (uint64_t)N * qrow);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(s, (uint64_t)N * C * 2);
    int64_t n = row0 + wave * 32 + r;
    const bool nvalid = n < N;
    n = nvalid ? n : N - 1;                      // rows past N reload the last row, not stored
    const uint32_t rowq = (uint32_t)n * qrow, hrow = rowq + (uint32_t)K / 2, rows = (uint32_t)n * C * 2;

    float acc[MF][4];
#pragma unroll
    for (int f = 0; f < MF; ++f)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[f][v] = 0.0f;
    const f16v zero = {};

    LaneCodes<BITS> cd[kSB];
    XStage xs;
    // prologue: segment 0's x split into buffer 0, its codes in flight
    load_x(xs, x, M, K, 0, t);
#pragma unroll
    for (int j = 0; j < kSB; ++j) cd[j] = load_codes<BITS>(qr, sr, rowq, hrow, rows, j < C ? j : C - 1, g);
    store_x<BITS, MF>(xs, M, lds, t);
    __syncthreads();

    for (int seg = 0; seg < nseg; ++seg) {
        const int b0 = seg * kSB;
        const uint8_t *buf = lds + (seg & 1) * Buf<MF>::BYTES;
        const float *E = reinterpret_cast<const float *>(buf + Buf<MF>::A_BYTES);
        if (seg + 1 < nseg) load_x(xs, x, M, K, b0 + kSB, t);
#pragma unroll
        for (int j = 0; j < kSB; ++j) {
            const int b = b0 + j;
            // this lane's x rows 8f + 4g .. 8f + 4g + 3: their factors of block j
            f4 ef[MF];
#pragma unroll
            for (int f = 0; f < MF; ++f) ef[f] = *reinterpret_cast<const f4 *>(E + j * 16 + 8 * f + 4 * g);
            h8 bw[2];
            unpack_codes<BITS>(cd[j], dc, dc5, bw);
            const float sc = b < C ? (float)__builtin_bit_cast(_Float16, (uint16_t)cd[j].sc) : 0.0f;
            // the next segment's codes for this slot, in flight during the rest
            if (seg + 1 < nseg) {
                const int bn = b + kSB < C ? b + kSB : C - 1;
                cd[j] = load_codes<BITS>(qr, sr, rowq, hrow, rows, bn, g);
            }
#pragma unroll
            for (int f = 0; f < MF; ++f) {
                const uint8_t *op = buf + f * kOpBytes;
                const h8 a0 = *reinterpret_cast<const h8 *>(op + aoff(r, j * 4 + 2 * g));
                const h8 a1 = *reinterpret_cast<const h8 *>(op + aoff(r, j * 4 + 2 * g + 1));
                f16v p = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, bw[0], zero, 0, 0, 0);
                p = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, bw[1], p, 0, 0, 0);
                // value v < 4 of lane (n, g): operand row 4g + v, i.e. x row
                // m = 8f + 4g + v (part 1); values v + 4 and v + 8: parts 2 and 3.
                // Rows m >= M hold no data and are never stored.
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    acc[f][v] = __builtin_fmaf(sc * ef[f][v], (p[v] + p[v + 4]) + p[v + 8], acc[f][v]);
                    asm volatile("" : "+v"(acc[f][v]));   // the block's scaling happens here
                }
            }
        }
        if (seg + 1 < nseg) {
            store_x<BITS, MF>(xs, M, lds + ((seg + 1) & 1) * Buf<MF>::BYTES, t);
            lds_barrier();                       // the next buffer is complete, this one free; codes stay in flight
        }
    }
    if (nvalid) {
#pragma unroll
        for (int f = 0; f < MF; ++f)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = 8 * f + 4 * g + v;
                if (m < M) y[(size_t)m * N + n] = acc[f][v];
            }
    }
}

template <int BITS, int MF>
__global__ __launch_bounds__(256) void mgemv_kernel(const float *__restrict__ x, int M, int K, int64_t N,
                                                    const uint8_t *__restrict__ q, const uint16_t *__restrict__ s,
                                                    float *__restrict__ y)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * Buf<MF>::BYTES];
    mgemv_item<BITS, MF>(x, M, K, N, q, s, y, (int64_t)blockIdx.x * kMgemvRows, lds);
}

template <int MF>
__global__ __launch_bounds__(256) void mgemv_grouped_kernel(const uint8_t *__restrict__ base,
                                                            const wq_desc *__restrict__ table, int count, int M)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * Buf<MF>::BYTES];
    const int64_t item = blockIdx.x;
    int lo = 0, hi = count - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (table[mid].tile_begin <= item) lo = mid; else hi = mid - 1;
    }
    const wq_desc d = table[lo];
    const uint8_t *q = base + d.q_off;
    const uint16_t *s = reinterpret_cast<const uint16_t *>(base + d.s_off);
    const int64_t row0 = (item - d.tile_begin) * kMgemvRows;
    if (d.bits == 4) mgemv_item<4, MF>(d.x, M, (int)d.K, d.N, q, s, d.y, row0, lds);
    else if (d.bits == 5) mgemv_item<5, MF>(d.x, M, (int)d.K, d.N, q, s, d.y, row0, lds);
    else mgemv_item<8, MF>(d.x, M, (int)d.K, d.N, q, s, d.y, row0, lds);
}

}  // namespace

hipError_t launch_mgemv(const float *x, int64_t M, int64_t K, int64_t N, int bits, const void *q,
                        const uint16_t *scales, float *y, hipStream_t stream)
{
    const unsigned grid = (unsigned)((N + kMgemvRows - 1) / kMgemvRows);
    const uint8_t *qb = (const uint8_t *)q;
    if (M <= 8) {
        if (bits == 4) mgemv_kernel<4, 1><<<grid, 256, 0, stream>>>(x, (int)M, (int)K, N, qb, scales, y);
        else if (bits == 5) mgemv_kernel<5, 1><<<grid, 256, 0, stream>>>(x, (int)M, (int)K, N, qb, scales, y);
        else mgemv_kernel<8, 1><<<grid, 256, 0, stream>>>(x, (int)M, (int)K, N, qb, scales, y);
    } else {
        if (bits == 4) mgemv_kernel<4, 2><<<grid, 256, 0, stream>>>(x, (int)M, (int)K, N, qb, scales, y);
        else if (bits == 5) mgemv_kernel<5, 2><<<grid, 256, 0, stream>>>(x, (int)M, (int)K, N, qb, scales, y);
        else mgemv_kernel<8, 2><<<grid, 256, 0, stream>>>(x, (int)M, (int)K, N, qb, scales, y);
    }
    return hipGetLastError();
}

hipError_t launch_mgemv_grouped(const void *base, const wq_desc *table_dev, int count, int64_t total_items,
                                int64_t M, hipStream_t stream)
{
    if (M <= 8)
        mgemv_grouped_kernel<1><<<(unsigned)total_items, 256, 0, stream>>>((const uint8_t *)base, table_dev, count, (int)M);
    else
        mgemv_grouped_kernel<2><<<(unsigned)total_items, 256, 0, stream>>>((const uint8_t *)base, table_dev, count, (int)M);
    return hipGetLastError();
}

}  // namespace wq
