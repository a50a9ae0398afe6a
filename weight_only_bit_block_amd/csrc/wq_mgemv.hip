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
//    product is exact and the matrix core sums in fp32. Only the operand rows
//    that carry data are stored in LDS (3 * MR of them, MR = 4 or 8 rows per
//    part); the lanes of the other rows read a stored row, and their results
//    are never used.
//  * Per block and operand, two chained v_mfma_f32_32x32x16_f16 from a zero
//    accumulator give P[32 x 32]; operand rows m, 8+m and 16+m land in one lane
//    (values v, v+4, v+8), so row m's block partial is P[v] + P[v+4] + P[v+8],
//    and acc[m] += (s[n,b] * 2^-e[m,b]) * partial in fp32 (the product of a
//    binary16 scale and a power of two is exact). The summation depth per
//    output is about 8 + K/32, far below the ~160 at which fp32 rounding could
//    reach 1e-5 * sum |x||w|.
//  * A workgroup of 4 wavefronts owns 128 consecutive weight rows (32 per
//    wavefront, one matrix column each) for all K, walked in segments of SB
//    blocks (seg_blocks). Each wavefront copies its rows' codes of the next
//    segment from HBM straight into a wave-private LDS buffer (direct-to-LDS
//    buffer loads, no registers), while x of the next segment is loaded
//    into registers and the current segment is computed; x is then split into
//    the other of two operand buffers. Lane (n, g) reads codes 16g..16g+15 of
//    each block of its row from LDS and unpacks them in registers. The operand
//    order of the 8 values of a k-group is the order the unpack produces,
//    identical for x and the codes.
//  * The operand rows are stored with a row-dependent XOR swizzle of their
//    16-byte slots, so the 16 lanes of each 128-bit LDS read hit distinct banks.
// x blocks whose largest magnitude is below 2^-112 lose relative precision (the
// factor 2^e is capped at 2^126 so that 2^-e stays a normal fp32 number); any
// other finite fp32 x is split exactly as above.
#include "wq_internal.h"
#include "wq_device.h"
#include "wq_decode.h"

namespace wq {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// Blocks per segment. With one operand a segment copies a whole 128-byte line
// of each of a wavefront's 32 rows for int4 (8 blocks) and int8 (4 blocks):
// with 4-block int4 segments (half lines) the mixed decode step at M = 4 took
// 5% longer and the all-int4 step 7% longer. int5 (80 + 16 bytes per 4
// blocks) and the two-operand form keep 4 blocks: 8 would raise the kernel's
// registers past 128 (int5) or the two-operand LDS to 66 KiB.
template <int BITS, int MF>
constexpr int seg_blocks() { return BITS == 4 && MF == 1 ? 8 : 4; }

// Operand buffer of a segment of SB blocks: MF operands of 3 * MR stored rows
// (binary16, row pitch SB * 64 bytes) and the factors 2^-e, [SB][16] floats.
template <int MF, int MR, int SB>
struct Buf {
    static constexpr int ROW_BYTES = SB * 32 * 2;
    static constexpr int OP_BYTES = 3 * MR * ROW_BYTES;
    static constexpr int A_BYTES = MF * OP_BYTES;
    static constexpr int BYTES = A_BYTES + 16 * SB * 4;
};

// Stored row of operand row r (0..31): part r / 8 (h1, h2, h3; 3 is unused),
// activation row r % 8. Lanes of rows without data read a stored row chosen
// so that each 16-lane group of a 128-bit LDS read still hits 16 distinct
// 16-byte bank groups or the same address: part 3 reads the rows of part 1,
// other rows past MR read stored row 0. (Part 3 on stored row 0 collided with
// row 16 in its group: LDS bank conflicts rose from 0.18 to 0.85 of the
// LDS-active cycles at M = 8.)
template <int MR>
__device__ __forceinline__ int stored_row(int r)
{
    const int part = (r >> 3) == 3 ? 1 : r >> 3;
    return (r & 7) < MR ? part * MR + (r & 7) : 0;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// 16-byte slot s of operand row r (4 * SB slots per row of a segment)
template <int SB>
__device__ __forceinline__ int aoff(int r, int s) { return r * (SB * 64) + ((s ^ r) & (4 * SB - 1)) * 16; }

// A wavefront's codes of one segment in LDS, copied there directly (no
// registers). Row rr of its 32 weight rows holds the segment's SB blocks in
// 16-byte pieces; piece p is stored at slot p ^ swz(rr) so that the matrix
// operand reads of 32 rows spread over the banks. int5 adds the rows' bit-4
// dwords, [32 rows][SB dwords].
template <int BITS, int SB>
struct BStage {
    static constexpr int SLOTS = SB * (BITS == 8 ? 2 : 1);       // 16-byte pieces per row
    static constexpr int ROW = SLOTS * 16;
    static constexpr int CODE_BYTES = 32 * ROW;
    static constexpr int H_BYTES = BITS == 5 ? 32 * SB * 4 : 0;
    static constexpr int WAVE_BYTES = CODE_BYTES + H_BYTES;
    static constexpr int BYTES = 4 * WAVE_BYTES;                  // the workgroup's 4 wavefronts
    // the rows read together by one LDS read hit distinct banks
    __device__ static constexpr int swz(int rr) { return (rr / (16 / SLOTS)) % SLOTS; }
};

template <int POLICY>
__device__ __forceinline__ void copy16(__amdgpu_buffer_rsrc_t r, uint8_t *lds_base, uint32_t off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds_base, 16, off, 0, 0,
                                             POLICY);
}

// Issue the copies of segment b0 .. b0+SB-1 of weight rows nrow0 .. nrow0+31
// into this wavefront's region dst: each instruction moves the segment's part
// of 64 / SLOTS rows. Reads past the tensor return zeros; blocks past K read
// the next row's codes, whose scale is taken as 0. Copies of whole 128-byte
// lines use the non-temporal policy (the codes are read once): with it the
// mixed decode step at M = 3..8 ran 4-5% faster. Partial lines (int5, int4 in
// 4-block segments) keep the default policy, which lets the cache serve the
// rest of the line to the next segment's copies: non-temporal copies of half
// lines made the step 8% slower.
template <int BITS, int SB>
__device__ __forceinline__ void stage_codes(__amdgpu_buffer_rsrc_t qr, uint32_t qrow, int K, int64_t nrow0, int64_t N,
                                            int b0, uint8_t *dst, int lane)
{
    using B = BStage<BITS, SB>;
    constexpr int RPI = 64 / B::SLOTS;             // rows per instruction
    constexpr int POL = BITS != 5 && B::ROW % 128 == 0 ? kNonTemporal : 0;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
        const int rr = i * RPI + lane / B::SLOTS;
        const int p = (lane % B::SLOTS) ^ B::swz(rr);
        int64_t n = nrow0 + rr;
        n = n < N ? n : N - 1;
        copy16<POL>(qr, dst + i * 1024, (uint32_t)n * qrow + (uint32_t)b0 * (B::ROW / SB) + (uint32_t)p * 16);
    }
    if constexpr (BITS == 5) {
        // the rows' bit-4 dwords: SB / 4 pieces of 16 bytes per row
        constexpr int PR = SB / 4;
        const int rr = lane / PR, h = lane % PR;    // dwords 4h .. 4h+3 of row rr
        if (rr < 32) {
            int64_t n = nrow0 + rr;
            n = n < N ? n : N - 1;
            copy16<0>(qr, dst + B::CODE_BYTES, (uint32_t)n * qrow + (uint32_t)K / 2 + (uint32_t)(b0 + 4 * h) * 4);
        }
    }
}

// Lane (r, g)'s codes of a segment: codes 16g .. 16g+15 of each block of its
// row, as raw packed words (int5: with their bit-4 bytes).
template <int BITS, int SB>
struct LaneCodes {
    u4 v[BITS == 8 ? SB : (SB + 1) / 2];   // int8: 16 bytes per block; int4/int5: 8 bytes per block
    uint32_t h[SB];                        // int5: bit 4 of the 16 codes of each block
};

template <int BITS, int SB>
__device__ __forceinline__ void read_codes(const uint8_t *src, int r, int g, LaneCodes<BITS, SB> &c)
{
    using B = BStage<BITS, SB>;
#pragma unroll
    for (int j = 0; j < SB; ++j) {
        if constexpr (BITS == 8) {
            c.v[j] = *reinterpret_cast<const u4 *>(src + r * B::ROW + ((2 * j + g) ^ B::swz(r)) * 16);
        } else {
            const u2 v = *reinterpret_cast<const u2 *>(src + r * B::ROW + (j ^ B::swz(r)) * 16 + g * 8);
            c.v[j / 2][2 * (j & 1)] = v.x;
            c.v[j / 2][2 * (j & 1) + 1] = v.y;
            if constexpr (BITS == 5)
                c.h[j] = *reinterpret_cast<const uint16_t *>(src + B::CODE_BYTES + r * (SB * 4) + j * 4 + g * 2);
        }
    }
}

// Block j of a lane's segment codes as two groups of 8 in unpack order.
template <int BITS, int SB>
__device__ __forceinline__ void lane_codes(const LaneCodes<BITS, SB> &c, int j, const DecodeConsts &dc,
                                           const Decode5Consts &dc5, h8 (&b)[2])
{
    if constexpr (BITS == 8) {
        b[0] = unpack8_int8(c.v[j].x, c.v[j].y, dc);
        b[1] = unpack8_int8(c.v[j].z, c.v[j].w, dc);
    } else {
        const uint32_t lo = c.v[j / 2][2 * (j & 1)], hi = c.v[j / 2][2 * (j & 1) + 1];
        if constexpr (BITS == 4) {
            b[0] = unpack8_int4(lo, dc);
            b[1] = unpack8_int4(hi, dc);
        } else {
            b[0] = unpack8_int5(lo, c.h[j] & 0xFF, dc5);
            b[1] = unpack8_int5(hi, c.h[j] >> 8, dc5);
        }
    }
}

// The scales of a segment for one row: SB binary16 values, packed two per
// dword (one load when the row's scales are aligned for it).
template <int SB>
struct Scales {
    uint32_t w[SB / 2];
};

template <int SB>
__device__ __forceinline__ Scales<SB> load_scales(__amdgpu_buffer_rsrc_t sr, uint32_t rows, int C, int b0)
{
    Scales<SB> r;
    if ((C & (SB - 1)) == 0) {
        if constexpr (SB == 8) {
            const u4 v = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(sr, rows + (uint32_t)b0 * 2, 0, 0));
            r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
        } else {
            const u2 v = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(sr, rows + (uint32_t)b0 * 2, 0, 0));
            r.w[0] = v.x; r.w[1] = v.y;
        }
        return r;
    }
#pragma unroll
    for (int j = 0; j < SB / 2; ++j)
        r.w[j] = __builtin_amdgcn_raw_buffer_load_b16(sr, rows + (uint32_t)(b0 + 2 * j) * 2, 0, 0) |
                 (__builtin_amdgcn_raw_buffer_load_b16(sr, rows + (uint32_t)(b0 + 2 * j + 1) * 2, 0, 0) << 16);
    return r;
}

// x of one segment: group i (8 values) of the segment is row m, block blk,
// k-group q (i = (m * SB + blk) * 4 + q); a thread holds XG groups (8 * MF
// rows; threads past them hold none).
template <int MF, int SB>
struct XStage {
    static constexpr int XG = 8 * MF * SB * 4 / 256 > 0 ? 8 * MF * SB * 4 / 256 : 1;
    f4 v[XG][2];
};

template <int MF, int SB>
__device__ __forceinline__ void load_x(XStage<MF, SB> &xs, const float *__restrict__ x, int M, int K, int b0, int t)
{
    const int C = K >> 5;
#pragma unroll
    for (int i = 0; i < XStage<MF, SB>::XG; ++i) {
        const int idx = t + i * 256;
        int m = idx / (SB * 4);
        const int blk = (idx / 4) % SB, q = idx & 3;
        int b = b0 + blk;
        m = m < M ? m : M - 1;                   // rows past M and blocks past K load valid data, unused
        b = b < C ? b : C - 1;
        const f4 *p = reinterpret_cast<const f4 *>(x + (size_t)m * K + b * 32 + q * 8);
        xs.v[i][0] = p[0];
        xs.v[i][1] = p[1];
    }
}

// Split the staged x into the operand rows and the per-(row, block) factors.
template <int BITS, int MF, int MR, int SB>
__device__ __forceinline__ void store_x(const XStage<MF, SB> &xs, int M, uint8_t *buf, int t)
{
    using A = Buf<MF, MR, SB>;
    float *E = reinterpret_cast<float *>(buf + A::A_BYTES);
#pragma unroll
    for (int i = 0; i < XStage<MF, SB>::XG; ++i) {
        const int idx = t + i * 256;
        const int m = idx / (SB * 4);
        const int blk = (idx / 4) % SB, q = idx & 3;
        // rows past M are neither split nor stored (their operand rows feed
        // outputs that are never stored); the 4 lanes of a (row, block) skip
        // together, and so does a wavefront whose 4 rows all lie past M
        if (m >= M) continue;
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
        const int s = blk * 4 + q;
        uint8_t *op = buf + (m >> 3) * A::OP_BYTES;
        const int mm = m & 7;                    // < MR
        *reinterpret_cast<h8 *>(op + aoff<SB>(mm, s)) = p1;
        *reinterpret_cast<h8 *>(op + aoff<SB>(MR + mm, s)) = p2;
        *reinterpret_cast<h8 *>(op + aoff<SB>(2 * MR + mm, s)) = p3;
        if (q == 0) E[blk * 16 + m] = __builtin_ldexpf(1.0f, -e);
    }
}

// One item: weight rows row0 .. row0+127 of one tensor, all M activation rows
// (M <= 8 * (MF - 1) + MR). bq: the LDS buffer of the codes (a separate array,
// so reads of the operand buffers never wait for copies into it). Each wavefront moves its
// codes of a segment from bq into registers when the segment starts, so the
// same buffer then takes the next segment's copies.
template <int BITS, int MF, int MR>
__device__ __forceinline__ void mgemv_item(const float *__restrict__ x, int M, int K, int64_t N,
                                           const uint8_t *__restrict__ q, const uint16_t *__restrict__ s,
                                           float *__restrict__ y, int64_t row0, uint8_t *__restrict__ lds,
                                           uint8_t *__restrict__ bq)
{
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int r = lane & 31, g = lane >> 5;
    const int ar = stored_row<MR>(r);            // the lane's operand row as stored
    constexpr int SB = seg_blocks<BITS, MF>();
    using A = Buf<MF, MR, SB>;
    using BS = BStage<BITS, SB>;
    const int C = K >> 5;
    const int nseg = (C + SB - 1) / SB;
    const uint32_t qrow = (uint32_t)K * BITS / 8;
    const DecodeConsts dc = DecodeConsts::make();
    Decode5Consts dc5;
    if constexpr (BITS == 5) dc5 = Decode5Consts::make();
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(q, (uint64_t)N * qrow);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(s, (uint64_t)N * C * 2);
    const int64_t nrow0 = row0 + wave * 32;
    int64_t n = nrow0 + r;
    const bool nvalid = n < N;
    n = nvalid ? n : N - 1;                      // rows past N reload the last row, not stored
    const uint32_t rows = (uint32_t)n * C * 2;
    uint8_t *const wq = bq + wave * BS::WAVE_BYTES;

    float acc[MF][4];
#pragma unroll
    for (int f = 0; f < MF; ++f)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[f][v] = 0.0f;
    const f16v zero = {};

    XStage<MF, SB> xs;
    Scales<SB> scv = load_scales<SB>(sr, rows, C, 0), scn = scv;
    // prologue: segment 0's codes copied, its x split into buffer 0
    stage_codes<BITS, SB>(qr, qrow, K, nrow0, N, 0, wq, lane);
    load_x<MF, SB>(xs, x, M, K, 0, t);
    store_x<BITS, MF, MR, SB>(xs, M, lds, t);
    lds_barrier();

    // One segment: codes from the buffer into registers, then the next
    // segment's codes into the buffer and its x into the other operand buffer.
    auto segment = [&](int seg) {
        const int b0 = seg * SB;
        const uint8_t *buf = lds + (seg & 1) * A::BYTES;
        const float *E = reinterpret_cast<const float *>(buf + A::A_BYTES);
        const bool more = seg + 1 < nseg;
        // Everything this wavefront issued so far has landed: the copies of this
        // segment's codes (issued one segment ago) and its scales.
        __builtin_amdgcn_s_waitcnt(0x0070);      // vmcnt(0) lgkmcnt(0)
        LaneCodes<BITS, SB> lc;
        read_codes<BITS, SB>(wq, r, g, lc);
        __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): the reads are done, the buffer is free
        asm volatile("" ::: "memory");
        if (more) {
            // next segment: x first (split at the end of this one), then the
            // code copies, which stay in flight the longest. Its scales: with
            // one operand they are loaded before this segment's last block,
            // when the codes of the other blocks no longer hold registers
            // (128 registers, four wavefronts per SIMD); with two, here.
            load_x<MF, SB>(xs, x, M, K, b0 + SB, t);
            if constexpr (MF == 2) scn = load_scales<SB>(sr, rows, C, b0 + SB);
            stage_codes<BITS, SB>(qr, qrow, K, nrow0, N, b0 + SB, wq, lane);
        }
        // A operands and factors one block ahead of their matrix instructions
        h8 na0[MF], na1[MF];
        f4 nef[MF];
#pragma unroll
        for (int f = 0; f < MF; ++f) {
            const uint8_t *op = buf + f * A::OP_BYTES;
            na0[f] = *reinterpret_cast<const h8 *>(op + aoff<SB>(ar, 2 * g));
            na1[f] = *reinterpret_cast<const h8 *>(op + aoff<SB>(ar, 2 * g + 1));
            nef[f] = *reinterpret_cast<const f4 *>(E + 8 * f + 4 * g);
        }
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            const int b = b0 + j;
            h8 ca0[MF], ca1[MF];
            f4 ef[MF];
#pragma unroll
            for (int f = 0; f < MF; ++f) { ca0[f] = na0[f]; ca1[f] = na1[f]; ef[f] = nef[f]; }
            if (j + 1 < SB) {
#pragma unroll
                for (int f = 0; f < MF; ++f) {
                    const uint8_t *op = buf + f * A::OP_BYTES;
                    na0[f] = *reinterpret_cast<const h8 *>(op + aoff<SB>(ar, (j + 1) * 4 + 2 * g));
                    na1[f] = *reinterpret_cast<const h8 *>(op + aoff<SB>(ar, (j + 1) * 4 + 2 * g + 1));
                    nef[f] = *reinterpret_cast<const f4 *>(E + (j + 1) * 16 + 8 * f + 4 * g);
                }
            }
            h8 bw[2];
            lane_codes<BITS, SB>(lc, j, dc, dc5, bw);
            const uint16_t sbits = (uint16_t)(scv.w[j >> 1] >> (16 * (j & 1)));
            const float sc = b < C ? (float)__builtin_bit_cast(_Float16, sbits) : 0.0f;
#pragma unroll
            for (int f = 0; f < MF; ++f) {
                const h8 a0 = ca0[f];
                const h8 a1 = ca1[f];
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
            if (MF == 1 && j == SB - 2 && more) scn = load_scales<SB>(sr, rows, C, b0 + SB);
            __builtin_amdgcn_sched_barrier(0);   // keep each block's work together (bounds live registers)
        }
        if (more) {
            scv = scn;
            store_x<BITS, MF, MR, SB>(xs, M, lds + ((seg + 1) & 1) * A::BYTES, t);
            lds_barrier();                       // the next operand buffer is complete, this one free
        }
    };
    for (int seg = 0; seg < nseg; ++seg) segment(seg);
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

template <int BITS, int MF, int MR>
__global__ __launch_bounds__(256) void mgemv_kernel(const float *__restrict__ x, int M, int K, int64_t N,
                                                    const uint8_t *__restrict__ q, const uint16_t *__restrict__ s,
                                                    float *__restrict__ y)
{
    constexpr int SB = seg_blocks<BITS, MF>();
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * Buf<MF, MR, SB>::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t bq[BStage<BITS, SB>::BYTES];
    mgemv_item<BITS, MF, MR>(x, M, K, N, q, s, y, (int64_t)blockIdx.x * kMgemvRows, lds, bq);
}

template <int A_, int B_>
constexpr int cmax() { return A_ > B_ ? A_ : B_; }

template <int MF, int MR>
__global__ __launch_bounds__(256) void mgemv_grouped_kernel(const uint8_t *__restrict__ base,
                                                            const wq_desc *__restrict__ table, int count, int M)
{
    // buffers sized for the largest of the three code widths
    constexpr int SB4 = seg_blocks<4, MF>(), SB5 = seg_blocks<5, MF>(), SB8 = seg_blocks<8, MF>();
    constexpr int AB = cmax<cmax<Buf<MF, MR, SB4>::BYTES, Buf<MF, MR, SB5>::BYTES>(), Buf<MF, MR, SB8>::BYTES>();
    constexpr int BB = cmax<cmax<BStage<4, SB4>::BYTES, BStage<5, SB5>::BYTES>(), BStage<8, SB8>::BYTES>();
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * AB];
    __shared__ __attribute__((aligned(16))) uint8_t bq[BB];
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
    if (d.bits == 4) mgemv_item<4, MF, MR>(d.x, M, (int)d.K, d.N, q, s, d.y, row0, lds, bq);
    else if (d.bits == 5) mgemv_item<5, MF, MR>(d.x, M, (int)d.K, d.N, q, s, d.y, row0, lds, bq);
    else mgemv_item<8, MF, MR>(d.x, M, (int)d.K, d.N, q, s, d.y, row0, lds, bq);
}

}  // namespace

hipError_t launch_mgemv(const float *x, int64_t M, int64_t K, int64_t N, int bits, const void *q,
                        const uint16_t *scales, float *y, hipStream_t stream)
{
    const unsigned grid = (unsigned)((N + kMgemvRows - 1) / kMgemvRows);
    const uint8_t *qb = (const uint8_t *)q;
    // MR: activation rows per operand part stored in LDS (4 keeps the LDS of a
    // workgroup at 29 KiB, four workgroups per compute unit)
    if (M <= 4) {
        if (bits == 4) mgemv_kernel<4, 1, 4><<<grid, 256, 0, stream>>>(x, (int)M, (int)K, N, qb, scales, y);
        else if (bits == 5) mgemv_kernel<5, 1, 4><<<grid, 256, 0, stream>>>(x, (int)M, (int)K, N, qb, scales, y);
        else mgemv_kernel<8, 1, 4><<<grid, 256, 0, stream>>>(x, (int)M, (int)K, N, qb, scales, y);
    } else if (M <= 8) {
        if (bits == 4) mgemv_kernel<4, 1, 8><<<grid, 256, 0, stream>>>(x, (int)M, (int)K, N, qb, scales, y);
        else if (bits == 5) mgemv_kernel<5, 1, 8><<<grid, 256, 0, stream>>>(x, (int)M, (int)K, N, qb, scales, y);
        else mgemv_kernel<8, 1, 8><<<grid, 256, 0, stream>>>(x, (int)M, (int)K, N, qb, scales, y);
    } else {
        if (bits == 4) mgemv_kernel<4, 2, 8><<<grid, 256, 0, stream>>>(x, (int)M, (int)K, N, qb, scales, y);
        else if (bits == 5) mgemv_kernel<5, 2, 8><<<grid, 256, 0, stream>>>(x, (int)M, (int)K, N, qb, scales, y);
        else mgemv_kernel<8, 2, 8><<<grid, 256, 0, stream>>>(x, (int)M, (int)K, N, qb, scales, y);
    }
    return hipGetLastError();
}

hipError_t launch_mgemv_grouped(const void *base, const wq_desc *table_dev, int count, int64_t total_items,
                                int64_t M, hipStream_t stream)
{
    if (M <= 4)
        mgemv_grouped_kernel<1, 4><<<(unsigned)total_items, 256, 0, stream>>>((const uint8_t *)base, table_dev, count, (int)M);
    else if (M <= 8)
        mgemv_grouped_kernel<1, 8><<<(unsigned)total_items, 256, 0, stream>>>((const uint8_t *)base, table_dev, count, (int)M);
    else
        mgemv_grouped_kernel<2, 8><<<(unsigned)total_items, 256, 0, stream>>>((const uint8_t *)base, table_dev, count, (int)M);
    return hipGetLastError();
}

}  // namespace wq
