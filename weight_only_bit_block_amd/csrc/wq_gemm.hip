// wq_gemm.hip -- prefill GEMM for block-32 int4 / int8 weights (any M, tuned for M >= 128).
//
// The TinyMOSS-Diarize devpost page ("How we built it") describes a blocked
// prefill GEMM that unpacks each weight group once and reuses it across all
// activation rows. On gfx950 (wave64, fp16 matrix cores, 160 KiB LDS):
//
//  * A workgroup of 4 wavefronts computes a BM x 128 tile of y (BM = 128, or 64
//    when M <= 64); wavefront w owns 32 output columns (2 fragments of 16) and
//    all BM rows (BM/16 fragments), so each weight code of the tile is unpacked
//    exactly once, in the registers of the wavefront that uses it, into an
//    exact binary16 integer, and that unpack is shared by BM/16 matrix-core
//    instructions.
//  * The K loop runs over stages of KT = 2 quantization blocks through two LDS
//    buffers. The packed codes, x (fp32) and the scales of a stage are loaded
//    into registers while the previous stage is computed, then written to the
//    other buffer: x rounded to binary16 (nearest even) in the order the unpack
//    produces the codes, with an XOR swizzle of its 16-byte pieces so that the
//    128-bit fragment reads of 16 rows hit distinct banks.
//  * Each block of 32 values is one v_mfma_f32_16x16x32_f16 per 16 x 16
//    fragment from a zero accumulator: the block's fp32 partial, which is then
//    scaled by the block scale of its column and added to the fp32 accumulator
//    (one fused multiply-add per output and block, taking the binary16 scale).
//  * Within a block the 32 values are visited in the order the unpack produces
//    them, identically for x and the weights, so each dot product is unchanged.
//  * Tiles are ordered so that the workgroups placed on one XCD (workgroup id
//    modulo 8) cover consecutive tiles of a row of tiles and share x in that
//    XCD's L2.
#include "wq_internal.h"
#include "wq_decode.h"

namespace wq {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int BN = 128;            // columns per workgroup tile (32 per wavefront)
constexpr int KT = 2;              // quantization blocks per stage
constexpr int kThreads = 256;
constexpr int kXcds = 8;

// LDS layout of one stage buffer (BM = 128 or 64 rows per workgroup tile).
//   A: x as binary16, [BM rows][KT*32 values]; row pitch 128 bytes, 16-byte
//      slot s of row r stored at slot s ^ ((r >> 1) & 7).
//   B: packed codes, [BN columns][KT * CB bytes].
//   S: binary16 scales, [BN columns][KT].
template <int BITS, int BM>
struct Stage {
    static constexpr int CB = BITS * 4;                    // code bytes per column per block
    static constexpr int A_BYTES = BM * KT * 64;
    static constexpr int B_BYTES = BN * KT * CB;
    static constexpr int S_BYTES = BN * KT * 2;
    static constexpr int BYTES = A_BYTES + B_BYTES + S_BYTES;
};

__device__ __forceinline__ int aslot(int r, int s) { return r * (KT * 4) + (s ^ ((r >> 1) & 7)); }

template <int BITS, int BM>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(const float *__restrict__ x, int M, int K, int N,
                                                           const uint8_t *__restrict__ q,
                                                           const uint16_t *__restrict__ s,
                                                           float *__restrict__ y, int tiles_m, int tiles_n)
{
    using L = Stage<BITS, BM>;
    constexpr int CB = L::CB;
    constexpr int RF = BM / 16;                     // row fragments per wavefront
    constexpr int XI = BM * KT * 4 / kThreads;      // 8-value x groups per thread per stage (4 or 2)
    constexpr int BP = BN * KT * CB / 16;           // 16-byte code pieces per stage (256 or 512)
    constexpr int QI = BP / kThreads;               // code pieces per thread per stage (1 or 2)
    static_assert(XI * kThreads == BM * KT * 4 && BP % kThreads == 0, "tile shape");
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * L::BYTES];

    // XCD-aware tile order: workgroups id, id+8, id+16, ... run on one XCD; give
    // them consecutive tiles (row-major over (tm, tn)).
    const int T = tiles_m * tiles_n;
    const int per = (T + kXcds - 1) / kXcds;
    const int tile = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
    if (tile >= T) return;
    const int tm = tile / tiles_n;
    const int tn = tile - tm * tiles_n;
    const int m0 = tm * BM, n0 = tn * BN;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int fr = lane & 15, fg = lane >> 4;    // fragment row / column, k-group
    const int C = K >> 5;                        // blocks per row
    const int NT = (C + KT - 1) / KT;            // stages
    const DecodeConsts dc = DecodeConsts::make();

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint64_t)M * K * 4);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(s, (uint64_t)N * C * 2);
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(q, (uint64_t)N * K * BITS / 8);
    const uint32_t qrow = (uint32_t)K * BITS / 8;

    // x: thread t loads XI groups of 8 values: row r, block tb, k-group g.
    uint32_t xoff[XI];
    int xblk[XI], xlds[XI];
#pragma unroll
    for (int i = 0; i < XI; ++i) {
        const int idx = t + i * kThreads;        // 0 .. BM*KT*4-1
        const int r = idx / (KT * 4), sl = idx % (KT * 4);
        int m = m0 + r;
        m = m < M ? m : M - 1;
        xoff[i] = ((uint32_t)m * (uint32_t)K + (uint32_t)(sl & 3) * 8) * 4;
        xblk[i] = sl >> 2;
        xlds[i] = aslot(r, sl) * 16;
    }
    // scales: thread t < BN loads the KT scales of column n0 + t
    int sn = n0 + (t & (BN - 1));
    sn = sn < N ? sn : N - 1;
    const uint32_t soff = (uint32_t)sn * (uint32_t)C * 2;
    // codes: thread t loads QI pieces of 16 bytes; piece pc of a stage is piece
    // pc % (KT*CB/16) of column pc / (KT*CB/16)'s KT*CB bytes
    uint32_t qoff[QI];
    int qblk[QI];
#pragma unroll
    for (int i = 0; i < QI; ++i) {
        const int pc = t + i * kThreads;
        const int c = pc / (KT * CB / 16);
        const int k = pc - c * (KT * CB / 16);
        int n = n0 + c;
        n = n < N ? n : N - 1;
        qoff[i] = (uint32_t)n * qrow + (uint32_t)((k * 16) % CB);
        qblk[i] = (k * 16) / CB;
    }
    f4 xv[XI][2];
    u4 qv[QI];
    uint16_t sv[KT];
    auto issue = [&](int st) {
        const int b0 = st * KT;
#pragma unroll
        for (int i = 0; i < QI; ++i) {
            int b = b0 + qblk[i];                // blocks past K reload the last one (scale 0)
            b = b < C ? b : C - 1;
            qv[i] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(qr, qoff[i] + (uint32_t)b * CB, 0, 0));
        }
#pragma unroll
        for (int i = 0; i < XI; ++i) {
            int b = b0 + xblk[i];
            b = b < C ? b : C - 1;
            const uint32_t o = xoff[i] + (uint32_t)b * 128;
            xv[i][0] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(xr, o, 0, 0));
            xv[i][1] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(xr, o + 16, 0, 0));
        }
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            const int b = b0 + k < C ? b0 + k : C - 1;
            sv[k] = __builtin_amdgcn_raw_buffer_load_b16(sr, soff + (uint32_t)b * 2, 0, 0);
        }
    };
    // x rounded to binary16 in operand order, the codes and the scales (zero past
    // K), into buffer buf
    auto commit = [&](int st, int buf) {
        uint8_t *base = lds + buf * L::BYTES;
#pragma unroll
        for (int i = 0; i < QI; ++i) *reinterpret_cast<u4 *>(base + L::A_BYTES + (t + i * kThreads) * 16) = qv[i];
#pragma unroll
        for (int i = 0; i < XI; ++i) {
            const float v[8] = {xv[i][0].x, xv[i][0].y, xv[i][0].z, xv[i][0].w,
                                xv[i][1].x, xv[i][1].y, xv[i][1].z, xv[i][1].w};
            h8 h;
#pragma unroll
            for (int k = 0; k < 8; ++k) h[operand_slot<BITS>(k)] = (_Float16)v[k];   // nearest even
            *reinterpret_cast<h8 *>(base + xlds[i]) = h;
        }
        if (t < BN) {
            uint16_t *S = reinterpret_cast<uint16_t *>(base + L::A_BYTES + L::B_BYTES);
            const int b0 = st * KT;
#pragma unroll
            for (int k = 0; k < KT; ++k) S[t * KT + k] = b0 + k < C ? sv[k] : (uint16_t)0;
        }
    };

    f4 acc[RF][2];
#pragma unroll
    for (int i = 0; i < RF; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f4{0.0f, 0.0f, 0.0f, 0.0f};

    issue(0);
    commit(0, 0);                                // waits for stage 0's loads
    __syncthreads();
    if (NT > 1) issue(1);

    const f4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int it = 0; it < NT; ++it) {
        const int cur = it & 1;
        const uint8_t *base = lds + cur * L::BYTES;
        const uint8_t *B = base + L::A_BYTES;
        const uint16_t *S = reinterpret_cast<const uint16_t *>(B + L::B_BYTES);
        // Fragment reads run one step ahead of their use: the codes and scales of
        // block kb+1 while block kb is computed, the x fragment of row i+1 while
        // row i is computed.
        auto read_codes = [&](int kb, uint32_t (&cw)[2][CB / 16], uint32_t &sw2) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int c = wave * 32 + j * 16 + fr;
                const uint8_t *qp = B + c * (KT * CB) + kb * CB + fg * (CB / 4);
                if (BITS == 4) {
                    cw[j][0] = *reinterpret_cast<const uint32_t *>(qp);
                } else {
                    const u2 v = *reinterpret_cast<const u2 *>(qp);
                    cw[j][0] = v.x;
                    cw[j][CB / 16 - 1] = v.y;
                }
            }
            const uint16_t s0 = S[(wave * 32 + fr) * KT + kb], s1 = S[(wave * 32 + 16 + fr) * KT + kb];
            sw2 = (uint32_t)s0 | ((uint32_t)s1 << 16);
        };
        auto read_a = [&](int kb, int i) {
            return *reinterpret_cast<const h8 *>(base + aslot(i * 16 + fr, kb * 4 + fg) * 16);
        };
        uint32_t cw[2][CB / 16], sw2;
        read_codes(0, cw, sw2);
        h8 an = read_a(0, 0);
        // The stage's KT*RF (block, row fragment) steps in order; step f issues the
        // matrix work of its two fragments, then scales the partials of step f-2
        // (two steps of matrix work in between, so the wave does not wait for them).
        h8 b[2];
        float sc[2], scp[2] = {0.0f, 0.0f};
        f4 p[3][2];
#pragma unroll
        for (int f = 0; f < KT * RF + 2; ++f) {
            const int kb = f / RF, i = f % RF;
            if (f < KT * RF) {
                if (i == 0) {
                    // this lane's codes and scales of block kb, for its 2 column fragments
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        b[j] = BITS == 4 ? unpack8_int4(cw[j][0], dc) : unpack8_int8(cw[j][0], cw[j][CB / 16 - 1], dc);
                    scp[0] = sc[0]; scp[1] = sc[1];
                    const h2 sp = as_h2(sw2);
                    sc[0] = (float)sp.x; sc[1] = (float)sp.y;
                    asm volatile("" : "+v"(sc[0]), "+v"(sc[1]));   // fp32 scales: plain FMAs below
                    if (kb + 1 < KT) read_codes(kb + 1, cw, sw2);
                }
                const h8 a = an;
                if (i + 1 < RF) an = read_a(kb, i + 1);
                else if (kb + 1 < KT) an = read_a(kb + 1, 0);
#pragma unroll
                for (int j = 0; j < 2; ++j) p[f % 3][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[j], zero, 0, 0, 0);
            }
            if (f >= 2) {
                const int g = f - 2, gi = g % RF;
                // step g's block is the current one, or the previous one when a new
                // block started within the last two steps
                const bool cur_block = f >= KT * RF || g / RF == kb;
                const float s0 = cur_block ? sc[0] : scp[0];
                const float s1 = cur_block ? sc[1] : scp[1];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    acc[gi][0][v] = __builtin_fmaf(s0, p[g % 3][0][v], acc[gi][0][v]);
                    acc[gi][1][v] = __builtin_fmaf(s1, p[g % 3][1][v], acc[gi][1][v]);
                }
                asm volatile("" : "+v"(acc[gi][0]), "+v"(acc[gi][1]));   // the scaling happens here
            }
        }
        if (it + 1 < NT) {
            commit(it + 1, cur ^ 1);             // waits for stage it+1's loads
            __syncthreads();                     // every wave is done with buffer cur
            if (it + 2 < NT) issue(it + 2);
        }
    }

    // D fragment layout: lane holds column (lane & 15), rows 4*(lane >> 4) + v.
#pragma unroll
    for (int i = 0; i < RF; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + wave * 32 + j * 16 + fr;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = m0 + i * 16 + 4 * fg + v;
                if (m < M && n < N) y[(size_t)m * N + n] = acc[i][j][v];
            }
        }
}

template <int BITS, int BM>
hipError_t launch_bits(const float *x, int64_t M, int64_t K, int64_t N, const void *q,
                       const uint16_t *scales, float *y, hipStream_t stream)
{
    const int tiles_m = (int)((M + BM - 1) / BM);
    const int tiles_n = (int)((N + BN - 1) / BN);
    const int T = tiles_m * tiles_n;
    const unsigned grid = (unsigned)(((T + kXcds - 1) / kXcds) * kXcds);
    gemm_kernel<BITS, BM><<<grid, kThreads, 0, stream>>>(x, (int)M, (int)K, (int)N, (const uint8_t *)q, scales,
                                                         y, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const float *x, int64_t M, int64_t K, int64_t N, int bits, const void *q,
                       const uint16_t *scales, float *y, hipStream_t stream)
{
    // 64-row tiles when M <= 64 (no matrix work on padding rows), else 128
    if (M <= 64) {
        if (bits == 4) return launch_bits<4, 64>(x, M, K, N, q, scales, y, stream);
        return launch_bits<8, 64>(x, M, K, N, q, scales, y, stream);
    }
    if (bits == 4) return launch_bits<4, 128>(x, M, K, N, q, scales, y, stream);
    return launch_bits<8, 128>(x, M, K, N, q, scales, y, stream);
}

}  // namespace wq
