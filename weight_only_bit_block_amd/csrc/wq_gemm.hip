// wq_gemm.hip -- prefill GEMM for block-32 int4 / int8 weights (any M, tuned for M >= 128).
//
// The TinyMOSS-Diarize devpost page ("How we built it") describes a blocked
// prefill GEMM that unpacks each weight group once and reuses it across all
// activation rows. On gfx950 (wave64, fp16 matrix cores, 160 KiB LDS):
//
//  * A workgroup of 4 wavefronts computes a BM x 256 tile of y. Wavefront w owns
//    64 output columns (4 fragments of 16) and all BM rows, so every weight code
//    of the tile is unpacked exactly once, in the registers of the wavefront that
//    uses it, into exact binary16 integers.
//  * The K loop runs over K-tiles of KT quantization blocks through two LDS
//    buffers. Each iteration first issues the global loads of the next K-tile
//    (packed codes, binary16 scales, fp32 x) into registers, then does the
//    matrix work of the current K-tile from LDS, then rounds the prefetched x to
//    binary16 (nearest even) and writes it, the packed codes and the scales to
//    the other buffer, then one barrier. Loads are consumed in the iteration
//    that issued them, so they overlap a whole K-tile of matrix work.
//  * Each block of 32 values is one v_mfma_f32_16x16x32_f16 per 16 x 16
//    fragment from a zero accumulator: the block's fp32 partial, which is then
//    scaled by the block scale of its column and added to the fp32 accumulator.
//  * Within a block the 32 values are visited in the order the unpack produces
//    them, identically for x and the weights, so each dot product is unchanged.
//  * Tiles are ordered so that the workgroups placed on one XCD (workgroup id
//    modulo 8) cover a compact patch of the output and share x and weights in
//    that XCD's L2.
#include "wq_internal.h"
#include "wq_decode.h"

namespace wq {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int BN = 256;            // columns per workgroup tile (64 per wavefront)
constexpr int kThreads = 256;
constexpr int kXcds = 8;

// LDS layout of one buffer: BM rows of x (binary16), BN rows of packed codes,
// KT blocks of binary16 scales.
template <int BITS, int BM, int KT>
struct Lds {
    static constexpr int AH = KT * 32 + 8;                  // halfs per x row (+16 B: conflict-free reads)
    static constexpr int QB = KT * BITS * 4 + 16;           // bytes per code row (+16 B)
    static constexpr int A_BYTES = BM * AH * 2;
    static constexpr int Q_BYTES = BN * QB;
    static constexpr int S_BYTES = KT * BN * 2;             // per block: [wave][fr][j] halfs
    static constexpr int BYTES = A_BYTES + Q_BYTES + S_BYTES;
};

template <int BITS, int BM, int KT, int NB>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(const float *__restrict__ x, int M, int K,
                                                           int N, const uint8_t *__restrict__ q,
                                                           const uint16_t *__restrict__ s,
                                                           float *__restrict__ y, int tiles_m,
                                                           int tiles_n)
{
    using L = Lds<BITS, BM, KT>;
    constexpr int MF = BM / 16;                 // m fragments per wavefront
    constexpr int CB = BITS * 4;                // code bytes per row per block
    constexpr int XG = BM * KT * 4 / kThreads;  // groups of 8 x values per thread per K-tile
    constexpr int PIECES = KT * CB / 16;        // 16-byte code pieces per row per K-tile
    constexpr int QV = BN * PIECES / kThreads;  // code pieces per thread per K-tile
    static_assert(XG >= 1 && QV >= 1 && BN * PIECES % kThreads == 0, "tile shape");
    __shared__ __attribute__((aligned(16))) uint8_t lds[NB * L::BYTES];

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
    const int lane = t & 63, wave = t >> 6;
    const int fr = lane & 15, fg = lane >> 4;   // fragment row / column, k-group
    const int C = K >> 5;
    const int NT = (C + KT - 1) / KT;           // K-tiles
    const DecodeConsts dc = DecodeConsts::make();

    // Loads: buffer descriptors in scalar registers and 32-bit per-lane offsets.
    // Blocks past the end of K are clamped to the last block; their scale is
    // written as zero, so they add nothing.
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(q, (uint64_t)N * K * BITS / 8);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(s, (uint64_t)N * C * 2);
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint64_t)M * K * 4);

    // x: thread loads XG groups of 8 values: row r, group gc (block gc/4, k-group gc%4)
    uint32_t xbase[XG];
    int xblk[XG], xlds[XG];
#pragma unroll
    for (int i = 0; i < XG; ++i) {
        const int idx = t + i * kThreads;       // 0 .. BM*KT*4-1
        const int r = idx / (KT * 4), gc = idx % (KT * 4);
        int m = m0 + r;
        m = m < M ? m : M - 1;
        xbase[i] = ((uint32_t)m * (uint32_t)K + (uint32_t)(gc & 3) * 8) * 4;
        xblk[i] = gc >> 2;
        xlds[i] = r * L::AH + gc * 8;
    }
    // codes: thread loads QV pieces of 16 B: row r, piece pc of the K-tile
    uint32_t qbase[QV];
    int qblk[QV], qlds[QV];
#pragma unroll
    for (int i = 0; i < QV; ++i) {
        const int idx = t + i * kThreads;       // 0 .. BN*PIECES-1
        const int r = idx / PIECES, pc = idx % PIECES;
        int n = n0 + r;
        n = n < N ? n : N - 1;
        qbase[i] = (uint32_t)n * (uint32_t)(K * BITS / 8) + (uint32_t)((pc * 16) % CB);
        qblk[i] = pc * 16 / CB;
        qlds[i] = r * L::QB + pc * 16;
    }
    // scales: thread t holds the KT scales of column n0 + t
    int sn = n0 + t;
    sn = sn < N ? sn : N - 1;
    const uint32_t sbase = (uint32_t)sn * (uint32_t)C * 2;
    const int slds = (((t >> 6) * 16 + (t & 15)) * 4 + ((t >> 4) & 3)) * 2;  // column t = w*64 + j*16 + fr

    f4 xv[XG][2];
    u4 qv[QV];
    uint16_t sv[KT];

    auto clampb = [&](int b) { return b < C ? b : C - 1; };
    auto issue = [&](int it) {
        const int kb0 = it * KT;
#pragma unroll
        for (int i = 0; i < XG; ++i) {
            const uint32_t o = xbase[i] + (uint32_t)clampb(kb0 + xblk[i]) * 128;
            xv[i][0] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(xr, o, 0, 0));
            xv[i][1] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(xr, o + 16, 0, 0));
        }
#pragma unroll
        for (int i = 0; i < QV; ++i) {
            const uint32_t o = qbase[i] + (uint32_t)clampb(kb0 + qblk[i]) * CB;
            qv[i] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(qr, o, 0, 0));
        }
#pragma unroll
        for (int k = 0; k < KT; ++k)
            sv[k] = __builtin_amdgcn_raw_buffer_load_b16(sr, sbase + (uint32_t)clampb(kb0 + k) * 2, 0, 0);
    };
    auto commit = [&](int buf, int it) {
        uint8_t *base = lds + buf * L::BYTES;
        _Float16 *A = reinterpret_cast<_Float16 *>(base);
        uint8_t *Q = base + L::A_BYTES;
        uint8_t *S = Q + L::Q_BYTES;
#pragma unroll
        for (int i = 0; i < XG; ++i) {
            const float v[8] = {xv[i][0].x, xv[i][0].y, xv[i][0].z, xv[i][0].w,
                                xv[i][1].x, xv[i][1].y, xv[i][1].z, xv[i][1].w};
            h8 h;
#pragma unroll
            for (int k = 0; k < 8; ++k) h[operand_slot<BITS>(k)] = (_Float16)v[k];   // nearest even
            *reinterpret_cast<h8 *>(&A[xlds[i]]) = h;
        }
#pragma unroll
        for (int i = 0; i < QV; ++i) *reinterpret_cast<u4 *>(Q + qlds[i]) = qv[i];
        const int kb0 = it * KT;
#pragma unroll
        for (int k = 0; k < KT; ++k)
            *reinterpret_cast<uint16_t *>(S + k * 512 + slds) = kb0 + k < C ? sv[k] : (uint16_t)0;
    };

    f4 acc[MF][4];
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f4{0.0f, 0.0f, 0.0f, 0.0f};

    issue(0);
    commit(0, 0);
    lds_barrier();

    const f4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int it = 0; it < NT; ++it) {
        const int cur = NB == 2 ? (it & 1) : 0;
        const int nit = it + 1 < NT ? it + 1 : it;       // the last iteration reloads itself
        issue(nit);

        const uint8_t *base = lds + cur * L::BYTES;
        const _Float16 *A = reinterpret_cast<const _Float16 *>(base);
        const uint8_t *Q = base + L::A_BYTES;
        const uint8_t *S = Q + L::Q_BYTES;
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            // this lane's codes of block k for its 4 column fragments, and the scales
            h8 b[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint8_t *qp = Q + (wave * 64 + j * 16 + fr) * L::QB + k * CB + fg * (CB / 4);
                if (BITS == 4) {
                    b[j] = unpack8_int4(*reinterpret_cast<const uint32_t *>(qp), dc);
                } else {
                    const u2 v = *reinterpret_cast<const u2 *>(qp);
                    b[j] = unpack8_int8(v.x, v.y, dc);
                }
            }
            const u2 sw = *reinterpret_cast<const u2 *>(S + k * 512 + (wave * 16 + fr) * 8);
            const h2 s01 = as_h2(sw.x), s23 = as_h2(sw.y);
            const float sc[4] = {(float)s01.x, (float)s01.y, (float)s23.x, (float)s23.y};

            f4 pa[4], pb[4];
            auto mfma_row = [&](int i, f4 (&p)[4]) {
                const h8 a = *reinterpret_cast<const h8 *>(&A[(i * 16 + fr) * L::AH + k * 32 + fg * 8]);
#pragma unroll
                for (int j = 0; j < 4; ++j) p[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[j], zero, 0, 0, 0);
            };
            auto scale_row = [&](int i, const f4 (&p)[4]) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[i][j][v] = __builtin_fmaf(sc[j], p[j][v], acc[i][j][v]);
            };
            // matrix work of row fragment i overlaps the scaling of fragment i-1
            mfma_row(0, pa);
#pragma unroll
            for (int i = 1; i < MF; ++i) {
                if (i & 1) { mfma_row(i, pb); scale_row(i - 1, pa); }
                else       { mfma_row(i, pa); scale_row(i - 1, pb); }
            }
            if ((MF - 1) & 1) scale_row(MF - 1, pb); else scale_row(MF - 1, pa);
        }

        if (NB == 1) lds_barrier();            // one buffer: everyone has finished reading it
        commit(NB == 2 ? (cur ^ 1) : 0, nit);
        lds_barrier();
    }

    // D fragment layout: lane holds column (lane & 15), rows 4*(lane >> 4) + v.
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + wave * 64 + j * 16 + fr;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = m0 + i * 16 + 4 * fg + v;
                if (m < M && n < N) y[(size_t)m * N + n] = acc[i][j][v];
            }
        }
}

template <int BITS, int BM, int KT, int NB>
hipError_t launch_cfg(const float *x, int64_t M, int64_t K, int64_t N, const void *q,
                      const uint16_t *scales, float *y, hipStream_t stream)
{
    const int tiles_m = (int)((M + BM - 1) / BM);
    const int tiles_n = (int)((N + BN - 1) / BN);
    const int T = tiles_m * tiles_n;
    const unsigned grid = (unsigned)(((T + kXcds - 1) / kXcds) * kXcds);
    gemm_kernel<BITS, BM, KT, NB><<<grid, kThreads, 0, stream>>>(x, (int)M, (int)K, (int)N, (const uint8_t *)q,
                                                             scales, y, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const float *x, int64_t M, int64_t K, int64_t N, int bits, const void *q,
                       const uint16_t *scales, float *y, hipStream_t stream)
{
    if (bits == 4) return launch_cfg<4, 64, 4, 2>(x, M, K, N, q, scales, y, stream);
    return launch_cfg<8, 64, 2, 2>(x, M, K, N, q, scales, y, stream);
}

}  // namespace wq
