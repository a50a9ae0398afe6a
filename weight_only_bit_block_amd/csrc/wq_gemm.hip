// wq_gemm.hip -- prefill GEMM for block-32 int4 / int5 / int8 weights (any M, tuned for M >= 128).
//
// The TinyMOSS-Diarize devpost page ("How we built it") describes a blocked
// prefill GEMM that unpacks each weight group once and reuses it across all
// activation rows. On gfx950 (wave64, fp16 matrix cores, 160 KiB LDS):
//
//  * A group of 4 wavefronts computes a BM x 128 tile of y (BM = 128 for long
//    prefills, 64, or 32 for small problems); wavefront w owns 32 output
//    columns and all BM rows (BM/32 fragments of 32 x 32), so each weight code
//    of the tile is unpacked exactly once, in the registers of the wavefront
//    that uses it, into an exact binary16 integer, and that unpack feeds every
//    row fragment.
//  * When there are too few tiles to occupy the chip, a workgroup holds S = 2
//    or 4 such groups that split the tile's K loop; groups 1..S-1 hand their
//    fp32 sums to group 0 through LDS, which adds them in group order, so the
//    result stays deterministic and no memory beyond y is written.
//  * The K loop runs over stages of KT = 2 quantization blocks through two LDS
//    buffers. The packed codes, x (fp32) and the scales of a stage are loaded
//    into registers while earlier stages are computed (one stage ahead, two
//    for 32-row tiles), then written to the free buffer: x rounded to binary16
//    (nearest even) in the order the unpack produces the codes, with an XOR
//    swizzle of its 16-byte pieces so that the 128-bit fragment reads of the
//    rows hit distinct banks. Each scale is loaded by one thread.
//  * Each block of 32 values is two chained v_mfma_f32_32x32x16_f16 per 32 x 32
//    fragment from a zero accumulator: the block's fp32 partial, which is then
//    scaled by the block scale of its column and added to the fp32 accumulator
//    (one fused multiply-add per output and block), while the matrix work of
//    the compute unit's other wavefronts runs. The 32x32x16 shape is used
//    rather than 16x16x32 because on gfx950 it sustains twice the fp16 matrix
//    throughput per instruction issued.
//  * Within a block the 32 values are visited in the order the unpack produces
//    them, identically for x and the weights, so each dot product is unchanged.
//  * Tiles are ordered so that the workgroups placed on one XCD (workgroup id
//    modulo 8) cover consecutive tiles of a row of tiles and share x in that
//    XCD's L2. y is written with non-temporal stores: it is not read again by
//    this kernel and would otherwise evict x from L2.
//  * The grouped form runs the tiles of every tensor of a planned table in one
//    launch (the projections of a layer), with the same tile body.
#include "wq_internal.h"
#include "wq_decode.h"

namespace wq {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));

constexpr int BN = 128;            // columns per workgroup tile (32 per wavefront)
constexpr int KT = 2;              // quantization blocks per stage
constexpr int kThreads = 256;
constexpr int kXcds = 8;

// LDS layout of one stage buffer (BM rows per workgroup tile: 32, 64 or 128).
//   A: x as binary16, [BM rows][KT*32 values]; row pitch 128 bytes, 16-byte
//      slot s of row r stored at slot s ^ ((r >> 1) & 7).
//   B: packed codes, [BN columns][KT * CB bytes] (int5: the low nibbles), each
//      column in 8-byte units rotated as CodeUnits describes.
//   H: int5 only, bit 4 of the codes, [BN columns][KT dwords].
//   S: binary16 scales, [BN columns][KT].
template <int BITS, int BM>
struct Stage {
    static constexpr int CB = BITS == 8 ? 32 : 16;         // code bytes per column per block (int5: nibbles)
    static constexpr int A_BYTES = BM * KT * 64;
    static constexpr int B_BYTES = BN * KT * CB;
    static constexpr int H_BYTES = BITS == 5 ? BN * KT * 4 : 0;   // int5: bit 4 of the codes
    static constexpr int S_BYTES = BN * KT * 2;
    static constexpr int BYTES = A_BYTES + B_BYTES + H_BYTES + S_BYTES;
};

__device__ __forceinline__ int aslot(int r, int s) { return r * (KT * 4) + (s ^ ((r >> 1) & 7)); }

// B holds column c's KT * CB code bytes in 8-byte units rotated by a
// column-dependent amount, so that the code reads of a wavefront's 32 columns
// (one unit index for all of them) hit distinct banks: unit u of column c is
// stored at unit (u + rot(c)) % P.
template <int CB>
struct CodeUnits {
    static constexpr int COLB = KT * CB;                 // bytes per column
    static constexpr int P = COLB / 8;                   // units per column (4 or 8)
    static constexpr int L = COLB == 32 ? 3 : 2;         // columns c, c + 2^L, ... share banks
    __device__ static constexpr int rot(int c) { return (c >> L) & (P - 1); }
    __device__ static constexpr int off(int c, int u) { return c * COLB + ((u + rot(c)) & (P - 1)) * 8; }
};

// Launch bounds of a workgroup of S groups: one 256-thread group (two
// workgroups per compute unit) or S groups of 256 threads.
#define WQ_GEMM_BOUNDS(S) __launch_bounds__(((S) == 1 ? kThreads : kThreads * (S)), ((S) == 1 ? 2 : 1))

// Stages whose loads are in flight while one is computed: 2 for 32-row tiles
// (short prefills, where a stage's few matrix instructions cannot cover a
// memory round trip), else 1 (registers are needed for the row fragments).
constexpr int gemm_prefetch(int BM) { return BM == 32 ? 2 : 1; }

// One BM x 128 output tile (tm, tn) of y = x W^T; every thread of the
// workgroup calls it. lds_all holds at least S * 2 * Stage<BITS, BM>::BYTES.
template <int BITS, int BM, int S, int PF = gemm_prefetch(BM)>
__device__ __forceinline__ void gemm_tile(const float *__restrict__ x, int M, int K, int N,
                                          const uint8_t *__restrict__ q, const uint16_t *__restrict__ s,
                                          float *__restrict__ y, int tm, int tn, uint8_t *lds_all)
{
    using L = Stage<BITS, BM>;
    constexpr int CB = L::CB;
    constexpr int RF = BM / 32;                     // 32-row fragments per wavefront
    constexpr int XI = BM * KT * 4 / kThreads;      // 8-value x groups per thread per stage (4 or 2)
    constexpr int BP = BN * KT * CB / 16;           // 16-byte code pieces per stage (256 or 512)
    constexpr int QI = BP / kThreads;               // code pieces per thread per stage (1 or 2)
    static_assert(XI * kThreads == BM * KT * 4 && BP % kThreads == 0, "tile shape");
    // S groups of 4 wavefronts split the K loop; each group has its own two stage
    // buffers, and the partial sums of groups 1..S-1 are reduced through them.
    static_assert((S - 1) * kThreads * RF * 16 * 4 <= S * 2 * L::BYTES, "reduction fits the stage buffers");
    const int m0 = tm * BM, n0 = tn * BN;

    const int t = threadIdx.x & (kThreads - 1);  // index within the K group
    const int h = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kThreads);   // K group
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int C = K >> 5;                        // blocks per row
    const int NT = (C + KT - 1) / KT;            // stages of the whole K loop
    const int NTh = (NT + S - 1) / S;            // stages of this group (past K: scale 0)
    const int st0 = h * NTh;                     // its first stage
    uint8_t *const lds = lds_all + h * 2 * L::BYTES;
    const DecodeConsts dc = DecodeConsts::make();
    Decode5Consts dc5;
    if constexpr (BITS == 5) dc5 = Decode5Consts::make();

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
    // scales (and int5 bit-4 dwords): a stage needs KT * BN of them, one per
    // thread: thread t loads block sk = t % KT of the stage for column t / KT,
    // so the KT lanes of a column read one cache line. Each lane of such a load
    // reads a different row of the scales; loading each value once, from as few
    // lines as possible, measured 10-30% faster than KT loads in every thread.
    static_assert(kThreads == BN * KT, "one scale per thread and stage");
    const int sk = t % KT;
    int sn = n0 + t / KT;
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
    // one stage's loads in registers; PF sets in flight
    struct Regs {
        f4 xv[XI][2];
        u4 qv[QI];
        uint16_t sv;                              // scale of block sk of column sn
        uint32_t hv;                              // int5: its bit-4 dword
    };
    Regs rs[PF];
    const uint32_t hoff = (uint32_t)sn * qrow + (uint32_t)K / 2;
    // loads of stage st (every address clamped into the tensors, so a stage
    // past the group's K range loads valid data that is never committed)
    auto issue = [&](int st, Regs &r) {
        auto &qv = r.qv;
        auto &xv = r.xv;
        auto &sv = r.sv;
        auto &hv = r.hv;
        const int b0 = (st0 + st) * KT;
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
        {
            const int b = b0 + sk < C ? b0 + sk : C - 1;
            sv = __builtin_amdgcn_raw_buffer_load_b16(sr, soff + (uint32_t)b * 2, 0, 0);
            if constexpr (BITS == 5) hv = __builtin_amdgcn_raw_buffer_load_b32(qr, hoff + (uint32_t)b * 4, 0, 0);
        }
    };
    // x rounded to binary16 in operand order, the codes and the scales (zero past
    // K), into buffer buf
    auto commit = [&](int st, int buf, const Regs &r) {
        const auto &qv = r.qv;
        const auto &xv = r.xv;
        const auto &sv = r.sv;
        const auto &hv = r.hv;
        uint8_t *base = lds + buf * L::BYTES;
#pragma unroll
        for (int i = 0; i < QI; ++i) {
            // piece pc = 16-byte piece k of column c: units 2k and 2k + 1
            using U = CodeUnits<CB>;
            const int pc = t + i * kThreads;
            const int cc = pc / (U::COLB / 16), k = pc - cc * (U::COLB / 16);
            *reinterpret_cast<u2 *>(base + L::A_BYTES + U::off(cc, 2 * k)) = u2{qv[i].x, qv[i].y};
            *reinterpret_cast<u2 *>(base + L::A_BYTES + U::off(cc, 2 * k + 1)) = u2{qv[i].z, qv[i].w};
        }
#pragma unroll
        for (int i = 0; i < XI; ++i) {
            const float v[8] = {xv[i][0].x, xv[i][0].y, xv[i][0].z, xv[i][0].w,
                                xv[i][1].x, xv[i][1].y, xv[i][1].z, xv[i][1].w};
            h8 h;
#pragma unroll
            for (int k = 0; k < 8; ++k) h[operand_slot<BITS>(k)] = (_Float16)v[k];   // nearest even
            *reinterpret_cast<h8 *>(base + xlds[i]) = h;
        }
        {
            uint16_t *Sc = reinterpret_cast<uint16_t *>(base + L::A_BYTES + L::B_BYTES + L::H_BYTES);
            const int b = (st0 + st) * KT + sk;
            Sc[t] = b < C ? sv : (uint16_t)0;    // column t / KT, block sk
            if constexpr (BITS == 5) {
                uint32_t *H = reinterpret_cast<uint32_t *>(base + L::A_BYTES + L::B_BYTES);
                H[t] = hv;
            }
        }
    };

    f16v acc[RF];
#pragma unroll
    for (int i = 0; i < RF; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;

    const f16v zero = {};
    const int c = wave * 32 + (lane & 31);       // this lane's column of the tile
    const int g = lane >> 5;                     // its k-group within a K-step of 16
    // the matrix work of stage it, from LDS buffer it & 1
    auto compute = [&](int it) {
        const int cur = it & 1;
        const uint8_t *base = lds + cur * L::BYTES;
        const uint8_t *B = base + L::A_BYTES;
        const uint8_t *H = B + L::B_BYTES;
        const uint16_t *Sc = reinterpret_cast<const uint16_t *>(H + L::H_BYTES);
        // A fragments one K-step ahead (K-step q of the stage is at slot 2q + g)
        h8 acur[RF];
#pragma unroll
        for (int i = 0; i < RF; ++i) acur[i] = *reinterpret_cast<const h8 *>(base + aslot(i * 32 + (lane & 31), g) * 16);
        // the stage's code words and scales of this lane, read together at the
        // stage start (one LDS wait for the whole stage)
        using U = CodeUnits<CB>;
        u2 cw[KT][2];
        uint32_t hbs[KT][2];
        uint16_t scb[KT];
#pragma unroll
        for (int kb = 0; kb < KT; ++kb) {
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                if constexpr (BITS == 8) {
                    cw[kb][st] = *reinterpret_cast<const u2 *>(B + U::off(c, 4 * kb + 2 * st + g));
                } else {
                    cw[kb][st].x = *reinterpret_cast<const uint32_t *>(B + U::off(c, 2 * kb + st) + g * 4);
                    if constexpr (BITS == 5) hbs[kb][st] = H[(c * KT + kb) * 4 + 2 * st + g];
                }
            }
            scb[kb] = Sc[c * KT + kb];
        }
#pragma unroll
        for (int kb = 0; kb < KT; ++kb) {
            // this lane's 8 codes of each K-step (k = 16*st + 8*g .. +7 of block kb),
            // unpacked once and used by every row fragment
            h8 b[2];
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                if constexpr (BITS == 4) b[st] = unpack8_int4(cw[kb][st].x, dc);
                else if constexpr (BITS == 5) b[st] = unpack8_int5(cw[kb][st].x, hbs[kb][st], dc5);
                else b[st] = unpack8_int8(cw[kb][st].x, cw[kb][st].y, dc);
            }
            float sc = (float)__builtin_bit_cast(_Float16, scb[kb]);
            asm volatile("" : "+v"(sc));             // fp32 scale: plain FMAs
            // block partial of every row fragment: two chained K-steps of 16
            f16v p[RF];
            h8 anx[RF];
#pragma unroll
            for (int i = 0; i < RF; ++i) anx[i] = *reinterpret_cast<const h8 *>(base + aslot(i * 32 + (lane & 31), kb * 4 + 2 + g) * 16);
#pragma unroll
            for (int i = 0; i < RF; ++i) p[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(acur[i], b[0], zero, 0, 0, 0);
            if (kb + 1 < KT) {
#pragma unroll
                for (int i = 0; i < RF; ++i) acur[i] = *reinterpret_cast<const h8 *>(base + aslot(i * 32 + (lane & 31), (kb + 1) * 4 + g) * 16);
            }
#pragma unroll
            for (int i = 0; i < RF; ++i) p[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(anx[i], b[1], p[i], 0, 0, 0);
            // acc += scale * partial, block by block; the matrix work of other
            // wavefronts runs meanwhile
#pragma unroll
            for (int i = 0; i < RF; ++i) {
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][v] = __builtin_fmaf(sc, p[i][v], acc[i][v]);
                asm volatile("" : "+v"(acc[i]));    // the scaling happens here
            }
        }
    };

    if constexpr (PF == 1) {
        issue(0, rs[0]);
        commit(0, 0, rs[0]);                     // waits for stage 0's loads
        __syncthreads();
        if (NTh > 1) issue(1, rs[0]);
        for (int it = 0; it < NTh; ++it) {
            compute(it);
            if (it + 1 < NTh) {
                commit(it + 1, (it + 1) & 1, rs[0]);   // waits for stage it+1's loads
                __syncthreads();                 // every wave is done with buffer it & 1
                if (it + 2 < NTh) issue(it + 2, rs[0]);
            }
        }
    } else {
        // stage j's loads go to register set j % 2, issued two stages ahead, always
        // (no load under a branch, so each commit waits only for its own set)
        static_assert(PF == 2, "prefetch depth 1 or 2");
        issue(0, rs[0]);
        issue(1, rs[1]);
        commit(0, 0, rs[0]);                     // waits for stage 0's loads only
        __syncthreads();
        issue(2, rs[0]);
        int it = 0;
        for (; it + 1 < NTh; it += 2) {
            compute(it);
            commit(it + 1, 1, rs[1]);
            __syncthreads();
            issue(it + 3, rs[1]);
            compute(it + 1);
            if (it + 2 < NTh) {
                commit(it + 2, 0, rs[0]);
                __syncthreads();
            }
            issue(it + 4, rs[0]);
        }
        if (it < NTh) compute(it);
    }
    if constexpr (S > 1) {
        // groups 1..S-1 hand their partial sums to group 0 through LDS, which
        // adds them in group order (a fixed order: results are deterministic)
        float *red = reinterpret_cast<float *>(lds_all);
        __syncthreads();                         // every group is done with its buffers
        if (h > 0) {
#pragma unroll
            for (int i = 0; i < RF; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) red[(((h - 1) * RF + i) * 16 + v) * kThreads + t] = acc[i][v];
        }
        __syncthreads();
        if (h > 0) return;
#pragma unroll
        for (int j = 1; j < S; ++j)
#pragma unroll
            for (int i = 0; i < RF; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][v] += red[(((j - 1) * RF + i) * 16 + v) * kThreads + t];
    }

    // 32 x 32 output fragment: value v of lane l is row 8*(v/4) + 4*(l/32) + v%4,
    // column l%32.
    const int n = n0 + c;
    if (m0 + BM <= M && n0 + BN <= N) {
        // a whole tile: no per-value bounds checks (no branches between the stores)
        float *yp = y + (size_t)(m0 + 4 * g) * N + n;
#pragma unroll
        for (int i = 0; i < RF; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                __builtin_nontemporal_store(acc[i][v], yp + (size_t)(i * 32 + 8 * (v >> 2) + (v & 3)) * N);
    } else {
#pragma unroll
        for (int i = 0; i < RF; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = m0 + i * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
                if (m < M && n < N) __builtin_nontemporal_store(acc[i][v], y + (size_t)m * N + n);
            }
    }
}

template <int BITS, int BM, int S>
__global__ WQ_GEMM_BOUNDS(S) void gemm_kernel(const float *__restrict__ x, int M, int K, int N,
                                             const uint8_t *__restrict__ q, const uint16_t *__restrict__ s,
                                             float *__restrict__ y, int tiles_m, int tiles_n)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds_all[S * 2 * Stage<BITS, BM>::BYTES];
    // XCD-aware tile order: workgroups id, id+8, id+16, ... run on one XCD; give
    // them consecutive tiles (row-major over (tm, tn)).
    const int T = tiles_m * tiles_n;
    const int per = (T + kXcds - 1) / kXcds;
    const int tile = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
    if (tile >= T) return;
    const int tm = tile / tiles_n;
    gemm_tile<BITS, BM, S>(x, M, K, N, q, s, y, tm, tile - tm * tiles_n, lds_all);
}

// Grouped prefill: the work items of every tensor of a planned table in one
// launch. Item i belongs to the entry whose [tile_begin, tile_begin + tiles)
// holds it; within an entry, item j is tile (j % tiles_m, j / tiles_m), so with
// entries starting at multiples of 8 the items of one XCD (i % 8) share row
// tiles of x. Items past an entry's tiles (alignment padding) do nothing.
template <int BM, int S>
__global__ WQ_GEMM_BOUNDS(S) void gemm_grouped_kernel(const uint8_t *__restrict__ base,
                                                      const wq_desc *__restrict__ table, int count, int M)
{
    // int8 has the largest stage of the three code widths
    static_assert(Stage<8, BM>::BYTES >= Stage<4, BM>::BYTES && Stage<8, BM>::BYTES >= Stage<5, BM>::BYTES, "");
    __shared__ __attribute__((aligned(16))) uint8_t lds_all[S * 2 * Stage<8, BM>::BYTES];
    const int64_t item = blockIdx.x;
    const int tiles_m = (M + BM - 1) / BM;
    int e = -1;
    for (int i = 0; i < count; ++i) {
        const int64_t tb = table[i].tile_begin;
        const int64_t tiles = (int64_t)tiles_m * ((table[i].N + BN - 1) / BN);
        if (item >= tb && item < tb + tiles) { e = i; break; }
    }
    if (e < 0) return;
    const wq_desc &d = table[e];
    const int j = (int)(item - d.tile_begin);
    const int tm = j % tiles_m, tn = j / tiles_m;
    const int K = (int)d.K, N = (int)d.N;
    const uint8_t *q = base + d.q_off;
    const uint16_t *sc = reinterpret_cast<const uint16_t *>(base + d.s_off);
    if (d.bits == 4) gemm_tile<4, BM, S>(d.x, M, K, N, q, sc, d.y, tm, tn, lds_all);
    else if (d.bits == 5) gemm_tile<5, BM, S>(d.x, M, K, N, q, sc, d.y, tm, tn, lds_all);
    else gemm_tile<8, BM, S>(d.x, M, K, N, q, sc, d.y, tm, tn, lds_all);
}

template <int BITS, int BM, int S>
hipError_t launch_bits(const float *x, int64_t M, int64_t K, int64_t N, const void *q,
                       const uint16_t *scales, float *y, hipStream_t stream)
{
    const int tiles_m = (int)((M + BM - 1) / BM);
    const int tiles_n = (int)((N + BN - 1) / BN);
    const int T = tiles_m * tiles_n;
    const unsigned grid = (unsigned)(((T + kXcds - 1) / kXcds) * kXcds);
    gemm_kernel<BITS, BM, S><<<grid, kThreads * S, 0, stream>>>(x, (int)M, (int)K, (int)N, (const uint8_t *)q,
                                                                scales, y, tiles_m, tiles_n);
    return hipGetLastError();
}

// Tile height and K split. With at least 256 tiles of 128 x 128 (M >= 256),
// 128-row tiles: each unpacked code feeds four row fragments (measured 3-9%
// faster than 64 rows at M = 4096); with fewer than 512 of them (under two per
// compute unit) the K loop of each is split over 2 groups (the M = 4096 down
// projection: 9% faster; splitting 768 tiles was 10% slower). Else with at
// least 256 tiles of 64 x 128,
// 64-row tiles; fewer: 32-row tiles with the K loop of each tile split over 4
// groups (2 when it has fewer than 4 stages), so every SIMD runs several
// wavefronts; the time of a tile is then about a quarter of its serial K loop.
template <int BITS>
hipError_t launch_shape(const float *x, int64_t M, int64_t K, int64_t N, const void *q,
                        const uint16_t *scales, float *y, hipStream_t stream)
{
    const int64_t tn = (N + BN - 1) / BN;
    const int64_t stages = (K / 32 + KT - 1) / KT;
    const int64_t t128 = ((M + 127) / 128) * tn;
    if (M >= 256 && t128 >= 256) {
        // fewer than two tiles per compute unit: split each tile's K loop in two
        if (t128 < 512) return launch_bits<BITS, 128, 2>(x, M, K, N, q, scales, y, stream);
        return launch_bits<BITS, 128, 1>(x, M, K, N, q, scales, y, stream);
    }
    if (((M + 63) / 64) * tn >= 256 || stages < 2) return launch_bits<BITS, 64, 1>(x, M, K, N, q, scales, y, stream);
    if (stages < 4) return launch_bits<BITS, 32, 2>(x, M, K, N, q, scales, y, stream);
    return launch_bits<BITS, 32, 4>(x, M, K, N, q, scales, y, stream);
}

template <int BM, int S>
hipError_t launch_grouped(const void *base, const wq_desc *table, int count, int64_t total_tiles, int64_t M,
                          hipStream_t stream)
{
    gemm_grouped_kernel<BM, S><<<(unsigned)total_tiles, kThreads * S, 0, stream>>>(
        (const uint8_t *)base, table, count, (int)M);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_grouped(const void *base, const wq_desc *table, int count, int64_t total_tiles,
                               int64_t M, hipStream_t stream)
{
    static_assert(BN == kGemmTileN, "tile width");
    const int bm = gemm_grouped_bm(M), sp = gemm_grouped_split(M);
    if (bm == 32 && sp == 4) return launch_grouped<32, 4>(base, table, count, total_tiles, M, stream);
    if (bm == 64 && sp == 1) return launch_grouped<64, 1>(base, table, count, total_tiles, M, stream);
    if (bm == 128 && sp == 1) return launch_grouped<128, 1>(base, table, count, total_tiles, M, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_gemm(const float *x, int64_t M, int64_t K, int64_t N, int bits, const void *q,
                       const uint16_t *scales, float *y, hipStream_t stream)
{
    if (bits == 4) return launch_shape<4>(x, M, K, N, q, scales, y, stream);
    if (bits == 5) return launch_shape<5>(x, M, K, N, q, scales, y, stream);
    return launch_shape<8>(x, M, K, N, q, scales, y, stream);
}

}  // namespace wq
