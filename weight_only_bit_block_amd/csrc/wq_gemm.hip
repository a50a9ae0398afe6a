// wq_gemm.hip -- prefill GEMM for block-32 int4 / int5 / int8 weights (any M >= 1).
//
// The TinyMOSS-Diarize devpost page ("How we built it") describes a blocked
// prefill GEMM that unpacks each weight group once and reuses it across all
// activation rows, with FP32 activations and dequantization fused into the
// matmul. On gfx950 (wave64, fp16 matrix cores, 160 KiB LDS per compute unit)
// the work is done in two kernels on the caller's stream:
//
//  1. xprep_kernel rounds x to binary16 once per call, into a workspace: each
//     row m is first scaled by a power of two 2^e_m chosen so that its largest
//     magnitude lands in [2^14, 2^15) (for x inside binary16's normal range
//     this changes nothing but the exponent: the rounded values are the plain
//     binary16 rounding of x times 2^e_m, and any finite row is representable),
//     and 2^-e_m is kept per row. Within each block of 32 values the prepared
//     row is stored in the order in which the matrix instructions consume it
//     (below), so that the GEMM copies it to LDS without touching it.
//  2. gemm_kernel: a workgroup of WN x SK wavefronts computes a BM x (32 WN)
//     tile of y. Wavefront (h, w) owns 32 output columns and all BM rows (BM/32
//     row fragments of 32 x 32) for the h-th of SK slices of the K loop, so
//     each weight code is unpacked exactly once per tile, in the registers of
//     the wavefront that uses it, into an exact binary16 integer, and that
//     unpack feeds every row fragment.
//
// Data movement: the K loop runs over stages of two quantization blocks. The
// prepared x of a stage (BM rows x 128 bytes), the packed codes and the block
// scales of the wavefront's 32 columns are copied from global memory straight
// into LDS by buffer loads with the LDS-direct form (no registers, no vector
// ALU work), into a ring of NS stage buffers: while stage s is computed the
// copies of stages s+1 .. s+NS-1 are in flight. Each stage starts with a wait
// for this wavefront's copies of the stage and one workgroup barrier.
//
// Matrix work: per block of 32 values and 32 x 32 fragment, two chained
// v_mfma_f32_32x32x16_f16 from a zero accumulator give the block's fp32
// partial, which is scaled by the block scale of its column and added to the
// fp32 accumulator (one fused multiply-add per output and block). Lane (c, g)
// of a wavefront (c = lane % 32, g = lane / 32) supplies, for K-step st of a
// block, the 8 codes of group q = 2g + st of its column (codes 8q .. 8q+7),
// and the x operand lane (row, g) supplies the same 8 k in the same order
// (the order the unpack produces them), so each dot product is unchanged.
// Lane (c, g) therefore reads the contiguous bytes of groups 2g and 2g+1 of a
// block. The prepared x stores the four groups of a block at positions
// 2 st + g, i.e. in group order 0, 2, 1, 3.
//
// LDS layout: a row of the stage's x occupies 128 bytes (8 slots of 16 bytes,
// slot 4 kb + 2 st + g); slot s of row r is stored at slot s ^ ((r >> 1) & 7),
// so the 16 lanes of each 128-bit operand read hit distinct banks. The copy
// instruction writes 64 consecutive 16-byte slots, so the swizzle is applied
// by choosing which global piece each lane fetches.
//
// Tiles are ordered so that the workgroups placed on one XCD (workgroup id
// modulo 8) cover consecutive tiles of a row of tiles and share x in that
// XCD's L2; y is written with non-temporal stores, scaled by the row's 2^-e_m.
// The grouped form runs the tiles of every tensor of a planned table in one
// launch (the projections of a layer), with the same tile body.
#include <cstddef>
#include <mutex>
#include <type_traits>

#include "wq_internal.h"
#include "wq_device.h"
#include "wq_decode.h"

namespace wq {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int KT = 2;          // quantization blocks per stage
constexpr int kXcds = 8;

// ---------------------------------------------------------------- prepared x

// Position, within a block, of natural group q (codes 8q .. 8q+7): group q is
// used by K-step st = q & 1 in lane half g = q >> 1, and stored at 2 st + g.
__device__ __forceinline__ constexpr int group_pos(int q) { return ((q & 1) << 1) | (q >> 1); }

// Power-of-two exponent e for a row whose largest magnitude is amax: amax * 2^e
// lands in [2^14, 2^15). Rows of zeros or with non-finite entries get e = 0;
// e is capped so that 2^-e stays a normal fp32 number.
__device__ __forceinline__ int row_exponent(float amax)
{
    if (!(amax > 0.0f) || !(amax <= 3.4028234663852886e38f)) return 0;
    int E;
    (void)frexpf(amax, &E);                  // amax = f * 2^E, f in [0.5, 1)
    int e = 15 - E;
    return e > 126 ? 126 : e;                // E >= -125 here except for fp32 subnormals
}

// Eight values of group q of a row -> binary16 (times 2^e), in the operand order
// of the code width.
template <int ORDER>
__device__ __forceinline__ h8 xprep_group(f4 a, f4 b, int e)
{
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    h8 hv;
#pragma unroll
    for (int k = 0; k < 8; ++k)
        hv[operand_slot<ORDER == 1 ? 8 : 4>(k)] = (_Float16)ldexpf(v[k], e);   // exact scaling, then nearest even
    return hv;
}

// 16-byte slot of group q within a prepared row: block q / 4, position
// group_pos(q % 4) within the block.
__device__ __forceinline__ int xprep_slot(int q) { return (q >> 2) * 4 + group_pos(q & 3); }

__device__ __forceinline__ float absmax8(f4 a, f4 b)
{
    return fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                 fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
}

// One row of x -> binary16 groups in operand order, handed to put(q, h8); one
// wavefront per row; returns the row's exponent e. Rows of up to 64 * XG
// groups of 8 values are read once into registers (all loads in flight
// together); longer rows are read twice.
template <int ORDER, int XG, class Put>
__device__ __forceinline__ int xprep_row(const float *__restrict__ xrow, int K, int lane, Put put)
{
    const int G = K >> 3;                    // groups of 8 values
    float amax = 0.0f;
    if (G <= 64 * XG) {
        f4 va[XG], vb[XG];
#pragma unroll
        for (int i = 0; i < XG; ++i) {
            const int q = lane + 64 * i;
            if (q < G) {
                va[i] = *reinterpret_cast<const f4 *>(xrow + 8 * q);
                vb[i] = *reinterpret_cast<const f4 *>(xrow + 8 * q + 4);
                amax = fmaxf(amax, absmax8(va[i], vb[i]));
            }
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
        const int e = row_exponent(amax);
#pragma unroll
        for (int i = 0; i < XG; ++i) {
            const int q = lane + 64 * i;
            if (q < G) put(q, xprep_group<ORDER>(va[i], vb[i], e));
        }
        return e;
    }
    for (int q = lane; q < G; q += 64) {
        const f4 a = *reinterpret_cast<const f4 *>(xrow + 8 * q);
        const f4 b = *reinterpret_cast<const f4 *>(xrow + 8 * q + 4);
        amax = fmaxf(amax, absmax8(a, b));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    const int e = row_exponent(amax);
    for (int q = lane; q < G; q += 64) {
        const f4 a = *reinterpret_cast<const f4 *>(xrow + 8 * q);
        const f4 b = *reinterpret_cast<const f4 *>(xrow + 8 * q + 4);
        put(q, xprep_group<ORDER>(a, b, e));
    }
    return e;
}

// One row of x into the prepared workspace layout (global memory).
template <int ORDER>
__device__ __forceinline__ void xprep_row_ws(const float *__restrict__ xrow, int K, _Float16 *__restrict__ orow,
                                             float *__restrict__ rinv_m, int lane)
{
    const int e = xprep_row<ORDER, 8>(xrow, K, lane,
                                   [&](int q, h8 hv) { *reinterpret_cast<h8 *>(orow + xprep_slot(q) * 8) = hv; });
    if (lane == 0) *rinv_m = ldexpf(1.0f, -e);
}

// Prepared rows of one x [M][K]: four rows per workgroup.
template <int ORDER>
__global__ __launch_bounds__(256) void xprep_kernel(const float *__restrict__ x, int M, int K,
                                                     _Float16 *__restrict__ x16, float *__restrict__ rinv)
{
    const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= M) return;
    xprep_row_ws<ORDER>(x + (size_t)m * K, K, x16 + (size_t)m * K, rinv + m, threadIdx.x & 63);
}

// Grouped: entry e (blockIdx.y) prepares its x unless it is empty or an earlier
// entry owns the same workspace slot (ws_slot < 0: entries that share an x and
// a code order share a slot).
__global__ __launch_bounds__(256) void xprep_grouped_kernel(const wq_desc *__restrict__ table, int count, int M,
                                                             uint8_t *__restrict__ ws, int nflags)
{
    // clear the split-K flags of this call (the GEMM launch that follows sets them)
    {
        uint32_t *flags = reinterpret_cast<uint32_t *>(ws);
        const int stride = (int)(gridDim.x * gridDim.y) * 256;
        for (int i = (int)(blockIdx.y * gridDim.x + blockIdx.x) * 256 + (int)threadIdx.x; i < nflags; i += stride)
            flags[i] = 0u;
    }
    if ((int)blockIdx.y >= count) return;
    const wq_desc &d = table[blockIdx.y];
    if (d.N == 0 || d.ws_slot < 0) return;      // no work (x may be unset), or prepared by another entry
    const int slot = d.ws_slot;
    const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= M) return;
    const int K = (int)d.K;
    uint8_t *base = ws + (size_t)slot * kGemmWsUnit;
    _Float16 *x16 = reinterpret_cast<_Float16 *>(base);
    float *rinv = reinterpret_cast<float *>(base + gemm_ws_x16_bytes(M, K));
    if (d.bits == 8) xprep_row_ws<1>(d.x + (size_t)m * K, K, x16 + (size_t)m * K, rinv + m, threadIdx.x & 63);
    else xprep_row_ws<0>(d.x + (size_t)m * K, K, x16 + (size_t)m * K, rinv + m, threadIdx.x & 63);
}

// ---------------------------------------------------------------- GEMM tile

// LDS of one stage of one K slice: the prepared x (BM rows x 128 bytes), then for
// each of the WN wavefronts its codes (B), int5 bit-4 dwords (H), scales (S: for
// each (block, column) the aligned dword holding that block's scale) and row
// factors (R: 2^-e of BM / WN tile rows, repeated over 64 dwords).
template <int BITS, int BM, int WN>
struct Lay {
    static constexpr int A = BM * 128;
    static constexpr int BW = 32 * KT * (BITS == 8 ? 32 : 16);   // codes of 32 columns
    static constexpr int HW = BITS == 5 ? 32 * KT * 4 : 0;
    static constexpr int SW = 32 * KT * 4;
    static constexpr int RW = 64 * 4;
    static constexpr int WAVE = BW + HW + SW + RW;
    static constexpr int STAGE = A + WN * WAVE;
};
template <int BM, int WN>
constexpr int stage_max() { return Lay<8, BM, WN>::STAGE; }   // int8 has the largest stage
static_assert(Lay<8, 128, 4>::STAGE >= Lay<5, 128, 4>::STAGE && Lay<8, 64, 4>::STAGE >= Lay<5, 64, 4>::STAGE, "");

// Buffer loads in the LDS-direct form: lane i writes its 16 (4) bytes at LDS
// byte address lds + 16 i (4 i); lds (in M0) and the resource are uniform. They
// are issued from inline assembly so that the compiler keeps no wait counting
// of its own for them (its alias tracking of such copies cannot tell the ring
// buffers apart and would drain the ring at every stage); every wait on them is
// the explicit vmcnt wait of the K loop. They write no registers.
typedef uint32_t sgpr4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ sgpr4 raw_rsrc(const void *p, uint64_t bytes)
{
    const uint64_t a = (uint64_t)p;
    sgpr4 r;
    r.x = __builtin_amdgcn_readfirstlane((uint32_t)a);
    r.y = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xFFFFu);   // stride 0
    r.z = __builtin_amdgcn_readfirstlane((uint32_t)bytes);
    r.w = 0x00020000u;                                                    // 32-bit untyped data
    return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

__device__ __forceinline__ void dma16(sgpr4 r, uint32_t lds, uint32_t voff, uint32_t soff)
{
    // s_nop: one wait state between the write of M0 and its read by the copy
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :: "v"(voff), "s"(r), "s"(soff), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma4(sgpr4 r, uint32_t lds, uint32_t voff, uint32_t soff)
{
    asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, %2 offen lds"
                 :: "v"(voff), "s"(r), "s"(soff), "{m0}"(lds) : "memory");
}

// s_waitcnt vmcnt(N) with the other counters left alone.
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
constexpr int cap63(int n) { return n < 63 ? n : 63; }

// Bytes of one K slice of a ring buffer: the stage, and with a K split at least
// the 16 KiB through which a slice hands one fragment of sums to slice 0.
template <int STAGE, int WN, int SK>
constexpr int slice_bytes() { return (SK > 1 && STAGE < WN * 4096) ? WN * 4096 : STAGE; }

// SL: bytes of one K slice of a ring buffer (from the code width's own stage for
// a single call, from the largest over code widths for a grouped launch).
template <int BITS, int BM, int WN, int SK, int NS, int SL = slice_bytes<Lay<BITS, BM, WN>::STAGE, WN, SK>()>
struct Tile {
    using L = Lay<BITS, BM, WN>;
    static constexpr int RF = BM / 32;                  // row fragments per wavefront
    static constexpr int AI = BM / (8 * WN);            // x copy instructions per wavefront and stage
    static constexpr int BI = BITS == 8 ? 2 : 1;        // code copy instructions
    static constexpr int V = AI + BI + (BITS == 5 ? 1 : 0) + 2;   // copies per wavefront and stage
    static constexpr int RPW = BM / WN;                 // tile rows whose factors a wavefront copies
    static constexpr int STORES = RF * 16;              // y stores per wavefront and tile (slice 0)
    static constexpr int SLICE = SL;
    static_assert(SL >= L::STAGE, "slice size");
    static constexpr int LDS = NS * SK * SLICE;
    static_assert(AI * 8 * WN == BM && RPW >= 8 && 32 % RPW == 0, "tile geometry");
    static_assert(NS >= 2 && NS <= 4, "ring depth");
    static_assert(V * (NS - 2) < 64, "vmcnt");
    static_assert(SK == 1 || WN * 64 * 16 * 4 <= SLICE, "reduction buffer");
};

// Resident workgroups per compute unit of a configuration (LDS and the
// launch bounds below).
template <int LDS, int WN, int SK>
constexpr int gemm_occupancy() { return WN * SK > 4 ? 1 : (LDS <= 53248 ? 3 : (LDS <= 81920 ? 2 : 1)); }

#define WQ_GEMM_BOUNDS(LDS, WN, SK) __launch_bounds__((WN) * (SK) * 64, (gemm_occupancy<LDS, WN, SK>()))

// The K range of a tile's work item and its part in a split across
// workgroups: stages [st_begin, st_begin + st_count) of the tile's K loop; with
// P > 1 pieces, piece kp < P - 1 leaves its fp32 partial tile at part + kp BM
// BN (floats, lane-major) and then sets flag[kp]; piece P - 1 waits for the
// flags of pieces 0 .. P-2 (workgroups of lower index, dispatched before it),
// adds their partials in piece order to its own, and stores the tile.
struct KPiece {
    int st_begin, st_count, kp, P;
    float *part;
    uint32_t *flag;
};

// The pieces of a split tile run on different XCDs, whose L2 caches are not
// kept coherent with each other. Partial tiles and flags are therefore written
// and read only with device-scope relaxed atomic accesses, which the hardware
// keeps coherent at device scope by themselves: such a store writes through
// the XCD's L2 and is complete at device scope once the wavefront's vmcnt has
// drained, and such a load does not return a line of its own L2. So neither
// side needs a device-scope fence, whose release writes back and whose acquire
// invalidates the whole L2 of its XCD (which all other workgroups there then
// pay for). The producer drains its stores before the workgroup barrier that
// precedes thread 0's flag store; the consumer issues its partial loads only
// after it has read every flag set (a compiler barrier keeps them there).

// Waits (bounded) until a piece's flag is set; false if it never was (the
// caller then poisons its tile with NaN, so a broken dispatch-order assumption
// shows as wrong output, never as a hang).
__device__ __forceinline__ bool wait_piece(const uint32_t *flag)
{
    for (int it = 0; it < (1 << 20); ++it) {
        if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) return true;
        __builtin_amdgcn_s_sleep(8);
    }
    return false;
}

// The tiles [u = 0, U) of one workgroup, as a stream of K stages: tile_of(u)
// gives (tm, tn) of the u-th tile. The copies of the next NS - 1 stages are in
// flight while a stage is computed, across tile boundaries, so a tile's first
// loads overlap the previous tile's last stages and its stores of y. Every
// thread of the workgroup calls it, with the same U. ring holds the NS stage
// buffers of SK * SLICE bytes each.
// ONE: the workgroup has a single tile (U == 1), whose end is handled after
// the K loop, once every copy has landed; SPLIT: that tile may be a piece of a
// K loop split across workgroups (kpc.P > 1).
template <int BITS, int BM, int WN, int SK, int NS, int SL, bool ONE = false, bool SPLIT = false, class TileOf>
__device__ __forceinline__ void gemm_stream(const _Float16 *__restrict__ x16, const float *__restrict__ rinv,
                                            int M, int K, int N, const uint8_t *__restrict__ q,
                                            const uint16_t *__restrict__ s, float *__restrict__ y, int U,
                                            TileOf tile_of, uint8_t *ring, KPiece kpc)
{
    using T = Tile<BITS, BM, WN, SK, NS, SL>;
    using L = typename T::L;
    constexpr int RF = T::RF, AI = T::AI, V = T::V, SLICE = T::SLICE, RPW = T::RPW;
    constexpr int BN = 32 * WN;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int h = wv / WN;                       // K slice
    const int w = wv - h * WN;                   // wavefront within the slice: columns 32w .. 32w+31
    const int C = K >> 5;                        // blocks per row
    const int NTh = (kpc.st_count + SK - 1) / SK;   // stages of each slice (past the range: scale 0)
    const int st0 = kpc.st_begin + h * NTh;
    const int st_end = kpc.st_begin + kpc.st_count;
    const uint32_t qrow = (uint32_t)K * BITS / 8;
    const int c = lane & 31, g = lane >> 5;     // column of the wavefront; lane half

    const sgpr4 xr = raw_rsrc(x16, (uint64_t)M * K * 2);
    const sgpr4 qr = raw_rsrc(q, (uint64_t)N * qrow);
    // Scales are copied as the aligned dwords that hold them. When N * K/32 is
    // odd the last dword reaches 2 bytes past the last scale; those bytes lie
    // in the same 16-byte granule as the scale (the array is 16-byte aligned),
    // hence in a mapped page, and are never used.
    const sgpr4 sr = raw_rsrc(s, ((uint64_t)N * C * 2 + 3) & ~(uint64_t)3);
    // Row factors: the region is padded to 256 bytes; tile rows past it read 0
    // (they are never stored).
    const sgpr4 rr = raw_rsrc(rinv, gemm_ws_rinv_bytes(M));

    // ---- issue cursor: the next stage to copy and the per-lane offsets of its tile
    int iu = 0, istl = 0;
    uint32_t xoff[AI], qoff = 0, hoff = 0, soff = 0, roff = 0;
    auto set_tile = [&](int u) {
        const auto tt = tile_of(u);
        const int m0 = tt.x * BM, n0 = tt.y * BN;
#pragma unroll
        for (int j = 0; j < AI; ++j) {
            const int r = (w * AI + j) * 8 + (lane >> 3);      // tile row written by this lane
            const int sl = (lane & 7) ^ ((r >> 1) & 7);        // the logical slot stored at slot lane & 7
            int m = m0 + r;
            m = m < M ? m : M - 1;
            xoff[j] = (uint32_t)m * (uint32_t)K * 2 + (uint32_t)(sl >> 2) * 64 + (uint32_t)(sl & 3) * 16;
        }
        int ncl = n0 + w * 32 + c;
        ncl = ncl < N ? ncl : N - 1;
        // codes: lane (c, g) copies block g of the stage for column c (int8: each
        // of the two copy instructions moves one 16-byte half of it)
        qoff = (uint32_t)ncl * qrow + (uint32_t)g * (BITS == 8 ? 32 : 16);
        hoff = (uint32_t)ncl * qrow + (uint32_t)K / 2 + (uint32_t)g * 4;
        // scales: the aligned dword holding the scale of block 2 st + g of column c
        soff = (((uint32_t)ncl * (uint32_t)C + (uint32_t)g) * 2) & ~3u;
        roff = (uint32_t)(m0 + w * RPW + lane % RPW) * 4;
    };
    set_tile(0);
    // Copies of the next stage into `ring`. Issued unconditionally (every
    // wavefront issues V copies per call, which the waits count); past the
    // last stage the last one is read again (cache hits) into a buffer that is
    // never read.
    auto issue = [&](uint8_t *ring) {
        const bool live = iu < U;
        const int st = st0 + (live ? istl : NTh - 1);
        uint8_t *base = ring + h * SLICE;
        uint8_t *wb = base + L::A + w * L::WAVE;
#pragma unroll
        for (int j = 0; j < AI; ++j) dma16(xr, lds_addr(base + (w * AI + j) * 1024), xoff[j], (uint32_t)st * 128);
        if constexpr (BITS == 8) {
            dma16(qr, lds_addr(wb), qoff, (uint32_t)st * 64);
            dma16(qr, lds_addr(wb + 1024), qoff + 16, (uint32_t)st * 64);
        } else {
            dma16(qr, lds_addr(wb), qoff, (uint32_t)st * 32);
            if constexpr (BITS == 5) dma4(qr, lds_addr(wb + L::BW), hoff, (uint32_t)st * 8);
        }
        dma4(sr, lds_addr(wb + L::BW + L::HW), soff, (uint32_t)st * 4);
        dma4(rr, lds_addr(wb + L::BW + L::HW + L::SW), roff, 0);
        if (live && ++istl == NTh) {
            istl = 0;
            if (++iu < U) set_tile(iu);
        }
    };

    // ---- per-lane read offsets
    const int t = g ^ ((c >> 1) & 7);           // operand row r = 32 i + c: swizzle (r >> 1) & 7
    uint32_t aoff[2 * KT];                       // K-step (kb, st): slot 4 kb + 2 st + g, stored at slot ^ swizzle
#pragma unroll
    for (int u = 0; u < 2 * KT; ++u) aoff[u] = (uint32_t)c * 128 + (uint32_t)(((2 * u) ^ t) << 4);
    const uint32_t boff = BITS == 8 ? (uint32_t)(g * 1024 + c * 16) : (uint32_t)(c * 16 + g * 8);
    const DecodeConsts dc = DecodeConsts::make();
    Decode5Consts dc5;
    if constexpr (BITS == 5) dc5 = Decode5Consts::make();

    f16v acc[RF];
#pragma unroll
    for (int i = 0; i < RF; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;
    const f16v zero = {};

    // ---- compute cursor
    int cu = 0, cstl = 0;
    int ssh[KT];                                 // which half of a copied dword holds block kb's scale
    auto set_scale_halves = [&](int u) {
        const auto tt = tile_of(u);
        int ncl = tt.y * BN + w * 32 + c;
        ncl = ncl < N ? ncl : N - 1;
        const uint32_t scol = (uint32_t)ncl * (uint32_t)C;
#pragma unroll
        for (int kb = 0; kb < KT; ++kb) ssh[kb] = (int)(((scol + kb) & 1) * 16);
    };
    set_scale_halves(0);

    auto compute = [&](const uint8_t *ring) {
        const int st = st0 + cstl;
        const uint8_t *A = ring + h * SLICE;
        const uint8_t *wb = A + L::A + w * L::WAVE;
#pragma unroll
        for (int kb = 0; kb < KT; ++kb) {
            h8 b[2];
            if constexpr (BITS == 8) {
                const u4 cw = *reinterpret_cast<const u4 *>(wb + kb * 512 + boff);
                b[0] = unpack8_int8(cw.x, cw.y, dc);
                b[1] = unpack8_int8(cw.z, cw.w, dc);
            } else {
                const u2 cw = *reinterpret_cast<const u2 *>(wb + kb * 512 + boff);
                if constexpr (BITS == 5) {
                    const uint32_t hb = *reinterpret_cast<const uint32_t *>(wb + L::BW + (kb * 32 + c) * 4) >> (16 * g);
                    b[0] = unpack8_int5(cw.x, hb & 0xFFu, dc5);
                    b[1] = unpack8_int5(cw.y, (hb >> 8) & 0xFFu, dc5);
                } else {
                    b[0] = unpack8_int4(cw.x, dc);
                    b[1] = unpack8_int4(cw.y, dc);
                }
            }
            const uint32_t sw = *reinterpret_cast<const uint32_t *>(wb + L::BW + L::HW + (kb * 32 + c) * 4);
            float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)(sw >> ssh[kb]));
            sc = (st < st_end && st * KT + kb < C) ? sc : 0.0f;   // blocks past the range contribute nothing
            asm volatile("" : "+v"(sc));
            h8 a0[RF], a1[RF];
#pragma unroll
            for (int i = 0; i < RF; ++i) {
                a0[i] = *reinterpret_cast<const h8 *>(A + aoff[2 * kb] + i * 4096);
                a1[i] = *reinterpret_cast<const h8 *>(A + aoff[2 * kb + 1] + i * 4096);
            }
            f16v p[RF];
#pragma unroll
            for (int i = 0; i < RF; ++i) p[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0[i], b[0], zero, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < RF; ++i) p[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1[i], b[1], p[i], 0, 0, 0);
#pragma unroll
            for (int i = 0; i < RF; ++i) {
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][v] = __builtin_fmaf(sc, p[i][v], acc[i][v]);
            }
        }
    };

    // The end of tile u, whose last stage was computed from `ring`: slices
    // 1..SK-1 hand their sums to slice 0 through their own parts of that buffer
    // (free until the next barrier), one fragment at a time in slice order (a
    // fixed order: deterministic); slice 0 scales by 2^-e_m and stores y with
    // buffer stores (out-of-range outputs go past the resource and are dropped,
    // so every wavefront of slice 0 issues exactly STORES stores).
    auto epilogue = [&](int u, const uint8_t *ring) {
        if constexpr (SK > 1) {
#pragma unroll
            for (int j = 1; j < SK; ++j) {
#pragma unroll
                for (int i = 0; i < RF; ++i) {
                    float *red = reinterpret_cast<float *>(const_cast<uint8_t *>(ring) + j * SLICE);
                    lds_barrier();
                    if (h == j) {
#pragma unroll
                        for (int v = 0; v < 16; ++v) red[(v * WN + w) * 64 + lane] = acc[i][v];
                    }
                    lds_barrier();
                    if (h == 0) {
#pragma unroll
                        for (int v = 0; v < 16; ++v) acc[i][v] += red[(v * WN + w) * 64 + lane];
                    }
                }
            }
        }
        bool store = true;
        if (SPLIT && kpc.P > 1) {
            if (kpc.kp < kpc.P - 1) {
                // a leading piece: its partial, then its flag, once every
                // wavefront's partial stores have completed
                if (h == 0) {
                    float *dst = kpc.part + (size_t)kpc.kp * BM * BN;
#pragma unroll
                    for (int i = 0; i < RF; ++i)
#pragma unroll
                        for (int v = 0; v < 16; ++v)
                            __hip_atomic_store(dst + ((i * 16 + v) * WN + w) * 64 + lane, acc[i][v], __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                    asm volatile("" ::: "memory");
                    wait_vm<0>();
                }
                __syncthreads();
                if (threadIdx.x == 0)
                    __hip_atomic_store(kpc.flag + kpc.kp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                store = false;
            } else if (h == 0) {
                // the last piece: partials of pieces 0 .. P-2 in order, then its own
                bool ok = true;
                for (int j = 0; j < kpc.P - 1; ++j) ok = wait_piece(kpc.flag + j) && ok;
                asm volatile("" ::: "memory");
                // one piece at a time, all of its loads in flight together
                f16v sum[RF];
                for (int j = 0; j < kpc.P - 1; ++j) {
                    const float *pj = kpc.part + (size_t)j * BM * BN + w * 64 + lane;
                    f16v t[RF];
#pragma unroll
                    for (int i = 0; i < RF; ++i)
#pragma unroll
                        for (int v = 0; v < 16; ++v)
                            t[i][v] = __hip_atomic_load(pj + (i * 16 + v) * WN * 64, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
                    for (int i = 0; i < RF; ++i) sum[i] = j == 0 ? t[i] : sum[i] + t[i];
                }
#pragma unroll
                for (int i = 0; i < RF; ++i)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[i][v] = ok ? sum[i][v] + acc[i][v] : __builtin_nanf("");
            }
        }
        if (h == 0 && store) {
            const auto tt = tile_of(u);
            const int m0 = tt.x * BM, n0 = tt.y * BN;
            const int rows = M - m0 < BM ? M - m0 : BM;
            const __amdgpu_buffer_rsrc_t yr = make_rsrc(y + (size_t)m0 * N, (uint64_t)rows * N * 4);
            const int n = n0 + w * 32 + c;
            // Output (r, n) of the tile is at byte (r N + n) 4 of yr: a per-lane part
            // (4 g rows and the column; past N: the resource size) in the vector
            // offset and the rest of the row in the scalar offset. The buffer range
            // check covers their sum, so rows past the tile's last and columns past
            // N land past the resource and are dropped (every kernel's writes are
            // checked against a guard region by the tests). (r + rows) N 4 < 2^32
            // as N < 2^22.
            const uint32_t lane_off = n < N ? (uint32_t)(4 * g * N + n) * 4 : (uint32_t)rows * N * 4;
            const uint8_t *R = ring + L::A + L::BW + L::HW + L::SW + 16 * g;   // slice 0's factors
            // 32 x 32 output fragment: value v of lane l is row 8*(v/4) + 4*(l/32) + v%4, column l%32
#pragma unroll
            for (int i = 0; i < RF; ++i) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int rg = i * 32 + 8 * j;                    // rows rg + 4 g .. rg + 4 g + 3
                    const f4 f = *reinterpret_cast<const f4 *>(R + (rg / RPW) * L::WAVE + (rg % RPW) * 4);
                    const float fv[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, acc[i][4 * j + v] * fv[v]),
                                                              yr, lane_off, (uint32_t)(rg + v) * N * 4, kNonTemporal);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < RF; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;
    };

    // Stage steps. Each waits for this wavefront's copies of the stage it
    // computes: NS - 2 later stages are in flight behind them, plus the stores
    // of tiles ended since those copies were issued, then a barrier (everyone's
    // copies have landed and everyone is done with the buffer about to be
    // refilled), refills that buffer with the stage NS - 1 ahead, computes.
    const int J = U * NTh;
    constexpr int SKS = SK * SLICE;
    issue(ring);
    if constexpr (NS >= 3) issue(ring + SKS);
    if constexpr (NS >= 4) issue(ring + 2 * SKS);
    int epi = 0;                                 // bit i: the step i + 1 steps back ended a tile
    int cs = 0;                                  // ring buffer of the stage computed next
    for (int j = 0; j < J; ++j) {
        if (h == 0 && (epi & ((1 << (NS - 1)) - 1)) != 0) {
            // stores were issued after this stage's copies: count at least one tile's
            // worth of them (capped: a smaller count only waits longer)
            wait_vm<cap63(V * (NS - 2) + T::STORES)>();
        } else {
            wait_vm<V * (NS - 2)>();
        }
        lds_barrier();
        const int ns = cs == 0 ? NS - 1 : cs - 1;   // the buffer computed last step: refill it
        issue(ring + ns * SKS);
        const uint8_t *cur = ring + cs * SKS;
        compute(cur);
        if constexpr (ONE) {
            ++cstl;                              // the single tile ends after the loop
        } else {
            epi <<= 1;
            if (++cstl == NTh) {
                epilogue(cu, cur);
                epi |= 1;
                cstl = 0;
                if (++cu < U) set_scale_halves(cu);
            }
        }
        cs = cs + 1 == NS ? 0 : cs + 1;
    }
    // the copies of the stages past the end are still in flight: let them land
    // before the LDS is released (or reused by the end of a single tile)
    wait_vm<0>();
    if constexpr (ONE) {
        lds_barrier();
        epilogue(0, ring);
    }
}

// Single call: a persistent grid of G workgroups (a multiple of 8). Workgroup b
// runs on XCD b % 8; XCD x owns the consecutive tiles [x per, (x + 1) per) of
// the row-major tile order (neighbouring tiles share rows of x in that XCD's
// L2), and its workgroups take them round-robin.
template <int BITS, int BM, int WN, int SK, int NS>
__global__ WQ_GEMM_BOUNDS((Tile<BITS, BM, WN, SK, NS>::LDS), WN, SK) void gemm_kernel(const _Float16 *__restrict__ x16,
                                                           const float *__restrict__ rinv, int M, int K, int N,
                                                           const uint8_t *__restrict__ q,
                                                           const uint16_t *__restrict__ s, float *__restrict__ y,
                                                           int tiles_m, int tiles_n)
{
    __shared__ __attribute__((aligned(16))) uint8_t ring[Tile<BITS, BM, WN, SK, NS>::LDS];
    const int T = tiles_m * tiles_n;
    const int per = (T + kXcds - 1) / kXcds;
    const int g8 = (int)gridDim.x / kXcds;
    const int x = blockIdx.x % kXcds, i = blockIdx.x / kXcds;
    const int first = x * per + i;
    const int end = (x + 1) * per < T ? (x + 1) * per : T;
    const int U = first < end ? (end - first + g8 - 1) / g8 : 0;
    if (U == 0) return;
    auto tile_of = [&](int u) {
        const int tt = first + u * g8;
        const int tm = tt / tiles_n;
        return make_int2(tm, tt - tm * tiles_n);
    };
    const KPiece whole = {0, ((K >> 5) + KT - 1) / KT, 0, 1, nullptr, nullptr};
    gemm_stream<BITS, BM, WN, SK, NS, Tile<BITS, BM, WN, SK, NS>::SLICE>(x16, rinv, M, K, N, q, s, y, U, tile_of, ring,
                                                                        whole);
}

// Grouped prefill: the work items of every tensor of a planned table in one
// launch, one tile per workgroup. Item i belongs to the entry whose
// [tile_begin, tile_begin + tiles) holds it; within an entry, item j is tile
// (j % tiles_m, j / tiles_m), so with entries starting at multiples of 8 the
// items of one XCD (i % 8) share row tiles of x. Items past an entry's tiles
// (alignment padding) do nothing.
template <int BM, int WN, int SK, int NS>
__global__ WQ_GEMM_BOUNDS((Tile<8, BM, WN, SK, NS, slice_bytes<stage_max<BM, WN>(), WN, SK>()>::LDS), WN, SK) void gemm_grouped_kernel(const uint8_t *__restrict__ base,
                                                                   const wq_desc *__restrict__ table, int count,
                                                                   int M, const uint8_t *__restrict__ ws)
{
    constexpr int SL = slice_bytes<stage_max<BM, WN>(), WN, SK>();
    __shared__ __attribute__((aligned(16))) uint8_t ring[Tile<8, BM, WN, SK, NS, SL>::LDS];
    const int64_t item = blockIdx.x;
    const int tiles_m = (M + BM - 1) / BM;
    // the entry whose [tile_begin, tile_begin + items) holds the item (at most
    // one does): 64 entries per step, one per lane, each lane reading its whole
    // descriptor, so that the one found is broadcast from registers (no second
    // round trip to the table)
    const int lane = threadIdx.x & 63;
    int e = -1, src = 0;
    u4 dd[4];
    for (int b0 = 0; b0 < count; b0 += 64) {
        const int i = b0 + lane;
        bool hit = false;
        if (i < count) {
            const u4 *pd = reinterpret_cast<const u4 *>(table + i);
#pragma unroll
            for (int k = 0; k < 4; ++k) dd[k] = pd[k];
            const int64_t tb = (int64_t)(((uint64_t)dd[3].w << 32) | dd[3].z);
            const int64_t n = (int64_t)(((uint64_t)dd[0].w << 32) | dd[0].z);
            const int64_t kk = (int64_t)(((uint64_t)dd[1].y << 32) | dd[1].x);
            const int64_t items = (int64_t)tiles_m * ((n + 32 * WN - 1) / (32 * WN)) * gemm_grouped_ksplit(M, kk);
            hit = item >= tb && item < tb + items;
        }
        const uint64_t m = __ballot(hit);
        if (m) {
            src = (int)__builtin_ctzll(m);
            e = b0 + src;
            break;
        }
    }
    if (e < 0) return;                           // alignment padding between entries
    static_assert(offsetof(wq_desc, ws_slot) == 4 && offsetof(wq_desc, N) == 8 && offsetof(wq_desc, K) == 16 &&
                      offsetof(wq_desc, q_off) == 24 && offsetof(wq_desc, s_off) == 32 &&
                      offsetof(wq_desc, x) == 40 && offsetof(wq_desc, y) == 48 && offsetof(wq_desc, tile_begin) == 56,
                  "descriptor dwords decoded below");
    auto rl = [&](uint32_t v) { return (uint32_t)__builtin_amdgcn_readlane((int)v, src); };
    auto rl64 = [&](uint32_t lo, uint32_t hi) { return ((uint64_t)rl(hi) << 32) | rl(lo); };
    wq_desc dl;
    dl.bits = (int32_t)rl(dd[0].x);
    dl.ws_slot = (int32_t)rl(dd[0].y);
    dl.N = (int64_t)rl64(dd[0].z, dd[0].w);
    dl.K = (int64_t)rl64(dd[1].x, dd[1].y);
    dl.q_off = rl64(dd[1].z, dd[1].w);
    dl.s_off = rl64(dd[2].x, dd[2].y);
    dl.x = reinterpret_cast<const float *>(rl64(dd[2].z, dd[2].w));
    dl.y = reinterpret_cast<float *>(rl64(dd[3].x, dd[3].y));
    dl.tile_begin = (int64_t)rl64(dd[3].z, dd[3].w);
    const wq_desc &d = dl;
    const int K = (int)d.K, N = (int)d.N;
    // item -> tile and piece of its K loop
    const int P = gemm_grouped_ksplit(M, K);
    const int j = (int)(item - d.tile_begin);
    const int t = j / P, kp = j - t * P;
    const int2 tile = make_int2(t % tiles_m, t / tiles_m);
    auto tile_of = [&](int) { return tile; };
    const int NT = ((K >> 5) + KT - 1) / KT;
    KPiece kpc;
    kpc.st_begin = kp * NT / P;
    kpc.st_count = (kp + 1) * NT / P - kpc.st_begin;
    kpc.kp = kp;
    kpc.P = P;
    const int64_t first = d.tile_begin + (int64_t)t * P;      // the tile's first item
    kpc.flag = reinterpret_cast<uint32_t *>(const_cast<uint8_t *>(ws)) + first;
    kpc.part = reinterpret_cast<float *>(const_cast<uint8_t *>(ws) + gemm_grouped_flag_bytes(M, gridDim.x)) +
               first * (BM * 32 * WN);
    const uint8_t *q = base + d.q_off;
    const uint16_t *sc = reinterpret_cast<const uint16_t *>(base + d.s_off);
    const uint8_t *slot = ws + (size_t)(d.ws_slot < 0 ? ~d.ws_slot : d.ws_slot) * kGemmWsUnit;
    const _Float16 *x16 = reinterpret_cast<const _Float16 *>(slot);
    const float *rinv = reinterpret_cast<const float *>(slot + gemm_ws_x16_bytes(M, K));
    if (d.bits == 4)
        gemm_stream<4, BM, WN, SK, NS, SL, true, BM == 64>(x16, rinv, M, K, N, q, sc, d.y, 1, tile_of, ring, kpc);
    else if (d.bits == 5)
        gemm_stream<5, BM, WN, SK, NS, SL, true, BM == 64>(x16, rinv, M, K, N, q, sc, d.y, 1, tile_of, ring, kpc);
    else
        gemm_stream<8, BM, WN, SK, NS, SL, true, BM == 64>(x16, rinv, M, K, N, q, sc, d.y, 1, tile_of, ring, kpc);
}

// Compute units of the current device (queried once per device).
int device_cus()
{
    static int cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

// ---------------------------------------------------------------- skinny GEMM
// With few rows (M <= 64) and many columns (the lm_head at M = 64) the GEMM is
// bound by streaming the weights from HBM, and the tile kernel above, which
// passes every operand through one LDS ring per workgroup, keeps too few bytes
// in flight per compute unit for that. Here one workgroup per compute unit
// first rounds all M rows of x to binary16 into LDS (the per-row power-of-two
// scaling and operand order of xprep_kernel, so no pre-pass and no workspace),
// where they stay for the whole launch; then each of its 8 wavefronts walks
// 32-column strips of the weights, loading the codes and scales of SB blocks
// at a time straight into registers with the next SKP - 1 batches in flight,
// and multiplies them against the resident x with the same per-block matrix
// instructions and fp32 scaling as the tile kernel. Strip t goes to workgroup
// t % G and, within it, wavefront (t / G) % 8, so the compute units' shares
// differ by at most one strip. x rows are stored with 16-byte slot j of row r
// at j ^ (r & 15) (rows are a multiple of 256 bytes long), so the 16 lanes of
// each 128-bit operand read hit distinct banks.
constexpr int kSkWaves = 8;
constexpr int kSkLdsX = 128 * 1024;           // resident x: 32 RF rows x K values x 2 bytes at most

template <int BITS, int SB>
struct SkBatch {
    using CW = typename std::conditional<BITS == 8, u4, u2>::type;    // a lane's codes of one block
    static constexpr int SV = SB >= 8 ? SB / 8 : 1;                   // loads of the column's SB scales
    using SW = typename std::conditional<SB >= 8, u4, u2>::type;      // 8 scales (or 4)
    static_assert(SB >= 4 && (SB == 4 || SB % 8 == 0), "batch size");
    CW code[SB];
    SW sc[SV];
};

template <typename V>
__device__ __forceinline__ V sk_load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    if constexpr (sizeof(V) == 16)
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
    else
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0));
}

template <int BITS, int RF, int SB, int SPS, int P>
__global__ __launch_bounds__(kSkWaves * 64, 1) void gemm_skinny_kernel(const float *__restrict__ x, int M, int N,
                                                                       const uint8_t *__restrict__ q,
                                                                       const uint16_t *__restrict__ s,
                                                                       float *__restrict__ y)
{
    constexpr int BM = 32 * RF;
    constexpr int C = SB * SPS;                  // blocks per row
    constexpr int K = 32 * C;
    constexpr int ROWB = K * 2;                  // bytes of a resident x row
    constexpr int QROW = K * BITS / 8;           // bytes of a column's codes
    constexpr int BPB = 32 * BITS / 8;           // code bytes per block and column
    constexpr int CB = BPB / 2;                  // ... per lane half
    static_assert(BM * ROWB <= kSkLdsX && ROWB % 256 == 0, "resident x");
    static_assert(SPS % P == 0, "batch ring slots repeat every strip");
    using B = SkBatch<BITS, SB>;
    // Row r = 32 i + c of x is stored as LDS row RF c + i, so the row fragments
    // of one lane are ROWB bytes apart (an immediate offset of the read).
    __shared__ __attribute__((aligned(16))) uint8_t lds[BM * ROWB + BM * 4];
    float *R = reinterpret_cast<float *>(lds + BM * ROWB);

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int c = lane & 31, g = lane >> 5;
    const int G = gridDim.x;
    const int strips = (N + 31) >> 5;
    const int first = (int)blockIdx.x + wv * G, step = kSkWaves * G;
    const int my = first < strips ? (strips - first + step - 1) / step : 0;   // strips of this wavefront

    const __amdgpu_buffer_rsrc_t qr = make_rsrc(q, (uint64_t)N * QROW);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(s, (uint64_t)N * C * 2);
    auto col_of = [&](int j) {                   // column of this lane in strip j (clamped: loads stay in range)
        const int n = (first + j * step) * 32 + c;
        return n < N ? n : N - 1;
    };
    auto load = [&](B &b, int ncl, int seg) {    // batch seg of the strip holding column ncl
        const uint32_t vq = (uint32_t)ncl * QROW + (uint32_t)g * CB;
#pragma unroll
        for (int kb = 0; kb < SB; ++kb)
            b.code[kb] = sk_load<typename B::CW>(qr, vq + kb * BPB, (uint32_t)seg * SB * BPB);
#pragma unroll
        for (int v = 0; v < B::SV; ++v)
            b.sc[v] = sk_load<typename B::SW>(sr, (uint32_t)ncl * C * 2 + v * 16, (uint32_t)seg * SB * 2);
    };

    // ---- resident x, loads: wavefront wv prepares rows wv + 8 t, all of their
    // loads in flight together. They are issued before the first code batches:
    // loads complete in order, so x issued after the batches waited for all of
    // them (the M=64 lm_head, back to back over rotated copies: 57.0 us that
    // way, 54.2 us this way).
    constexpr int RPW = BM / kSkWaves;           // rows per wavefront
    constexpr int XGS = K / 512;                 // groups of 8 values per lane and row
    static_assert(XGS >= 1 && K % 512 == 0, "x rows are whole multiples of 64 groups");
    f4 va[RPW][XGS], vb[RPW][XGS];
#pragma unroll
    for (int t = 0; t < RPW; ++t) {
        const int r = wv + kSkWaves * t;
        const float *xr = x + (size_t)(r < M ? r : 0) * K;
#pragma unroll
        for (int i = 0; i < XGS; ++i) {
            const int qg = lane + 64 * i;
            va[t][i] = *reinterpret_cast<const f4 *>(xr + 8 * qg);
            vb[t][i] = *reinterpret_cast<const f4 *>(xr + 8 * qg + 4);
        }
    }

    // The first batches of this wavefront's first strip, then as many stores as
    // a strip's end issues, all dropped (past the resource): the loop is then
    // entered with the same memory operations in flight, in the same order, as
    // it is re-entered from a strip's end, and the wait counts derived for it
    // keep the later batches in flight.
    const uint32_t ybytes = (uint32_t)M * (uint32_t)N * 4;
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(y, ybytes);
    B ring[P];
    {
        const int n0 = col_of(0);
#pragma unroll
        for (int p = 0; p < P - 1; ++p) load(ring[p], n0, p);
#pragma unroll
        for (int i = 0; i < RF * 16; ++i)
            __builtin_amdgcn_raw_buffer_store_b32(0u, yr, ybytes + (uint32_t)i * N * 4, 0, kNonTemporal);
    }

    // ---- resident x, rounding: the scaling and operand order of xprep_kernel;
    // rows past M are zeros. The x values pass through an empty asm first, so
    // no use of them is moved up between their loads (which would wait for the
    // first row before the other rows' loads are issued).
#pragma unroll
    for (int t = 0; t < RPW; ++t)
#pragma unroll
        for (int i = 0; i < XGS; ++i) asm volatile("" : "+v"(va[t][i]), "+v"(vb[t][i]));
    {
#pragma unroll
        for (int t = 0; t < RPW; ++t) {
            const int r = wv + kSkWaves * t;
            uint8_t *row = lds + ((r & 31) * RF + (r >> 5)) * ROWB;
            const int key = r & 15;
            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < XGS; ++i) amax = fmaxf(amax, absmax8(va[t][i], vb[t][i]));
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
            const int e = row_exponent(amax);
            const bool live = r < M;
#pragma unroll
            for (int i = 0; i < XGS; ++i) {
                const int qg = lane + 64 * i;
                const h8 hv = live ? xprep_group<BITS == 8 ? 1 : 0>(va[t][i], vb[t][i], e) : h8{};
                *reinterpret_cast<h8 *>(row + ((xprep_slot(qg) ^ key) << 4)) = hv;
            }
            if (lane == 0) R[r] = live ? ldexpf(1.0f, -e) : 0.0f;
        }
    }
    __syncthreads();

    // ---- per-lane LDS offsets: slot (4 (blk & 3) + 2 st + g) ^ (c & 15) of the lane's row
    uint32_t aoff[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)                  // u = 2 (blk & 3) + st
        aoff[u] = (uint32_t)(c * RF) * ROWB + (uint32_t)((((u >> 1) * 4 + (u & 1) * 2 + g) ^ (c & 15)) << 4);
    const DecodeConsts dc = DecodeConsts::make();
    const f16v zero = {};
    f16v acc[RF];
#pragma unroll
    for (int i = 0; i < RF; ++i) acc[i] = zero;

    auto compute = [&](const B &b, int seg) {
#pragma unroll
        for (int kb = 0; kb < SB; ++kb) {
            const int blk = seg * SB + kb;       // constant after unrolling
            h8 w0, w1;
            if constexpr (BITS == 8) {
                w0 = unpack8_int8(b.code[kb].x, b.code[kb].y, dc);
                w1 = unpack8_int8(b.code[kb].z, b.code[kb].w, dc);
            } else {
                w0 = unpack8_int4(b.code[kb].x, dc);
                w1 = unpack8_int4(b.code[kb].y, dc);
            }
            const uint32_t sw = b.sc[kb >> 3][(kb >> 1) & 3];
            float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)(sw >> (16 * (kb & 1))));
            // converted once: otherwise each scaling FMA takes the binary16
            // scale as a mixed-precision operand, which issues at half rate
            asm volatile("" : "+v"(sc));
            const uint32_t bo = (uint32_t)(blk & ~3) * 64;
            const int u = 2 * (blk & 3);
#pragma unroll
            for (int i = 0; i < RF; ++i) {
                const h8 a0 = *reinterpret_cast<const h8 *>(lds + aoff[u] + i * ROWB + bo);
                const h8 a1 = *reinterpret_cast<const h8 *>(lds + aoff[u + 1] + i * ROWB + bo);
                f16v p = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, w0, zero, 0, 0, 0);
                p = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, w1, p, 0, 0, 0);
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][v] = __builtin_fmaf(sc, p[v], acc[i][v]);
            }
            __builtin_amdgcn_sched_barrier(0);   // one block at a time: bounded live ranges
        }
    };

    // Output (r, n) is at byte (r N + n) 4 of yr: the lane's part (4 g rows and
    // its column; past N the resource size) plus the rest of the row, both in
    // the vector offset, which alone is range-checked: rows past M and columns
    // past N land past the resource and are dropped.
    for (int j = 0; j < my; ++j) {
        const int ncl = col_of(j);
        const int nxt = col_of(j + 1 < my ? j + 1 : j);
#pragma unroll
        for (int sg = 0; sg < SPS; ++sg) {
            const int ts = sg + P - 1;        // the batch issued now: ts of this strip or ts - SPS of the next
            if (ts < SPS) load(ring[ts % P], ncl, ts);
            else load(ring[ts % P], nxt, ts - SPS);
            compute(ring[sg % P], sg);
        }
        const int n = (first + j * step) * 32 + c;
        const uint32_t lane_off = n < N ? (uint32_t)(4 * g * N + n) * 4 : ybytes;
#pragma unroll
        for (int i = 0; i < RF; ++i) {
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
                const int rg = i * 32 + 8 * j4;  // rows rg + 4 g .. rg + 4 g + 3
                const f4 f = *reinterpret_cast<const f4 *>(R + rg + 4 * g);
                const float fv[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, acc[i][4 * j4 + v] * fv[v]), yr,
                                                          lane_off + (uint32_t)(rg + v) * N * 4, 0, kNonTemporal);
            }
            acc[i] = zero;
        }
    }
    wait_vm<0>();                                // the batches loaded past the last strip
}

template <int BITS, int RF, int SB, int SPS, int P>
hipError_t launch_skinny(const float *x, int64_t M, int64_t N, const void *q, const uint16_t *scales, float *y,
                         hipStream_t stream)
{
    const int64_t strips = (N + 31) / 32;
    const int64_t want = (strips + kSkWaves - 1) / kSkWaves;
    const int64_t cus = device_cus();
    const unsigned grid = (unsigned)(want < cus ? want : cus);
    gemm_skinny_kernel<BITS, RF, SB, SPS, P><<<grid, kSkWaves * 64, 0, stream>>>(x, (int)M, (int)N,
                                                                                (const uint8_t *)q, scales, y);
    return hipGetLastError();
}

template <int BITS, int BM, int WN, int SK, int NS>
hipError_t launch_cfg(const _Float16 *x16, const float *rinv, int64_t M, int64_t K, int64_t N, const void *q,
                      const uint16_t *scales, float *y, hipStream_t stream)
{
    const int tiles_m = (int)((M + BM - 1) / BM);
    const int tiles_n = (int)((N + 32 * WN - 1) / (32 * WN));
    const int64_t T = (int64_t)tiles_m * tiles_n;
    // persistent grid: every resident workgroup slot, a multiple of 8 (one per XCD)
    const int64_t slots =
        (int64_t)device_cus() * gemm_occupancy<Tile<BITS, BM, WN, SK, NS>::LDS, WN, SK>() / kXcds * kXcds;
    const int64_t want = (T + kXcds - 1) / kXcds * kXcds;
    const unsigned grid = (unsigned)(want < slots ? want : slots);
    gemm_kernel<BITS, BM, WN, SK, NS><<<grid, WN * SK * 64, 0, stream>>>(
        x16, rinv, (int)M, (int)K, (int)N, (const uint8_t *)q, scales, y, tiles_m, tiles_n);
    return hipGetLastError();
}

// Tile shape, K split and ring depth of a single call (C compute units):
//  - long prefills (at least 2 C tiles of 128 x 128): 128-row tiles, each code
//    unpack feeding four row fragments; three workgroups per compute unit with
//    two stages in flight when that gives no more tiles per compute unit than
//    two workgroups with three stages (the M = 4096 gate projection: 768 tiles,
//    one per workgroup, measured 11% faster), else the latter. int5 always
//    takes the latter: under the register limit of three workgroups (168) its
//    K loop spills (the bit-4 dwords and their unpack constants), and the
//    M = 4096 int5 gate projection took 79.8 us cold against 63.2 us with two;
//  - C .. 2 C such tiles: the same tiles with the K loop of each split over two
//    wavefront groups of one workgroup;
//  - fewer: 64-row tiles (the M = 64 int8 lm_head has 1187 of them) with four
//    stages in flight, or for few of those, 64-row tiles with a two-way split.
// The grid is persistent (every resident workgroup slot), so the tiles of a
// workgroup stream through one copy ring.
template <int BITS>
hipError_t launch_shape(const _Float16 *x16, const float *rinv, int64_t M, int64_t K, int64_t N, const void *q,
                        const uint16_t *scales, float *y, hipStream_t stream)
{
    const int64_t cus = device_cus();
    const int64_t tn = (N + 127) / 128;
    const int64_t t128 = ((M + 127) / 128) * tn;
    const int64_t t64 = ((M + 63) / 64) * tn;
    if (M > 64 && t128 >= 2 * cus) {
        if constexpr (BITS != 5) {
            const int64_t per3 = 3 * ((t128 + 3 * cus - 1) / (3 * cus)), per2 = 2 * ((t128 + 2 * cus - 1) / (2 * cus));
            if (per3 <= per2) return launch_cfg<BITS, 128, 4, 1, 2>(x16, rinv, M, K, N, q, scales, y, stream);
        }
        return launch_cfg<BITS, 128, 4, 1, 3>(x16, rinv, M, K, N, q, scales, y, stream);
    }
    if (M > 64 && t128 >= cus) return launch_cfg<BITS, 128, 4, 2, 3>(x16, rinv, M, K, N, q, scales, y, stream);
    if (t64 >= cus) return launch_cfg<BITS, 64, 4, 1, 4>(x16, rinv, M, K, N, q, scales, y, stream);
    return launch_cfg<BITS, 64, 4, 2, 3>(x16, rinv, M, K, N, q, scales, y, stream);
}

template <int BM, int WN, int SK, int NS>
hipError_t launch_grouped(const void *base, const wq_desc *table, int count, int64_t total_tiles, int64_t M,
                          const void *ws, hipStream_t stream)
{
    gemm_grouped_kernel<BM, WN, SK, NS><<<(unsigned)total_tiles, WN * SK * 64, 0, stream>>>(
        (const uint8_t *)base, table, count, (int)M, (const uint8_t *)ws);
    return hipGetLastError();
}

// Scratch of the allocation-free prefill entry point: the prepared x and row
// factors of one call, in device memory that exists as long as the library is
// loaded. Host code addresses it only through the pointer hipGetSymbolAddress
// returns for the current device (the array's name is a host stand-in).
static __device__ __align__(256) uint8_t scratch[kGemmNoAllocScratch];

std::mutex g_scratch_mu;
void *g_scratch_ptr[64] = {};

}  // namespace

hipError_t gemm_noalloc_scratch(void **ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

bool gemm_skinny(int64_t M, int64_t K, int64_t N, int bits)
{
    if ((bits != 4 && bits != 8) || M < 1 || M > 64) return false;
    if (!(K == 512 || K == 1024 || (K == 2048 && M <= 32))) return false;
    return (N + 31) / 32 >= 4 * (int64_t)device_cus();      // at least 4 strips per compute unit
}

// Batches of SB blocks of the strip's 32 columns: kSkSB blocks per batch, up to
// kSkP batches in registers (one fewer in flight), no more than a strip holds.
constexpr int kSkSB8 = 4, kSkSB4 = 4;          // blocks per batch: int8, int4
constexpr int kSkP = 4;
template <int BITS, int RF, int K>
hipError_t launch_skinny_kk(const float *x, int64_t M, int64_t N, const void *q, const uint16_t *scales, float *y,
                            hipStream_t stream)
{
    constexpr int SB0 = BITS == 8 ? kSkSB8 : kSkSB4;
    constexpr int SB = SB0 < K / 32 ? SB0 : K / 32;
    constexpr int SPS = K / 32 / SB;
    constexpr int P = SPS < kSkP ? SPS : kSkP;
    return launch_skinny<BITS, RF, SB, SPS, P>(x, M, N, q, scales, y, stream);
}

template <int BITS>
hipError_t launch_skinny_k(const float *x, int64_t M, int64_t K, int64_t N, const void *q, const uint16_t *scales,
                           float *y, hipStream_t stream)
{
    if (K == 512) {
        if (M <= 32) return launch_skinny_kk<BITS, 1, 512>(x, M, N, q, scales, y, stream);
        return launch_skinny_kk<BITS, 2, 512>(x, M, N, q, scales, y, stream);
    }
    if (K == 1024) {
        if (M <= 32) return launch_skinny_kk<BITS, 1, 1024>(x, M, N, q, scales, y, stream);
        return launch_skinny_kk<BITS, 2, 1024>(x, M, N, q, scales, y, stream);
    }
    return launch_skinny_kk<BITS, 1, 2048>(x, M, N, q, scales, y, stream);   // M <= 32
}

hipError_t launch_gemm(const float *x, int64_t M, int64_t K, int64_t N, int bits, const void *q,
                       const uint16_t *scales, float *y, void *ws, hipStream_t stream)
{
    if (gemm_skinny(M, K, N, bits)) {
        return bits == 8 ? launch_skinny_k<8>(x, M, K, N, q, scales, y, stream)
                         : launch_skinny_k<4>(x, M, K, N, q, scales, y, stream);
    }
    _Float16 *x16 = reinterpret_cast<_Float16 *>(ws);
    float *rinv = reinterpret_cast<float *>((uint8_t *)ws + gemm_ws_x16_bytes(M, K));
    const unsigned pgrid = (unsigned)((M + 3) / 4);
    if (bits == 8) xprep_kernel<1><<<pgrid, 256, 0, stream>>>(x, (int)M, (int)K, x16, rinv);
    else xprep_kernel<0><<<pgrid, 256, 0, stream>>>(x, (int)M, (int)K, x16, rinv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (bits == 4) return launch_shape<4>(x16, rinv, M, K, N, q, scales, y, stream);
    if (bits == 5) return launch_shape<5>(x16, rinv, M, K, N, q, scales, y, stream);
    return launch_shape<8>(x16, rinv, M, K, N, q, scales, y, stream);
}

hipError_t launch_gemm_grouped(const void *base, const wq_desc *table, int count, int64_t total_tiles, int64_t M,
                               void *ws, hipStream_t stream)
{
    static_assert(kGemmTileN == 128, "tile width of every grouped shape");
    dim3 pgrid((unsigned)((M + 3) / 4), (unsigned)count);
    const int nflags = gemm_grouped_flag_bytes(M, total_tiles) ? (int)total_tiles : 0;
    xprep_grouped_kernel<<<pgrid, 256, 0, stream>>>(table, count, (int)M, (uint8_t *)ws, nflags);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int bm = gemm_grouped_bm(M), sp = gemm_grouped_split(M);
    if (bm == 64 && sp == 2) return launch_grouped<64, 4, 2, 3>(base, table, count, total_tiles, M, ws, stream);
    if (bm == 128 && sp == 1) return launch_grouped<128, 4, 1, 3>(base, table, count, total_tiles, M, ws, stream);
    return hipErrorInvalidValue;
}

}  // namespace wq
