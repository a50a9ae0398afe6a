// wq_gemv.hip -- decode GEMV for block-32 int4 / int5 / int8 weights, M <= 2
// activation rows (3 <= M <= 16 run on the matrix cores, wq_mgemv.hip).
//
// The devpost page for TinyMOSS-Diarize ("How we built it") describes a
// separate GEMV path for decode that multiplies straight out of the packed
// weights, activations in FP32, dequantization fused, nothing materialized.
// This is that path designed for gfx950, where it is bound by the HBM stream of
// packed codes:
//
//  * Work items. A workgroup (4 wavefronts) computes one item: IROWS
//    consecutive rows of one tensor for all M activation rows. G lanes of a
//    wavefront share a row and each lane owns the 16-byte chunks li, li+G,
//    li+2G, ... of it (one int4 block, or half an int8 block, per chunk), so
//    the lanes of a row read G*16 contiguous bytes per load (geometry in
//    wq_internal.h). In the fast form a lane owns four rows and walks them in
//    segments of two chunks per row: the segment's eight chunks are loaded with
//    non-temporal 128-bit loads straight into registers, and memory and
//    arithmetic overlap across the many items resident on each compute unit.
//    Items hold 32-128 KiB of codes at the decoder's shapes, so a launch has
//    thousands of them and its tail is short.
//  * x and the item's scales are copied into LDS by direct-to-LDS loads
//    (global_load_lds_dwordx4: no registers), issued before the code loads; a
//    barrier that waits only for those copies lets the code loads stay in
//    flight across it, and the arithmetic starts on each chunk as it lands. x
//    is stored unpadded with an XOR swizzle of its 16-byte pieces so that the
//    128-bit reads of 16 lanes hit distinct banks.
//  * int5 rows are read as int4 chunks of low nibbles plus, per chunk, the 4
//    bytes of its codes' bit 4 (a second load from the row's bit-4 plane).
//  * Unpack in registers without int->float conversions (wq_decode.h): with
//    one activation row the fp32 FMA takes the binary16 code directly as an
//    operand (v_fma_mix_f32); with two, codes go straight to exact fp32 values
//    by bit operations and the FMAs are plain v_fma_f32. Either way each
//    product q*x is exact and is accumulated in fp32.
//  * Per chunk: two partial chains over its codes, then acc += scale * partial
//    in fp32; lanes of a row are reduced with a DPP butterfly, so every lane of
//    the group holds the same bits. The arithmetic of an output depends only on
//    (K, bits, M): not on J, the item or the launch (single tensor or
//    grouped), so every launch gives bitwise identical results.
//
// Error: summation depth per output is 16 + 1 + CC/G + log2(G) (CC chunks per
// row), far below the depth of ~160 at which fp32 rounding could reach
// 1e-5 * sum |x||w|.
#include "wq_internal.h"
#include "wq_device.h"
#include "wq_decode.h"

namespace wq {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// A code as fp32 (exact). With one activation row the conversion folds into
// v_fma_mix_f32; with several, each code is converted once and the MT products
// use the full-rate v_fma_f32 (v_fma_mix_f32 issues at half rate on gfx950).
// The arithmetic is the same either way: exact product, one rounding.
template <int MT>
__device__ __forceinline__ float code_f32(_Float16 w)
{
    float f = (float)w;
    if constexpr (MT > 1) asm volatile("" : "+v"(f));
    return f;
}

// y pointers come from kernel arguments or the tensor table; both are global
// memory, so store through the global address space.
__device__ __forceinline__ void store_global(float *p, float v)
{
    *(__attribute__((address_space(1))) float *)p = v;
}

// Butterfly sums over aligned groups of G lanes (G a power of two <= 16, one
// DPP row). Both lanes of every exchanged pair add the same two values, so every
// lane of a group ends with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int N_>
__device__ __forceinline__ void group_sums(float (&v)[N_], int G)
{
    if (G >= 2) {
#pragma unroll
        for (int i = 0; i < N_; ++i) v[i] += dpp<0xB1>(v[i]);     // quad_perm [1,0,3,2]: lane ^ 1
    }
    if (G >= 4) {
#pragma unroll
        for (int i = 0; i < N_; ++i) v[i] += dpp<0x4E>(v[i]);     // quad_perm [2,3,0,1]: lane ^ 2
    }
    if (G >= 8) {
#pragma unroll
        for (int i = 0; i < N_; ++i) v[i] += dpp<0x141>(v[i]);    // row_half_mirror: other quad of 8
    }
    if (G >= 16) {
#pragma unroll
        for (int i = 0; i < N_; ++i) v[i] += dpp<0x140>(v[i]);    // row_mirror: other 8 of 16
    }
}

// Direct-to-LDS copy of 16 bytes per active lane: lane i of the wavefront
// writes lds_base + 16 * i (lds_base is the same for every lane).
__device__ __forceinline__ void dma16(const void *src, void *lds_base)
{
    __builtin_amdgcn_global_load_lds(src, lds_base, 16, 0, 0);
}

// Copies `pieces` 16-byte pieces into LDS, spread over the 4 wavefronts: piece
// pc (0 <= pc < pieces) is read from src(pc) and lands at dst + 16 * pc.
template <typename F>
__device__ __forceinline__ void copy_pieces(int pieces, uint8_t *dst, int wave, int lane, F src)
{
    for (int base = wave * kWave; base < pieces; base += kGemvThreads) {
        const int pc = base + lane;
        if (pc < pieces) dma16(src(pc), dst + (size_t)base * 16);
    }
}

// Workgroup barrier after this wave's LDS writes and copies into LDS: waits
// until at most N vector-memory operations of the wave are outstanding (the
// copies were issued before the last N loads) and its LDS operations are done,
// then s_barrier. Unlike __syncthreads() it does not wait for every global load,
// so the last N loads stay in flight across it. The empty asm statements keep
// the compiler from moving memory accesses across the barrier.
template <int N_>
__device__ __forceinline__ void copies_barrier()
{
    static_assert(N_ >= 0 && N_ < 64, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N_ & 15) | (7 << 4) | ((N_ >> 4) << 14));   // vmcnt(N_) expcnt(7) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Slot (in 16-byte pieces) of piece p (0..7) of block b in a staged x row.
// Blocks b..b+15 read at one piece index land in 16 distinct bank groups.
__device__ __forceinline__ int xslot(int b, int p) { return b * 8 + (p ^ ((b >> 1) & 7)); }

// x rows [mg, mg+MT) over blocks [b0, b0+nb) into LDS, 16-byte pieces, swizzled.
template <int MT>
__device__ __forceinline__ void stage_x(const float *__restrict__ x, int M, int K, int mg, int b0, int nb,
                                        uint8_t *xs, int wave, int lane)
{
    copy_pieces(MT * nb * 8, xs, wave, lane, [&](int pc) {
        const int m = pc / (nb * 8);
        const int rem = pc - m * nb * 8;
        const int b = rem >> 3;
        const int p = (rem & 7) ^ ((b >> 1) & 7);                       // piece that belongs in this slot
        const int mm = mg + m < M ? mg + m : M - 1;
        return reinterpret_cast<const uint8_t *>(x + (size_t)mm * K + (size_t)(b0 + b) * kBlock + p * 4);
    });
}

// The arithmetic of one chunk index for the J rows of a lane: codes w[j] (16
// bytes of row j) times the staged x of the chunk's block (read once for all J
// rows), into two partial chains per (j, m); then acc += scale * partial.
// Piece p of the block's x row m is at xp[p] + m * xstride. Two forms, by the
// number of activation rows; both give exact products and fp32 sums:
//  * one row (chunk_fma_h): codes as binary16, two per packed fp16 op, and one
//    v_fma_mix_f32 per product, the fewest instructions per code;
//  * two rows (chunk_fma_f): codes straight to fp32 with full-rate bit ops and
//    one subtract (no conversion), then full-rate v_fma_f32 per product.
// Measured on the decode step: the second form is 7% faster at M = 2 and 5%
// slower at M = 1.
template <int BITS, int MT, int J>
__device__ __forceinline__ void chunk_fma_h(const u4 (&w)[J], const uint8_t *const (&xp)[8], int xstride,
                                            const DecodeConsts &dc, const float (&sc)[J], float (&acc)[J][MT])
{
    float p0[J][MT], p1[J][MT];
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
        for (int m = 0; m < MT; ++m) { p0[j][m] = 0.0f; p1[j][m] = 0.0f; }
#pragma unroll
    for (int h = 0; h < (BITS == 4 ? 4 : 2); ++h) {       // groups of 8 codes: x pieces 2h, 2h+1 of xp
        f4 xa[MT], xb[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            xa[m] = *reinterpret_cast<const f4 *>(xp[2 * h] + m * xstride);
            xb[m] = *reinterpret_cast<const f4 *>(xp[2 * h + 1] + m * xstride);
        }
#pragma unroll
        for (int j = 0; j < J; ++j) {
            h2 t0, t1, t2, t3;
            if (BITS == 4) {
                decode_int4(w[j][h], dc, t0, t1, t2, t3);     // (k0,k4) (k1,k5) (k2,k6) (k3,k7)
                const float ft0x = code_f32<MT>(t0.x);
                const float ft0y = code_f32<MT>(t0.y);
                const float ft1x = code_f32<MT>(t1.x);
                const float ft1y = code_f32<MT>(t1.y);
                const float ft2x = code_f32<MT>(t2.x);
                const float ft2y = code_f32<MT>(t2.y);
                const float ft3x = code_f32<MT>(t3.x);
                const float ft3y = code_f32<MT>(t3.y);
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    p0[j][m] = __builtin_fmaf(ft0x, xa[m].x, p0[j][m]);
                    p1[j][m] = __builtin_fmaf(ft0y, xb[m].x, p1[j][m]);
                    p0[j][m] = __builtin_fmaf(ft1x, xa[m].y, p0[j][m]);
                    p1[j][m] = __builtin_fmaf(ft1y, xb[m].y, p1[j][m]);
                    p0[j][m] = __builtin_fmaf(ft2x, xa[m].z, p0[j][m]);
                    p1[j][m] = __builtin_fmaf(ft2y, xb[m].z, p1[j][m]);
                    p0[j][m] = __builtin_fmaf(ft3x, xa[m].w, p0[j][m]);
                    p1[j][m] = __builtin_fmaf(ft3y, xb[m].w, p1[j][m]);
                }
            } else {
                decode_int8(w[j][2 * h], dc, t0, t1);         // (k0,k2) (k1,k3)
                decode_int8(w[j][2 * h + 1], dc, t2, t3);     // (k4,k6) (k5,k7)
                const float ft0x = code_f32<MT>(t0.x);
                const float ft0y = code_f32<MT>(t0.y);
                const float ft1x = code_f32<MT>(t1.x);
                const float ft1y = code_f32<MT>(t1.y);
                const float ft2x = code_f32<MT>(t2.x);
                const float ft2y = code_f32<MT>(t2.y);
                const float ft3x = code_f32<MT>(t3.x);
                const float ft3y = code_f32<MT>(t3.y);
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    p0[j][m] = __builtin_fmaf(ft0x, xa[m].x, p0[j][m]);
                    p1[j][m] = __builtin_fmaf(ft0y, xa[m].z, p1[j][m]);
                    p0[j][m] = __builtin_fmaf(ft1x, xa[m].y, p0[j][m]);
                    p1[j][m] = __builtin_fmaf(ft1y, xa[m].w, p1[j][m]);
                    p0[j][m] = __builtin_fmaf(ft2x, xb[m].x, p0[j][m]);
                    p1[j][m] = __builtin_fmaf(ft2y, xb[m].z, p1[j][m]);
                    p0[j][m] = __builtin_fmaf(ft3x, xb[m].y, p0[j][m]);
                    p1[j][m] = __builtin_fmaf(ft3y, xb[m].w, p1[j][m]);
                }
            }
        }
    }
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[j][m] = __builtin_fmaf(sc[j], p0[j][m] + p1[j][m], acc[j][m]);
}

template <int BITS, int MT, int J>
__device__ __forceinline__ void chunk_fma_f(const u4 (&w)[J], const uint8_t *const (&xp)[8], int xstride,
                                            const DecodeF32Consts &dc, const float (&sc)[J], float (&acc)[J][MT])
{
    // plo: codes at even positions; phi: codes at odd positions, times 16 (int4)
    // or 256 (int8) as decoded
    float plo[J][MT], phi[J][MT];
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
        for (int m = 0; m < MT; ++m) { plo[j][m] = 0.0f; phi[j][m] = 0.0f; }
#pragma unroll
    for (int h = 0; h < (BITS == 4 ? 4 : 2); ++h) {       // groups of 8 codes: x pieces 2h, 2h+1 of xp
        f4 xa[MT], xb[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            xa[m] = *reinterpret_cast<const f4 *>(xp[2 * h] + m * xstride);
            xb[m] = *reinterpret_cast<const f4 *>(xp[2 * h + 1] + m * xstride);
        }
#pragma unroll
        for (int j = 0; j < J; ++j) {
            // the 8 codes and their x values: c[0..7] with x in xa.xyzw, xb.xyzw
            float lo[4], hi[4];
            if (BITS == 4) {
                decode_int4_f32(w[j][h], dc, lo, hi);        // lo: k0 k2 k4 k6; hi: 16 * (k1 k3 k5 k7)
            } else {
                float l0[2], h0[2], l1[2], h1[2];
                decode_int8_f32(w[j][2 * h], dc, l0, h0);     // k0 k2 | 256 * (k1 k3)
                decode_int8_f32(w[j][2 * h + 1], dc, l1, h1); // k4 k6 | 256 * (k5 k7)
                lo[0] = l0[0]; lo[1] = l0[1]; lo[2] = l1[0]; lo[3] = l1[1];
                hi[0] = h0[0]; hi[1] = h0[1]; hi[2] = h1[0]; hi[3] = h1[1];
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                plo[j][m] = __builtin_fmaf(lo[0], xa[m].x, plo[j][m]);
                phi[j][m] = __builtin_fmaf(hi[0], xa[m].y, phi[j][m]);
                plo[j][m] = __builtin_fmaf(lo[1], xa[m].z, plo[j][m]);
                phi[j][m] = __builtin_fmaf(hi[1], xa[m].w, phi[j][m]);
                plo[j][m] = __builtin_fmaf(lo[2], xb[m].x, plo[j][m]);
                phi[j][m] = __builtin_fmaf(hi[2], xb[m].y, phi[j][m]);
                plo[j][m] = __builtin_fmaf(lo[3], xb[m].z, plo[j][m]);
                phi[j][m] = __builtin_fmaf(hi[3], xb[m].w, phi[j][m]);
            }
        }
    }
    constexpr float kHi = BITS == 4 ? 0.0625f : 0.00390625f;   // 1/16 or 1/256: exact
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
        for (int m = 0; m < MT; ++m)
            acc[j][m] = __builtin_fmaf(sc[j], __builtin_fmaf(phi[j][m], kHi, plo[j][m]), acc[j][m]);
}

// Unpack constants of the chunk form for MT activation rows.
template <int MT> struct ChunkConsts { using type = DecodeConsts; };
template <> struct ChunkConsts<2> { using type = DecodeF32Consts; };

template <int BITS, int MT, int J>
__device__ __forceinline__ void chunk_fma(const u4 (&w)[J], const uint8_t *const (&xp)[8], int xstride,
                                          const typename ChunkConsts<MT>::type &dc, const float (&sc)[J],
                                          float (&acc)[J][MT])
{
    if constexpr (MT == 1) chunk_fma_h<BITS, MT, J>(w, xp, xstride, dc, sc, acc);
    else chunk_fma_f<BITS, MT, J>(w, xp, xstride, dc, sc, acc);
}

// int5 chunk: the int4 arithmetic above with the codes decoded from the chunk's
// low nibbles and its 4 bytes of bit 4 (byte h covers codes 8h .. 8h+7).
template <int MT, int J>
__device__ __forceinline__ void chunk_fma5(const u4 (&w)[J], const uint32_t (&hb)[J], const uint8_t *const (&xp)[8],
                                           int xstride, const Decode5Consts &dc, const float (&sc)[J],
                                           float (&acc)[J][MT])
{
    float p0[J][MT], p1[J][MT];
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
        for (int m = 0; m < MT; ++m) { p0[j][m] = 0.0f; p1[j][m] = 0.0f; }
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        f4 xa[MT], xb[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            xa[m] = *reinterpret_cast<const f4 *>(xp[2 * h] + m * xstride);
            xb[m] = *reinterpret_cast<const f4 *>(xp[2 * h + 1] + m * xstride);
        }
#pragma unroll
        for (int j = 0; j < J; ++j) {
            h2 t0, t1, t2, t3;
            decode_int5(w[j][h], hb[j] >> (8 * h), dc, t0, t1, t2, t3);   // (k0,k4) (k1,k5) (k2,k6) (k3,k7)
            const float ft0x = code_f32<MT>(t0.x);
            const float ft0y = code_f32<MT>(t0.y);
            const float ft1x = code_f32<MT>(t1.x);
            const float ft1y = code_f32<MT>(t1.y);
            const float ft2x = code_f32<MT>(t2.x);
            const float ft2y = code_f32<MT>(t2.y);
            const float ft3x = code_f32<MT>(t3.x);
            const float ft3y = code_f32<MT>(t3.y);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                p0[j][m] = __builtin_fmaf(ft0x, xa[m].x, p0[j][m]);
                p1[j][m] = __builtin_fmaf(ft0y, xb[m].x, p1[j][m]);
                p0[j][m] = __builtin_fmaf(ft1x, xa[m].y, p0[j][m]);
                p1[j][m] = __builtin_fmaf(ft1y, xb[m].y, p1[j][m]);
                p0[j][m] = __builtin_fmaf(ft2x, xa[m].z, p0[j][m]);
                p1[j][m] = __builtin_fmaf(ft2y, xb[m].z, p1[j][m]);
                p0[j][m] = __builtin_fmaf(ft3x, xa[m].w, p0[j][m]);
                p1[j][m] = __builtin_fmaf(ft3y, xb[m].w, p1[j][m]);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[j][m] = __builtin_fmaf(sc[j], p0[j][m] + p1[j][m], acc[j][m]);
}

// The 8 x-piece pointers a lane reads for the chunk of block `blk` of a staged
// segment, in the order its codes use them (int8: the chunk's half of the
// block, pieces 4*half .. 4*half+3).
template <int BITS>
__device__ __forceinline__ void piece_ptrs(const uint8_t *xs, int blk, int half, const uint8_t *(&xp)[8])
{
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int p = BITS != 8 ? k : half * 4 + (k & 3);
        xp[k] = xs + xslot(blk, p) * 16;
    }
}

// Reduce acc over the G lanes of each row and store rows [r0, r0 + J) for
// activation rows [mg, mg + MT) (lane li stores the values whose index is li
// modulo G).
template <int MT, int J>
__device__ __forceinline__ void reduce_store(float (&acc)[J][MT], int G, int li, int64_t r0, int64_t N, int mg,
                                             int M, float *__restrict__ y)
{
    group_sums(reinterpret_cast<float (&)[J * MT]>(acc), G);
    const int mc = (M - mg) < MT ? (M - mg) : MT;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int64_t r = r0 + j;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int idx = j * MT + m;
            if ((idx & (G - 1)) == li && m < mc && r < N) store_global(y + (size_t)(mg + m) * N + r, acc[j][m]);
        }
    }
}

// Fast item form: G == 16 and K % 256 == 0. The row is walked in CPL/S full
// segments of S chunks per lane; per segment the x blocks and the item's scales
// are copied into LDS, then the J*S code loads are issued, and the barrier
// waits for the copies only. All M <= MT activation rows in one pass.
template <int BITS, int MT, int J, int S>
__device__ __forceinline__ void gemv_item_fast(const float *__restrict__ x, int M, int K, int64_t N,
                                               const uint8_t *__restrict__ q, const uint16_t *__restrict__ s,
                                               float *__restrict__ y, int64_t row0, int CPL,
                                               uint8_t *__restrict__ lds)
{
    constexpr int G = 16, CPB = BITS / 4;
    constexpr int RW = kWave / G;
    constexpr int IROWS = kGemvWaves * RW * J;
    constexpr int NB = S * G / CPB;            // blocks per segment (a multiple of 8)
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & (G - 1);
    const int lrow0 = wave * RW * J + (lane >> 4) * J;
    const int C = K >> 5;
    const uint32_t qrow = (uint32_t)K * BITS / 8;     // bytes per row of codes
    const int nseg = CPL / S;
    typename ChunkConsts<MT>::type dc;
    if constexpr (BITS != 5) dc = ChunkConsts<MT>::type::make();
    Decode5Consts dc5;
    if constexpr (BITS == 5) dc5 = Decode5Consts::make();
    constexpr int NL = BITS == 5 ? 2 * J * S : J * S;   // loads per segment (int5: + bit-4 dwords)
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(q, (uint64_t)N * qrow);   // N * qrow < 2^32 (host check)
    uint8_t *xs = lds;                                                      // [MT][NB][8] pieces
    uint16_t *ss = reinterpret_cast<uint16_t *>(lds + MT * NB * 128);       // [IROWS][NB]
    uint32_t rowq[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        int64_t r = row0 + lrow0 + j;
        r = r < N ? r : N - 1;                 // rows past the end reload the last row
        rowq[j] = (uint32_t)r * qrow;
    }

    u4 w[J][S];
    uint32_t hw[J][S];                          // int5: the chunks' bit-4 dwords
    float acc[J][MT];
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[j][m] = 0.0f;
    {
        for (int seg = 0; seg < nseg; ++seg) {
            const int b0 = seg * NB;
            if (seg > 0) copies_barrier<0>();                          // earlier readers of LDS are done
            // the item's scales for the segment: IROWS rows of NB binary16 values
            copy_pieces(IROWS * NB / 8, reinterpret_cast<uint8_t *>(ss), wave, lane, [&](int pc) {
                const int r = pc / (NB / 8);
                const int k8 = pc - r * (NB / 8);
                int64_t row = row0 + r;
                row = row < N ? row : N - 1;
                return reinterpret_cast<const uint8_t *>(s + (size_t)row * C + b0 + k8 * 8);
            });
            stage_x<MT>(x, M, K, 0, b0, NB, xs, wave, lane);
#pragma unroll
            for (int c = 0; c < S; ++c)
#pragma unroll
                for (int j = 0; j < J; ++j)
                    w[j][c] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(
                                                         qr, rowq[j] + (uint32_t)((seg * S + c) * G + li) * 16,
                                                         0, kNonTemporal));
            if constexpr (BITS == 5) {
#pragma unroll
                for (int c = 0; c < S; ++c)
#pragma unroll
                    for (int j = 0; j < J; ++j)
                        hw[j][c] = __builtin_amdgcn_raw_buffer_load_b32(
                            qr, rowq[j] + (uint32_t)K / 2 + (uint32_t)((seg * S + c) * G + li) * 4, 0, kNonTemporal);
            }
            copies_barrier<NL>();                                        // codes stay in flight
            // Lane li reads block blk(c) = c * 16 / CPB + blk0 of the segment; the
            // swizzle of its pieces depends on li only (int4) or on li and the parity
            // of c (int8), so the piece pointers are set once and each chunk adds a
            // constant: the LDS reads take immediate offsets.
            const int blk0 = li / CPB;
            const uint8_t *xpe[8], *xpo[8];
            piece_ptrs<BITS>(xs, blk0, li & 1, xpe);
            if (BITS == 8) piece_ptrs<BITS>(xs, blk0 + 8, li & 1, xpo);
#pragma unroll
            for (int c = 0; c < S; ++c) {
                const int blk = c * G / CPB + blk0;                      // block within the segment
                const int cofs = (BITS != 8 ? c : (c & ~1)) * (G / CPB) * 128;
                const uint8_t *xp[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) xp[k] = ((BITS == 8 && (c & 1)) ? xpo[k] : xpe[k]) + cofs;
                float sc[J];
                u4 wc[J];
                uint32_t hc[J];
#pragma unroll
                for (int j = 0; j < J; ++j) {
                    sc[j] = (float)__builtin_bit_cast(_Float16, ss[(lrow0 + j) * NB + blk]);
                    wc[j] = w[j][c];
                    hc[j] = hw[j][c];
                }
                if constexpr (BITS == 5) chunk_fma5<MT, J>(wc, hc, xp, NB * 128, dc5, sc, acc);
                else chunk_fma<BITS, MT, J>(wc, xp, NB * 128, dc, sc, acc);
                __builtin_amdgcn_sched_barrier(0);   // keep each chunk's work together (bounds live registers)
            }
        }
        reduce_store<MT, J>(acc, G, li, row0 + lrow0, N, 0, M, y);
    }
}

// General item form (any K % 32 == 0): one row per lane, chunk by chunk. x is
// staged per segment of up to kGemvGenBlocks blocks; scales are read directly.
template <int BITS, int MT>
__device__ __forceinline__ void gemv_item_general(const float *__restrict__ x, int M, int K, int64_t N,
                                                  const uint8_t *__restrict__ q,
                                                  const uint16_t *__restrict__ s, float *__restrict__ y,
                                                  int64_t row0, const GemvGeom &g, uint8_t *__restrict__ lds)
{
    constexpr int CPB = BITS / 4;
    const int G = g.G;
    const int lg = __builtin_ctz(G);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & (G - 1);
    const int lrow = wave * (kWave >> lg) + (lane >> lg);
    const int C = K >> 5;
    const int CC = C * CPB;
    const uint32_t qrow = (uint32_t)K * BITS / 8;
    const uint32_t hoff = (uint32_t)K / 2;      // int5: offset of the bit-4 plane in a row
    typename ChunkConsts<MT>::type dc;
    if constexpr (BITS != 5) dc = ChunkConsts<MT>::type::make();
    Decode5Consts dc5;
    if constexpr (BITS == 5) dc5 = Decode5Consts::make();
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(q, (uint64_t)N * qrow);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(s, (uint64_t)N * C * 2);
    int64_t r = row0 + lrow;
    r = r < N ? r : N - 1;
    const uint32_t rq = (uint32_t)r * qrow, rs = (uint32_t)r * (uint32_t)C * 2;
    const int seg_chunks = g.nb * CPB;         // chunks of a row per segment (x blocks staged at once)
    {
        float acc[1][MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[0][m] = 0.0f;
        for (int c0 = 0; c0 < CC; c0 += seg_chunks) {
            const int b0 = c0 / CPB;
            const int nbs = ((CC - c0) < seg_chunks ? (CC - c0) : seg_chunks) / CPB;
            if (c0 > 0) copies_barrier<0>();
            stage_x<MT>(x, M, K, 0, b0, nbs, lds, wave, lane);
            copies_barrier<0>();
#pragma unroll 1
            for (int ch = c0 + li; ch < c0 + nbs * CPB; ch += G) {
                u4 wc[1];
                wc[0] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(qr, rq + (uint32_t)ch * 16, 0,
                                                                                     kNonTemporal));
                float sc[1];
                sc[0] = (float)__builtin_bit_cast(
                    _Float16, (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(sr, rs + (uint32_t)(ch / CPB) * 2, 0, 0));
                const uint8_t *xp[8];
                piece_ptrs<BITS>(lds, ch / CPB - b0, ch & 1, xp);
                if constexpr (BITS == 5) {
                    const uint32_t hb[1] = {
                        (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(qr, rq + hoff + (uint32_t)ch * 4, 0, kNonTemporal)};
                    chunk_fma5<MT, 1>(wc, hb, xp, nbs * 128, dc5, sc, acc);
                } else {
                    chunk_fma<BITS, MT, 1>(wc, xp, nbs * 128, dc, sc, acc);
                }
            }
        }
        reduce_store<MT, 1>(acc, G, li, row0 + lrow, N, 0, M, y);
    }
}

template <int BITS, int MT, int J, int S>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(const float *__restrict__ x, int M, int K, int64_t N,
                                                           const uint8_t *__restrict__ q,
                                                           const uint16_t *__restrict__ s,
                                                           float *__restrict__ y)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const GemvGeom g = gemv_geom(K, BITS, N, false);
    const int64_t row0 = (int64_t)blockIdx.x * g.rows;
    if constexpr (S == 0) gemv_item_general<BITS, MT>(x, M, K, N, q, s, y, row0, g, lds);
    else gemv_item_fast<BITS, MT, J, S>(x, M, K, N, q, s, y, row0, g.CPL, lds);
}

// Grouped launch: workgroup b computes item b - tile_begin of the last table
// entry whose tile_begin <= b.
template <int BITS, int MT>
__device__ __forceinline__ void grouped_item(const wq_desc &d, int M, const uint8_t *__restrict__ q,
                                             const uint16_t *__restrict__ s, int64_t item, uint8_t *lds)
{
    const int K = (int)d.K;
    const GemvGeom g = gemv_geom(K, BITS, d.N, true);
    const int64_t row0 = item * g.rows;
    // the shapes gemv_geom gives a grouped launch
    if constexpr (BITS == 5) {
        if (g.kind == kGemvJ2S2) gemv_item_fast<BITS, MT, 2, 2>(d.x, M, K, d.N, q, s, d.y, row0, g.CPL, lds);
        else gemv_item_general<BITS, MT>(d.x, M, K, d.N, q, s, d.y, row0, g, lds);
    } else {
        if (g.kind == kGemvJ4S2) gemv_item_fast<BITS, MT, 4, 2>(d.x, M, K, d.N, q, s, d.y, row0, g.CPL, lds);
        else gemv_item_general<BITS, MT>(d.x, M, K, d.N, q, s, d.y, row0, g, lds);
    }
}

// Wavefronts per SIMD the grouped kernel is compiled for: the kernel holds every
// item form, and without a bound its registers follow the largest of them.
template <int MT>
constexpr int grouped_waves_per_simd() { return MT == 1 ? 5 : 4; }

template <int MT>
__global__ __launch_bounds__(kGemvThreads, (grouped_waves_per_simd<MT>())) void gemv_grouped_kernel(const uint8_t *__restrict__ base,
                                                                   const wq_desc *__restrict__ table,
                                                                   int count, int M)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int64_t item = blockIdx.x;
    int lo = 0, hi = count - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (table[mid].tile_begin <= item) lo = mid; else hi = mid - 1;
    }
    const wq_desc d = table[lo];
    const uint8_t *q = base + d.q_off;
    const uint16_t *s = reinterpret_cast<const uint16_t *>(base + d.s_off);
    if (d.bits == 4) grouped_item<4, MT>(d, M, q, s, item - d.tile_begin, lds);
    else if (d.bits == 5) grouped_item<5, MT>(d, M, q, s, item - d.tile_begin, lds);
    else grouped_item<8, MT>(d, M, q, s, item - d.tile_begin, lds);
}

template <int BITS, int MT, int J, int S>
hipError_t launch_kind(const float *x, int64_t M, int64_t K, int64_t N, const void *q, const uint16_t *s,
                       float *y, const GemvGeom &g, hipStream_t stream)
{
    const int64_t items = (N + g.rows - 1) / g.rows;
    gemv_kernel<BITS, MT, J, S><<<(unsigned)items, kGemvThreads, gemv_lds_bytes(MT, g), stream>>>(
        x, (int)M, (int)K, N, (const uint8_t *)q, s, y);
    return hipGetLastError();
}

template <int BITS, int MT>
hipError_t launch_gemv_mt(const float *x, int64_t M, int64_t K, int64_t N, const void *q,
                          const uint16_t *s, float *y, hipStream_t stream)
{
    const GemvGeom g = gemv_geom(K, BITS, N, false);
    switch (g.kind) {
    case kGemvJ4S2: return launch_kind<BITS, MT, BITS == 5 ? 2 : 4, 2>(x, M, K, N, q, s, y, g, stream);
    case kGemvJ2S2: return launch_kind<BITS, MT, 2, 2>(x, M, K, N, q, s, y, g, stream);
    case kGemvJ1S2: return launch_kind<BITS, MT, 1, 2>(x, M, K, N, q, s, y, g, stream);
    default: return launch_kind<BITS, MT, 1, 0>(x, M, K, N, q, s, y, g, stream);
    }
}

template <int BITS>
hipError_t launch_gemv_bits(const float *x, int64_t M, int64_t K, int64_t N, const void *q,
                            const uint16_t *s, float *y, hipStream_t stream)
{
    if (M == 1) return launch_gemv_mt<BITS, 1>(x, M, K, N, q, s, y, stream);
    return launch_gemv_mt<BITS, 2>(x, M, K, N, q, s, y, stream);
}

template <int MT>
hipError_t launch_grouped_mt(const void *base, const wq_desc *table, int count, int64_t items, int64_t M,
                             hipStream_t stream)
{
    gemv_grouped_kernel<MT><<<(unsigned)items, kGemvThreads, gemv_lds_bytes_max(MT), stream>>>(
        (const uint8_t *)base, table, count, (int)M);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const float *x, int64_t M, int64_t K, int64_t N, int bits, const void *q,
                       const uint16_t *scales, float *y, hipStream_t stream)
{
    if (M < 1 || M > kGemvMaxMT) return hipErrorInvalidValue;   // 3 <= M goes to the matrix-core kernel
    if (bits == 4) return launch_gemv_bits<4>(x, M, K, N, q, scales, y, stream);
    if (bits == 5) return launch_gemv_bits<5>(x, M, K, N, q, scales, y, stream);
    return launch_gemv_bits<8>(x, M, K, N, q, scales, y, stream);
}

hipError_t launch_gemv_grouped(const void *base, const wq_desc *table_dev, int count,
                               int64_t total_items, int64_t M, hipStream_t stream)
{
    if (M < 1 || M > kGemvMaxMT) return hipErrorInvalidValue;
    if (M == 1) return launch_grouped_mt<1>(base, table_dev, count, total_items, M, stream);
    return launch_grouped_mt<2>(base, table_dev, count, total_items, M, stream);
}

}  // namespace wq
