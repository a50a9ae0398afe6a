// wq_internal.h -- shared geometry and launcher declarations of the HIP library.
// Everything here is product code for gfx950; nothing is shared with the CPU
// oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wq.h"

namespace wq {

constexpr int kBlock = 32;          // quantization block along K
constexpr int kWave = 64;           // gfx950 wavefront size

// ---------------------------------------------------------------- GEMV geometry
// A row of K codes is read in chunks of 16 bytes: one quantization block of
// int4 codes, or half a block of int8 codes, CC = (K/32) * (bits/4) chunks per
// row. G lanes of a wavefront share a row (G the largest power of two <= 16
// dividing CC); lane li owns the chunks li, li+G, li+2G, ... (CPL = CC/G of
// them), so the lanes of a row read G*16 contiguous bytes per load. A
// workgroup item is IROWS = 4 * (64/G) * J consecutive rows of one tensor.
//
// int5 rows (the low-nibble plane, then the bit-4 plane) are read as int4
// chunks plus each chunk's 4 bytes of bit 4, in either form.
//
// Fast form (G == 16, K % 256 == 0 and an even CPL: every shape of the
// decoder): a lane owns J rows and holds S = 2 of its chunks per row in
// registers at a time; the row is walked in CPL/2 segments. General form (any
// K % 32 == 0): one row per lane, one chunk at a time.
//
// This kernel serves M <= 2 activation rows (the matrix-core kernel takes
// 3 <= M <= 16).
constexpr int kGemvThreads = 256;   // 4 wavefronts per workgroup
constexpr int kGemvWaves = kGemvThreads / kWave;
constexpr int kGemvMaxMT = 2;       // activation rows of the fp32-FMA kernel
constexpr int kGemvGenBlocks = 96;  // blocks of x staged per segment in the general form
constexpr int kNonTemporal = 2;     // cache policy of the weight loads: streamed once

enum GemvKind { kGemvJ4S2 = 0, kGemvJ2S2, kGemvJ1S2, kGemvGeneral };

struct GemvGeom {
    int G;           // lanes per row
    int CPL;         // chunks per lane per row
    int kind;        // GemvKind
    int J;           // rows per lane
    int S;           // chunks per lane per segment (fast form)
    int64_t rows;    // rows per item (workgroup)
    int nb;          // blocks of x (and, fast form, of scales) staged per segment
};

// Fast shapes take four rows per lane, so each staged x piece read from LDS
// serves four weight rows (measured 3-5% faster at M = 1 and 2 than two rows
// per lane, and 9% faster at M = 2 than one row per lane with longer
// segments); single launches with few items take one row per lane to spread
// over the chip. J and S never change the arithmetic of an output (it depends
// on K and bits only), so every shape and the grouped launch give the same
// bits.
__host__ __device__ inline GemvGeom gemv_geom(int64_t K, int bits, int64_t N, bool grouped)
{
    GemvGeom g;
    const int cpb = bits / 4;
    const int64_t C = K / kBlock;
    const int64_t CC = C * cpb;
    int G = 16;
    while (CC % G) G >>= 1;
    g.G = G;
    g.CPL = (int)(CC / G);
    g.J = 1;
    g.S = 1;
    g.kind = kGemvGeneral;
    if (G == 16 && K % 256 == 0 && g.CPL % 2 == 0) {
        // int5 holds a bit-4 dword per chunk besides the codes: two rows per lane
        const int jf = bits == 5 ? 2 : 4;
        const int64_t rows_f = (int64_t)kGemvWaves * 4 * jf;
        const bool few = !grouped && (N + rows_f - 1) / rows_f < 256;
        g.kind = few ? kGemvJ1S2 : (jf == 4 ? kGemvJ4S2 : kGemvJ2S2);
        g.J = few ? 1 : jf;
        g.S = 2;
    }
    g.rows = (int64_t)kGemvWaves * (kWave / G) * g.J;
    if (g.kind == kGemvGeneral) {
        g.nb = (int)(C < kGemvGenBlocks ? C : kGemvGenBlocks);
    } else {
        g.nb = g.S * 16 / cpb;
    }
    return g;
}

// Decode with 3..16 activation rows runs on the matrix cores (wq_mgemv.hip),
// where the fp32-FMA form is bound by its LDS reads of x: a work item is 128
// consecutive weight rows of one tensor.
constexpr int kMgemvRows = 128;
constexpr int kMgemvMinM = 3;
static_assert(kMgemvMinM == kGemvMaxMT + 1, "every M has one decode kernel");

// Rows per work item of a decode call with M activation rows.
__host__ __device__ inline int64_t decode_item_rows(int64_t K, int bits, int64_t N, bool grouped, int64_t M)
{
    return M >= kMgemvMinM ? (int64_t)kMgemvRows : gemv_geom(K, bits, N, grouped).rows;
}

// LDS of an item: MT staged x rows (128 bytes per block) and, in the fast form,
// the item's scales for one segment.
__host__ __device__ inline size_t gemv_lds_bytes(int MT, const GemvGeom &g)
{
    const size_t sc = g.kind == kGemvGeneral ? 0 : (size_t)g.rows * g.nb * 2;
    return (size_t)MT * g.nb * 128 + sc;
}
// Upper bound over every shape: nb <= 96 and rows * nb <= 32 * 96 in the fast form.
__host__ __device__ inline size_t gemv_lds_bytes_max(int MT) { return (size_t)MT * 96 * 128 + 32 * 96 * 2; }

// ---------------------------------------------------------------- prefill workspace
// The prefill GEMM rounds x to binary16 once per call (after a per-row
// power-of-two normalisation) into a workspace: the prepared x [M][K]
// (binary16), then the per-row factors 2^-e [M] (fp32), each region padded to
// 256 bytes. A grouped call holds one such slot per distinct (x, code order),
// at a multiple of 256 bytes (wq_desc.ws_slot, in 256-byte units).
constexpr uint64_t kGemmWsUnit = 256;
__host__ __device__ inline uint64_t gemm_ws_round(uint64_t b) { return (b + kGemmWsUnit - 1) / kGemmWsUnit * kGemmWsUnit; }
__host__ __device__ inline uint64_t gemm_ws_x16_bytes(int64_t M, int64_t K) { return gemm_ws_round((uint64_t)M * (uint64_t)K * 2); }
__host__ __device__ inline uint64_t gemm_ws_rinv_bytes(int64_t M) { return gemm_ws_round((uint64_t)M * 4); }
__host__ __device__ inline uint64_t gemm_ws_bytes(int64_t M, int64_t K) { return gemm_ws_x16_bytes(M, K) + gemm_ws_rinv_bytes(M); }

// Scratch of wq_gemm_noalloc: one per device, for the workspace above.
constexpr uint64_t kGemmNoAllocScratch = (uint64_t)32 << 20;
static_assert(kGemmNoAllocScratch == WQ_NOALLOC_SCRATCH_BYTES, "wq.h states the scratch size");

// ---------------------------------------------------------------- grouped prefill geometry
// A grouped prefill launch uses one tile shape for every tensor, chosen by M
// alone: BM-row x 128-column tiles, with the K loop of each tile split over S
// groups of 256 threads. Short prefills (M <= 128) take 64-row tiles split
// two ways; longer ones 128-row tiles, unsplit.
//
// Short prefills also split long K loops across workgroups, so that every
// work item covers at most about 1024 of K whatever the tensor's K: a tile of
// a tensor with K >= 2048 becomes P = min(K / 1024, 8) consecutive work items,
// item k covering stages [k NT / P, (k + 1) NT / P) of its NT stages. Items
// 0 .. P-2 leave their fp32 partial tile in the workspace and raise a flag;
// item P-1 (the highest index of the tile, so it waits only on workgroups
// dispatched before it) adds the partials in item order to its own, then
// scales and stores the tile: deterministic, and no read-modify-write atomics.
constexpr int kGemmTileN = 128;
constexpr int kGemmGroupAlign = 8;  // entries start at multiples of 8 items (one per XCD)
constexpr int64_t kGemmKSplitMaxM = 128;
__host__ __device__ inline int gemm_grouped_bm(int64_t M) { return M <= 128 ? 64 : 128; }
__host__ __device__ inline int gemm_grouped_split(int64_t M) { return gemm_grouped_bm(M) == 64 ? 2 : 1; }
__host__ __device__ inline int gemm_grouped_ksplit(int64_t M, int64_t K)
{
    if (M > kGemmKSplitMaxM) return 1;
    const int64_t p = K / 1024;
    return (int)(p < 1 ? 1 : p > 8 ? 8 : p);
}
__host__ __device__ inline int64_t gemm_grouped_items(int64_t M, int64_t N, int64_t K)
{
    const int bm = gemm_grouped_bm(M);
    return ((M + bm - 1) / bm) * ((N + kGemmTileN - 1) / kGemmTileN) * gemm_grouped_ksplit(M, K);
}
// Workspace header of a grouped prefill launch of `items` work items, before
// the prepared-x slots: one 32-bit flag per item (cleared by the preparation
// kernel of every call), then one fp32 partial tile per item.
__host__ __device__ inline uint64_t gemm_grouped_flag_bytes(int64_t M, int64_t items)
{
    return M > kGemmKSplitMaxM ? 0 : gemm_ws_round((uint64_t)items * 4);
}
__host__ __device__ inline uint64_t gemm_grouped_header_bytes(int64_t M, int64_t items)
{
    return M > kGemmKSplitMaxM ? 0
                               : gemm_grouped_flag_bytes(M, items) +
                                     (uint64_t)items * gemm_grouped_bm(M) * kGemmTileN * 4;
}

// ---------------------------------------------------------------- launchers
hipError_t launch_pack(const float *w, int64_t N, int64_t K, int bits, void *q,
                       uint16_t *scales, hipStream_t stream);
hipError_t launch_unpack(const void *q, int64_t N, int64_t K, int bits, int8_t *codes,
                         hipStream_t stream);
hipError_t launch_gemv(const float *x, int64_t M, int64_t K, int64_t N, int bits,
                       const void *q, const uint16_t *scales, float *y, hipStream_t stream);
hipError_t launch_gemv_grouped(const void *base, const wq_desc *table_dev, int count,
                               int64_t total_tiles, int64_t M, hipStream_t stream);
// Shapes that run on the skinny GEMM, which prepares x itself: launch_gemm
// then reads no workspace (ws may be null).
bool gemm_skinny(int64_t M, int64_t K, int64_t N, int bits);
// ws: gemm_ws_bytes(M, K) bytes (single call) or the planned workspace (grouped)
hipError_t launch_gemm(const float *x, int64_t M, int64_t K, int64_t N, int bits,
                       const void *q, const uint16_t *scales, float *y, void *ws, hipStream_t stream);
hipError_t launch_gemm_grouped(const void *base, const wq_desc *table_dev, int count,
                               int64_t total_tiles, int64_t M, void *ws, hipStream_t stream);
// Device address of this device's scratch of wq_gemm_noalloc (looked up once per device).
hipError_t gemm_noalloc_scratch(void **ptr);
hipError_t launch_mgemv(const float *x, int64_t M, int64_t K, int64_t N, int bits, const void *q,
                        const uint16_t *scales, float *y, hipStream_t stream);
hipError_t launch_mgemv_grouped(const void *base, const wq_desc *table_dev, int count, int64_t total_items,
                                int64_t M, hipStream_t stream);
hipError_t launch_embed(const int32_t *ids, int64_t n_ids, int64_t K, int64_t N, int bits,
                        const void *q, const uint16_t *scales, float *out, hipStream_t stream);

}  // namespace wq

static_assert(sizeof(wq_desc) == WQ_TABLE_ALIGN, "tensor-table entries are 64 bytes");
