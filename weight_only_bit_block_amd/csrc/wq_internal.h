// wq_internal.h -- shared geometry and launcher declarations of the HIP library.
// Everything here is product code for gfx950; nothing is shared with the CPU
// oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/wq.h"

namespace wq {

constexpr int kBlock = 32;          // quantization block along K
constexpr int kWave = 64;           // gfx950 wavefront size

// ---------------------------------------------------------------- GEMV geometry
// A row of K values is C = K/32 chunks; one chunk is one quantization block
// (16 bytes of int4 codes or 32 bytes of int8 codes). G lanes of a wavefront
// share a row: G is the largest power of two <= 64 dividing C, so each lane
// owns C/G chunks of the row (chunks li, li+G, li+2G, ...) and a wavefront
// covers 64/G rows per pass. Each lane carries J rows ("J row passes").
constexpr int kGemvThreads = 256;   // 4 wavefronts per workgroup
constexpr int kGemvWaves = kGemvThreads / kWave;
constexpr int kGemvMaxMT = 4;       // activation rows per pass over the weights
constexpr int kGemvLdsBytes = 64 * 1024;
constexpr int kGemvChunkPad = 36;   // floats per staged 32-float x chunk (bank spread)

__host__ __device__ inline int gemv_group(int64_t K)
{
    const int64_t C = K / kBlock;
    int g = 64;
    while (C % g) g >>= 1;
    return g;
}

__host__ __device__ inline int64_t gemv_rows_per_tile(int64_t K, int J)
{
    return (int64_t)kGemvWaves * (kWave / gemv_group(K)) * J;
}

// Rows of x staged in LDS at once, and rounds of chunks per staged segment.
__host__ __device__ inline int gemv_mt(int64_t M) { return M < kGemvMaxMT ? (int)M : kGemvMaxMT; }

// J used by the grouped launch for a given MT (fixed so that the host plan and
// the kernel agree).
__host__ __device__ inline int gemv_grouped_j(int MT) { return MT <= 2 ? 8 : 4; }

// ---------------------------------------------------------------- launchers
hipError_t launch_pack(const float *w, int64_t N, int64_t K, int bits, void *q,
                       uint16_t *scales, hipStream_t stream);
hipError_t launch_unpack(const void *q, int64_t N, int64_t K, int bits, int8_t *codes,
                         hipStream_t stream);
hipError_t launch_gemv(const float *x, int64_t M, int64_t K, int64_t N, int bits,
                       const void *q, const uint16_t *scales, float *y, hipStream_t stream);
hipError_t launch_gemv_grouped(const void *base, const wq_desc *table_dev, int count,
                               int64_t total_tiles, int64_t M, hipStream_t stream);
hipError_t launch_gemm(const float *x, int64_t M, int64_t K, int64_t N, int bits,
                       const void *q, const uint16_t *scales, float *y, hipStream_t stream);

}  // namespace wq

static_assert(sizeof(wq_desc) == WQ_TABLE_ALIGN, "tensor-table entries are 64 bytes");
