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
// A row of K values is C = K/32 chunks; one chunk is one quantization block
// (16 bytes of int4 codes or 32 bytes of int8 codes). G lanes of a wavefront
// share a row: G is the largest power of two <= 64 dividing C, so each lane
// owns C/G chunks of the row (chunks li, li+G, li+2G, ... : one "round" each)
// and a wavefront covers 64/G rows per pass. A tile is J passes of the four
// wavefronts: every lane keeps J rows (J x 16 or 32 bytes) in flight.
constexpr int kGemvThreads = 256;   // 4 wavefronts per workgroup
constexpr int kGemvWaves = kGemvThreads / kWave;
constexpr int kGemvMaxMT = 4;       // activation rows per pass over the weights
constexpr int kGemvChunkPad = 36;   // floats per staged 32-float x chunk (bank spread)
constexpr int kGemvLdsFloatsPerMT = 4608;   // x staging budget: 18 KiB per activation row
constexpr int kGroupedTilesPerWg = 4;       // consecutive tiles of one tensor per workgroup

__host__ __device__ inline int gemv_group(int64_t K)
{
    const int64_t C = K / kBlock;
    int g = 64;
    while (C % g) g >>= 1;
    return g;
}

// Activation rows staged at once (m-group size).
__host__ __device__ inline int gemv_mt(int64_t M) { return M < kGemvMaxMT ? (int)M : kGemvMaxMT; }

// Rows in flight per lane in the grouped launch: 128 B of codes per lane for
// MT <= 2, 64 B above (register budget).
__host__ __device__ inline int gemv_grouped_j(int bits, int MT)
{
    return bits == 4 ? (MT <= 2 ? 8 : 4) : (MT <= 2 ? 4 : 2);
}

__host__ __device__ inline int64_t gemv_rows_per_tile(int64_t K, int J)
{
    return (int64_t)kGemvWaves * (kWave / gemv_group(K)) * J;
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS operations,
// then s_barrier. Unlike __syncthreads() it does not wait for outstanding global
// loads, so prefetched registers stay in flight across the barrier.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);        // lgkmcnt(0); vmcnt and expcnt untouched
    __builtin_amdgcn_s_barrier();
}

// Raw buffer descriptor over [p, p + bytes) (bytes < 2^32). Dword 3 selects
// 32-bit untyped data (raw buffer loads ignore the format otherwise).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)(uint32_t)bytes, 0x00020000);
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
hipError_t launch_gemm(const float *x, int64_t M, int64_t K, int64_t N, int bits,
                       const void *q, const uint16_t *scales, float *y, hipStream_t stream);

}  // namespace wq

static_assert(sizeof(wq_desc) == WQ_TABLE_ALIGN, "tensor-table entries are 64 bytes");
