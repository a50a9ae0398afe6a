// wq_device.h -- device-side helpers shared by the kernels (included by the
// .hip sources only; the host-side ABI layer needs none of it).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wq {

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

}  // namespace wq
