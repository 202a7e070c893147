// tile_common.h -- small device helpers shared by the attention kernels
// (forward and backward): workgroup barrier on LDS traffic, NaN-propagating
// max, cross-half reductions, loads straight into LDS, and the swizzle of
// K-layout tiles.
#pragma once
#include "sla_device.h"

namespace sla {
namespace {

// Workgroup barrier that waits for this wave's LDS (and scalar) traffic
// only: global loads issued before it stay in flight.  The wait goes through
// the builtin so that the compiler's own wait placement knows about it; the
// memory clobber keeps the compiler from moving memory accesses across the
// barrier.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);                  // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
}

// maximum that propagates NaN instead of quieting it (v_maximum3_f32 on
// gfx950): it takes MFMA results without canonicalising them first
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// max and sum across the two 32-lane halves of the wave
__device__ __forceinline__ float half_swap_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}



// 16 bytes per lane from a buffer into LDS at lds + 16 * lane (lds is wave-uniform)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, const void *lds, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)


// swizzle of the K tile: chunk c of row r sits at chunk c ^ kswz(r)
template <int D> __device__ __forceinline__ int kswz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }

}  // namespace
}  // namespace sla
