// tile_common.h -- small device helpers shared by the attention kernels
// (forward and backward): workgroup barrier on LDS traffic, NaN-propagating
// max, cross-half reductions, loads straight into LDS, and the swizzle of
// K-layout tiles with the offsets of their row and transposing reads.
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


// offset of the first token of the block's part 1 (a frame boundary inside
// the block), 64 when the block lies in one frame; frames of fp >= 64 tokens
__device__ __forceinline__ int frame_split(int blk, int fp) {
    const int start = 64 * blk;
    const int bnd = (start / fp + 1) * fp - start;
    return bnd < 64 ? bnd : 64;
}

// swizzle of the K tile: chunk c of row r sits at chunk c ^ kswz(r). Row
// reads (a lane per row, 16 bytes each) touch every bank once per 16 lanes,
// and the transposing reads of tr_offsets every bank exactly twice: the two
// low row bits pick the high chunk bits and the next two the low ones
template <int D> __device__ __forceinline__ int kswz(int r) {
    return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3))
                    : (((r >> 1) & 1) | (((r >> 3) & 1) << 1) | (((r >> 2) & 1) << 2));
}

// swizzle of a tile that is only read transposed (V): chunk c of row r sits
// at chunk c ^ vswz(r), so that the 8 rows x 4 chunks of one transposing read
// (see tr_offsets) land on every bank exactly twice
template <int D> __device__ __forceinline__ int vswz(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

// 1 KB block u of this wave's share of a 64 x D tile: source offset of its
// lane in the K layout (rows of 2D bytes, 16-byte chunks swizzled by kswz,
// or by vswz with V = true)
template <int D, bool V = false> __device__ __forceinline__ uint32_t off_klayout(int byte) {
    const int r = byte / (2 * D), pk = (byte % (2 * D)) / 16;
    return (uint32_t)(r * 2 * D + (pk ^ (V ? vswz<D>(r) : kswz<D>(r))) * 16);
}
// Transposing reads of a K-layout tile as the A operand [channel][row] of
// rows 32 half .. +31, rows in the accumulator order of a 32 x 32 tile: k
// slot e of step ks is row 16 ks + (e < 4 ? 4 hh + e : 8 + 4 hh + e - 4).
// Lane L of a 16-lane group points at row 8 x + 4 hh + L / 4 of the step and
// channels 32 ct + 16 (group & 1) + 4 (L % 4) .. +3, found through the
// row's chunk swizzle (which only depends on the row modulo 16).
template <int D, bool V = false> __device__ __forceinline__ void tr_offsets(int lane, int (&toff)[D / 32][2]) {
    const int grp = lane >> 4, L = lane & 15, hh = lane >> 5;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
        const int rr = 8 * x + 4 * hh + (L >> 2);
        const int sw = V ? vswz<D>(rr) : kswz<D>(rr);
#pragma unroll
        for (int ct = 0; ct < D / 32; ++ct)
            toff[ct][x] = rr * D + ((4 * ct + 2 * (grp & 1) + ((L & 3) >> 1)) ^ sw) * 8 + 4 * (L & 1);
    }
}

template <typename T, int D>
__device__ __forceinline__ void read_tr(const T *tile, int half, const int (&toff)[D / 32][2], v8<T> (&a)[D / 32][2]) {
#pragma unroll
    for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const T *base = tile + (32 * half + 16 * ks) * D;
            a[ct][ks] = cat8<T>(lds_tr_raw<T>(base + toff[ct][0]), lds_tr_raw<T>(base + toff[ct][1]));
        }
}

}  // namespace
}  // namespace sla
