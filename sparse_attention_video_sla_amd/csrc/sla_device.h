// sla_device.h -- device helpers shared by the gfx950 kernels of libsla.
//
// MFMA fragment convention used by every kernel (CDNA3/CDNA4 32x32 layouts):
//   v_mfma_f32_32x32x16_{bf16,f16}: lane l supplies A[m = l%32][k = 8*(l/32) + e] and
//   B[k = 8*(l/32) + e][n = l%32] for e = 0..7; the 16 accumulator registers r of
//   lane l hold D[row = 8*(r/4) + 4*(l/32) + r%4][col = l%32].
// A float "fragment" is the same 8 k-slots per lane fed to eight
// v_mfma_f32_32x32x2f32 (instruction e uses slot e), which yields the same
// 32x32 sum over 16 k values and the same accumulator layout.
//
// When the B operand of a product is taken from the accumulator of a previous
// one (P^T after softmax, a projected tile), lane (n, h) holds the rows
// {4h..4h+3, 8+4h..8+4h+3} of each 16-row group.  Any k order is valid as long
// as A and B agree, so such products read A with that same permutation
// ("permuted k"): slot e <-> k = 16s + (e < 4 ? 4h + e : 8 + 4h + e - 4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sla {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename E> struct V8;
template <> struct V8<bf16> { typedef bf16 type __attribute__((ext_vector_type(8))); };
template <> struct V8<f16> { typedef f16 type __attribute__((ext_vector_type(8))); };
template <> struct V8<float> { typedef float type __attribute__((ext_vector_type(8))); };
template <typename E> using v8 = typename V8<E>::type;

template <typename E> struct V4;
template <> struct V4<bf16> { typedef bf16 type __attribute__((ext_vector_type(4))); };
template <> struct V4<f16> { typedef f16 type __attribute__((ext_vector_type(4))); };
template <> struct V4<float> { typedef float type __attribute__((ext_vector_type(4))); };
template <typename E> using v4 = typename V4<E>::type;

// ---------------------------------------------------------------- MFMA wrappers
__device__ __forceinline__ void mma16(f32x16 &acc, const v8<bf16> &a, const v8<bf16> &b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x16 &acc, const v8<f16> &a, const v8<f16> &b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x16 &acc, const v8<float> &a, const v8<float> &b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], acc, 0, 0, 0);
}

// ---------------------------------------------------------------- conversions
template <typename E> __device__ __forceinline__ E from_f32(float x);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ f16 from_f32<f16>(float x) { return (f16)x; }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

template <typename E> __device__ __forceinline__ float to_f32(E x) { return (float)x; }

template <typename E, typename Src>
__device__ __forceinline__ v8<E> cvt8(const Src &x) {
    v8<E> r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = from_f32<E>((float)x[e]);
    return r;
}

template <typename E> __device__ __forceinline__ v8<E> zero8() {
    v8<E> r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = from_f32<E>(0.f);
    return r;
}

// ---------------------------------------------------------------- 16-byte chunks
struct alignas(16) Chunk { uint32_t w[4]; };

__device__ __forceinline__ Chunk ld_chunk(const void *p) { return *reinterpret_cast<const Chunk *>(p); }
__device__ __forceinline__ void st_chunk(void *p, const Chunk &c) { *reinterpret_cast<Chunk *>(p) = c; }
__device__ __forceinline__ Chunk zero_chunk() { Chunk c; c.w[0] = c.w[1] = c.w[2] = c.w[3] = 0u; return c; }

// 8 consecutive elements (16 or 32 bytes, 16-byte aligned)
template <typename E> __device__ __forceinline__ v8<E> ld8(const E *p) {
    v8<E> r;
    __builtin_memcpy(&r, p, sizeof(r));
    return r;
}
template <typename E> __device__ __forceinline__ v4<E> ld4(const E *p) {
    v4<E> r;
    __builtin_memcpy(&r, p, sizeof(r));
    return r;
}
// 8 elements from two 4-element runs (the permuted-k A operand)
template <typename E> __device__ __forceinline__ v8<E> ld4x2(const E *p0, const E *p1) {
    v4<E> a = ld4(p0), b = ld4(p1);
    v8<E> r;
#pragma unroll
    for (int e = 0; e < 4; ++e) { r[e] = a[e]; r[e + 4] = b[e]; }
    return r;
}

// ---------------------------------------------------------------- buffer loads
// Raw buffer loads through a 128-bit resource: the hardware checks each
// access against num_records and returns zeros past the end, so a tile that
// runs over the end of a head needs no per-lane guard.  The resource covers
// one head, so a ragged last block reads zeros, never the next head.  Every
// offset that must be checked goes into the per-lane offset (voff): callers
// pass 0 as the scalar offset.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ Chunk buf_ld(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    Chunk c;
    c.w[0] = v[0]; c.w[1] = v[1]; c.w[2] = v[2]; c.w[3] = v[3];
    return c;
}
// 16 bytes to LDS at an address that is only 8-byte aligned
__device__ __forceinline__ void st_chunk8(void *p, const Chunk &c) {
    uint32_t *q = reinterpret_cast<uint32_t *>(p);
    *reinterpret_cast<uint64_t *>(q) = (uint64_t)c.w[0] | ((uint64_t)c.w[1] << 32);
    *reinterpret_cast<uint64_t *>(q + 2) = (uint64_t)c.w[2] | ((uint64_t)c.w[3] << 32);
}

// ---------------------------------------------------------------- LDS transposing reads
// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, lane L supplies
// the address of 4 consecutive 16-bit elements (row L of a 16 x 4 block) and
// lane i receives the elements (4e + i/4, i%4), e = 0..3.  Pointing lane L at
// T[k0 + L/4][n0 + 4*(L%4)] of a row-major LDS tile T therefore hands lane i
// the column run T[k0 + e][n0 + i], e = 0..3: four consecutive k-values of one
// MFMA row/column, read from a tile stored with that row/column contiguous.
// (k0, n0) are the same for the 16 lanes of a group.  32-bit data has no
// transposing read; it takes the same values with four scalar reads.
template <typename E> __device__ __forceinline__ v4<E> lds_tr_raw(const E *p);
template <> __device__ __forceinline__ v4<bf16> lds_tr_raw<bf16>(const bf16 *p) {
    typedef __bf16 raw4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
    const raw4 r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) raw4 *)(p));
    v4<bf16> o;
    __builtin_memcpy(&o, &r, sizeof(o));
    return o;
}
template <> __device__ __forceinline__ v4<f16> lds_tr_raw<f16>(const f16 *p) {
    typedef __fp16 raw4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
    const raw4 r = __builtin_amdgcn_ds_read_tr16_b64_v4f16((__attribute__((address_space(3))) raw4 *)(p));
    v4<f16> o;
    __builtin_memcpy(&o, &r, sizeof(o));
    return o;
}
// The column run T[k0 .. k0+3][n0 + lane%16] of a row-major LDS tile (stride in elements).
template <typename E>
__device__ __forceinline__ v4<E> lds_col4(const E *tile, int stride, int k0, int n0, int lane) {
    const int L = lane & 15;
    if constexpr (sizeof(E) == 2) {
        return lds_tr_raw<E>(tile + (k0 + (L >> 2)) * stride + n0 + 4 * (L & 3));
    } else {
        v4<E> o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = tile[(k0 + e) * stride + n0 + L];
        return o;
    }
}
template <typename E> __device__ __forceinline__ v8<E> cat8(const v4<E> &a, const v4<E> &b) {
    v8<E> r;
#pragma unroll
    for (int e = 0; e < 4; ++e) { r[e] = a[e]; r[e + 4] = b[e]; }
    return r;
}

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ float shfl_xor32(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace sla
