// state.hip -- per-key-block linear-attention states (SLA article, section 3:
// linear attention over the marginal blocks computes phi(K)^T V first, with
// phi = softmax over the channels, section 5).
//
// One workgroup per key block j (64 tokens), D/32 waves; wave w owns output
// channels c in 32w..32w+31.
//   phi(k_t) = softmax over the d channels of each valid token (pad tokens 0).
//   The projection W of the linear branch is folded in here: the block state
//   is h'_j = phi(K_j)^T (V_j W^T), computed as V'_j = V_j W^T then
//   h'_j = phi(K_j)^T V'_j, both on MFMA.  The linear output is
//   phi(q) H / (phi(q).Z) with H a sum of block states, so applying W^T per
//   block is the same linear map as applying it to the output.
//   z_j = sum_t phi(k_t).
// Stored per block as one row of Lp values, scaled by 1/64 (exact) so that
// values stay within the range of the fp16 staging type:
//   [h'^T row-major (column c*d + a holds h'[a][c]), z (d), zero pad].
// Blocks past Nb up to Nbc (the next multiple of 64) are written as zero rows.
#include <algorithm>

#include "sla_device.h"
#include "sla_launch.h"

namespace sla {

// W in the state type, once per call (d x d)
template <typename S>
__global__ __launch_bounds__(256) void w_to_state_kernel(const float *__restrict__ w, S *__restrict__ ws, int n) {
    const int x = blockIdx.x * 256 + threadIdx.x;
    if (x < n) ws[x] = from_f32<S>(w[x]);
}

template <typename T, typename S, int D>
__global__ __launch_bounds__(2 * D) void state_kernel(const T *__restrict__ k, const T *__restrict__ v,
                                                      const S *__restrict__ w, int N, int Nb, int Nbc,
                                                      S *__restrict__ hs, int Lp) {
    constexpr int NT = 2 * D;
    constexpr int EPC = 16 / sizeof(T);      // input elements per 16-byte chunk
    constexpr int CPR = D / EPC;             // chunks per token row
    constexpr int NCH = 64 * CPR / NT;       // chunks per thread
    constexpr int SE = 16 / sizeof(S);
    constexpr int SSTR = D + SE;             // V row stride in LDS (state type)
    constexpr int PSTR = D + (sizeof(S) == 2 ? 16 : 4);   // phi row stride: 8 dwords mod 64 for transposing reads
    __shared__ __attribute__((aligned(16))) S Vs[64 * SSTR];
    __shared__ __attribute__((aligned(16))) S Ph[64 * PSTR];

    const long blk = blockIdx.x;             // bh * Nbc + j
    const int j = (int)(blk % Nbc);
    const long bh = blk / Nbc;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    S *hsb = hs + blk * (long)Lp;
    if (j >= Nb) {                           // padding block: a zero row
        for (int x = tid; x < Lp; x += NT) hsb[x] = from_f32<S>(0.f);
        return;
    }
    const int n = min(64, N - 64 * j);
    const T *kb = k + (bh * N + 64L * j) * D;
    const T *vb = v + (bh * N + 64L * j) * D;

    Chunk kc[NCH], vc[NCH];
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
        const int ch = tid + NT * u, row = ch / CPR, cc = ch % CPR;
        const bool ok = row < n;
        kc[u] = ok ? ld_chunk(kb + (long)row * D + cc * EPC) : zero_chunk();
        vc[u] = ok ? ld_chunk(vb + (long)row * D + cc * EPC) : zero_chunk();
    }

    // phi(K) per token row: the CPR threads of a row are CPR consecutive lanes.
    // phi and V go to LDS row-major in the state type.
    constexpr float LOG2E = 1.4426950408889634f;
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
        const int ch = tid + NT * u, row = ch / CPR, cc = ch % CPR;
        const T *x = reinterpret_cast<const T *>(&kc[u]);
        float xf[EPC];
        float mx = -__builtin_inff();
#pragma unroll
        for (int e = 0; e < EPC; ++e) { xf[e] = to_f32<T>(x[e]); mx = fmaxf(mx, xf[e]); }
#pragma unroll
        for (int off = 1; off < CPR; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) { xf[e] = fast_exp2((xf[e] - mx) * LOG2E); sum += xf[e]; }
#pragma unroll
        for (int off = 1; off < CPR; off <<= 1) sum += __shfl_xor(sum, off, 64);
        const float inv = (row < n) ? 1.f / sum : 0.f;
        S ph[EPC], vv[EPC];
        const T *y = reinterpret_cast<const T *>(&vc[u]);
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
            ph[e] = from_f32<S>(xf[e] * inv);
            vv[e] = from_f32<S>(to_f32<T>(y[e]));
        }
        __builtin_memcpy(&Ph[row * PSTR + cc * EPC], ph, sizeof(ph));
        __builtin_memcpy(&Vs[row * SSTR + cc * EPC], vv, sizeof(vv));
    }
    __syncthreads();

    // V'[t][c] = sum_b V[t][b] W[c][b]: M = t (2 tiles), N = c (this wave's tile), K = b
    f32x16 accv[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) accv[mt][r] = 0.f;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        const v8<S> bw = ld8<S>(w + (long)(32 * wave + l32) * D + 16 * s + 8 * hh);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const v8<S> a = ld8<S>(&Vs[(32 * mt + l32) * SSTR + 16 * s + 8 * hh]);
            mma16(accv[mt], a, bw);
        }
    }
    // h'[a][c] = sum_t phi[t][a] V'[t][c]: M = a, N = c (this wave's tile), K = t.
    // V' is the B operand straight from its accumulator, so t runs in the
    // accumulator's permuted order; the phi^T operand takes the same t runs as
    // columns of the row-major phi tile (transposing reads).
    const int grp = lane >> 4;
    f32x16 acch[D / 32];
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acch[mt][r] = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        v8<S> b;
#pragma unroll
        for (int e = 0; e < 8; ++e) b[e] = from_f32<S>(accv[s >> 1][8 * (s & 1) + e]);
        const int k0 = 16 * s + 4 * (grp >> 1);
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) {
            const int n0 = 32 * mt + 16 * (grp & 1);
            mma16(acch[mt], cat8<S>(lds_col4<S>(Ph, PSTR, k0, n0, lane), lds_col4<S>(Ph, PSTR, k0 + 8, n0, lane)), b);
        }
    }

    // lane (c, h) holds h'[a][c] for a = 32mt + 8g + 4h + 0..3: four consecutive
    // columns c*d + a of the state row
    const float scale = 1.f / 64.f;
    const int c = 32 * wave + l32;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            v4<S> y;
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = from_f32<S>(acch[mt][4 * g + e] * scale);
            __builtin_memcpy(hsb + c * D + 32 * mt + 8 * g + 4 * hh, &y, sizeof(y));
        }
    if (tid < D) {
        float z = 0.f;
        for (int t = 0; t < 64; ++t) z += to_f32<S>(Ph[t * PSTR + tid]);
        hsb[D * D + tid] = from_f32<S>(z * scale);
    }
    for (int x = D * D + D + tid; x < Lp; x += NT) hsb[x] = from_f32<S>(0.f);
}

// workgroup barrier that leaves global loads in flight (the prefetched block)
// Reductions over aligned groups of W = 8 or 16 lanes (a token row's
// channel chunks) with DPP moves instead of LDS permutes: after the two quad
// steps every lane of a quad holds the quad's result; a mirror inside each
// half row (row) then pairs every lane with one of the other quad (half).
__device__ __forceinline__ float dpp_f(float x, int ctrl_sel) {
    int r;
    switch (ctrl_sel) {                      // the control word must be a constant
    case 0: r = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false); break;   // quad_perm 1,0,3,2
    case 1: r = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false); break;   // quad_perm 2,3,0,1
    case 2: r = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false); break;  // row_half_mirror
    default: r = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false); break; // row_mirror
    }
    return __int_as_float(r);
}
template <int W> __device__ __forceinline__ float group_max(float x) {
    static_assert(W == 8 || W == 16, "8- or 16-lane groups");
#pragma unroll
    for (int t = 0; t < (W == 16 ? 4 : 3); ++t) x = fmaxf(x, dpp_f(x, t));
    return x;
}
template <int W> __device__ __forceinline__ float group_sum(float x) {
    static_assert(W == 8 || W == 16, "8- or 16-lane groups");
#pragma unroll
    for (int t = 0; t < (W == 16 ? 4 : 3); ++t) x += dpp_f(x, t);
    return x;
}

// Sum over the lanes l, l ^ W, l ^ 2W, ... of a wave (W = 8 or 16): the
// lanes that hold the same channel chunk of different token rows.  Each
// swap of rows (16-lane groups) or halves gives every lane the pair's other
// value.
template <int W> __device__ __forceinline__ float column_sum(float x) {
    static_assert(W == 8 || W == 16, "8- or 16-lane groups");
    if constexpr (W == 8) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));   // row_ror:8
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(h[0]) + __uint_as_float(h[1]);
}

__device__ __forceinline__ void st_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);                  // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
}

// bf16 inputs, fp16 states: a persistent grid of two workgroups per CU, each
// zeroing its share of the padding rows, then walking the real key blocks
// b = bh * Nb + j = blockIdx.x, + gridDim.x, ...  W stays in LDS for the
// workgroup's lifetime (each workgroup converts the float W itself).  The
// next block's K and V are loaded into the registers that held the current
// block's as soon as phi and V are in LDS, so the loads run under the
// products of the current block; they are waited for before the block's
// stores (and once before the loop), so that no wait in the loop counts the
// stores: these drain under the next block's work.  z comes
// from per-thread partial sums of phi, reduced across lanes and waves.  The
// state h'^T goes out through LDS (8-byte units swizzled by row) as whole
// contiguous rows.
template <int D>
__global__ __launch_bounds__(2 * D, 2) void state16_kernel(const bf16 *__restrict__ k, const bf16 *__restrict__ v,
                                                          const float *__restrict__ w, int N, int Nb, int Nbc,
                                                          long total, f16 *__restrict__ hs, int Lp) {
    constexpr int NT = 2 * D;
    constexpr int CPR = D / 8;               // 16-byte chunks per token row
    constexpr int NCH = 64 * CPR / NT;       // chunks per thread and tensor
    constexpr int SSTR = D + 8;              // V row stride in LDS
    constexpr int PSTR = D + 16;             // phi row stride: 8 dwords mod 64 for transposing reads
    constexpr int WSTR = D + 8;              // W row stride: conflict-free 16-byte B-fragment reads
    constexpr int UPR = D / 4;               // 8-byte units per staged state row
    constexpr int RPI = 64 / UPR;            // staged rows per wave-wide read
    __shared__ __attribute__((aligned(16))) f16 Vs[64 * SSTR];
    __shared__ __attribute__((aligned(16))) f16 Ph[64 * PSTR];
    __shared__ __attribute__((aligned(16))) f16 Ws[D * WSTR];
    __shared__ __attribute__((aligned(16))) float Zp[NT / 64][D];   // z partial sums per wave
    static_assert(32 * D * 2 <= 64 * SSTR * 2 && 32 * D * 2 <= 64 * PSTR * 2, "staging fits");
    static_assert(NCH * NT == 64 * CPR && 64 % (NT / CPR) == 0, "thread t holds rows t / CPR + (NT / CPR) u");

    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5, grp = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    for (int x = tid; x < D * CPR; x += NT) {   // W (float) to LDS in fp16
        const int r = x / CPR, c = x % CPR;
        const Chunk a = ld_chunk(w + (long)r * D + 8 * c), b = ld_chunk(w + (long)r * D + 8 * c + 4);
        const float *fa = reinterpret_cast<const float *>(&a), *fb = reinterpret_cast<const float *>(&b);
        f16 h[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) { h[e] = (f16)fa[e]; h[e + 4] = (f16)fb[e]; }
        __builtin_memcpy(&Ws[r * WSTR + 8 * c], h, sizeof(h));
    }

    Chunk kc[NCH], vc[NCH];
    // buffer loads over the block's valid rows: pad rows (and padding
    // blocks) read zeros without a per-lane branch, so the prefetched
    // registers are the same on every path
    auto load = [&](long bb) {                // bb = bh * Nb + j, a real block
        const int j = (int)(bb % Nb);
        const long bh = bb / Nb;
        const int n = min(64, N - 64 * j);
        const bf16 *kb = k + (bh * N + 64L * j) * D;
        const bf16 *vb = v + (bh * N + 64L * j) * D;
#pragma unroll
        for (int u = 0; u < NCH; ++u) {
            const int ch = tid + NT * u, row = ch / CPR, cc = ch % CPR;
            const bool ok = row < n;
            kc[u] = ok ? ld_chunk(kb + (long)row * D + cc * 8) : zero_chunk();
            vc[u] = ok ? ld_chunk(vb + (long)row * D + cc * 8) : zero_chunk();
        }
    };
    const long G = gridDim.x;
    // rows of the padding blocks (Nb <= j < Nbc) are zero
    const int npad = Nbc - Nb;
    for (long p = blockIdx.x; p < total / Nb * npad; p += G) {
        f16 *hsb = hs + ((p / npad) * Nbc + Nb + p % npad) * (long)Lp;
        for (int x = tid; x < Lp; x += NT) hsb[x] = (f16)0.f;
    }
    long b = blockIdx.x;
    if (b < total) load(b);
    __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0): the loop's head then never waits for memory
    st_barrier();                            // W in LDS

    constexpr float LOG2E = 1.4426950408889634f;
    const float scale = 1.f / 64.f;
    for (; b < total; b += G) {              // the real blocks b = bh * Nb + j
        const int j = (int)(b % Nb);
        f16 *hsb = hs + ((b / Nb) * Nbc + j) * (long)Lp;
        const int n = min(64, N - 64 * j);
        // phi(K) per token row (the CPR threads of a row are consecutive lanes);
        // phi and V to LDS in fp16; zp: this thread's share of z (its rows,
        // channel chunk tid % CPR), summed from the fp16 phi values
        float zp[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) zp[e] = 0.f;
#pragma unroll
        for (int u = 0; u < NCH; ++u) {
            const int ch = tid + NT * u, row = ch / CPR, cc = ch % CPR;
            const bf16 *x = reinterpret_cast<const bf16 *>(&kc[u]);
            float xf[8];
            float mx = -__builtin_inff();
#pragma unroll
            for (int e = 0; e < 8; ++e) { xf[e] = (float)x[e]; mx = fmaxf(mx, xf[e]); }
            mx = group_max<CPR>(mx);
            float sum = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) { xf[e] = fast_exp2((xf[e] - mx) * LOG2E); sum += xf[e]; }
            sum = group_sum<CPR>(sum);
            const float inv = (row < n) ? 1.f / sum : 0.f;
            f16 ph[8], vv[8];
            const bf16 *y = reinterpret_cast<const bf16 *>(&vc[u]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                ph[e] = (f16)(xf[e] * inv);
                vv[e] = (f16)(float)y[e];
                zp[e] += (float)ph[e];
            }
            __builtin_memcpy(&Ph[row * PSTR + cc * 8], ph, sizeof(ph));
            __builtin_memcpy(&Vs[row * SSTR + cc * 8], vv, sizeof(vv));
        }
        // z over the wave's rows: lanes l, l ^ CPR, ... hold the same channels
#pragma unroll
        for (int e = 0; e < 8; ++e) zp[e] = column_sum<CPR>(zp[e]);
        if (lane < CPR) {
#pragma unroll
            for (int e = 0; e < 8; e += 4)
                *reinterpret_cast<f32x4 *>(&Zp[wave][lane * 8 + e]) = f32x4{zp[e], zp[e + 1], zp[e + 2], zp[e + 3]};
        }
        st_barrier();
        if (b + G < total) load(b + G);      // next block, under this block's products and stores

        // V'[t][c] = sum_b V[t][b] W[c][b]: M = t (2 tiles), N = c (this wave's tile), K = b
        f32x16 accv[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) accv[mt][r] = 0.f;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            const v8<f16> bw = ld8<f16>(&Ws[(32 * wave + l32) * WSTR + 16 * s + 8 * hh]);
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) mma16(accv[mt], ld8<f16>(&Vs[(32 * mt + l32) * SSTR + 16 * s + 8 * hh]), bw);
        }
        // h'[a][c] = sum_t phi[t][a] V'[t][c]: M = a, N = c, K = t in the
        // accumulator's permuted order (the phi^T operand takes the same t runs
        // with transposing reads of the row-major phi tile)
        f32x16 acch[D / 32];
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acch[mt][r] = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            v8<f16> bv;
#pragma unroll
            for (int e = 0; e < 8; ++e) bv[e] = (f16)accv[s >> 1][8 * (s & 1) + e];
            const int k0 = 16 * s + 4 * (grp >> 1);
#pragma unroll
            for (int mt = 0; mt < D / 32; ++mt) {
                const int n0 = 32 * mt + 16 * (grp & 1);
                mma16(acch[mt], cat8<f16>(lds_col4<f16>(Ph, PSTR, k0, n0, lane), lds_col4<f16>(Ph, PSTR, k0 + 8, n0, lane)), bv);
            }
        }
        if (tid < D) {                       // z = sum over the block's tokens of phi: the waves' shares in order
            float z = Zp[0][tid];
#pragma unroll
            for (int w = 1; w < NT / 64; ++w) z += Zp[w][tid];
            hsb[D * D + tid] = (f16)(z * scale);
        }
        for (int x = D * D + D + tid; x < Lp; x += NT) hsb[x] = (f16)0.f;
        st_barrier();                        // Vs and Ph free: stage the state

        // lane (c, h) holds h'[a][c] for a = 32 mt + 8 g + 4 h + 0..3, i.e. the
        // 8-byte unit u = 8 mt + 2 g + h of row c; the wave's 32 rows c go
        // through a private LDS slice with unit u of row r at u ^ (r % UPR)
        f16 *stg = (wave < 2 ? Vs : Ph) + (wave & 1) * (32 * D);
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int u = 8 * mt + 2 * g + hh;
                v4<f16> y;
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = (f16)(acch[mt][4 * g + e] * scale);
                __builtin_memcpy(&stg[l32 * D + 4 * (u ^ (l32 % UPR))], &y, sizeof(y));
            }
        // The next block's K and V (loaded since the first barrier) are
        // waited for here, before this block's stores: loads and stores share
        // one counter, so a wait after the stores would also wait for the
        // writes to complete; this way the stores drain under the next
        // block's softmax and products.
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        f16 *orow = hsb + (long)(32 * wave) * D;
#pragma unroll
        for (int x = 0; x < 32 / RPI; ++x) {
            const int r = RPI * x + lane / UPR, u = lane % UPR;
            const v4<f16> y = ld4<f16>(&stg[r * D + 4 * (u ^ (r % UPR))]);
            __builtin_memcpy(orow + r * D + 4 * u, &y, sizeof(y));
        }
        st_barrier();                        // staging read before the next block's phi and V
    }
}

template <int D>
static hipError_t launch_state16_t(const StateArgs &a, hipStream_t st) {
    hipError_t e;
    int dev = 0, cus = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    const long total = a.BH * a.Nb;          // real blocks; the kernel also zeroes the padding rows
    const long grid = std::min<long>(std::max<long>(total, a.BH * (a.Nbc - a.Nb)), 2L * cus);
    state16_kernel<D><<<(unsigned)grid, 2 * D, 0, st>>>((const bf16 *)a.k, (const bf16 *)a.v, a.w,
                                                        a.N, a.Nb, a.Nbc, total, (f16 *)a.hs, a.Lp);
    return hipGetLastError();
}

template <typename T, typename S, int D>
static hipError_t launch_state_t(const StateArgs &a, hipStream_t st) {
    const int Nbc = a.Nbc;
    w_to_state_kernel<S><<<(D * D + 255) / 256, 256, 0, st>>>(a.w, (S *)a.wstate, D * D);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned grid = (unsigned)(a.BH * Nbc);
    state_kernel<T, S, D><<<grid, 2 * D, 0, st>>>((const T *)a.k, (const T *)a.v, (const S *)a.wstate, a.N,
                                                  a.Nb, Nbc, (S *)a.hs, a.Lp);
    return hipGetLastError();
}

hipError_t launch_state(const StateArgs &a, hipStream_t st) {
    if (a.bf16_in) return a.D == 64 ? launch_state16_t<64>(a, st) : launch_state16_t<128>(a, st);
    return a.D == 64 ? launch_state_t<float, float, 64>(a, st) : launch_state_t<float, float, 128>(a, st);
}

}  // namespace sla
