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
// Blocks past Nb up to the next multiple of 32 are written as zero rows.
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

template <typename T, typename S, int D>
static hipError_t launch_state_t(const StateArgs &a, hipStream_t st) {
    const int Nbc = (a.Nb + 31) / 32 * 32;
    w_to_state_kernel<S><<<(D * D + 255) / 256, 256, 0, st>>>(a.w, (S *)a.wstate, D * D);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned grid = (unsigned)(a.BH * Nbc);
    state_kernel<T, S, D><<<grid, 2 * D, 0, st>>>((const T *)a.k, (const T *)a.v, (const S *)a.wstate, a.N,
                                                  a.Nb, Nbc, (S *)a.hs, a.Lp);
    return hipGetLastError();
}

hipError_t launch_state(const StateArgs &a, hipStream_t st) {
    if (a.bf16_in)
        return a.D == 64 ? launch_state_t<bf16, f16, 64>(a, st) : launch_state_t<bf16, f16, 128>(a, st);
    return a.D == 64 ? launch_state_t<float, float, 64>(a, st) : launch_state_t<float, float, 128>(a, st);
}

}  // namespace sla
