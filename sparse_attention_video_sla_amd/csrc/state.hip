// state.hip -- per-key-block linear-attention states (SLA article, section 3:
// linear attention over the marginal blocks computes phi(K)^T V first, with
// phi = softmax over the channels, section 5).
//
// One workgroup per key block j (64 tokens), D/32 waves; wave w owns output
// channels 32w..32w+31.
//   phi(k_t) = softmax over the d channels of each valid token (pad tokens 0).
//   The projection W of the linear branch is folded in here: the block state
//   is h'_j^T = (phi(K_j)^T V_j W^T)^T, computed as V'_j = V_j W^T then
//   h'_j^T = V'_j^T phi(K_j), both on MFMA.  Since the linear output is
//   phi(q) H / (phi(q).Z) with H a sum of h_j, applying W^T to H per block is
//   the same linear map as applying it to the output.
//   z_j = sum_t phi(k_t).
// Stored per block, scaled by 1/64 (exact) so that values stay within the
// range of the fp16 staging type, as one "column" vector of Lp values
// [h'^T row-major (d*d), z (d), zero pad] per block.  The blocks are
// interleaved by 8: value (block j, column x) sits at ((j/8)*Lp + x)*8 + j%8,
// so that the assembly GEMM reads 8 consecutive blocks of one column as one
// 16-byte MFMA fragment.  Blocks past Nb up to the next multiple of 32 are
// written as zeros.  Workgroups are mapped so that the 8 blocks of a group run
// back to back on one XCD, whose L2 then merges their interleaved stores.
// The same kernel writes V_j transposed ([d][64], pad tokens zero) in the
// input dtype, the layout the fused kernel streams through LDS.
#include "sla_device.h"
#include "sla_launch.h"

namespace sla {

template <typename T, typename S, int D>
__global__ __launch_bounds__(2 * D) void state_kernel(const T *__restrict__ k, const T *__restrict__ v,
                                                      const float *__restrict__ w, int N, int Nb, int Nbc,
                                                      long G, int per_xcd, T *__restrict__ vt,
                                                      S *__restrict__ hs, int Lp, int do_states, int do_vt) {
    constexpr int NT = 2 * D;
    constexpr int EPC = 16 / sizeof(T);      // input elements per 16-byte chunk
    constexpr int CPR = D / EPC;             // chunks per token row
    constexpr int NCH = 64 * CPR / NT;       // chunks per thread
    constexpr int SE = 16 / sizeof(S);
    constexpr int SSTR = D + SE;             // V row stride in LDS (state type)
    constexpr int PSTR = 64 + SE;            // phi^T row stride in LDS
    __shared__ S Vs[64 * SSTR];
    __shared__ S Pt[D * PSTR];

    const long logical = (long)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);   // bh * Nbc + j
    if (logical >= G) return;
    const int j = (int)(logical % Nbc);
    const long bh = logical / Nbc;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    // interleaved state column of this block: element x at hsb[x * 8]
    S *hsb = hs + ((bh * (Nbc / 8) + j / 8) * (long)Lp) * 8 + (j % 8);
    if (j >= Nb) {                           // padding block: zero states only
        if (do_states)
            for (int x = tid; x < Lp; x += NT) hsb[(long)x * 8] = from_f32<S>(0.f);
        return;
    }
    const long blk = bh * Nb + j;
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
    if (do_vt) {
        T *vtb = vt + blk * (long)D * 64;
#pragma unroll
        for (int u = 0; u < NCH; ++u) {
            const int ch = tid + NT * u, row = ch / CPR, cc = ch % CPR;
            const T *x = reinterpret_cast<const T *>(&vc[u]);
#pragma unroll
            for (int e = 0; e < EPC; ++e) vtb[(long)(cc * EPC + e) * 64 + row] = x[e];
        }
    }
    if (!do_states) return;

    // phi(K) per token row: the CPR threads of a row are CPR consecutive lanes
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
        for (int e = 0; e < EPC; ++e) { xf[e] = expf(xf[e] - mx); sum += xf[e]; }
#pragma unroll
        for (int off = 1; off < CPR; off <<= 1) sum += __shfl_xor(sum, off, 64);
        const float inv = (row < n) ? 1.f / sum : 0.f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) Pt[(cc * EPC + e) * PSTR + row] = from_f32<S>(xf[e] * inv);
        // V in the state type, row-major
        const T *y = reinterpret_cast<const T *>(&vc[u]);
#pragma unroll
        for (int e = 0; e < EPC; ++e) Vs[row * SSTR + cc * EPC + e] = from_f32<S>(to_f32<T>(y[e]));
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
        const v8<S> bw = cvt8<S>(ld8<float>(w + (long)(32 * wave + l32) * D + 16 * s + 8 * hh));
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const v8<S> a = ld8<S>(&Vs[(32 * mt + l32) * SSTR + 16 * s + 8 * hh]);
            mma16(accv[mt], a, bw);
        }
    }
    // h'^T[c][a] = sum_t V'[t][c] phi[t][a]: M = c, N = a, K = t taken in the
    // accumulator's permuted row order (see sla_device.h)
    f32x16 acch[D / 32];
#pragma unroll
    for (int nt = 0; nt < D / 32; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acch[nt][r] = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        v8<S> a;
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = from_f32<S>(accv[s >> 1][8 * (s & 1) + e]);
#pragma unroll
        for (int nt = 0; nt < D / 32; ++nt) {
            const S *p = &Pt[(32 * nt + l32) * PSTR + 16 * s + 4 * hh];
            mma16(acch[nt], a, ld4x2<S>(p, p + 8));
        }
    }

    const float scale = 1.f / 64.f;
#pragma unroll
    for (int nt = 0; nt < D / 32; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int c = 32 * wave + 8 * (r >> 2) + 4 * hh + (r & 3);
            hsb[(long)(c * D + 32 * nt + l32) * 8] = from_f32<S>(acch[nt][r] * scale);
        }
    if (tid < D) {
        float z = 0.f;
        for (int t = 0; t < 64; ++t) z += to_f32<S>(Pt[tid * PSTR + t]);
        hsb[(long)(D * D + tid) * 8] = from_f32<S>(z * scale);
    }
    for (int x = D * D + D + tid; x < Lp; x += NT) hsb[(long)x * 8] = from_f32<S>(0.f);
}

template <typename T, typename S, int D>
static hipError_t launch_state_t(const StateArgs &a, hipStream_t st) {
    const int Nbc = (a.Nb + 31) / 32 * 32;
    const long G = a.BH * (a.do_states ? Nbc : a.Nb);
    const int per = (int)((G + 7) / 8);
    // without states there is no padding: the grid is then bh * Nb blocks, j < Nb
    const int nbc = a.do_states ? Nbc : a.Nb;
    state_kernel<T, S, D><<<(unsigned)(8L * per), 2 * D, 0, st>>>((const T *)a.k, (const T *)a.v, a.w, a.N, a.Nb,
                                                                  nbc, G, per, (T *)a.vt, (S *)a.hs, a.Lp,
                                                                  a.do_states, a.do_vt);
    return hipGetLastError();
}

hipError_t launch_state(const StateArgs &a, hipStream_t st) {
    if (a.bf16_in)
        return a.D == 64 ? launch_state_t<bf16, f16, 64>(a, st) : launch_state_t<bf16, f16, 128>(a, st);
    return a.D == 64 ? launch_state_t<float, float, 64>(a, st) : launch_state_t<float, float, 128>(a, st);
}

}  // namespace sla
