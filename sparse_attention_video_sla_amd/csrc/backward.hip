// backward.hip -- gradients of the SLA forward pass (SLA article, section 三:
// the backward splits like the forward, FlashAttention gradients for the
// sparse part and linear-attention gradients for the linear part), bf16
// inputs, fp32 gradients.  The block labels are held fixed.
//
// Sparse part, with P = softmax of the critical keys (recomputed from the
// log-sum-exp the forward kernel writes) and D_r = dO_r . O_s,r:
//   dS = P * (dO V^T - D),  dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d),
//   dV = P^T dO;
// bwd_dq_kernel walks each query block's critical blocks, bwd_dkv_kernel
// each key block's list of query blocks that chose it (transposed lists).
//
// Linear part, with the marginal states as the forward keeps them (Ĥ'_i^T,
// Ẑ_i, both divided by the row's marginal token count m_i, the projection
// folded in: y_r = phi(q_r) Ĥ'_i / phi(q_r).Ẑ_i):
//   rows:  g_r = dO_r . y_r,  dphi(q_r) = (Ĥ'_i dO_r - g_r Ẑ_i) / den_r,
//          dĤ'_i = sum_r phi(q_r) dO_r^T / den_r,  dẐ_i = -sum_r g_r phi(q_r) / den_r
//          (den_r = phi(q_r).Ẑ_i with the true, unscaled states);
//   sums:  dh'_j = sum of dĤ'_i over the rows i for which j is marginal
//          (the transposed 0/1 product);
//   keys:  v'_u = W v_u, dphi(k_u) = dh'_j v'_u + dz_j, dv'_u = dh'_j^T phi(k_u),
//          dv_u += W^T dv'_u, dW += sum_u dv'_u v_u^T;
//   phi = softmax over channels: dx = phi * (dphi - phi . dphi).
#include "sla_device.h"
#include "sla_launch.h"
#include "tile_common.h"

#include <algorithm>

namespace sla {

namespace {
constexpr float NEG_INF_B = -__builtin_inff();
}

// ---- transposed lists and indicator ------------------------------------------

// thread per (head, key block j): the query blocks i with j critical, ascending
__global__ __launch_bounds__(256) void bwd_tlists_kernel(const int8_t *__restrict__ mask, long BH, int Nb,
                                                         uint16_t *__restrict__ tlist, int32_t *__restrict__ tcnt) {
    const long t = (long)blockIdx.x * 256 + threadIdx.x;
    if (t >= BH * Nb) return;
    const long bh = t / Nb;
    const int j = (int)(t % Nb);
    const int8_t *m = mask + bh * Nb * (long)Nb + j;
    uint16_t *out = tlist + t * (long)Nb;
    int c = 0;
    for (int i = 0; i < Nb; ++i)
        if (m[(long)i * Nb] == 1) out[c++] = (uint16_t)i;
    tcnt[t] = c;
}

// margT[bh][j][i] = 1 when key block j is marginal for query block i (i < Nbc, 0 past Nb);
// unit[bh][j] = 64 so that the marginal-state product applies no row scale
__global__ __launch_bounds__(256) void bwd_margT_kernel(const int8_t *__restrict__ mask, long BH, int Nb, int Nbc,
                                                        float *__restrict__ margT, int32_t *__restrict__ unit) {
    const long t = (long)blockIdx.x * 256 + threadIdx.x;
    if (t >= BH * Nb * (long)Nbc) return;
    const int i = (int)(t % Nbc);
    const long r = t / Nbc;
    const int j = (int)(r % Nb);
    const long bh = r / Nb;
    margT[t] = (i < Nb && mask[(bh * Nb + i) * (long)Nb + j] == 0) ? 1.f : 0.f;
    if (i == 0) unit[r] = 64;
}

__global__ __launch_bounds__(256) void bwd_zero_kernel(float *__restrict__ p, long n) {
    const long t = (long)blockIdx.x * 256 + threadIdx.x;
    if (t < n) p[t] = 0.f;
}

// ---- sparse part ------------------------------------------------------------

namespace {

// 1 KB block u of this wave's share of a 64 x D tile: source offsets of its
// lane in the K layout (rows of 2D bytes, 16-byte chunks swizzled) and the V
// layout (groups of 4 rows, chunk-major inside a group)
template <int D> __device__ __forceinline__ uint32_t off_klayout(int byte) {
    const int r = byte / (2 * D), pk = (byte % (2 * D)) / 16;
    return (uint32_t)(r * 2 * D + (pk ^ kswz<D>(r)) * 16);
}
template <int D> __device__ __forceinline__ uint32_t off_vlayout(int byte) {
    const int g = byte / (8 * D), qv = (byte % (8 * D)) / 16;
    return (uint32_t)((4 * g + (qv & 3)) * 2 * D + (qv >> 2) * 16);
}
// transposing reads of rows 32*half .. +31 of a V-layout tile as the A
// operand [channel][row], rows in the accumulator order of a 32 x 32 tile
template <typename T, int D>
__device__ __forceinline__ void read_tr(const T *tile, int vb, v8<T> (&a)[D / 32][2]) {
    const T *Vs = tile + vb;
#pragma unroll
    for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            a[ct][ks] = cat8<T>(lds_tr_raw<T>(Vs + ks * 16 * D + ct * 128), lds_tr_raw<T>(Vs + ks * 16 * D + 8 * D + ct * 128));
}
__device__ __forceinline__ int vbase_of(int half, int lane, int D) {
    const int grp = lane >> 4, L = lane & 15;
    return ((8 * half + (grp >> 1)) * 8 * D + ((2 * (grp & 1) + ((L & 3) >> 1)) * 4 + (L >> 2)) * 16 + (L & 1) * 8) / 2;
}

}  // namespace

// One workgroup of 4 waves per query block i: wave (rh, kh) takes query rows
// 32rh .. +31 against key half kh of every critical block.  Per block: S^T =
// K Q^T and dP^T = V dO^T on the matrix core (K, V rows from LDS, Q and dO
// in registers), dS^T in the VALU, dQ^T += K^T dS^T (transposing reads of K).
// Tiles go global -> LDS through a two-slot ring, one barrier per block.
template <int D>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                                                        const bf16 *__restrict__ v, const bf16 *__restrict__ dout,
                                                        const float *__restrict__ o_s, const float *__restrict__ lse,
                                                        const int32_t *__restrict__ crit, int kc,
                                                        float *__restrict__ dq, float *__restrict__ dbuf, long G,
                                                        int per_xcd, int N, int Nb, float sl2, float scale) {
    using T = bf16;
    constexpr int TILE = 64 * D, NS = D / 16, NCT = D / 32, NCH = NCT / 2, NBW = D / 32;
    __shared__ __attribute__((aligned(1024))) T Kk[2][TILE];
    __shared__ __attribute__((aligned(1024))) T Kv[2][TILE];
    __shared__ __attribute__((aligned(1024))) T Vk[2][TILE];
    const long logical = (long)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (logical >= G) return;
    const long bh = logical / Nb;
    const int i = (int)(logical % Nb);
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, hh = lane >> 5;
    const int rh = wave >> 1, kh = wave & 1;
    const int qrow = 64 * i + 32 * rh + l32;
    const bool qvalid = qrow < N;
    v8<T> qf[NS], df[NS];
    float Dr = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const long base = (bh * N + qrow) * (long)D + 16 * s + 8 * hh;
        qf[s] = qvalid ? ld8<T>(q + base) : zero8<T>();
        df[s] = qvalid ? ld8<T>(dout + base) : zero8<T>();
        if (qvalid) {
#pragma unroll
            for (int e = 0; e < 8; ++e) Dr += to_f32<T>(df[s][e]) * o_s[base + e];
        }
    }
    Dr = half_swap_sum(Dr);
    if (kh == 0 && hh == 0 && qvalid) dbuf[bh * N + qrow] = Dr;
    const float lse2 = qvalid ? lse[bh * N + qrow] : __builtin_inff();

    int koff[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int r = 32 * kh + l32;
        koff[s] = r * D + ((2 * s + hh) ^ kswz<D>(r)) * 8;
    }
    const int vb = vbase_of(kh, lane, D);
    uint32_t ok_[NBW], ov_[NBW];
#pragma unroll
    for (int u = 0; u < NBW; ++u) {
        const int byte = (wave * NBW + u) * 1024 + 16 * lane;
        ok_[u] = off_klayout<D>(byte);
        ov_[u] = off_vlayout<D>(byte);
    }
    const uint32_t head_bytes = (uint32_t)((long)N * D * sizeof(T));
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + bh * N * (long)D, head_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + bh * N * (long)D, head_bytes);
    const int32_t *cl = crit + (bh * Nb + i) * (long)kc;
    auto load = [&](int c, int slot) __attribute__((always_inline)) {
        const uint32_t off = (uint32_t)(64L * cl[c] * D * sizeof(T));
#pragma unroll
        for (int u = 0; u < NBW; ++u) {
            dma16(rk, &Kk[slot][(wave * NBW + u) * 512], ok_[u] + off, 0);
            dma16(rk, &Kv[slot][(wave * NBW + u) * 512], ov_[u] + off, 0);
            dma16(rv, &Vk[slot][(wave * NBW + u) * 512], ok_[u] + off, 0);
        }
    };
    f32x16 dqt[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqt[ct][r] = 0.f;
    auto compute = [&](int c, int slot) __attribute__((always_inline)) {
        const int j = cl[c];
        v8<T> a[NS];
        f32x16 sacc, pacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = pacc[r] = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s) a[s] = ld8<T>(&Kk[slot][koff[s]]);
#pragma unroll
        for (int s = 0; s < NS; ++s) mma16(sacc, a[s], qf[s]);
#pragma unroll
        for (int s = 0; s < NS; ++s) a[s] = ld8<T>(&Vk[slot][koff[s]]);
#pragma unroll
        for (int s = 0; s < NS; ++s) mma16(pacc, a[s], df[s]);
        v8<T> dsb[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = 64 * j + 32 * kh + 8 * (r >> 2) + 4 * hh + (r & 3);
            const float p = key < N ? fast_exp2(__builtin_fmaf(sacc[r], sl2, -lse2)) : 0.f;
            dsb[r >> 3][r & 7] = from_f32<T>(p * (pacc[r] - Dr));
        }
        v8<T> at[NCT][2];
        read_tr<T, D>(Kv[slot], vb, at);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) mma16(dqt[ct], at[ct][ks], dsb[ks]);
    };
    if (kc > 0) {
        load(0, 0);
        wait_vm0();
        lds_barrier();
        int c = 0;
        for (; c + 1 < kc; c += 2) {
            load(c + 1, 1);
            compute(c, 0);
            wait_vm0();
            lds_barrier();
            if (c + 2 < kc) load(c + 2, 0);
            compute(c + 1, 1);
            wait_vm0();
            lds_barrier();
        }
        if (c < kc) {
            compute(c, 0);
            lds_barrier();
        }
    }
    wait_vm0();
    // sum the two key halves: wave kh keeps channel tiles NCH*kh .. +NCH-1
    float *xo = reinterpret_cast<float *>(&Kk[0][0]);     // [4 waves][NCH*4][64] f32x4
    f32x16 mine[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        mine[c] = kh == 0 ? dqt[c] : dqt[NCH + c];
        const f32x16 give = kh == 0 ? dqt[NCH + c] : dqt[c];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 y = {give[4 * g], give[4 * g + 1], give[4 * g + 2], give[4 * g + 3]};
            *reinterpret_cast<f32x4 *>(xo + ((wave * NCH * 4 + c * 4 + g) * 64 + lane) * 4) = y;
        }
    }
    lds_barrier();
    const int partner = wave ^ 1;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 y = *reinterpret_cast<const f32x4 *>(xo + ((partner * NCH * 4 + c * 4 + g) * 64 + lane) * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) mine[c][4 * g + e] += y[e];
        }
    if (!qvalid) return;
    float *orow = dq + (bh * N + qrow) * (long)D;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int c0 = 32 * (NCH * kh + c);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 y = {mine[c][4 * g] * scale, mine[c][4 * g + 1] * scale, mine[c][4 * g + 2] * scale,
                             mine[c][4 * g + 3] * scale};
            *reinterpret_cast<f32x4 *>(orow + c0 + 8 * g + 4 * hh) = y;
        }
    }
}

// One workgroup of 4 waves per key block j: wave (kh, rh) takes keys 32kh ..
// +31 against query rows 32rh .. +31 of every query block that chose j.  Per
// query block: S = Q K^T and dP = dO V^T on the matrix core (Q, dO rows from
// LDS, K and V rows in registers), dS in the VALU, dV^T += dO^T P and dK^T +=
// Q^T dS (transposing reads of dO and Q).
template <int D>
__global__ __launch_bounds__(256, 1) void bwd_dkv_kernel(const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                                                         const bf16 *__restrict__ v, const bf16 *__restrict__ dout,
                                                         const float *__restrict__ lse, const float *__restrict__ dbuf,
                                                         const uint16_t *__restrict__ tlist,
                                                         const int32_t *__restrict__ tcnt, float *__restrict__ dk,
                                                         float *__restrict__ dv, long G, int per_xcd, int N, int Nb,
                                                         float sl2, float scale) {
    using T = bf16;
    constexpr int TILE = 64 * D, NS = D / 16, NCT = D / 32, NCH = NCT / 2, NBW = D / 32;
    __shared__ __attribute__((aligned(1024))) T Qk[2][TILE];
    __shared__ __attribute__((aligned(1024))) T Qv[2][TILE];
    __shared__ __attribute__((aligned(1024))) T Ok[2][TILE];
    __shared__ __attribute__((aligned(1024))) T Ov[2][TILE];
    const long logical = (long)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (logical >= G) return;
    const long bh = logical / Nb;
    const int j = (int)(logical % Nb);
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, hh = lane >> 5;
    const int kh = wave >> 1, rh = wave & 1;
    const int krow = 64 * j + 32 * kh + l32;
    const bool kvalid = krow < N;
    v8<T> kf[NS], vf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const long base = (bh * N + krow) * (long)D + 16 * s + 8 * hh;
        kf[s] = kvalid ? ld8<T>(k + base) : zero8<T>();
        vf[s] = kvalid ? ld8<T>(v + base) : zero8<T>();
    }
    int koff[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int r = 32 * rh + l32;
        koff[s] = r * D + ((2 * s + hh) ^ kswz<D>(r)) * 8;
    }
    const int vb = vbase_of(rh, lane, D);
    uint32_t ok_[NBW], ov_[NBW];
#pragma unroll
    for (int u = 0; u < NBW; ++u) {
        const int byte = (wave * NBW + u) * 1024 + 16 * lane;
        ok_[u] = off_klayout<D>(byte);
        ov_[u] = off_vlayout<D>(byte);
    }
    const uint32_t head_bytes = (uint32_t)((long)N * D * sizeof(T));
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + bh * N * (long)D, head_bytes);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(dout + bh * N * (long)D, head_bytes);
    const uint16_t *tl = tlist + (bh * Nb + j) * (long)Nb;
    const int cnt = tcnt[bh * Nb + j];
    auto load = [&](int c, int slot) __attribute__((always_inline)) {
        const uint32_t off = (uint32_t)(64L * tl[c] * D * sizeof(T));
#pragma unroll
        for (int u = 0; u < NBW; ++u) {
            dma16(rq, &Qk[slot][(wave * NBW + u) * 512], ok_[u] + off, 0);
            dma16(rq, &Qv[slot][(wave * NBW + u) * 512], ov_[u] + off, 0);
            dma16(ro, &Ok[slot][(wave * NBW + u) * 512], ok_[u] + off, 0);
            dma16(ro, &Ov[slot][(wave * NBW + u) * 512], ov_[u] + off, 0);
        }
    };
    f32x16 dvt[NCT], dkt[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) dvt[ct][r] = dkt[ct][r] = 0.f;
    auto compute = [&](int c, int slot) __attribute__((always_inline)) {
        const int i = tl[c];
        // the rows of the accumulator this lane holds, their lse and D
        float lr[16], dr[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 64 * i + 32 * rh + 8 * (r >> 2) + 4 * hh + (r & 3);
            lr[r] = row < N ? lse[bh * N + row] : __builtin_inff();
            dr[r] = row < N ? dbuf[bh * N + row] : 0.f;
        }
        v8<T> a[NS];
        f32x16 sacc, pacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = pacc[r] = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s) a[s] = ld8<T>(&Qk[slot][koff[s]]);
#pragma unroll
        for (int s = 0; s < NS; ++s) mma16(sacc, a[s], kf[s]);
#pragma unroll
        for (int s = 0; s < NS; ++s) a[s] = ld8<T>(&Ok[slot][koff[s]]);
#pragma unroll
        for (int s = 0; s < NS; ++s) mma16(pacc, a[s], vf[s]);
        v8<T> pb[2], dsb[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = kvalid ? fast_exp2(__builtin_fmaf(sacc[r], sl2, -lr[r])) : 0.f;
            pb[r >> 3][r & 7] = from_f32<T>(p);
            dsb[r >> 3][r & 7] = from_f32<T>(p * (pacc[r] - dr[r]));
        }
        v8<T> at[NCT][2];
        read_tr<T, D>(Ov[slot], vb, at);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) mma16(dvt[ct], at[ct][ks], pb[ks]);
        read_tr<T, D>(Qv[slot], vb, at);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) mma16(dkt[ct], at[ct][ks], dsb[ks]);
    };
    if (cnt > 0) {
        load(0, 0);
        wait_vm0();
        lds_barrier();
        int c = 0;
        for (; c + 1 < cnt; c += 2) {
            load(c + 1, 1);
            compute(c, 0);
            wait_vm0();
            lds_barrier();
            if (c + 2 < cnt) load(c + 2, 0);
            compute(c + 1, 1);
            wait_vm0();
            lds_barrier();
        }
        if (c < cnt) {
            compute(c, 0);
            lds_barrier();
        }
    }
    wait_vm0();
    // sum the two row halves: wave rh keeps channel tiles NCH*rh .. +NCH-1 of dV and dK
    float *xv = reinterpret_cast<float *>(&Qk[0][0]);     // [4 waves][NCH*4][64] f32x4 (dV)
    float *xk = reinterpret_cast<float *>(&Ok[0][0]);     // same for dK
    f32x16 mv[NCH], mk[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        mv[c] = rh == 0 ? dvt[c] : dvt[NCH + c];
        mk[c] = rh == 0 ? dkt[c] : dkt[NCH + c];
        const f32x16 gv = rh == 0 ? dvt[NCH + c] : dvt[c];
        const f32x16 gk = rh == 0 ? dkt[NCH + c] : dkt[c];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 y = {gv[4 * g], gv[4 * g + 1], gv[4 * g + 2], gv[4 * g + 3]};
            const f32x4 z = {gk[4 * g], gk[4 * g + 1], gk[4 * g + 2], gk[4 * g + 3]};
            *reinterpret_cast<f32x4 *>(xv + ((wave * NCH * 4 + c * 4 + g) * 64 + lane) * 4) = y;
            *reinterpret_cast<f32x4 *>(xk + ((wave * NCH * 4 + c * 4 + g) * 64 + lane) * 4) = z;
        }
    }
    lds_barrier();
    const int partner = wave ^ 1;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 y = *reinterpret_cast<const f32x4 *>(xv + ((partner * NCH * 4 + c * 4 + g) * 64 + lane) * 4);
            const f32x4 z = *reinterpret_cast<const f32x4 *>(xk + ((partner * NCH * 4 + c * 4 + g) * 64 + lane) * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                mv[c][4 * g + e] += y[e];
                mk[c][4 * g + e] += z[e];
            }
        }
    if (!kvalid) return;
    float *vrow = dv + (bh * N + krow) * (long)D;
    float *krw = dk + (bh * N + krow) * (long)D;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int c0 = 32 * (NCH * rh + c);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 y = {mv[c][4 * g], mv[c][4 * g + 1], mv[c][4 * g + 2], mv[c][4 * g + 3]};
            const f32x4 z = {mk[c][4 * g] * scale, mk[c][4 * g + 1] * scale, mk[c][4 * g + 2] * scale,
                             mk[c][4 * g + 3] * scale};
            *reinterpret_cast<f32x4 *>(vrow + c0 + 8 * g + 4 * hh) = y;
            *reinterpret_cast<f32x4 *>(krw + c0 + 8 * g + 4 * hh) = z;
        }
    }
}

// ---- linear part --------------------------------------------------------------

namespace {
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
}  // namespace

// One workgroup per query block i (rows past Nb, and rows without marginal
// blocks, write zero states).  Rows: wave w takes rows 16w .. +15, each lane
// D/64 channels.  Then dĤ' (stored transposed like Ĥ': [c][a]) and dẐ.
template <int D>
__global__ __launch_bounds__(256) void bwd_lin_row_kernel(const bf16 *__restrict__ q, const bf16 *__restrict__ dout,
                                                          const f16 *__restrict__ hhat, const int32_t *__restrict__ mcount,
                                                          int Lp, float *__restrict__ dq, float *__restrict__ dhrow,
                                                          long BH, int N, int Nb, int Nbc) {
    constexpr int CPL = D / 64;                          // channels per lane
    constexpr int HS = D + 1;                            // padded row stride of Hs
    __shared__ float Hs[D * HS];                         // stored [c][a]
    __shared__ float Zs[D];
    __shared__ float Pn[64 * D];                         // phi(q_r) / den_r (scaled states)
    __shared__ float Do[64 * D];
    __shared__ float Gr[64];
    const long blk = blockIdx.x;
    const long bh = blk / Nbc;
    const int i = (int)(blk % Nbc);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float *drow = dhrow + blk * (long)Lp;
    const int mc = i < Nb ? mcount[bh * Nb + i] : 0;
    if (mc == 0) {
        for (int x = tid; x < Lp; x += 256) drow[x] = 0.f;
        return;
    }
    const f16 *hr = hhat + (bh * Nb + i) * (long)Lp;
    for (int x = tid; x < D * D; x += 256) Hs[(x / D) * HS + (x % D)] = (float)hr[x];
    for (int x = tid; x < D; x += 256) Zs[x] = (float)hr[D * D + x];
    for (int x = D * D + D + tid; x < Lp; x += 256) drow[x] = 0.f;
    __syncthreads();
    for (int rr = 0; rr < 16; ++rr) {
        const int r = 16 * wave + rr;
        const int row = 64 * i + r;
        float ph[CPL], dov[CPL];
        if (row < N) {
            const long base = (bh * N + row) * (long)D;
            float qv[CPL], mx = NEG_INF_B;
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
                qv[e] = to_f32<bf16>(q[base + lane + 64 * e]);
                dov[e] = to_f32<bf16>(dout[base + lane + 64 * e]);
                mx = fmaxf(mx, qv[e]);
            }
            mx = wave_max(mx);
            float se = 0.f;
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
                ph[e] = __expf(qv[e] - mx);
                se += ph[e];
            }
            se = wave_sum(se);
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
                ph[e] /= se;
                Pn[r * D + lane + 64 * e] = ph[e];
                Do[r * D + lane + 64 * e] = dov[e];
            }
        } else {
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
                ph[e] = 0.f;
                dov[e] = 0.f;
                Pn[r * D + lane + 64 * e] = 0.f;
                Do[r * D + lane + 64 * e] = 0.f;
            }
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        if (row >= N) {
            if (lane == 0) Gr[r] = 0.f;
            continue;
        }
        float den = 0.f;
#pragma unroll
        for (int e = 0; e < CPL; ++e) den += ph[e] * Zs[lane + 64 * e];
        den = wave_sum(den);
        // y[c] = sum_a phi_a H[c][a] / den (this lane's c), g = dO . y
        float g = 0.f;
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            const int c = lane + 64 * e;
            float y = 0.f;
            for (int a = 0; a < D; ++a) y += Pn[r * D + a] * Hs[c * HS + a];
            g += dov[e] * y / den;
        }
        g = wave_sum(g);
        // dphi[a] = (sum_c H[c][a] dO_c - g Z[a]) / den (this lane's a)
        float dph[CPL], pd = 0.f;
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            const int a = lane + 64 * e;
            float x = 0.f;
            for (int c = 0; c < D; ++c) x += Hs[c * HS + a] * Do[r * D + c];
            dph[e] = (x - g * Zs[a]) / den;
            pd += ph[e] * dph[e];
        }
        pd = wave_sum(pd);
        float *qg = dq + (bh * N + row) * (long)D;
#pragma unroll
        for (int e = 0; e < CPL; ++e) qg[lane + 64 * e] += ph[e] * (dph[e] - pd);
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
        for (int e = 0; e < CPL; ++e) Pn[r * D + lane + 64 * e] = ph[e] / den;
        if (lane == 0) Gr[r] = g;
    }
    __syncthreads();
    // dĤ'[c][a] = (1/m) sum_r Pn[r][a] Do[r][c]; wave w: a = lane + 64 (w & 1) ... per D
    const float inv_m = 1.f / (float)mc;
    constexpr int AW = D / 64;                           // waves along a
    constexpr int CB = D / (4 / AW);                     // c's per wave
    const int a = lane + 64 * (wave % AW);
    const int c0 = (wave / AW) * CB;
    float acc[CB];
#pragma unroll
    for (int x = 0; x < CB; ++x) acc[x] = 0.f;
    float zacc = 0.f;
    for (int r = 0; r < 64; ++r) {
        const float p = Pn[r * D + a];
#pragma unroll
        for (int x = 0; x < CB; ++x) acc[x] += p * Do[r * D + c0 + x];
        zacc += Gr[r] * p;
    }
#pragma unroll
    for (int x = 0; x < CB; ++x) drow[(c0 + x) * D + a] = acc[x] * inv_m;
    if (wave / AW == 0) drow[D * D + a] = -zacc * inv_m;
}

// One workgroup per key block j, persistent over a stride of blocks so that
// dW is added once per workgroup.  W and dh' (stored [c][a]) live in LDS
// with padded rows; the 64 rows of a block go in four passes of 16.
template <int D>
__global__ __launch_bounds__(256) void bwd_lin_key_kernel(const bf16 *__restrict__ k, const bf16 *__restrict__ v,
                                                          const float *__restrict__ w, const float *__restrict__ dhs,
                                                          int Lp, float *__restrict__ dk, float *__restrict__ dv,
                                                          float *__restrict__ dw, long BH, int N, int Nb) {
    constexpr int CPL = D / 64;
    constexpr int HS = D + 1;
    constexpr int RB = 16;                               // rows per pass
    __shared__ float Wl[D * HS];
    __shared__ float Dh[D * HS];
    __shared__ float Dz[D];
    __shared__ float Ph[RB * D];                         // phi(k_u)
    __shared__ float Vr[RB * D];                         // v_u
    __shared__ float Vp[RB * D];                         // v'_u = W v_u, then dv'_u
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int x = tid; x < D * D; x += 256) Wl[(x / D) * HS + (x % D)] = w[x];
    constexpr int WC = D * D / 256;                      // dW accumulators: (c block, e = tid % D)
    const int we = tid % D, wc0 = (tid / D) * WC;
    float wacc[WC];
#pragma unroll
    for (int x = 0; x < WC; ++x) wacc[x] = 0.f;
    const long total = BH * Nb;
    for (long blk = blockIdx.x; blk < total; blk += gridDim.x) {
        const long bh = blk / Nb;
        const int j = (int)(blk % Nb);
        const float *hrow = dhs + blk * (long)Lp;
        __syncthreads();
        for (int x = tid; x < D * D; x += 256) Dh[(x / D) * HS + (x % D)] = hrow[x];
        for (int x = tid; x < D; x += 256) Dz[x] = hrow[D * D + x];
        for (int pass = 0; pass < 64 / RB; ++pass) {
            __syncthreads();
            // rows of this pass: phi(k_u), v_u (wave w: rows 4w .. 4w+3)
            for (int rr = 0; rr < RB / 4; ++rr) {
                const int r = (RB / 4) * wave + rr;
                const int row = 64 * j + RB * pass + r;
                if (row < N) {
                    const long base = (bh * N + row) * (long)D;
                    float kv[CPL], mx = NEG_INF_B;
#pragma unroll
                    for (int e = 0; e < CPL; ++e) {
                        kv[e] = to_f32<bf16>(k[base + lane + 64 * e]);
                        Vr[r * D + lane + 64 * e] = to_f32<bf16>(v[base + lane + 64 * e]);
                        mx = fmaxf(mx, kv[e]);
                    }
                    mx = wave_max(mx);
                    float se = 0.f;
#pragma unroll
                    for (int e = 0; e < CPL; ++e) {
                        kv[e] = __expf(kv[e] - mx);
                        se += kv[e];
                    }
                    se = wave_sum(se);
#pragma unroll
                    for (int e = 0; e < CPL; ++e) Ph[r * D + lane + 64 * e] = kv[e] / se;
                } else {
#pragma unroll
                    for (int e = 0; e < CPL; ++e) {
                        Ph[r * D + lane + 64 * e] = 0.f;
                        Vr[r * D + lane + 64 * e] = 0.f;
                    }
                }
            }
            __syncthreads();
            // v'_u[c] = sum_e W[c][e] v_u[e]: thread (c = tid % D, rows tid / D + (256 / D) n)
            for (int r = tid / D; r < RB; r += 256 / D) {
                const int c = tid % D;
                float x = 0.f;
                for (int e = 0; e < D; ++e) x += Wl[c * HS + e] * Vr[r * D + e];
                Vp[r * D + c] = x;
            }
            __syncthreads();
            // dphi[a] = sum_c dh[c][a] v'[c] + dz[a]; dk += phi * (dphi - phi . dphi)
            for (int rr = 0; rr < RB / 4; ++rr) {
                const int r = (RB / 4) * wave + rr;
                const int row = 64 * j + RB * pass + r;
                if (row >= N) continue;
                float dph[CPL], pd = 0.f;
#pragma unroll
                for (int e = 0; e < CPL; ++e) {
                    const int a = lane + 64 * e;
                    float x = Dz[a];
                    for (int c = 0; c < D; ++c) x += Dh[c * HS + a] * Vp[r * D + c];
                    dph[e] = x;
                    pd += Ph[r * D + a] * x;
                }
                pd = wave_sum(pd);
                float *kg = dk + (bh * N + row) * (long)D;
#pragma unroll
                for (int e = 0; e < CPL; ++e) {
                    const int a = lane + 64 * e;
                    kg[a] += Ph[r * D + a] * (dph[e] - pd);
                }
            }
            __syncthreads();
            // dv'_u[c] = sum_a phi_a dh[c][a], kept in Vp
            for (int r = tid / D; r < RB; r += 256 / D) {
                const int c = tid % D;
                float x = 0.f;
                for (int a = 0; a < D; ++a) x += Ph[r * D + a] * Dh[c * HS + a];
                Vp[r * D + c] = x;
            }
            __syncthreads();
            // dv_u[e] += sum_c dv'_u[c] W[c][e]
            for (int r = tid / D; r < RB; r += 256 / D) {
                const int e = tid % D;
                const int row = 64 * j + RB * pass + r;
                if (row >= N) continue;
                float x = 0.f;
                for (int c = 0; c < D; ++c) x += Vp[r * D + c] * Wl[c * HS + e];
                dv[(bh * N + row) * (long)D + e] += x;
            }
            // dW[c][e] += sum_u dv'_u[c] v_u[e]
            for (int r = 0; r < RB; ++r) {
                const float ve = Vr[r * D + we];
#pragma unroll
                for (int x = 0; x < WC; ++x) wacc[x] += Vp[r * D + wc0 + x] * ve;
            }
        }
    }
#pragma unroll
    for (int x = 0; x < WC; ++x) atomicAdd(&dw[(wc0 + x) * D + we], wacc[x]);
}

// ---- launchers -----------------------------------------------------------------

hipError_t launch_zero(float *p, long n, hipStream_t st) {
    bwd_zero_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(p, n);
    return hipGetLastError();
}

hipError_t launch_backward_dq(const BackwardArgs &a, hipStream_t st) {
    const long Gq = a.BH * a.Nb;
    const int per = (int)((Gq + 7) / 8);
    const float sl2 = 1.4426950408889634f / sqrtf((float)a.D), scale = 1.f / sqrtf((float)a.D);
    const unsigned g1 = (unsigned)((a.BH * a.Nb + 255) / 256);
    bwd_tlists_kernel<<<g1, 256, 0, st>>>(a.mask, a.BH, a.Nb, a.tlist, a.tcnt);
    if (a.D == 64)
        bwd_dq_kernel<64><<<(unsigned)(8L * per), 256, 0, st>>>((const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v,
            (const bf16 *)a.dout, a.o_s, a.lse, a.crit, a.kc, a.dq, a.dbuf, Gq, per, a.N, a.Nb, sl2, scale);
    else
        bwd_dq_kernel<128><<<(unsigned)(8L * per), 256, 0, st>>>((const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v,
            (const bf16 *)a.dout, a.o_s, a.lse, a.crit, a.kc, a.dq, a.dbuf, Gq, per, a.N, a.Nb, sl2, scale);
    return hipGetLastError();
}

hipError_t launch_backward_dkv(const BackwardArgs &a, hipStream_t st) {
    const long Gq = a.BH * a.Nb;
    const int per = (int)((Gq + 7) / 8);
    const float sl2 = 1.4426950408889634f / sqrtf((float)a.D), scale = 1.f / sqrtf((float)a.D);
    if (a.D == 64)
        bwd_dkv_kernel<64><<<(unsigned)(8L * per), 256, 0, st>>>((const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v,
            (const bf16 *)a.dout, a.lse, a.dbuf, a.tlist, a.tcnt, a.dk, a.dv, Gq, per, a.N, a.Nb, sl2, scale);
    else
        bwd_dkv_kernel<128><<<(unsigned)(8L * per), 256, 0, st>>>((const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v,
            (const bf16 *)a.dout, a.lse, a.dbuf, a.tlist, a.tcnt, a.dk, a.dv, Gq, per, a.N, a.Nb, sl2, scale);
    return hipGetLastError();
}

hipError_t launch_backward_lin_rows(const BackwardArgs &a, hipStream_t st) {
    // zero dW, the transposed indicator and its unit counts
    bwd_zero_kernel<<<(unsigned)((a.D * a.D + 255) / 256), 256, 0, st>>>(a.dw, (long)a.D * a.D);
    const long nt = a.BH * a.Nb * (long)a.Nbc;
    bwd_margT_kernel<<<(unsigned)((nt + 255) / 256), 256, 0, st>>>(a.mask, a.BH, a.Nb, a.Nbc, a.margT, a.unit);
    const unsigned rows = (unsigned)(a.BH * a.Nbc);
    if (a.D == 64)
        bwd_lin_row_kernel<64><<<rows, 256, 0, st>>>((const bf16 *)a.q, (const bf16 *)a.dout, (const f16 *)a.hhat,
                                                     a.mcount, a.Lp, a.dq, a.dhrow, a.BH, a.N, a.Nb, a.Nbc);
    else
        bwd_lin_row_kernel<128><<<rows, 256, 0, st>>>((const bf16 *)a.q, (const bf16 *)a.dout, (const f16 *)a.hhat,
                                                      a.mcount, a.Lp, a.dq, a.dhrow, a.BH, a.N, a.Nb, a.Nbc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    AssembleArgs as{};
    as.marg = a.margT; as.hs = a.dhrow; as.mcount = a.unit; as.hhat = a.dhs;
    as.BH = a.BH; as.Nb = a.Nb; as.Nbc = a.Nbc; as.Nbp = a.Nbc; as.Lp = a.Lp; as.f32 = true;
    return launch_assemble(as, st);
}

hipError_t launch_backward_lin_keys(const BackwardArgs &a, hipStream_t st) {
    int dev = 0, cus = 0;
    hipGetDevice(&dev);
    hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const unsigned gk = (unsigned)std::min<long>(a.BH * a.Nb, (long)std::max(cus, 1));
    if (a.D == 64)
        bwd_lin_key_kernel<64><<<gk, 256, 0, st>>>((const bf16 *)a.k, (const bf16 *)a.v, a.w, a.dhs, a.Lp, a.dk, a.dv,
                                                   a.dw, a.BH, a.N, a.Nb);
    else
        bwd_lin_key_kernel<128><<<gk, 256, 0, st>>>((const bf16 *)a.k, (const bf16 *)a.v, a.w, a.dhs, a.Lp, a.dk, a.dv,
                                                    a.dw, a.BH, a.N, a.Nb);
    return hipGetLastError();
}

}  // namespace sla
