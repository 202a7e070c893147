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
// Every product of the linear part runs on fp16 MFMA with fp32 accumulation;
// operands derived from dO (dO, dh'_j, dv') carry a power of two per block
// that puts the block's largest magnitude in [0.5, 1); the per-row state
// gradients dĤ'_i are stored as fp16 with such an exponent per row, and the
// transposed sum applies the exponents in its 0/1 operand.
#include "sla_device.h"
#include "sla_launch.h"
#include "tile_common.h"

#include <algorithm>

namespace sla {

namespace {
constexpr float NEG_INF_B = -__builtin_inff();
constexpr int EXP_ZERO = -(1 << 20);                     // exponent of an all-zero state-gradient row
}

// ---- transposed lists and indicator ------------------------------------------

// one wave per (head, key block j): the query blocks i with j critical, ascending
__global__ __launch_bounds__(256) void bwd_tlists_kernel(const int8_t *__restrict__ mask, long BH, int Nb,
                                                         int32_t *__restrict__ tlist, int32_t *__restrict__ tcnt) {
    const long t = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= BH * Nb) return;
    const int lane = threadIdx.x & 63;
    const long bh = t / Nb;
    const int j = (int)(t % Nb);
    const int8_t *m = mask + bh * Nb * (long)Nb + j;
    int32_t *out = tlist + t * (long)Nb;
    int c = 0;
    for (int i0 = 0; i0 < Nb; i0 += 64) {
        const int i = i0 + lane;
        const bool hit = i < Nb && m[(long)i * Nb] == 1;
        const uint64_t bal = __ballot(hit);
        if (hit) out[c + __popcll(bal & ((1ull << lane) - 1))] = i;
        c += __popcll(bal);
    }
    if (lane == 0) tcnt[t] = c;
}

// mbits[bh][w][j] (w < Nbc / 32, j < Nbp): bit b set when key block j is
// marginal for query block i = 32 w + b (i, j < Nb): the transposed marginal
// indicator as bits
__global__ __launch_bounds__(256) void bwd_mbitsT_kernel(const int8_t *__restrict__ mask, long BH, int Nb, int Nbc,
                                                         int Nbp, uint32_t *__restrict__ mbits) {
    const long t = (long)blockIdx.x * 256 + threadIdx.x;
    const int nw = Nbc / 32;
    if (t >= BH * nw * (long)Nbp) return;
    const int j = (int)(t % Nbp);
    const long r = t / Nbp;
    const int wd = (int)(r % nw);
    const long bh = r / nw;
    const int i0 = 32 * wd;
    uint32_t bits = 0;
    if (j < Nb)
        for (int b = 0; b < 32; ++b) {
            const int i = i0 + b;
            if (i < Nb && mask[(bh * Nb + i) * (long)Nb + j] == 0) bits |= 1u << b;
        }
    mbits[t] = bits;
}

// one workgroup per head: R = the largest exponent of the head's state-
// gradient rows; per row k its fp16 exponent byte for the transposed sum,
// that of 2^(E_k - R + 14) (0 for rows more than 28 below R), and the
// head's output exponent R + c, c = ceil(log2 Nbc)
__global__ __launch_bounds__(256) void bwd_rowexp_kernel(const int32_t *__restrict__ dexp, int Nbc,
                                                         uint8_t *__restrict__ kbyte, int32_t *__restrict__ hexp) {
    __shared__ int Rw[4];
    const long bh = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int32_t *e = dexp + bh * (long)Nbc;
    int r = EXP_ZERO;
    for (int k = tid; k < Nbc; k += 256) r = max(r, e[k]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) r = max(r, __shfl_xor(r, o));
    if (lane == 0) Rw[wave] = r;
    __syncthreads();
    const int R = max(max(Rw[0], Rw[1]), max(Rw[2], Rw[3]));
    for (int k = tid; k < Nbc; k += 256) {
        const int dlt = e[k] - R;
        kbyte[bh * Nbc + k] = dlt >= -28 ? (uint8_t)((dlt + 29) << 2) : (uint8_t)0;
    }
    if (tid == 0) hexp[bh] = R + (32 - __clz(Nbc - 1));
}

__global__ __launch_bounds__(256) void bwd_zero_kernel(float *__restrict__ p, long n) {
    const long t = (long)blockIdx.x * 256 + threadIdx.x;
    if (t < n) p[t] = 0.f;
}

// ---- sparse part ------------------------------------------------------------

// One workgroup of 4 waves per query block i: wave (rh, kh) takes query rows
// 32rh .. +31 against key half kh of every critical block.  Per block: S^T =
// K Q^T and dP^T = V dO^T on the matrix core (K, V rows from LDS, Q and dO
// in registers), dS^T in the VALU, dQ^T += K^T dS^T (transposing reads of the
// same K tile).  Tiles go global -> LDS through a two-slot ring, one barrier
// per block; 64 KB of LDS lets two workgroups share a compute unit.
template <int D>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                                                        const bf16 *__restrict__ v, const bf16 *__restrict__ dout,
                                                        const float *__restrict__ o_s, const float *__restrict__ lse,
                                                        const int32_t *__restrict__ crit, int kc,
                                                        float *__restrict__ dq, float *__restrict__ dbuf, long G,
                                                        int per_xcd, int N, int Nb, float sl2, float scale) {
    using T = bf16;
    constexpr int TILE = 64 * D, NS = D / 16, NCT = D / 32, NCH = NCT / 2, NBW = D / 32;
    // each slot of the K and V rings is an array of its own, so that reads of
    // one slot do not wait for loads still landing in the other
    __shared__ __attribute__((aligned(1024))) T Kk0[TILE];
    __shared__ __attribute__((aligned(1024))) T Kk1[TILE];
    __shared__ __attribute__((aligned(1024))) T Vk0[TILE];
    __shared__ __attribute__((aligned(1024))) T Vk1[TILE];
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
    if (kh == 0 && hh == 0 && qvalid) dbuf[bh * (64L * Nb) + qrow] = Dr;
    const float lse2 = qvalid ? lse[bh * (64L * Nb) + qrow] : __builtin_inff();

    int koff[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int r = 32 * kh + l32;
        koff[s] = r * D + ((2 * s + hh) ^ kswz<D>(r)) * 8;
    }
    int toff[NCT][2];
    tr_offsets<D>(lane, toff);
    uint32_t ok_[NBW];
#pragma unroll
    for (int u = 0; u < NBW; ++u) ok_[u] = off_klayout<D>((wave * NBW + u) * 1024 + 16 * lane);
    const uint32_t head_bytes = (uint32_t)((long)N * D * sizeof(T));
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + bh * N * (long)D, head_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + bh * N * (long)D, head_bytes);
    const int32_t *cl = crit + (bh * Nb + i) * (long)kc;
    auto load = [&](int c, int slot) __attribute__((always_inline)) {
        const uint32_t off = (uint32_t)(64L * cl[c] * D * sizeof(T));
#pragma unroll
        for (int u = 0; u < NBW; ++u) {
            dma16(rk, (slot ? Kk1 : Kk0) + (wave * NBW + u) * 512, ok_[u] + off, 0);
            dma16(rv, (slot ? Vk1 : Vk0) + (wave * NBW + u) * 512, ok_[u] + off, 0);
        }
    };
    f32x16 dqt[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqt[ct][r] = 0.f;
    auto compute = [&](int c, int slot) __attribute__((always_inline)) {
        // only a list's last block can be the ragged last key block (the
        // lists are ascending); its list entry is read only there
        const bool rag = c == kc - 1 && 64 * cl[c] + 64 > N;
        v8<T> a[NS];
        f32x16 sacc, pacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = pacc[r] = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s) a[s] = ld8<T>((slot ? Kk1 : Kk0) + koff[s]);
#pragma unroll
        for (int s = 0; s < NS; ++s) mma16(sacc, a[s], qf[s]);
#pragma unroll
        for (int s = 0; s < NS; ++s) a[s] = ld8<T>((slot ? Vk1 : Vk0) + koff[s]);
#pragma unroll
        for (int s = 0; s < NS; ++s) mma16(pacc, a[s], df[s]);
        v8<T> dsb[2];
        if (rag) {
            const int lim = N - 64 * cl[c];              // keys of the block below N
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 32 * kh + 8 * (r >> 2) + 4 * hh + (r & 3);
                const float p = key < lim ? fast_exp2(__builtin_fmaf(sacc[r], sl2, -lse2)) : 0.f;
                dsb[r >> 3][r & 7] = from_f32<T>(p * (pacc[r] - Dr));
            }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = fast_exp2(__builtin_fmaf(sacc[r], sl2, -lse2));
                dsb[r >> 3][r & 7] = from_f32<T>(p * (pacc[r] - Dr));
            }
        }
        v8<T> at[NCT][2];
        read_tr<T, D>(slot ? Kk1 : Kk0, kh, toff, at);
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
    // [2 waves][NCH*4][64] f32x4: waves 0, 1 in the first K slot, 2, 3 in the second
    float *xo = reinterpret_cast<float *>(wave < 2 ? Kk0 : Kk1);
    static_assert(2 * NCH * 4 * 64 * 16 <= TILE * 2, "two waves' exchange fits a slot");
    f32x16 mine[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        mine[c] = kh == 0 ? dqt[c] : dqt[NCH + c];
        const f32x16 give = kh == 0 ? dqt[NCH + c] : dqt[c];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 y = {give[4 * g], give[4 * g + 1], give[4 * g + 2], give[4 * g + 3]};
            *reinterpret_cast<f32x4 *>(xo + (((wave & 1) * NCH * 4 + c * 4 + g) * 64 + lane) * 4) = y;
        }
    }
    lds_barrier();
    const int partner = wave ^ 1;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 y = *reinterpret_cast<const f32x4 *>(xo + (((partner & 1) * NCH * 4 + c * 4 + g) * 64 + lane) * 4);
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

// One workgroup of 4 waves per key block j, two workgroups per compute unit.
// Per query block i of j's list, in two steps with a barrier between them:
//   produce, wave (kh, rh): keys 32kh .. +31 against query rows 32rh .. +31:
//     S = Q K^T and dP = dO V^T on the matrix core (Q, dO rows from LDS, K
//     and V rows in registers), P and dS = P (dP - D) in the VALU, written as
//     bf16 MFMA operands to the wave's LDS slot;
//   consume, wave (kh, ch): for both row halves, dV^T += dO^T P and dK^T +=
//     Q^T dS for the channels of half ch (transposing reads of the same dO
//     and Q tiles, P and dS from the producers' slots).
// Each wave thus owns a quarter of dK and dV, so no partial sums are merged.
template <int D>
__global__ __launch_bounds__(256, 2) void bwd_dkv_kernel(const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                                                         const bf16 *__restrict__ v, const bf16 *__restrict__ dout,
                                                         const float *__restrict__ lse, const float *__restrict__ dbuf,
                                                         const int32_t *__restrict__ tlist,
                                                         const int32_t *__restrict__ tcnt, float *__restrict__ dk,
                                                         float *__restrict__ dv, long G, int per_xcd, int N, int Nb,
                                                         float sl2, float scale) {
    using T = bf16;
    constexpr int TILE = 64 * D, NS = D / 16, NCT = D / 32, NCH = NCT / 2, NBW = D / 32;
    // each ring slot an array of its own (see the dQ kernel)
    __shared__ __attribute__((aligned(1024))) T Qk0[TILE];
    __shared__ __attribute__((aligned(1024))) T Qk1[TILE];
    __shared__ __attribute__((aligned(1024))) T Ok0[TILE];
    __shared__ __attribute__((aligned(1024))) T Ok1[TILE];
    __shared__ __attribute__((aligned(16))) v8<T> PB[4][4][64];     // [wave][pb0, pb1, ds0, ds1][lane]
    const long logical = (long)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (logical >= G) return;
    const long bh = logical / Nb;
    const int j = (int)(logical % Nb);
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, hh = lane >> 5;
    const int kh = wave >> 1, rh = wave & 1, ch = wave & 1;
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
    int toff[NCT][2];
    tr_offsets<D>(lane, toff);
    int tofc[NCH][2];                                    // the consumer's channel tiles only
#pragma unroll
    for (int c2 = 0; c2 < NCH; ++c2) {
        tofc[c2][0] = ch ? toff[NCH + c2][0] : toff[c2][0];
        tofc[c2][1] = ch ? toff[NCH + c2][1] : toff[c2][1];
    }
    uint32_t ok_[NBW];
#pragma unroll
    for (int u = 0; u < NBW; ++u) ok_[u] = off_klayout<D>((wave * NBW + u) * 1024 + 16 * lane);
    const uint32_t head_bytes = (uint32_t)((long)N * D * sizeof(T));
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + bh * N * (long)D, head_bytes);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(dout + bh * N * (long)D, head_bytes);
    // 32-bit entries: uniform, so they come through the scalar cache and no
    // wait for them waits for the tile loads in flight
    const int32_t *tl = tlist + (bh * Nb + j) * (long)Nb;
    const int cnt = tcnt[bh * Nb + j];
    auto load = [&](int c, int slot) __attribute__((always_inline)) {
        const uint32_t off = (uint32_t)(64L * tl[c] * D * sizeof(T));
#pragma unroll
        for (int u = 0; u < NBW; ++u) {
            dma16(rq, (slot ? Qk1 : Qk0) + (wave * NBW + u) * 512, ok_[u] + off, 0);
            dma16(ro, (slot ? Ok1 : Ok0) + (wave * NBW + u) * 512, ok_[u] + off, 0);
        }
    };
    f32x16 dvt[NCH], dkt[NCH];
#pragma unroll
    for (int ct = 0; ct < NCH; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) dvt[ct][r] = dkt[ct][r] = 0.f;
    // the rows of the accumulator this lane holds (four runs of four, 16-byte
    // aligned in the per-head rows of 64 Nb), their lse and D; issued before
    // the next tile's loads, so that waiting for them does not wait for those
    auto fetch = [&](int c, f32x4 (&lv)[4], f32x4 (&dv4)[4]) __attribute__((always_inline)) {
        const long rb = bh * (64L * Nb) + 64 * tl[c] + 32 * rh + 4 * hh;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            lv[g] = *reinterpret_cast<const f32x4 *>(lse + rb + 8 * g);
            dv4[g] = *reinterpret_cast<const f32x4 *>(dbuf + rb + 8 * g);
        }
        __builtin_amdgcn_sched_barrier(0);               // keep them ahead of the tile loads
    };
    auto produce = [&](int c, int slot, const f32x4 (&lv)[4], const f32x4 (&dv4)[4]) __attribute__((always_inline)) {
        const int i = tl[c];
        float lr[16], dr[16];
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool ok = 64 * i + 32 * rh + 8 * g + 4 * hh + e < N;
                lr[4 * g + e] = ok ? lv[g][e] : __builtin_inff();
                dr[4 * g + e] = ok ? dv4[g][e] : 0.f;
            }
        f32x16 sacc, pacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = pacc[r] = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s) mma16(sacc, ld8<T>((slot ? Qk1 : Qk0) + koff[s]), kf[s]);
#pragma unroll
        for (int s = 0; s < NS; ++s) mma16(pacc, ld8<T>((slot ? Ok1 : Ok0) + koff[s]), vf[s]);
        v8<T> pb[2], dsb[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = kvalid ? fast_exp2(__builtin_fmaf(sacc[r], sl2, -lr[r])) : 0.f;
            pb[r >> 3][r & 7] = from_f32<T>(p);
            dsb[r >> 3][r & 7] = from_f32<T>(p * (pacc[r] - dr[r]));
        }
        PB[wave][0][lane] = pb[0];
        PB[wave][1][lane] = pb[1];
        PB[wave][2][lane] = dsb[0];
        PB[wave][3][lane] = dsb[1];
    };
    auto consume = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2) {
            const int src = 2 * kh + r2;
            const v8<T> p0 = PB[src][0][lane], p1 = PB[src][1][lane];
            const v8<T> d0 = PB[src][2][lane], d1 = PB[src][3][lane];
#pragma unroll
            for (int c2 = 0; c2 < NCH; ++c2) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const T *bo = (slot ? Ok1 : Ok0) + (32 * r2 + 16 * ks) * D;
                    const T *bq = (slot ? Qk1 : Qk0) + (32 * r2 + 16 * ks) * D;
                    mma16(dvt[c2], cat8<T>(lds_tr_raw<T>(bo + tofc[c2][0]), lds_tr_raw<T>(bo + tofc[c2][1])),
                          ks ? p1 : p0);
                    mma16(dkt[c2], cat8<T>(lds_tr_raw<T>(bq + tofc[c2][0]), lds_tr_raw<T>(bq + tofc[c2][1])),
                          ks ? d1 : d0);
                }
            }
        }
    };
    if (cnt > 0) {
        load(0, 0);
        wait_vm0();
        lds_barrier();
        int c = 0;
        f32x4 lv[4], dv4[4];
        for (; c + 1 < cnt; c += 2) {
            fetch(c, lv, dv4);
            load(c + 1, 1);
            produce(c, 0, lv, dv4);
            lds_barrier();
            consume(0);
            wait_vm0();
            lds_barrier();
            fetch(c + 1, lv, dv4);
            // past the end it loads the last block again (slot 0 is free):
            // every path then has the same loads in flight, which keeps the
            // compiler's waits for the rows partial
            load(min(c + 2, cnt - 1), 0);
            produce(c + 1, 1, lv, dv4);
            lds_barrier();
            consume(1);
            wait_vm0();
            lds_barrier();
        }
        if (c < cnt) {
            fetch(c, lv, dv4);
            produce(c, 0, lv, dv4);
            lds_barrier();
            consume(0);
        }
        wait_vm0();                                      // no load into LDS outlives the loop
    }
    if (!kvalid) return;
    float *vrow = dv + (bh * N + krow) * (long)D;
    float *krw = dk + (bh * N + krow) * (long)D;
#pragma unroll
    for (int c2 = 0; c2 < NCH; ++c2) {
        const int c0 = 32 * (NCH * ch + c2);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 y = {dvt[c2][4 * g], dvt[c2][4 * g + 1], dvt[c2][4 * g + 2], dvt[c2][4 * g + 3]};
            const f32x4 z = {dkt[c2][4 * g] * scale, dkt[c2][4 * g + 1] * scale, dkt[c2][4 * g + 2] * scale,
                             dkt[c2][4 * g + 3] * scale};
            *reinterpret_cast<f32x4 *>(vrow + c0 + 8 * g + 4 * hh) = y;
            *reinterpret_cast<f32x4 *>(krw + c0 + 8 * g + 4 * hh) = z;
        }
    }
}

// ---- linear part --------------------------------------------------------------

namespace {
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
// power of two that brings the largest magnitude m of a tile into [0.5, 1)
// (1 for m = 0 or not finite), so that f16 operands keep their precision
// whatever the scale of the gradient
__device__ __forceinline__ float pow2_scale(float m) {
    if (!(m > 0.f) || !(m < __builtin_inff())) return 1.f;
    int ex = 0;
    frexpf(m, &ex);
    return ldexpf(1.f, -max(ex, -125));
}
}  // namespace

// One workgroup of 4 waves per query block i (blocks past Nb and rows without
// marginal blocks write zero state gradients).
//  1. VALU, a thread per 8-channel chunk of a row: Pn_r = phi(q_r) / den_r
//     and s dO_r (s a power of two shared by the block) as f16 rows in LDS,
//     with Ĥ'_i^T (stored [c][a]).
//  2. matrix core, wave (rh, ch): y^T = H Pn^T (channels c of half ch,
//     tokens of half rh) and s X^T = H^T (s dO)^T (channels a of half ch);
//     per token g = dO.y, e_a = X_a - g Ẑ_a, t = Pn.e (the two channel halves
//     summed through LDS), dq_a += Pn_a (e_a - den t).
//  3. matrix core: dĤ'_i = dO^T Pn / m_i, VALU: dẐ_i = -g^T Pn / m_i; with
//     M = f 2^E (f in [0.5, 1)) the row's largest magnitude, written as fp16
//     values times 2^-E, and E (EXP_ZERO for a zero row) in dexp.
template <int D>
__global__ __launch_bounds__(256, 2) void bwd_lin_row_kernel(const bf16 *__restrict__ q, const bf16 *__restrict__ dout,
                                                             const f16 *__restrict__ hhat,
                                                             const int32_t *__restrict__ mcount, int Lp,
                                                             float *__restrict__ dq, f16 *__restrict__ dhr,
                                                             int32_t *__restrict__ dexp, long BH, int N, int Nb,
                                                             int Nbc) {
    constexpr int STR = D + 8;                           // padded row stride of the f16 tiles
    constexpr int CPR = D / 8, RPP = 256 / CPR, NP = 64 / RPP;
    constexpr int NCT = D / 64;                          // 32-channel tiles per channel half
    constexpr int TPW = (D / 32) * (D / 32) / 4;         // dĤ' tiles per wave
    __shared__ __attribute__((aligned(16))) f16 Hs[D * STR];
    __shared__ __attribute__((aligned(16))) f16 Pn[64 * STR];
    __shared__ __attribute__((aligned(16))) f16 Ds[64 * STR];
    __shared__ float Zs[D], Dn[64], Gr[64], Gx[2][64], Tx[2][64], Red[4];

    const long blk = blockIdx.x;
    const long bh = blk / Nbc;
    const int i = (int)(blk % Nbc);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5, grp = lane >> 4;
    f16 *dh = dhr + (bh * Nbc + i) * (long)Lp;
    const int mc = i < Nb ? mcount[bh * Nb + i] : 0;
    if (mc == 0) {
        for (int x = tid; x < Lp / 8; x += 256) st_chunk(dh + 8 * x, zero_chunk());
        if (tid == 0) dexp[bh * Nbc + i] = EXP_ZERO;
        return;
    }
    const f16 *hr = hhat + (bh * Nb + i) * (long)Lp;
    for (int x = tid; x < D * CPR; x += 256) st_chunk(&Hs[(x / CPR) * STR + 8 * (x % CPR)], ld_chunk(hr + 8 * x));
    if (tid < D) Zs[tid] = (float)hr[D * D + tid];

    // 1. rows
    const int p = tid % CPR;
    float zf[8];
    {
        const Chunk zc = ld_chunk(hr + D * D + 8 * p);
        const f16 *z = reinterpret_cast<const f16 *>(&zc);
#pragma unroll
        for (int e = 0; e < 8; ++e) zf[e] = (float)z[e];
    }
    Chunk dc[NP];
    float dmax = 0.f;
#pragma unroll
    for (int n = 0; n < NP; ++n) {
        const int r = RPP * n + tid / CPR, row = 64 * i + r;
        const bool ok = row < N;
        const long base = (bh * N + row) * (long)D + 8 * p;
        const Chunk qc = ok ? ld_chunk(q + base) : zero_chunk();
        dc[n] = ok ? ld_chunk(dout + base) : zero_chunk();
        const bf16 *qx = reinterpret_cast<const bf16 *>(&qc);
        float ph[8], mx = NEG_INF_B;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            ph[e] = (float)qx[e];
            mx = fmaxf(mx, ph[e]);
        }
#pragma unroll
        for (int o = 1; o < CPR; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        float se = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            ph[e] = __expf(ph[e] - mx);
            se += ph[e];
        }
#pragma unroll
        for (int o = 1; o < CPR; o <<= 1) se += __shfl_xor(se, o);
        const float ise = 1.f / se;
        float den = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            ph[e] *= ise;
            den += ph[e] * zf[e];
        }
#pragma unroll
        for (int o = 1; o < CPR; o <<= 1) den += __shfl_xor(den, o);
        const float inv = ok ? 1.f / den : 0.f;
        f16 pn[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pn[e] = (f16)(ph[e] * inv);
        __builtin_memcpy(&Pn[r * STR + 8 * p], pn, sizeof(pn));
        if (p == 0) Dn[r] = ok ? den : 1.f;
        const bf16 *dx = reinterpret_cast<const bf16 *>(&dc[n]);
#pragma unroll
        for (int e = 0; e < 8; ++e) dmax = fmaxf(dmax, fabsf((float)dx[e]));
    }
    dmax = wave_max(dmax);
    if (lane == 0) Red[wave] = dmax;
    __syncthreads();
    const float sc = pow2_scale(fmaxf(fmaxf(Red[0], Red[1]), fmaxf(Red[2], Red[3])));
#pragma unroll
    for (int n = 0; n < NP; ++n) {
        const int r = RPP * n + tid / CPR;
        const bf16 *dx = reinterpret_cast<const bf16 *>(&dc[n]);
        f16 ds[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) ds[e] = (f16)((float)dx[e] * sc);
        __builtin_memcpy(&Ds[r * STR + 8 * p], ds, sizeof(ds));
    }
    __syncthreads();

    // 2. y^T and s X^T for the wave's channel half and token half
    const int rh = wave & 1, chh = wave >> 1;
    const int r = 32 * rh + l32;                         // this lane's token
    const int row = 64 * i + r;
    float *qg = dq + (bh * N + row) * (long)D;
    // this lane's dQ values, read now so that the load overlaps the products
    f32x4 dqv[NCT][4];
#pragma unroll
    for (int mt = 0; mt < NCT; ++mt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int a0 = (D / 2) * chh + 32 * mt + 8 * g + 4 * hh;
            dqv[mt][g] = row < N ? *reinterpret_cast<const f32x4 *>(qg + a0) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    f32x16 yt[NCT], xt[NCT];
#pragma unroll
    for (int mt = 0; mt < NCT; ++mt)
#pragma unroll
        for (int x = 0; x < 16; ++x) yt[mt][x] = xt[mt][x] = 0.f;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        const int k0 = 16 * s + 8 * hh;
        const v8<f16> bp = ld8<f16>(&Pn[r * STR + k0]);
        const v8<f16> bd = ld8<f16>(&Ds[r * STR + k0]);
#pragma unroll
        for (int mt = 0; mt < NCT; ++mt) {
            const int t0 = (D / 2) * chh + 32 * mt, n0 = t0 + 16 * (grp & 1);
            mma16(yt[mt], ld8<f16>(&Hs[(t0 + l32) * STR + k0]), bp);
            mma16(xt[mt], cat8<f16>(lds_col4<f16>(Hs, STR, k0, n0, lane), lds_col4<f16>(Hs, STR, k0 + 4, n0, lane)), bd);
        }
    }
    // lane (r, hh) holds channels 64 ch + 32 mt + 8 g + 4 hh + 0..3 of token r
    float gp = 0.f;
#pragma unroll
    for (int mt = 0; mt < NCT; ++mt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const v4<f16> dd = ld4<f16>(&Ds[r * STR + (D / 2) * chh + 32 * mt + 8 * g + 4 * hh]);
#pragma unroll
            for (int e = 0; e < 4; ++e) gp += (float)dd[e] * yt[mt][4 * g + e];
        }
    gp = half_swap_sum(gp);
    if (hh == 0) Gx[chh][r] = gp;
    __syncthreads();
    const float gs = Gx[0][r] + Gx[1][r];                // s g_r
    v4<f16> pn4[NCT][4];
    float tp = 0.f;
#pragma unroll
    for (int mt = 0; mt < NCT; ++mt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int a0 = (D / 2) * chh + 32 * mt + 8 * g + 4 * hh;
            pn4[mt][g] = ld4<f16>(&Pn[r * STR + a0]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xt[mt][4 * g + e] -= gs * Zs[a0 + e];    // s e_a
                tp += (float)pn4[mt][g][e] * xt[mt][4 * g + e];
            }
        }
    tp = half_swap_sum(tp);
    if (hh == 0) {
        Tx[chh][r] = tp;
        if (chh == 0) Gr[r] = gs / sc;
    }
    __syncthreads();
    const float dts = Dn[r] * (Tx[0][r] + Tx[1][r]), isc = 1.f / sc;
    if (row < N) {
#pragma unroll
        for (int mt = 0; mt < NCT; ++mt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int a0 = (D / 2) * chh + 32 * mt + 8 * g + 4 * hh;
                f32x4 cur = dqv[mt][g];
#pragma unroll
                for (int e = 0; e < 4; ++e) cur[e] += (float)pn4[mt][g][e] * (xt[mt][4 * g + e] - dts) * isc;
                *reinterpret_cast<f32x4 *>(qg + a0) = cur;
            }
    }

    // 3. dĤ'[c][a] = sum_r dO[r][c] Pn[r][a] / m: tiles (ct, at), K = the 64 tokens
    const float osc = 1.f / ((float)mc * sc), inv_m = 1.f / (float)mc;
    f32x16 acc[TPW];
    float vmax = 0.f;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int x = wave * TPW + t, ct = x / (D / 32), at = x % (D / 32);
        const int nc = 32 * ct + 16 * (grp & 1), na = 32 * at + 16 * (grp & 1);
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int k0 = 16 * s + 8 * hh;
            mma16(acc[t], cat8<f16>(lds_col4<f16>(Ds, STR, k0, nc, lane), lds_col4<f16>(Ds, STR, k0 + 4, nc, lane)),
                  cat8<f16>(lds_col4<f16>(Pn, STR, k0, na, lane), lds_col4<f16>(Pn, STR, k0 + 4, na, lane)));
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            acc[t][e] *= osc;
            vmax = fmaxf(vmax, fabsf(acc[t][e]));
        }
    }
    float z = 0.f;
    if (tid < D) {
        for (int r2 = 0; r2 < 64; ++r2) z += Gr[r2] * (float)Pn[r2 * STR + tid];
        z = -z * inv_m;
        vmax = fmaxf(vmax, fabsf(z));
    }
    vmax = wave_max(vmax);
    if (lane == 0) Red[wave] = vmax;                     // its earlier reads ended two barriers ago
    __syncthreads();
    const float M = fmaxf(fmaxf(Red[0], Red[1]), fmaxf(Red[2], Red[3]));
    int E = EXP_ZERO;
    if (M > 0.f) {
        frexpf(M, &E);
        E = min(max(E, -125), 125);
    }
    const float xs = M > 0.f ? ldexpf(1.f, -E) : 0.f;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int x = wave * TPW + t, ct = x / (D / 32), at = x % (D / 32);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int c = 32 * ct + 8 * (e >> 2) + 4 * hh + (e & 3);
            dh[(long)c * D + 32 * at + l32] = (f16)(acc[t][e] * xs);
        }
    }
    if (tid < D) dh[D * D + tid] = (f16)(z * xs);
    for (int x = D * D + D + tid; x < Lp; x += 256) dh[x] = (f16)0.f;
    if (tid == 0) dexp[bh * Nbc + i] = E;
}

// Linear part, keys: persistent workgroups of D/16 waves over the key blocks
// j (W as f16 in LDS once per workgroup; dW summed in registers and added
// once at the end).  Per block, with dh'_j (stored [c][a]) times a power of
// two s as f16 in LDS:
//  1. VALU: phi(k_u) and v_u as f16 rows.
//  2. matrix core, wave (x, ut), x a 32-channel tile, ut a 32-token half:
//     v'^T = W V^T and s dv'^T = (s dh') phi^T, both to LDS as rows [u][c].
//  3. matrix core: s dphi^T = (s dh')^T v'^T (a tile x), s dv^T = W^T s dv'^T
//     (e tile x), dW tiles += s dv'^T V / s; VALU: dphi = (.)/s + dz,
//     pd = phi.dphi (tiles summed through LDS), dk += phi (dphi - pd),
//     dv += (.)/s.
// dh'_j comes as fp16 values x with dh'_j = x 2^Q, Q the head's output
// exponent of the transposed sum.
template <int D>
__global__ __launch_bounds__(4 * D) void bwd_lin_key_kernel(const bf16 *__restrict__ k, const bf16 *__restrict__ v,
                                                            const float *__restrict__ w, const f16 *__restrict__ dhs,
                                                            const int32_t *__restrict__ hexp, int Lp,
                                                            float *__restrict__ dk, float *__restrict__ dv,
                                                            float *__restrict__ dwp, long BH, int N, int Nb) {
    constexpr int NT = 4 * D, NW = NT / 64;              // threads, waves (2 tiles of tokens x D/32 of channels)
    constexpr int STR = D + 8;
    constexpr int CPR = D / 8, RPP = NT / CPR, NP = 64 / RPP;
    constexpr int HPT = D * D / 8 / NT;                  // 8-value chunks of dh' per thread
    constexpr int TPW = (D / 32) * (D / 32) / NW;        // dW tiles per wave
    __shared__ __attribute__((aligned(16))) f16 Wh[D * STR];
    __shared__ __attribute__((aligned(16))) f16 Dh[D * STR];
    __shared__ __attribute__((aligned(16))) f16 Pk[64 * STR];
    __shared__ __attribute__((aligned(16))) f16 Vs[64 * STR];
    __shared__ __attribute__((aligned(16))) f16 Vp[64 * STR];
    __shared__ __attribute__((aligned(16))) f16 Dv[64 * STR];
    __shared__ float Dz[D], Px[D / 32][64], Red[NW];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5, grp = lane >> 4;
    const int ut = wave & 1, xt = wave >> 1, u = 32 * ut + l32;
    const int p = tid % CPR;
    for (int x = tid; x < D * D; x += NT) Wh[(x / D) * STR + x % D] = (f16)w[x];
    f32x16 wacc[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) wacc[t][e] = 0.f;
    const long total = BH * Nb;
    for (long blk = blockIdx.x; blk < total; blk += gridDim.x) {
        const long bh = blk / Nb;
        const int j = (int)(blk % Nb);
        const f16 *hrow = dhs + blk * (long)Lp;
        const int Q = hexp[bh];
        __syncthreads();                                 // the previous block's reads of the tiles are done
        Chunk hv[HPT];
        float hmax = 0.f;
#pragma unroll
        for (int x = 0; x < HPT; ++x) {
            hv[x] = ld_chunk(hrow + 8 * (tid + NT * x));
            const f16 *hx = reinterpret_cast<const f16 *>(&hv[x]);
#pragma unroll
            for (int e = 0; e < 8; ++e) hmax = fmaxf(hmax, fabsf((float)hx[e]));
        }
        if (tid < D) Dz[tid] = ldexpf((float)hrow[D * D + tid], Q);
        // 1. phi(k_u), v_u
#pragma unroll
        for (int n = 0; n < NP; ++n) {
            const int r = RPP * n + tid / CPR, row = 64 * j + r;
            const bool ok = row < N;
            const long base = (bh * N + row) * (long)D + 8 * p;
            const Chunk kc = ok ? ld_chunk(k + base) : zero_chunk();
            const Chunk vc = ok ? ld_chunk(v + base) : zero_chunk();
            const bf16 *kx = reinterpret_cast<const bf16 *>(&kc);
            const bf16 *vx = reinterpret_cast<const bf16 *>(&vc);
            float ph[8], mx = NEG_INF_B;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                ph[e] = (float)kx[e];
                mx = fmaxf(mx, ph[e]);
            }
#pragma unroll
            for (int o = 1; o < CPR; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
            float se = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                ph[e] = __expf(ph[e] - mx);
                se += ph[e];
            }
#pragma unroll
            for (int o = 1; o < CPR; o <<= 1) se += __shfl_xor(se, o);
            const float ise = ok ? 1.f / se : 0.f;
            f16 pk[8], vv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pk[e] = (f16)(ph[e] * ise);
                vv[e] = (f16)(float)vx[e];
            }
            __builtin_memcpy(&Pk[r * STR + 8 * p], pk, sizeof(pk));
            __builtin_memcpy(&Vs[r * STR + 8 * p], vv, sizeof(vv));
        }
        hmax = wave_max(hmax);
        if (lane == 0) Red[wave] = hmax;
        __syncthreads();
        float bm = Red[0];
#pragma unroll
        for (int x = 1; x < NW; ++x) bm = fmaxf(bm, Red[x]);
        // the fp16 copy x sc (exact: sc is a power of two that brings the
        // largest |x| into [0.5, 1)); the true values are the copy / sc 2^Q
        const float sc = pow2_scale(bm), isc = ldexpf(1.f / sc, Q);
#pragma unroll
        for (int x = 0; x < HPT; ++x) {
            const int e0 = 8 * (tid + NT * x);
            const f16 *hx = reinterpret_cast<const f16 *>(&hv[x]);
            f16 h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = (f16)((float)hx[e] * sc);
            __builtin_memcpy(&Dh[(e0 / D) * STR + e0 % D], h, sizeof(h));
        }
        __syncthreads();

        // 2. v'^T and s dv'^T, channel tile xt, tokens of half ut
        {
            f32x16 av, ad;
#pragma unroll
            for (int e = 0; e < 16; ++e) av[e] = ad[e] = 0.f;
#pragma unroll
            for (int s = 0; s < D / 16; ++s) {
                const int k0 = 16 * s + 8 * hh;
                mma16(av, ld8<f16>(&Wh[(32 * xt + l32) * STR + k0]), ld8<f16>(&Vs[u * STR + k0]));
                mma16(ad, ld8<f16>(&Dh[(32 * xt + l32) * STR + k0]), ld8<f16>(&Pk[u * STR + k0]));
            }
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c0 = 32 * xt + 8 * g + 4 * hh;
                v4<f16> y1, y2;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    y1[e] = (f16)av[4 * g + e];
                    y2[e] = (f16)ad[4 * g + e];
                }
                __builtin_memcpy(&Vp[u * STR + c0], &y1, sizeof(y1));
                __builtin_memcpy(&Dv[u * STR + c0], &y2, sizeof(y2));
            }
        }
        __syncthreads();

        // 3. s dphi^T (a tile xt), s dv^T (e tile xt), dW tiles
        f32x16 ap, aq;
#pragma unroll
        for (int e = 0; e < 16; ++e) ap[e] = aq[e] = 0.f;
        const int n0 = 32 * xt + 16 * (grp & 1);
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            const int k0 = 16 * s + 8 * hh;
            mma16(ap, cat8<f16>(lds_col4<f16>(Dh, STR, k0, n0, lane), lds_col4<f16>(Dh, STR, k0 + 4, n0, lane)),
                  ld8<f16>(&Vp[u * STR + k0]));
            mma16(aq, cat8<f16>(lds_col4<f16>(Wh, STR, k0, n0, lane), lds_col4<f16>(Wh, STR, k0 + 4, n0, lane)),
                  ld8<f16>(&Dv[u * STR + k0]));
        }
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int x = wave * TPW + t, ct = x / (D / 32), et = x % (D / 32);
            const int nc = 32 * ct + 16 * (grp & 1), ne = 32 * et + 16 * (grp & 1);
            f32x16 tmp;
#pragma unroll
            for (int e = 0; e < 16; ++e) tmp[e] = 0.f;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int k0 = 16 * s + 8 * hh;
                mma16(tmp, cat8<f16>(lds_col4<f16>(Dv, STR, k0, nc, lane), lds_col4<f16>(Dv, STR, k0 + 4, nc, lane)),
                      cat8<f16>(lds_col4<f16>(Vs, STR, k0, ne, lane), lds_col4<f16>(Vs, STR, k0 + 4, ne, lane)));
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) wacc[t][e] += tmp[e] * isc;
        }
        // lane (u, hh) holds channels 32 xt + 8 g + 4 hh + 0..3 of token u
        v4<f16> ph4[4];
        float pp = 0.f;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int a0 = 32 * xt + 8 * g + 4 * hh;
            ph4[g] = ld4<f16>(&Pk[u * STR + a0]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ap[4 * g + e] = ap[4 * g + e] * isc + Dz[a0 + e];
                pp += (float)ph4[g][e] * ap[4 * g + e];
            }
        }
        pp = half_swap_sum(pp);
        if (hh == 0) Px[xt][u] = pp;
        __syncthreads();
        float pd = 0.f;
#pragma unroll
        for (int x = 0; x < D / 32; ++x) pd += Px[x][u];
        const int row = 64 * j + u;
        if (row < N) {
            float *kg = dk + (bh * N + row) * (long)D;
            float *vg = dv + (bh * N + row) * (long)D;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int a0 = 32 * xt + 8 * g + 4 * hh;
                f32x4 ck = *reinterpret_cast<const f32x4 *>(kg + a0);
                f32x4 cv = *reinterpret_cast<const f32x4 *>(vg + a0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ck[e] += (float)ph4[g][e] * (ap[4 * g + e] - pd);
                    cv[e] += aq[4 * g + e] * isc;
                }
                *reinterpret_cast<f32x4 *>(kg + a0) = ck;
                *reinterpret_cast<f32x4 *>(vg + a0) = cv;
            }
        }
    }
    // this workgroup's partial dW, summed over the workgroups in a fixed order
    // by bwd_dw_reduce_kernel
    float *part = dwp + (long)blockIdx.x * D * D;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int x = wave * TPW + t, ct = x / (D / 32), et = x % (D / 32);
#pragma unroll
        for (int e = 0; e < 16; ++e) part[(32 * ct + 8 * (e >> 2) + 4 * hh + (e & 3)) * D + 32 * et + l32] = wacc[t][e];
    }
}

// dW = the sum of the linear-keys workgroups' partials in a fixed order (the
// same bits on every run): for 64 consecutive elements, wave w adds the
// partials of the w-th contiguous quarter of the workgroups in ascending
// order, and the four quarter sums are added in ascending order (four
// independent chains per element, loads of whole 256-byte rows)
__global__ __launch_bounds__(256) void bwd_dw_reduce_kernel(const float *__restrict__ part, int groups, long n,
                                                            float *__restrict__ dw) {
    __shared__ float qs[4][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const long t = (long)blockIdx.x * 64 + lane;
    const int per = (groups + 3) / 4, g0 = w * per, g1 = min(groups, g0 + per);
    float s = 0.f;
    if (t < n) {
#pragma unroll 8
        for (int g = g0; g < g1; ++g) s += part[(long)g * n + t];
    }
    qs[w][lane] = s;
    __syncthreads();
    if (w == 0 && t < n) dw[t] = ((qs[0][lane] + qs[1][lane]) + qs[2][lane]) + qs[3][lane];
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
    bwd_tlists_kernel<<<(unsigned)((a.BH * a.Nb + 3) / 4), 256, 0, st>>>(a.mask, a.BH, a.Nb, a.tlist, a.tcnt);
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
    // the transposed indicator bits
    const long nt = a.BH * (a.Nbc / 32) * (long)a.Nbp;
    bwd_mbitsT_kernel<<<(unsigned)((nt + 255) / 256), 256, 0, st>>>(a.mask, a.BH, a.Nb, a.Nbc, a.Nbp, a.mbitsT);
    const unsigned rows = (unsigned)(a.BH * a.Nbc);
    if (a.D == 64)
        bwd_lin_row_kernel<64><<<rows, 256, 0, st>>>((const bf16 *)a.q, (const bf16 *)a.dout, (const f16 *)a.hhat,
                                                     a.mcount, a.Lp, a.dq, (f16 *)a.dhr, a.dexp, a.BH, a.N, a.Nb,
                                                     a.Nbc);
    else
        bwd_lin_row_kernel<128><<<rows, 256, 0, st>>>((const bf16 *)a.q, (const bf16 *)a.dout, (const f16 *)a.hhat,
                                                      a.mcount, a.Lp, a.dq, (f16 *)a.dhr, a.dexp, a.BH, a.N, a.Nb,
                                                      a.Nbc);
    bwd_rowexp_kernel<<<(unsigned)a.BH, 256, 0, st>>>(a.dexp, a.Nbc, a.kbyte, a.hexp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // dh'_j = sum over the query blocks i with j marginal of dĤ'_i: the 0/1
    // product in scaled mode (each row's exponent in its B values)
    AssembleArgs as{};
    as.mbits = a.mbitsT; as.hs = a.dhr; as.hhat = a.dhs; as.kbyte = a.kbyte;
    as.oshift = 14 + (32 - __builtin_clz((unsigned)a.Nbc - 1));
    as.BH = a.BH; as.Nb = a.Nb; as.Nbc = a.Nbc; as.Nbp = a.Nbp; as.Lp = a.Lp;
    return launch_assemble(as, st);
}

// one workgroup per compute unit of an MI355X (256), two for d = 64 (they
// fit a compute unit's LDS twice); a fixed number, not the device's
long backward_key_groups(long BH, int Nb, int D) {
    const long per_cu = D == 64 ? 2 : 1;
    return std::min<long>(BH * Nb, per_cu * 256);
}

hipError_t launch_backward_lin_keys(const BackwardArgs &a, hipStream_t st) {
    const unsigned gk = (unsigned)backward_key_groups(a.BH, a.Nb, a.D);
    if (a.D == 64)
        bwd_lin_key_kernel<64><<<gk, 256, 0, st>>>((const bf16 *)a.k, (const bf16 *)a.v, a.w, (const f16 *)a.dhs,
                                                   a.hexp, a.Lp, a.dk, a.dv, a.dwp, a.BH, a.N, a.Nb);
    else
        bwd_lin_key_kernel<128><<<gk, 512, 0, st>>>((const bf16 *)a.k, (const bf16 *)a.v, a.w, (const f16 *)a.dhs,
                                                    a.hexp, a.Lp, a.dk, a.dv, a.dwp, a.BH, a.N, a.Nb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long n = (long)a.D * a.D;
    bwd_dw_reduce_kernel<<<(unsigned)((n + 63) / 64), 256, 0, st>>>(a.dwp, (int)gk, n, a.dw);
    return hipGetLastError();
}

}  // namespace sla
