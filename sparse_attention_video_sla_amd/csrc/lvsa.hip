// lvsa.hip -- LVSA frame-level attention sets built on the device (the LVSA
// page, training-free sparse attention for long-video diffusion: "Core
// method" and "Method steps in detail"), and the slot schedule of the 16-bit
// fused kernel that makes every query token of frame t attend exactly the
// tokens of the frames in A(t) = G_s u W(t).
//
// The page builds the index lists on the host per denoising step and copies
// them over; here two small kernels build them in the stream (no host round
// trip).  Steps, in the page's order:
//   T_per = ceil(T / (C - (2W + 1)))                          (host)
//   G_s = {(s mod T_per + i T_per) mod T}, i < ceil(T / T_per): f is in G_s
//     when f - o or f - o + T (o = s mod T_per) is a multiple i T_per with
//     i < ceil(T / T_per); the values stay below 2T, so one wrap at most
//   basic window [w_lo, w_lo + 2W] clipped to T - 1, w_lo = max(0, min(t - W, T - 1 - 2W))
//   expansion: while the window holds fewer non-global frames than
//     min(2W + 1, T - |G_s|), add one frame on the side with more frames
//     left outside it (the earlier side on a tie)
//   A(t) = G_s u window.
// Token n belongs to frame n / P; a 64-token block holds at most two frames
// (P >= 64): its part 0 before the frame boundary inside it, part 1 after.
// A query-block row takes every key block that holds a token of a frame in
// A(f) for a frame f of the row's parts; a key block whose parts are not all
// seen by all the row's parts carries frame marks (bit 2a + c: query part a
// does not see key part c).  The schedule does not depend on the head, so
// one schedule serves every head.
#include "sla_device.h"
#include "sla_launch.h"
#include "slot_merge.h"

namespace sla {

namespace {

__device__ __forceinline__ bool lvsa_global(int f, const LvsaParams &p) {
    const int o = p.s % p.Tper;
    const int x1 = f - o, x2 = f - o + p.T;
    return (x1 >= 0 && x1 % p.Tper == 0 && x1 / p.Tper < p.m) || (x2 % p.Tper == 0 && x2 / p.Tper < p.m);
}

// the expanded window [lo, hi] of frame t
__device__ __forceinline__ void lvsa_window(int t, const LvsaParams &p, int &lo, int &hi) {
    lo = max(0, min(t - p.W, p.T - 1 - 2 * p.W));
    hi = min(p.T - 1, lo + 2 * p.W);
    const int target = min(2 * p.W + 1, p.T - p.m);
    int have = 0;
    for (int f = lo; f <= hi; ++f) have += lvsa_global(f, p) ? 0 : 1;
    // there are T - |G_s| >= target non-global frames: the loop ends within T steps
    for (int it = 0; have < target && it < p.T; ++it) {
        const int left = lo, right = p.T - 1 - hi;
        if (left >= right && left > 0) {
            --lo;
            have += lvsa_global(lo, p) ? 0 : 1;
        } else {
            ++hi;
            have += lvsa_global(hi, p) ? 0 : 1;
        }
    }
}

__device__ __forceinline__ bool lvsa_in_set(int t, int f, const int32_t *lohi, const LvsaParams &p) {
    return (f >= lohi[2 * t] && f <= lohi[2 * t + 1]) || lvsa_global(f, p);
}

}  // namespace

// one thread per frame: the expanded window, and (when sets is not null) the
// ascending frame set A(t) with its size
__global__ __launch_bounds__(256) void lvsa_frames_kernel(LvsaParams p, int32_t *__restrict__ lohi,
                                                          int32_t *__restrict__ sets, int32_t *__restrict__ counts,
                                                          int max_frames) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= p.T) return;
    int lo, hi;
    lvsa_window(t, p, lo, hi);
    if (lohi) {
        lohi[2 * t] = lo;
        lohi[2 * t + 1] = hi;
    }
    if (sets) {
        int c = 0;
        for (int f = 0; f < p.T; ++f)
            if ((f >= lo && f <= hi) || lvsa_global(f, p)) {
                if (c < max_frames) sets[(long)t * max_frames + c] = f;
                ++c;
            }
        counts[t] = c;
    }
}

// one wave per pair of query-block rows
template <int KM>
__global__ __launch_bounds__(256) void lvsa_slots_kernel(LvsaParams p, int P, int N, int Nb,
                                                         const int32_t *__restrict__ lohi, int kmax,
                                                         uint32_t *__restrict__ slots, int32_t *__restrict__ pcount) {
    extern __shared__ uint32_t bits[];
    const int Np = (Nb + 1) / 2;
    const int W = (Nb + 31) / 32;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int pair = blockIdx.x * 4 + wave;
    if (pair >= Np) return;
    const bool has_b = 2 * pair + 1 < Nb;
    uint32_t *ba = bits + wave * 2 * W, *bb = ba + W;
    for (int x = lane; x < 2 * W; x += 64) ba[x] = 0u;
    wave_lds_fence();
    // query frames of the parts of the two rows
    const int ia = 2 * pair, ib = min(2 * pair + 1, Nb - 1);
    const int qa0 = 64 * ia / P, qa1 = min(64 * ia + 63, N - 1) / P;
    const int qb0 = 64 * ib / P, qb1 = min(64 * ib + 63, N - 1) / P;
    for (int r = 0; r < 2; ++r) {
        if (r == 1 && !has_b) break;
        uint32_t *bm = r == 0 ? ba : bb;
        const int q0 = r == 0 ? qa0 : qb0, q1 = r == 0 ? qa1 : qb1;
        for (int f = lane; f < p.T; f += 64) {
            if (!lvsa_in_set(q0, f, lohi, p) && !lvsa_in_set(q1, f, lohi, p)) continue;
            const int b0 = (int)((long)f * P / 64), b1 = (int)(((long)f * P + P - 1) / 64);
            for (int w = b0 >> 5; w <= (b1 >> 5); ++w) {
                const int lo = max(b0, 32 * w) - 32 * w, hi = min(b1, 32 * w + 31) - 32 * w;
                const uint32_t m = (hi == 31 ? 0xFFFFFFFFu : ((1u << (hi + 1)) - 1u)) & ~((1u << lo) - 1u);
                atomicOr(&bm[w], m);
            }
        }
    }
    wave_lds_fence();
    auto mark = [&](int r, int j) -> uint32_t {
        const int kf0 = 64 * j / P, kf1 = min(64 * j + 63, N - 1) / P;
        const int q0 = r == 0 ? qa0 : qb0, q1 = r == 0 ? qa1 : qb1;
        uint32_t mk = 0u;
        if (!lvsa_in_set(q0, kf0, lohi, p)) mk |= 1u;
        if (!lvsa_in_set(q0, kf1, lohi, p)) mk |= 2u;
        if (!lvsa_in_set(q1, kf0, lohi, p)) mk |= 4u;
        if (!lvsa_in_set(q1, kf1, lohi, p)) mk |= 8u;
        return mk;
    };
    uint16_t *sl = reinterpret_cast<uint16_t *>(slots + (long)pair * kmax);
    const int n = merge_pair<KM>(ba, bb, has_b, Nb, kmax, sl, mark);
    if (lane == 0) pcount[pair] = n;
}

hipError_t launch_lvsa_frames(const LvsaParams &p, int32_t *lohi, int32_t *sets, int32_t *counts, int max_frames,
                              hipStream_t st) {
    lvsa_frames_kernel<<<(unsigned)((p.T + 255) / 256), 256, 0, st>>>(p, lohi, sets, counts, max_frames);
    return hipGetLastError();
}

hipError_t launch_lvsa_slots(const LvsaParams &p, int P, int N, int Nb, const int32_t *lohi, int kmax,
                             uint32_t *slots, int32_t *pcount, hipStream_t st) {
    const int Np = (Nb + 1) / 2;
    const unsigned grid = (unsigned)((Np + 3) / 4);
    const size_t lds = sizeof(uint32_t) * 4 * 2 * ((Nb + 31) / 32);
    const int ne = (Nb + 63) / 64;
    if (ne <= 8) lvsa_slots_kernel<8><<<grid, 256, lds, st>>>(p, P, N, Nb, lohi, kmax, slots, pcount);
    else if (ne <= 16) lvsa_slots_kernel<16><<<grid, 256, lds, st>>>(p, P, N, Nb, lohi, kmax, slots, pcount);
    else if (ne <= 32) lvsa_slots_kernel<32><<<grid, 256, lds, st>>>(p, P, N, Nb, lohi, kmax, slots, pcount);
    else lvsa_slots_kernel<64><<<grid, 256, lds, st>>>(p, P, N, Nb, lohi, kmax, slots, pcount);
    return hipGetLastError();
}

// out[t] = sum_m 2^(lse_m - L) O_m / sum_m 2^(lse_m - L), L the largest
// finite lse_m of the token (a share with lse = +inf had no key: weight 0;
// a token with no key in any share gets zeros).  One thread per 8 channels;
// the NC shares' log-sum-exps and 16-byte pieces are all loaded before any
// is used.
template <typename TO, int NC>
__global__ __launch_bounds__(256) void chunk_merge_kernel(const f16 *__restrict__ part,
                                                          const float *__restrict__ plse, long BH, int N,
                                                          int Nb, int D, TO *__restrict__ out) {
    const long t = (long)blockIdx.x * 256 + threadIdx.x;
    const int c8 = D / 8;
    if (t >= BH * N * c8) return;
    const long row = t / c8;
    const int c = (int)(t % c8) * 8;
    const long bh = row / N, tok = row % N;
    const long lstride = BH * 64L * Nb, pstride = lstride * D;
    float x[NC];
    v8<f16> o[NC];
#pragma unroll
    for (int m = 0; m < NC; ++m) {
        x[m] = plse[m * lstride + bh * 64L * Nb + tok];
        o[m] = ld8<f16>(part + m * pstride + row * D + c);
    }
    float L = -__builtin_inff();
#pragma unroll
    for (int m = 0; m < NC; ++m)
        if (x[m] < __builtin_inff()) L = fmaxf(L, x[m]);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (L > -__builtin_inff()) {
        float den = 0.f;
#pragma unroll
        for (int m = 0; m < NC; ++m) {
            const float w = x[m] < __builtin_inff() ? __builtin_amdgcn_exp2f(x[m] - L) : 0.f;
            den += w;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(w, (float)o[m][e], acc[e]);
        }
        const float inv = 1.f / den;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= inv;
    }
    if constexpr (__is_same(TO, float)) {
        *reinterpret_cast<f32x4 *>(out + row * D + c) = f32x4{acc[0], acc[1], acc[2], acc[3]};
        *reinterpret_cast<f32x4 *>(out + row * D + c + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    } else {
        v8<bf16> y;
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = (bf16)acc[e];
        __builtin_memcpy(out + row * D + c, &y, sizeof(y));
    }
}

hipError_t launch_chunk_merge(const f16 *part, const float *plse, int nchunk, long BH, int N, int Nb, int D,
                              void *out, bool bf16_out, hipStream_t st) {
    if (nchunk != 4) return hipErrorInvalidValue;        // the slot schedules are split in 4 shares
    const long n = BH * N * (D / 8);
    const unsigned grid = (unsigned)((n + 255) / 256);
    if (bf16_out)
        chunk_merge_kernel<bf16, 4><<<grid, 256, 0, st>>>(part, plse, BH, N, Nb, D, (bf16 *)out);
    else
        chunk_merge_kernel<float, 4><<<grid, 256, 0, st>>>(part, plse, BH, N, Nb, D, (float *)out);
    return hipGetLastError();
}

}  // namespace sla
