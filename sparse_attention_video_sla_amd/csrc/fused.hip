// fused.hip -- float inputs: one kernel for the three branches of SLA (SLA article,
// section 3: exact sparse FlashAttention over the critical blocks, linear
// attention over the marginal ones, negligible ones skipped, all in one GPU
// kernel, with the learnable projection on the linear output).
//
// One workgroup per pair of consecutive query blocks (2p, 2p+1) of one head,
// 4 waves: wave (b, qh) owns query rows 32qh..32qh+31 of block 2p+b and the
// full width of every key tile.
//   Sparse part: the workgroup streams the ascending union of the two blocks'
//   critical lists (built by the classifier, each entry tagged with the
//   blocks that selected it) through double-buffered LDS, so a key block
//   both rows selected is loaded once.  K and V tiles are staged as they lie
//   in memory; per tile a wave whose block selected it computes
//   S^T = K Q^T on 32x32x16 MFMA (Q held in registers as the B operand),
//   online softmax in the log2 domain with the 1/sqrt(d) scale folded into one
//   multiply-add and lazy rescaling, P^T converted to the input type straight
//   from the accumulator, O^T += V^T P^T on MFMA with V^T read from LDS by
//   transposing reads.  Keys past N (ragged last block) score -inf.  The
//   softmax runs over the union of all critical keys of the row (block-sparse
//   normalisation of the LVSA page, method steps).
//   Linear part: phi(q) = softmax over channels from the Q registers;
//   y = phi(q) Hhat_i^T on MFMA, divided by phi(q).Zhat_i.  Hhat_i already
//   holds the projection W (folded into the block states).
//   O = O_sparse + y, written once.
// Workgroups are remapped so that each XCD (own L2) takes a contiguous run of
// (head, pair): neighbouring query blocks share most critical tiles.
#include "sla_device.h"
#include "sla_launch.h"

namespace sla {

template <typename TO> __device__ __forceinline__ void store4(TO *p, float a, float b, float c, float d);
template <> __device__ __forceinline__ void store4<float>(float *p, float a, float b, float c, float d) {
    f32x4 v = {a, b, c, d};
    *reinterpret_cast<f32x4 *>(p) = v;
}
template <> __device__ __forceinline__ void store4<bf16>(bf16 *p, float a, float b, float c, float d) {
    v4<bf16> v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
    __builtin_memcpy(p, &v, sizeof(v));
}

template <typename T, typename S, int D, typename TO>
__global__ __launch_bounds__(256, 2) void fused_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                       const T *__restrict__ v,
                                                       const uint32_t *__restrict__ ulist,
                                                       const int32_t *__restrict__ ucount, int kc,
                                                       const S *__restrict__ hhat,
                                                       const int32_t *__restrict__ mcount, int Lp,
                                                       TO *__restrict__ out, long G, int per_xcd, int N,
                                                       int Nb, float sl2) {
    constexpr int EPC = 16 / sizeof(T);
    constexpr int KSTR = D + EPC;                        // K tile row stride: conflict-free 16-byte reads
    constexpr int VSTR = D + (sizeof(T) == 2 ? 16 : 4);  // V tile row stride: 8 dwords mod 64 for transposing reads
    constexpr int KT = 64 * KSTR, VT = 64 * VSTR;
    constexpr int CPR = D / EPC;                         // 16-byte chunks per token row
    constexpr int NK = 64 * CPR / 256;                   // chunks per thread per tile (K, and again V)
    constexpr int NS = D / 16;                           // k-steps over channels
    constexpr int NCT = D / 32;                          // 32-channel tiles
    constexpr float NEG_INF = -__builtin_inff();
    constexpr float TAU = 8.f;                           // lazy rescale: P may reach 2^TAU before O is rescaled
    __shared__ __attribute__((aligned(16))) T lds[2 * (KT + VT)];

    const long logical = (long)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (logical >= G) return;
    const int Np = (Nb + 1) / 2;
    const long bh = logical / Np;
    const int pr = (int)(logical % Np);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5, grp = lane >> 4;
    const int b = wave >> 1, qh = wave & 1;
    const int i = 2 * pr + b;                            // this wave's query block
    const bool bvalid = i < Nb;
    const uint32_t mybit = 1u << (16 + b);

    // Q rows of this wave as B fragments: lane (q, h) holds channels 16s + 8h .. +7
    const int qrow = 64 * i + 32 * qh + l32;
    const bool qvalid = bvalid && qrow < N;
    v8<T> qf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s)
        qf[s] = qvalid ? ld8<T>(q + (bh * N + qrow) * (long)D + 16 * s + 8 * hh) : zero8<T>();

    float m = NEG_INF, l = 0.f;
    f32x16 o[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[ct][r] = 0.f;

    const long pair = bh * Np + pr;
    const uint32_t *ul = ulist + pair * (2L * kc);
    const int nu = (kc > 0) ? min(max(ucount[pair], 0), 2 * kc) : 0;
    // one buffer resource per head: loads past the head's end come back as zeros
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + bh * N * (long)D, (uint32_t)((long)N * D * sizeof(T)));
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + bh * N * (long)D, (uint32_t)((long)N * D * sizeof(T)));
    uint32_t voff[NK];
#pragma unroll
    for (int u = 0; u < NK; ++u) {
        const int ch = tid + 256 * u;
        voff[u] = (uint32_t)(((ch / CPR) * D + (ch % CPR) * EPC) * sizeof(T));
    }

    // Two register stages (A, B) and two LDS buffers: while tile n is computed
    // from LDS, tile n+1 sits in one register stage (issued an iteration ago)
    // and tile n+2 is being fetched into the other, so every load has two
    // tile times to land.  The stages alternate by an unrolled pair of
    // iterations, so they are always indexed statically.
    struct Stage { Chunk k[NK], v[NK]; };
    Stage ra, rb;
    auto gload = [&](Stage &st, int j) {
        const uint32_t so = (uint32_t)(64L * j * D * sizeof(T));
#pragma unroll
        for (int u = 0; u < NK; ++u) st.k[u] = buf_ld(rk, voff[u] + so, 0);
#pragma unroll
        for (int u = 0; u < NK; ++u) st.v[u] = buf_ld(rv, voff[u] + so, 0);
    };
    auto lstore = [&](const Stage &st, int buf) {
        T *Ks = lds + buf * (KT + VT);
        T *Vs = Ks + KT;
#pragma unroll
        for (int u = 0; u < NK; ++u) {
            const int ch = tid + 256 * u, row = ch / CPR, cc = ch % CPR;
            st_chunk(Ks + row * KSTR + cc * EPC, st.k[u]);
            st_chunk(Vs + row * VSTR + cc * EPC, st.v[u]);
        }
    };
    // one key tile from LDS buffer `buf` (key block j) for this wave's 32 queries
    auto compute = [&](int buf, int j) {
        const T *Ks = lds + buf * (KT + VT);
        const T *Vs = Ks + KT;
        // S^T: keys 32mt.. of the tile x this wave's 32 queries
        f32x16 sacc[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[mt][r] = 0.f;
#pragma unroll
            for (int s = 0; s < NS; ++s)
                mma16(sacc[mt], ld8<T>(Ks + (32 * mt + l32) * KSTR + 16 * s + 8 * hh), qf[s]);
        }
        if (64 * j + 64 > N) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = 64 * j + 32 * mt + 8 * (r >> 2) + 4 * hh + (r & 3);
                    if (key >= N) sacc[mt][r] = NEG_INF;
                }
        }
        float mx = fmaxf(sacc[0][0], sacc[1][0]);
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(sacc[0][r], sacc[1][r]));
        mx = fmaxf(mx, shfl_xor32(mx)) * sl2;
        // lazy rescale: move the running max only when the tile exceeds it by TAU
        if (__ballot(mx > m + TAU)) {
            const float mnew = fmaxf(m, mx);
            const float alpha = (mnew == NEG_INF) ? 1.f : fast_exp2(m - mnew);
            l *= alpha;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[ct][r] *= alpha;
            m = mnew;
        }
        const float msub = (m == NEG_INF) ? 0.f : m;
        // P^T as B fragments: k-step ks covers keys 16ks..16ks+15 in the
        // accumulator's permuted order
        v8<T> pb[4];
        float ps = 0.f;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = fast_exp2(__builtin_fmaf(sacc[mt][r], sl2, -msub));
                ps += p;
                pb[2 * mt + (r >> 3)][r & 7] = from_f32<T>(p);
            }
        l += ps;
        // O^T (channels x queries) += V^T P^T: slots 0-3 of k-step ks are keys
        // 16ks+4h+0..3, slots 4-7 keys 16ks+8+4h+0..3, each run read as a column
        // of the V tile
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const int n0 = 32 * ct + 16 * (grp & 1);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int k0 = 16 * ks + 4 * (grp >> 1);
                mma16(o[ct], cat8<T>(lds_col4<T>(Vs, VSTR, k0, n0, lane), lds_col4<T>(Vs, VSTR, k0 + 8, n0, lane)),
                      pb[ks]);
            }
        }
    };

    if (nu > 0) {
        // list entries are clamped to [0, Nb) so that no index can leave the tensors
        auto blk_at = [&](int n) { return min((int)(ul[n] & 0xFFFFu), Nb - 1); };
        auto mine = [&](int n) { return (ul[n] & mybit) != 0; };
        gload(ra, blk_at(0));
        if (nu > 1) gload(rb, blk_at(1));
        lstore(ra, 0);
        __syncthreads();
        // invariant at the top of iteration n: LDS buffer n&1 holds tile n and the
        // register stage of parity (n+1) holds tile n+1 (in flight)
        int n = 0;
        for (; n + 1 < nu; n += 2) {
            if (n + 2 < nu) gload(ra, blk_at(n + 2));
            if (mine(n)) compute(0, blk_at(n));
            lstore(rb, 1);
            __syncthreads();
            if (n + 3 < nu) gload(rb, blk_at(n + 3));
            if (mine(n + 1)) compute(1, blk_at(n + 1));
            if (n + 2 < nu) lstore(ra, 0);
            __syncthreads();
        }
        if (n < nu && mine(n)) compute(0, blk_at(n));   // odd length: the last tile, already in buffer 0
    }
    if (!bvalid) return;

    l += shfl_xor32(l);
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[ct][r] *= inv;

    // linear part
    const long rid = bh * Nb + i;
    if (mcount != nullptr && mcount[rid] > 0) {
        const S *hr = hhat + rid * (long)Lp;
        constexpr float LOG2E = 1.4426950408889634f;
        float mq = NEG_INF;
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) mq = fmaxf(mq, to_f32<T>(qf[s][e]));
        mq = fmaxf(mq, shfl_xor32(mq));
        float ex[NS][8];
        float se = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                ex[s][e] = fast_exp2((to_f32<T>(qf[s][e]) - mq) * LOG2E);
                se += ex[s][e];
            }
        se += shfl_xor32(se);
        const float inv_se = 1.f / se;
        v8<S> ph[NS];
        float den = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const v8<S> z = ld8<S>(hr + D * D + 16 * s + 8 * hh);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                ph[s][e] = from_f32<S>(ex[s][e] * inv_se);
                den += to_f32<S>(ph[s][e]) * to_f32<S>(z[e]);
            }
        }
        den += shfl_xor32(den);
        const float rden = 1.f / den;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            f32x16 y;
#pragma unroll
            for (int r = 0; r < 16; ++r) y[r] = 0.f;
#pragma unroll
            for (int s = 0; s < NS; ++s) mma16(y, ld8<S>(hr + (32 * ct + l32) * D + 16 * s + 8 * hh), ph[s]);
#pragma unroll
            for (int r = 0; r < 16; ++r) o[ct][r] += y[r] * rden;
        }
    }

    if (qvalid) {
        TO *orow = out + (bh * N + qrow) * (long)D;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                store4<TO>(orow + 32 * ct + 8 * g + 4 * hh, o[ct][4 * g], o[ct][4 * g + 1], o[ct][4 * g + 2],
                           o[ct][4 * g + 3]);
    }
}

template <typename T, typename S, int D, typename TO>
static hipError_t launch_fused_t(const FusedArgs &a, hipStream_t st) {
    const long G = a.BH * ((a.Nb + 1) / 2);
    const int per = (int)((G + 7) / 8);
    const float sl2 = 1.4426950408889634f / sqrtf((float)D);
    fused_kernel<T, S, D, TO><<<(unsigned)(8L * per), 256, 0, st>>>(
        (const T *)a.q, (const T *)a.k, (const T *)a.v, a.ulist, a.ucount, a.kc, (const S *)a.hhat, a.mcount,
        a.Lp, (TO *)a.out, G, per, a.N, a.Nb, sl2);
    return hipGetLastError();
}

hipError_t launch_fused(const FusedArgs &a, hipStream_t st) {
    if (a.bf16_in) return hipErrorInvalidValue;           // 16-bit inputs run fused16s_kernel
    return a.D == 64 ? launch_fused_t<float, float, 64, float>(a, st) : launch_fused_t<float, float, 128, float>(a, st);
}

}  // namespace sla
