// classify.hip -- compressed block scores and the three-way labels (SLA
// article, section 3: the top share of each row's compressed map is critical
// (+1), the bottom share negligible (-1), the rest marginal (0)).
//
// A workgroup of 8 waves owns R consecutive query-block rows of one head.
//   1. Scores s_ij = sum_c Qbar_i[c] * Kbar_j[c] in fp64, ascending c, one
//      thread per key block j with R rows kept in registers (the products of
//      two float32 values are exact in fp64, so the fused multiply-add gives
//      the same value as a separate multiply and add).  Rows go to LDS.
//   2. One wave per row.  Each lane holds the order-preserving 64-bit keys of
//      blocks j = lane + 64e.  The k-th largest key is found bit by bit from
//      the top: a candidate prefix is kept when at least k keys are >= it
//      (counted with ballots); the search stops early once exactly k keys are
//      >= the prefix.  Ties on the threshold key are resolved by block index
//      (lower index ranks higher), so the first k_c of the order (score desc,
//      index asc) are critical and its last k_n negligible.  The bottom search
//      runs on inverted keys with ties taken from the highest index down.
//   3. The row's outputs: int8 labels, ascending critical list, optional
//      ascending excluded list, optional P_c, and for the forward pass the
//      0/1 marginal indicator row used by the marginal-state GEMM (float
//      values for float inputs, bits otherwise) and the number of marginal
//      tokens of the row.
//   4. For the forward pass, per pair of rows (2p, 2p+1): the ascending union
//      of their critical lists, each entry j | in_row_2p << 16 | in_row_2p+1 << 17
//      (32-bit, so that the fused kernel reads it with scalar loads), and its
//      length.  The float fused kernel streams a pair's union once.
#include "sla_device.h"
#include "sla_launch.h"

namespace sla {

static constexpr int CL_THREADS = 512;

__device__ __forceinline__ uint64_t order_key(double s) {
    uint64_t b = (uint64_t)__double_as_longlong(s);
    if (b == 0x8000000000000000ull) b = 0;              // -0 ranks like +0
    return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// The keys of one row live in registers: lane l holds blocks j = l + 64e,
// e < KM, as order-preserving 64-bit keys (0 past the row end, which no
// candidate, always >= 1, can reach).  The inverted keys of the bottom search
// are the complements of the valid ones.
template <int KM> struct RowKeys { uint64_t k[KM]; };

template <int KM>
__device__ __forceinline__ uint64_t key_of(const RowKeys<KM> &rk, int e, int j, int Nb, bool inv) {
    return (j >= Nb) ? 0ull : (inv ? ~rk.k[e] : rk.k[e]);
}

// Largest v with #{keys >= v} >= k (k >= 1); `exact` when that count is exactly k,
// which lets the search stop as soon as the prefix separates k keys.
template <int KM>
__device__ uint64_t kth_largest(const RowKeys<KM> &rk, int Nb, int lane, bool inv, int k, bool &exact) {
    uint64_t lo = 0;
    exact = false;
    for (int bit = 63; bit >= 0; --bit) {
        const uint64_t cand = lo | (1ull << bit);
        int cnt = 0;
#pragma unroll
        for (int e = 0; e < KM; ++e) cnt += __popcll(__ballot(key_of(rk, e, lane + 64 * e, Nb, inv) >= cand));
        if (cnt >= k) {
            lo = cand;
            if (cnt == k) { exact = true; break; }
        }
    }
    return lo;
}

// Label +1 (inv = false, sign = 1) or -1 (inv = true, sign = -1) for the k
// blocks ranked first by (key desc, index asc) / (inverted key desc, index desc).
template <int KM>
__device__ void mark(const RowKeys<KM> &rk, int8_t *lab, int Nb, int lane, bool inv, int k, int8_t sign) {
    bool exact;
    const uint64_t t = kth_largest(rk, Nb, lane, inv, k, exact);
    int need = 0;
    if (!exact) {
        int g = 0;
#pragma unroll
        for (int e = 0; e < KM; ++e) g += __popcll(__ballot(key_of(rk, e, lane + 64 * e, Nb, inv) > t));
        need = k - g;
    }
    const uint64_t lt = (1ull << lane) - 1ull;
    const uint64_t gt = (lane == 63) ? 0ull : (~0ull << (lane + 1));
    int run = 0;
#pragma unroll
    for (int x = 0; x < KM; ++x) {
        const int e = inv ? KM - 1 - x : x;      // ties: ascending index for +1, descending for -1
        const int j = lane + 64 * e;
        const uint64_t key = key_of(rk, e, j, Nb, inv);
        bool on = exact ? key >= t : key > t;
        const uint64_t tie = __ballot(!exact && key == t);
        if (!exact && key == t) on = run + __popcll(tie & (inv ? gt : lt)) < need;
        run += __popcll(tie);
        if (on && j < Nb) lab[j] = sign;
    }
}

template <int D, int R, int KM>
__global__ __launch_bounds__(CL_THREADS) void classify_kernel(
    const float *__restrict__ qp, const float *__restrict__ kp, int Nb, int kc, int kn,
    int8_t *__restrict__ mask, int32_t *__restrict__ crit, int32_t *__restrict__ excl,
    float *__restrict__ pc, float *__restrict__ marg, uint32_t *__restrict__ mbits, int Nbc, int Nbp,
    int32_t *__restrict__ mcount, int n_last,
    uint32_t *__restrict__ ulist, int32_t *__restrict__ ucount,
    double inv_sqrt_d) {
    extern __shared__ double smem[];
    double *qd = smem;                                        // [R][D]
    double *sc = smem + R * D;                                // [R][Nb]
    int8_t *labs = reinterpret_cast<int8_t *>(sc + R * Nb);   // [R][Nb]
    const int tiles = (Nb + R - 1) / R;
    const long bh = blockIdx.x / tiles;
    const int i0 = (blockIdx.x % tiles) * R;
    const int nr = min(R, Nb - i0);
    const int tid = threadIdx.x;

    for (int x = tid; x < R * D; x += CL_THREADS)
        qd[x] = (x < nr * D) ? (double)qp[(bh * Nb + i0) * D + x] : 0.0;
    for (int x = tid; x < R * Nb; x += CL_THREADS) labs[x] = 0;
    __syncthreads();

    for (int j = tid; j < Nb; j += CL_THREADS) {
        const float *kj = kp + (bh * Nb + j) * D;
        double acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = 0.0;
#pragma unroll 2
        for (int c = 0; c < D; c += 4) {
            const f32x4 kv = *reinterpret_cast<const f32x4 *>(kj + c);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const double kd = (double)kv[u];
#pragma unroll
                for (int r = 0; r < R; ++r) acc[r] = __builtin_fma(qd[r * D + c + u], kd, acc[r]);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (r < nr) sc[r * Nb + j] = acc[r];
    }
    __syncthreads();

    const int wave = tid >> 6, lane = tid & 63;
    const int ne = (Nb + 63) >> 6;
    const uint64_t lt = (1ull << lane) - 1ull;
    for (int r = wave; r < nr; r += CL_THREADS / 64) {
        const long row = bh * Nb + i0 + r;
        const double *s = sc + r * Nb;
        int8_t *lab = labs + r * Nb;
        RowKeys<KM> rk;
#pragma unroll
        for (int e = 0; e < KM; ++e) {
            const int j = lane + 64 * e;
            rk.k[e] = (j < Nb) ? order_key(s[j]) : 0ull;
        }
        if (kc > 0) mark(rk, lab, Nb, lane, false, kc, 1);
        if (kn > 0) mark(rk, lab, Nb, lane, true, kn, -1);
        int run_c = 0, run_x = 0, n_marg = 0;
        bool last_marg = false;
        for (int e = 0; e < ne; ++e) {
            const int j = lane + 64 * e;
            const bool ok = j < Nb;
            const int lb = ok ? lab[j] : 0;
            if (ok) mask[row * Nb + j] = (int8_t)lb;
            const uint64_t bc = __ballot(ok && lb == 1);
            const int pc_pos = run_c + __popcll(bc & lt);
            if (ok && lb == 1 && pc_pos < kc) crit[row * kc + pc_pos] = j;
            run_c += __popcll(bc);
            const uint64_t bx = __ballot(ok && lb != 0);
            const int px_pos = run_x + __popcll(bx & lt);
            if (excl && ok && lb != 0 && px_pos < kc + kn) excl[row * (kc + kn) + px_pos] = j;
            run_x += __popcll(bx);
            const uint64_t bm = __ballot(ok && lb == 0);
            n_marg += __popcll(bm);
            if (mbits && lane == 0) {                  // Nbc is a multiple of 64: both words exist
                uint32_t *wp = mbits + (bh * (Nbc / 32) + 2 * e) * (long)Nbp + i0 + r;
                wp[0] = (uint32_t)bm;
                wp[Nbp] = (uint32_t)(bm >> 32);
            }
            if (ok && lb == 0 && j == Nb - 1) last_marg = true;
            if (marg && j < Nbc) marg[row * Nbc + j] = (ok && lb == 0) ? 1.f : 0.f;
        }
        if (mcount) {
            const bool lm = __ballot(last_marg) != 0ull;
            if (lane == 0) mcount[row] = n_marg * 64 - (lm ? 64 - n_last : 0);
        }
        if (pc) {
            double m = -__builtin_inf();
            for (int j = lane; j < Nb; j += 64) m = fmax(m, s[j]);
            for (int off = 32; off > 0; off >>= 1) m = fmax(m, __shfl_xor(m, off, 64));
            double z = 0.0;
            for (int j = lane; j < Nb; j += 64) z += exp((s[j] - m) * inv_sqrt_d);
            for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off, 64);
            for (int j = lane; j < Nb; j += 64) pc[row * Nb + j] = (float)(exp((s[j] - m) * inv_sqrt_d) / z);
        }
    }
    if (ulist == nullptr) return;
    __syncthreads();
    // union of the critical lists of each row pair (R is even, i0 is even)
    const int Np = (Nb + 1) / 2;
    for (int pr = wave; ulist != nullptr && 2 * pr < nr; pr += CL_THREADS / 64) {
        const long pair = bh * Np + (i0 / 2 + pr);
        const int8_t *la = labs + (2 * pr) * Nb;
        const int8_t *lb = (2 * pr + 1 < nr) ? labs + (2 * pr + 1) * Nb : nullptr;
        int run = 0;
        for (int e = 0; e < ne; ++e) {
            const int j = lane + 64 * e;
            const bool a = j < Nb && la[j] == 1;
            const bool b = j < Nb && lb != nullptr && lb[j] == 1;
            const uint64_t bu = __ballot(a || b);
            const int pos = run + __popcll(bu & lt);
            if ((a || b) && pos < 2 * kc)
                ulist[pair * (2 * kc) + pos] = (uint32_t)j | (a ? 1u << 16 : 0u) | (b ? 1u << 17 : 0u);
            run += __popcll(bu);
        }
        if (lane == 0) ucount[pair] = run;
    }
}

template <int D, int R, int KM>
static hipError_t launch_cls_k(const ClassifyArgs &a, hipStream_t st) {
    const size_t lds = classify_lds_bytes(R, D, a.Nb);
    auto kern = classify_kernel<D, R, KM>;
    hipError_t err = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    const long tiles = (a.Nb + R - 1) / R;
    const unsigned grid = (unsigned)(a.BH * tiles);
    kern<<<grid, CL_THREADS, lds, st>>>(a.qp, a.kp, a.Nb, a.kc, a.kn, a.mask, a.crit, a.excl, a.pc,
                                        a.marg, a.mbits, a.Nbc, a.Nbp, a.mcount, a.n_last, a.ulist, a.ucount,
                                        a.inv_sqrt_d);
    return hipGetLastError();
}

// keys per lane: ceil(Nb / 64) rounded up to 8, 16, 24, 32 or 38 registers pairs
template <int D, int R>
static hipError_t launch_cls_r(const ClassifyArgs &a, hipStream_t st) {
    const int ne = (a.Nb + 63) / 64;
    if (ne <= 8) return launch_cls_k<D, R, 8>(a, st);
    if (ne <= 16) return launch_cls_k<D, R, 16>(a, st);
    if (ne <= 24) return launch_cls_k<D, R, 24>(a, st);
    if (ne <= 32) return launch_cls_k<D, R, 32>(a, st);
    return launch_cls_k<D, R, 38>(a, st);
}

template <int D>
static hipError_t launch_cls_d(const ClassifyArgs &a, hipStream_t st) {
    const int R = classify_rows_per_group(a.Nb, D);
    switch (R) {
    case 8: return launch_cls_r<D, 8>(a, st);
    case 4: return launch_cls_r<D, 4>(a, st);
    case 2: return launch_cls_r<D, 2>(a, st);
    default: return launch_cls_r<D, 2>(a, st);
    }
}

size_t classify_lds_bytes(int R, int D, int Nb) {
    return sizeof(double) * (size_t)R * (D + Nb) + (size_t)R * Nb;
}

int classify_rows_per_group(int Nb, int D) {
    const size_t limit = 160 * 1024;
    for (int R = 8; R > 2; R >>= 1)
        if (classify_lds_bytes(R, D, Nb) <= limit) return R;
    return 2;   // rows come in pairs; two rows fit for every supported Nb
}

hipError_t launch_classify(const ClassifyArgs &a, hipStream_t st) {
    return a.D == 64 ? launch_cls_d<64>(a, st) : launch_cls_d<128>(a, st);
}

}  // namespace sla
