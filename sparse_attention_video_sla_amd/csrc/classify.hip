// classify.hip -- compressed block scores and the three-way labels (SLA
// article, section 3: the top share of each row's compressed map is critical
// (+1), the bottom share negligible (-1), the rest marginal (0)).
//
// A workgroup of 4 waves owns R consecutive query-block rows of one head.
//   1. Scores s_ij = sum_c Qbar_i[c] * Kbar_j[c] in fp64, ascending c (the
//      products of two float32 values are exact in fp64, so the fused
//      multiply-add gives the same value as a separate multiply and add).
//      A thread owns two key blocks j and the R rows: per channel it reads
//      the R query means (fp64, broadcast reads from LDS) and its two key
//      means, and does 2R multiply-adds.  The key means come either from
//      the pool kernel's channel-packed copy ([c/4][j][4]: a wave reads one
//      contiguous run per step) or, for the public classify entry point,
//      from the [j][c] rows.  The order-preserving 64-bit keys of the scores
//      go to LDS.
//   2. One wave per row.  Each lane holds the keys of blocks j = lane + 64e.
//      The k-th largest key is found bit by bit with ballot counts, starting
//      below the bits that every key of the row shares, and stopping once
//      the prefix separates exactly k keys; the critical (top k_c) and the
//      negligible (bottom k_n, on the complemented keys) searches share the
//      passes.  Equal keys at a cut rank the lower block index first, so the
//      first k_c of the order (score desc, index asc) are critical and its
//      last k_n negligible.
//   3. The row's outputs: int8 labels, ascending critical list, optional
//      ascending excluded list, optional P_c, and for the forward pass the
//      0/1 marginal indicator row used by the marginal-state GEMM (float
//      values for float inputs, bits otherwise) and the number of marginal
//      tokens of the row.
//   4. For the forward pass with float inputs, per pair of rows (2p, 2p+1):
//      the ascending union of their critical lists, each entry
//      j | in_row_2p << 16 | in_row_2p+1 << 17, and its length.
#include "sla_device.h"
#include "sla_launch.h"

namespace sla {

static constexpr int CL_THREADS = 256;
static constexpr int CL_WAVES = CL_THREADS / 64;
// what a launch reads and writes: the public entry point ([j][c] key means,
// optional excluded lists and P_c), or the forward pass (packed key means,
// fp64 query means, marginal indicator bits and counts for 16-bit inputs;
// float indicator rows, counts and pair unions for float inputs)
enum { CL_API = 0, CL_FWD16 = 1, CL_FWD32 = 2 };

__device__ __forceinline__ uint64_t order_key(double s) {
    uint64_t b = (uint64_t)__double_as_longlong(s);
    if (b == 0x8000000000000000ull) b = 0;              // -0 ranks like +0
    return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}
__device__ __forceinline__ double key_value(uint64_t key) {
    return __longlong_as_double((long long)((key >> 63) ? (key & 0x7FFFFFFFFFFFFFFFull) : ~key));
}

// Labels of one row.  The k-th largest of the wave's valid keys is the
// largest value t with #{keys >= t} >= k, found bit by bit from the top with
// ballot counts; the bits above the highest bit in which the row's keys
// differ are common to every key and are taken as they are.  The search
// stops as soon as exactly k keys are >= the prefix.  The top search (the
// k_c critical blocks) and the bottom search (the k_n negligible blocks, on
// the complemented keys) run in the same passes.  Where the k-th value is
// shared by several keys, the lower block indices rank first in the top
// search and the higher ones first in the bottom search (the last k_n of
// the order score desc, index asc).
// Bit e of cm / nm: block lane + 64 e is critical / negligible.
__device__ __forceinline__ uint64_t uniform64(uint64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
    return (uint64_t)hi << 32 | lo;
}

// (Slots past Nb hold key 0.)
template <int KM>
__device__ void label_row(const uint64_t (&key)[KM], int Nb, int lane, int kc, int kn, uint64_t &cm, uint64_t &nm) {
    auto valid = [&](int e) __attribute__((always_inline)) { return lane + 64 * e < Nb; };
    uint64_t a = ~0ull, o = 0ull;
#pragma unroll
    for (int e = 0; e < KM; ++e)
        if (valid(e)) { a &= key[e]; o |= key[e]; }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        a &= __shfl_xor(a, off, 64);
        o |= __shfl_xor(o, off, 64);
    }
    // every lane holds the same values now: say so, so that the search runs
    // as a scalar loop
    a = uniform64(a);
    o = uniform64(o);
    const uint64_t diff = a ^ o;
    int bit = diff ? 63 - __builtin_clzll(diff) : -1;
    const uint64_t high = bit >= 0 ? ~((2ull << bit) - 1ull) : ~0ull;   // the common bits
    uint64_t tc = a & high, tn = ~o & high;              // prefixes of the two searches
    bool ec = false, en = false;                         // exact: k keys are >= the prefix
    bool dc = kc == 0, dn = kn == 0;
    // The slots past Nb hold key 0, which no candidate of the top search
    // (>= 1) reaches; in the bottom search (~key >= cand, i.e. key <= ~cand)
    // every one of them counts, so their number is taken off.
    const int n_pad = 64 * KM - Nb;
    for (; bit >= 0 && !(dc && dn); --bit) {
        const uint64_t b = 1ull << bit;
        if (!dc) {
            const uint64_t cand = tc | b;
            int cnt = 0;
#pragma unroll
            for (int e = 0; e < KM; ++e) cnt += __popcll(__ballot(key[e] >= cand));
            if (cnt >= kc) {
                tc = cand;
                if (cnt == kc) ec = dc = true;
            }
        }
        if (!dn) {
            const uint64_t cand = tn | b, lim = ~cand;
            int cnt = -n_pad;
#pragma unroll
            for (int e = 0; e < KM; ++e) cnt += __popcll(__ballot(key[e] <= lim));
            if (cnt >= kn) {
                tn = cand;
                if (cnt == kn) en = dn = true;
            }
        }
    }
    static_assert(KM <= 64, "one label bit per key slot");
    cm = nm = 0ull;
    const uint64_t lt = (1ull << lane) - 1ull;
    const uint64_t gt = (lane == 63) ? 0ull : (~0ull << (lane + 1));
    // keys strictly above each threshold, to know how many of the tied ones to take
    int gc = 0, gn = 0;
    if (kc > 0 && !ec) {
#pragma unroll
        for (int e = 0; e < KM; ++e) gc += __popcll(__ballot(valid(e) && key[e] > tc));
    }
    if (kn > 0 && !en) {
#pragma unroll
        for (int e = 0; e < KM; ++e) gn += __popcll(__ballot(valid(e) && ~key[e] > tn));
    }
    int run = 0;
#pragma unroll
    for (int e = 0; e < KM; ++e) {                       // critical: ties by ascending index
        if (kc == 0) break;
        const bool v = valid(e);
        bool on = v && (ec ? key[e] >= tc : key[e] > tc);
        if (!ec) {
            const bool tie = v && key[e] == tc;
            const uint64_t tb = __ballot(tie);
            if (tie) on = run + __popcll(tb & lt) < kc - gc;
            run += __popcll(tb);
        }
        if (on) cm |= 1ull << e;
    }
    run = 0;
#pragma unroll
    for (int x = 0; x < KM; ++x) {                       // negligible: ties by descending index
        if (kn == 0) break;
        const int e = KM - 1 - x;
        const bool v = valid(e);
        const uint64_t ik = ~key[e];
        bool on = v && (en ? ik >= tn : ik > tn);
        if (!en) {
            const bool tie = v && ik == tn;
            const uint64_t tb = __ballot(tie);
            if (tie) on = run + __popcll(tb & gt) < kn - gn;
            run += __popcll(tb);
        }
        if (on) nm |= 1ull << e;
    }
}

template <int D, int R, int KM, int MODE>
__device__ __forceinline__ void classify_body(
    const float *__restrict__ qp, const float *__restrict__ kp, int Nb, int Nb2, int kc, int kn,
    int8_t *__restrict__ mask, int32_t *__restrict__ crit, int32_t *__restrict__ excl,
    float *__restrict__ pc, float *__restrict__ marg, uint32_t *__restrict__ mbits, int Nbc, int Nbp,
    int32_t *__restrict__ mcount, int n_last,
    uint32_t *__restrict__ ulist, int32_t *__restrict__ ucount,
    double inv_sqrt_d) {
    extern __shared__ __attribute__((aligned(16))) double smem[];
    double *qd = smem;                                        // [D][R]
    uint64_t *keys = reinterpret_cast<uint64_t *>(smem + R * D);
    int8_t *labs = reinterpret_cast<int8_t *>(keys + R * Nb);   // [R][Nb], only with ulist
    const int tiles = (Nb + R - 1) / R;
    const long bh = blockIdx.x / tiles;
    const int i0 = (blockIdx.x % tiles) * R;
    const int nr = min(R, Nb - i0);
    const int tid = threadIdx.x;

    // the query means of the R rows in LDS, [c][r] in fp64
    for (int x = tid; x < R * D; x += CL_THREADS) {
        const int c = x / R, r = x % R;
        qd[x] = r < nr ? (double)qp[(bh * Nb + i0 + r) * D + c] : 0.0;
    }
    __syncthreads();

    // 1. scores of the R rows against key blocks j0 = 2p, j1 = 2p + 1
    for (int p = tid; 2 * p < Nb; p += CL_THREADS) {
        const int j0 = 2 * p, j1 = 2 * p + 1;
        double acc[R][2];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][0] = acc[r][1] = 0.0;
        auto load = [&](int c4, f32x4 &a, f32x4 &b) __attribute__((always_inline)) {
            if constexpr (MODE != CL_API) {
                const float *src = kp + ((bh * (D / 4) + c4) * (long)Nb2 + j0) * 4;
                a = *reinterpret_cast<const f32x4 *>(src);
                b = *reinterpret_cast<const f32x4 *>(src + 4);
            } else {
                a = *reinterpret_cast<const f32x4 *>(kp + (bh * Nb + j0) * D + 4 * c4);
                b = j1 < Nb ? *reinterpret_cast<const f32x4 *>(kp + (bh * Nb + j1) * D + 4 * c4) : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        };
        // the next step's key means in flight during the current products
        f32x4 ka, kb;
        load(0, ka, kb);
#pragma unroll 2
        for (int c4 = 0; c4 < D / 4; ++c4) {
            f32x4 na = ka, nb = kb;
            if (c4 + 1 < D / 4) load(c4 + 1, na, nb);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const double k0 = (double)ka[u], k1 = (double)kb[u];
                const double *qc = qd + (4 * c4 + u) * R;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    acc[r][0] = __builtin_fma(qc[r], k0, acc[r][0]);
                    acc[r][1] = __builtin_fma(qc[r], k1, acc[r][1]);
                }
            }
            ka = na;
            kb = nb;
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (r < nr) {
                keys[r * Nb + j0] = order_key(acc[r][0]);
                if (j1 < Nb) keys[r * Nb + j1] = order_key(acc[r][1]);
            }
        }
    }
    __syncthreads();

    // 2.-3. one wave per row
    const int wave = tid >> 6, lane = tid & 63;
    const int ne = (Nb + 63) >> 6;
    const uint64_t lt = (1ull << lane) - 1ull;
    for (int r = wave; r < nr; r += CL_WAVES) {
        const long row = bh * Nb + i0 + r;
        const uint64_t *kr = keys + r * Nb;
        uint64_t key[KM];
#pragma unroll
        for (int e = 0; e < KM; ++e) {
            const int j = lane + 64 * e;
            key[e] = j < Nb ? kr[j] : 0ull;
        }
        uint64_t cm, nm;
        label_row(key, Nb, lane, kc, kn, cm, nm);
        int run_c = 0, run_x = 0, n_marg = 0;
        bool last_marg = false;
#pragma unroll
        for (int e = 0; e < KM; ++e) {
            if (e >= ne) break;
            const int j = lane + 64 * e;
            const bool okj = j < Nb;
            const int lb = ((cm >> e) & 1) ? 1 : (((nm >> e) & 1) ? -1 : 0);
            if (okj) mask[row * Nb + j] = (int8_t)lb;
            if (MODE == CL_FWD32 && ulist && okj) labs[r * Nb + j] = (int8_t)lb;
            const uint64_t bc = __ballot(okj && lb == 1);
            const int pc_pos = run_c + __popcll(bc & lt);
            if (okj && lb == 1 && pc_pos < kc) crit[row * kc + pc_pos] = j;
            run_c += __popcll(bc);
            const uint64_t bx = __ballot(okj && lb != 0);
            const int px_pos = run_x + __popcll(bx & lt);
            if (MODE == CL_API && excl && okj && lb != 0 && px_pos < kc + kn) excl[row * (kc + kn) + px_pos] = j;
            run_x += __popcll(bx);
            const uint64_t bm = __ballot(okj && lb == 0);
            n_marg += __popcll(bm);
            if (MODE == CL_FWD16 && mbits && lane == 0) {   // Nbc is a multiple of 64: both words exist
                uint32_t *wp = mbits + (bh * (Nbc / 32) + 2 * e) * (long)Nbp + i0 + r;
                wp[0] = (uint32_t)bm;
                wp[Nbp] = (uint32_t)(bm >> 32);
            }
            if (okj && lb == 0 && j == Nb - 1) last_marg = true;
            if (MODE == CL_FWD32 && marg && j < Nbc) marg[row * Nbc + j] = (okj && lb == 0) ? 1.f : 0.f;
        }
        if (MODE != CL_API && mcount) {
            const bool lm = __ballot(last_marg) != 0ull;
            if (lane == 0) mcount[row] = n_marg * 64 - (lm ? 64 - n_last : 0);
        }
        if (MODE == CL_API && pc) {
            double m = -__builtin_inf();
#pragma unroll
            for (int e = 0; e < KM; ++e)
                if (lane + 64 * e < Nb) m = fmax(m, key_value(key[e]));
            for (int off = 32; off > 0; off >>= 1) m = fmax(m, __shfl_xor(m, off, 64));
            double z = 0.0;
#pragma unroll
            for (int e = 0; e < KM; ++e)
                if (lane + 64 * e < Nb) z += exp((key_value(key[e]) - m) * inv_sqrt_d);
            for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off, 64);
#pragma unroll
            for (int e = 0; e < KM; ++e)
                if (lane + 64 * e < Nb) pc[row * Nb + lane + 64 * e] = (float)(exp((key_value(key[e]) - m) * inv_sqrt_d) / z);
        }
    }
    if (MODE != CL_FWD32 || ulist == nullptr) return;
    __syncthreads();
    // union of the critical lists of each row pair (R is even, i0 is even)
    const int Np = (Nb + 1) / 2;
    for (int pr = wave; 2 * pr < nr; pr += CL_WAVES) {
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

#define SLA_CLASSIFY_ARGS                                                                                        \
    const float *__restrict__ qp, const float *__restrict__ kp, int Nb, int Nb2, int kc, int kn,                    \
        int8_t *__restrict__ mask, int32_t *__restrict__ crit, int32_t *__restrict__ excl, float *__restrict__ pc,  \
        float *__restrict__ marg, uint32_t *__restrict__ mbits, int Nbc, int Nbp, int32_t *__restrict__ mcount,     \
        int n_last, uint32_t *__restrict__ ulist, int32_t *__restrict__ ucount, double inv_sqrt_d
#define SLA_CLASSIFY_PASS qp, kp, Nb, Nb2, kc, kn, mask, crit, excl, pc, marg, mbits, Nbc, Nbp, mcount, n_last, ulist, ucount, inv_sqrt_d

// three waves per SIMD; rows of up to 32 keys per lane fit its registers
template <int D, int R, int KM, int MODE>
__global__ __launch_bounds__(CL_THREADS, 3) void classify_kernel(SLA_CLASSIFY_ARGS) {
    classify_body<D, R, KM, MODE>(SLA_CLASSIFY_PASS);
}
// two waves per SIMD, for rows of more than 2048 blocks (38 keys per lane)
template <int D, int R, int KM, int MODE>
__global__ __launch_bounds__(CL_THREADS, 2) void classify_wide_kernel(SLA_CLASSIFY_ARGS) {
    classify_body<D, R, KM, MODE>(SLA_CLASSIFY_PASS);
}

template <int D, int R, int KM, int MODE>
static hipError_t launch_cls_k(const ClassifyArgs &a, hipStream_t st) {
    const size_t lds = classify_lds_bytes(R, D, a.Nb);
    auto kern = [] {
        if constexpr (KM > 32) return classify_wide_kernel<D, R, KM, MODE>;
        else return classify_kernel<D, R, KM, MODE>;
    }();
    hipError_t err = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    const long tiles = (a.Nb + R - 1) / R;
    const unsigned grid = (unsigned)(a.BH * tiles);
    kern<<<grid, CL_THREADS, lds, st>>>(a.qp, MODE != CL_API ? a.kpack : a.kp, a.Nb, classify_packed_keys(a.Nb), a.kc, a.kn,
                                        a.mask, a.crit, a.excl, a.pc, a.marg, a.mbits, a.Nbc, a.Nbp, a.mcount,
                                        a.n_last, a.ulist, a.ucount, a.inv_sqrt_d);
    return hipGetLastError();
}

// keys per lane: ceil(Nb / 64) rounded up to 8, 16, 24, 32 or 38
// (eight rows per workgroup only fit the LDS limit below 1025 blocks)
template <int D, int R, int MODE>
static hipError_t launch_cls_r(const ClassifyArgs &a, hipStream_t st) {
    const int ne = (a.Nb + 63) / 64;
    if (ne <= 8) return launch_cls_k<D, R, 8, MODE>(a, st);
    if (ne <= 16) return launch_cls_k<D, R, 16, MODE>(a, st);
    if constexpr (R < 8) {
        if (ne <= 24) return launch_cls_k<D, R, 24, MODE>(a, st);
        if (ne <= 32) return launch_cls_k<D, R, 32, MODE>(a, st);
        return launch_cls_k<D, R, 38, MODE>(a, st);
    }
    return hipErrorInvalidValue;
}

template <int D, int MODE>
static hipError_t launch_cls_d(const ClassifyArgs &a, hipStream_t st) {
    switch (classify_rows_per_group(a.Nb, D)) {
    case 8: return launch_cls_r<D, 8, MODE>(a, st);
    case 4: return launch_cls_r<D, 4, MODE>(a, st);
    default: return launch_cls_r<D, 2, MODE>(a, st);
    }
}

int classify_packed_keys(int Nb) { return (Nb + 1) & ~1; }

size_t classify_lds_bytes(int R, int D, int Nb) {
    return sizeof(double) * (size_t)R * D + sizeof(uint64_t) * (size_t)R * Nb + (size_t)R * Nb;
}

// the most rows per workgroup with two workgroups' LDS in a compute unit
// (eight rows only up to 1024 blocks, 16 keys per lane)
int classify_rows_per_group(int Nb, int D) {
    const size_t limit = 80 * 1024;
    if (Nb <= 1024 && classify_lds_bytes(8, D, Nb) <= limit) return 8;
    if (classify_lds_bytes(4, D, Nb) <= limit) return 4;
    return 2;   // rows come in pairs; two rows fit for every supported Nb
}

// The forward pass passes the packed key means; float inputs also the pair
// unions (the indicator outputs of either mode are null when the row has no
// linear branch).
hipError_t launch_classify(const ClassifyArgs &a, hipStream_t st) {
    if (!a.kpack) return a.D == 64 ? launch_cls_d<64, CL_API>(a, st) : launch_cls_d<128, CL_API>(a, st);
    if (a.ulist) return a.D == 64 ? launch_cls_d<64, CL_FWD32>(a, st) : launch_cls_d<128, CL_FWD32>(a, st);
    return a.D == 64 ? launch_cls_d<64, CL_FWD16>(a, st) : launch_cls_d<128, CL_FWD16>(a, st);
}

}  // namespace sla
