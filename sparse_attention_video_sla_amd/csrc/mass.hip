// mass.hip -- exact block attention mass, a diagnostic of the three-way mask
// (SLA article, section 2: a few attention weights carry most of the mass;
// the mask keeps the blocks that hold it).
//
//   mass[bh][i][j] = mean over the valid rows r of query block i of the sum,
//                    over the valid keys u of key block j, of the softmax of
//                    q_r . k_u / sqrt(d) over all N keys of the head.
//
// Each row of blocks sums to 1.  bf16 inputs, d in {64, 128}.
//
// One workgroup of 8 waves per 4 consecutive query blocks of a head (wave w:
// query rows 32w .. 32w+31 of the 256), two passes over the key blocks of
// the head: the running row max and sum, then the block sums of the
// normalised probabilities.  Each 64-key tile goes through LDS once per pass
// for the 8 waves (register-staged double buffer, one barrier per tile);
// S^T = K Q^T on bf16 MFMA with Q in registers and K rows read from a
// swizzled tile (16-byte chunk c of row r at chunk c ^ f(r): conflict-free).
// Per tile and wave, the probabilities of its 32 rows are summed in the lanes
// and across the wave into LDS; the two waves of a query block are added in a
// fixed order at the end, so the result is the same on every run.
#include "sla_device.h"
#include "sla_launch.h"

namespace sla {

namespace {

// swizzle of the staged K tile: chunk c of row r sits at chunk c ^ mswz(r)
template <int D> __device__ __forceinline__ int mswz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}
__device__ __forceinline__ float half_max(float x) { return fmaxf(x, __shfl_xor(x, 32, 64)); }
__device__ __forceinline__ float half_sum(float x) { return x + __shfl_xor(x, 32, 64); }

}  // namespace

template <int D>
__global__ __launch_bounds__(512) void block_mass16_kernel(const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                                                           int N, int Nb, int tiles_i, float sl2,
                                                           float *__restrict__ mass) {
    constexpr int NS = D / 16;               // k-steps over channels
    constexpr int CPR = D / 8;               // 16-byte chunks per key row
    constexpr int NCH = 64 * CPR / 512;      // staged chunks per thread and tile
    constexpr float NEG_INF = -__builtin_inff();
    __shared__ __attribute__((aligned(16))) bf16 Kt[2][64 * D];
    extern __shared__ float part[];          // [8 waves][Nb] partial masses

    const int it = blockIdx.x % tiles_i;
    const long bh = blockIdx.x / tiles_i;
    const int i0 = 4 * it;                   // first query block of the workgroup
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hh = lane >> 5;

    // Q rows of this wave as B fragments: lane (q, h) holds channels 16s + 8h .. +7
    const int qrow = 64 * i0 + 32 * wave + l32;
    const bool qvalid = qrow < N;
    v8<bf16> qf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = qvalid ? ld8<bf16>(q + (bh * N + qrow) * (long)D + 16 * s + 8 * hh) : zero8<bf16>();

    const bf16 *kh = k + bh * (long)N * D;
    Chunk kc[NCH];
    auto gload = [&](int j) {
#pragma unroll
        for (int u = 0; u < NCH; ++u) {
            const int ch = tid + 512 * u, row = ch / CPR, c = ch % CPR;
            const int key = 64 * j + row;
            kc[u] = key < N ? ld_chunk(kh + (long)key * D + 8 * c) : zero_chunk();
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int u = 0; u < NCH; ++u) {
            const int ch = tid + 512 * u, row = ch / CPR, c = ch % CPR;
            st_chunk(&Kt[buf][row * D + 8 * (c ^ mswz<D>(row))], kc[u]);
        }
    };
    // S^T for the two 32-key halves of tile K: sa[kt][r] is the score of key
    // 32 kt + 8 (r >> 2) + 4 hh + (r & 3) of the tile against query l32
    f32x16 sa[2];
    auto tile_scores = [&](const bf16 *K) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sa[kt][r] = 0.f;
            const int row = 32 * kt + l32;
#pragma unroll
            for (int s = 0; s < NS; ++s)
                mma16(sa[kt], ld8<bf16>(K + row * D + 8 * ((2 * s + hh) ^ mswz<D>(row))), qf[s]);
        }
    };
    auto key_of = [&](int j, int kt, int r) { return 64 * j + 32 * kt + 8 * (r >> 2) + 4 * hh + (r & 3); };

    // pass 1: running max m (log2 units) and sum l of the row of query l32
    float m = NEG_INF, l = 0.f;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int j = 0; j < Nb; ++j) {
        if (j + 1 < Nb) gload(j + 1);
        tile_scores(Kt[j & 1]);
        const bool ragged = 64 * j + 64 > N;
        float mx = NEG_INF;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if (ragged && key_of(j, kt, r) >= N) sa[kt][r] = NEG_INF;
                mx = fmaxf(mx, sa[kt][r]);
            }
        const float mnew = fmaxf(m, half_max(mx) * sl2);
        float se = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) se += fast_exp2(__builtin_fmaf(sa[kt][r], sl2, -mnew));
        l = l * fast_exp2(m - mnew) + half_sum(se);
        m = mnew;
        if (j + 1 < Nb) lstore((j + 1) & 1);
        __syncthreads();
    }

    // pass 2: the normalised probabilities of this wave's rows summed per key block
    const float inv_l = (qvalid && l > 0.f) ? 1.f / l : 0.f;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int j = 0; j < Nb; ++j) {
        if (j + 1 < Nb) gload(j + 1);
        tile_scores(Kt[j & 1]);
        const bool ragged = 64 * j + 64 > N;
        float ps = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = fast_exp2(__builtin_fmaf(sa[kt][r], sl2, -m));
                ps += (ragged && key_of(j, kt, r) >= N) ? 0.f : p;
            }
        ps = wave_sum(ps * inv_l);
        if (lane == 0) part[wave * Nb + j] = ps;
        if (j + 1 < Nb) lstore((j + 1) & 1);
        __syncthreads();
    }

    // the two waves of each query block, in a fixed order, over its valid rows
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int i = i0 + b;
        if (i >= Nb) break;
        const float inv_n = 1.f / (float)min(64, N - 64 * i);
        float *row = mass + (bh * Nb + i) * (long)Nb;
        for (int j = tid; j < Nb; j += 512) row[j] = (part[(2 * b) * Nb + j] + part[(2 * b + 1) * Nb + j]) * inv_n;
    }
}

// Per row of blocks (one wave per row (bh, i)), from the mass row and the
// labels: the mass on the critical (+1), marginal (0) and negligible (-1)
// blocks, and the 95 % block density: the smallest number of blocks, taken
// by decreasing mass, whose mass reaches 0.95 of the row's total, over Nb.
// The count comes from a bitwise search for the threshold t (masses are >= 0,
// so their bit patterns order like their values): the largest t with
// sum{mass >= t} >= target; then #{mass > t} plus the blocks equal to t
// added one at a time until the target is reached.  Every sum is in fp64
// (per-lane partials in block order, then a fixed wave reduction), so the
// count is the one an fp64 cumulative sum over the sorted masses gives,
// except for a row whose cumulative mass lies within fp64 rounding of the
// target.
__device__ __forceinline__ double wave_sum_f64(double x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

template <int KM>
__global__ __launch_bounds__(256) void mask_stats_kernel(const float *__restrict__ mass, const int8_t *__restrict__ mask,
                                                         long rows, int Nb, float *__restrict__ stats) {
    const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int lane = threadIdx.x & 63;
    const float *mr = mass + row * Nb;
    const int8_t *lr = mask + row * Nb;
    uint32_t key[KM];
    double cls[3] = {0.0, 0.0, 0.0};                     // negligible, marginal, critical
    double tot = 0.0;
#pragma unroll
    for (int e = 0; e < KM; ++e) {
        const int j = lane + 64 * e;
        const float x = j < Nb ? fmaxf(mr[j], 0.f) : 0.f;
        key[e] = __float_as_uint(x);
        if (j < Nb) {
            const int lb = lr[j];
            cls[lb + 1] += (double)x;
            tot += (double)x;
        }
    }
#pragma unroll
    for (int c = 0; c < 3; ++c) cls[c] = wave_sum_f64(cls[c]);
    tot = wave_sum_f64(tot);
    const double target = 0.95 * tot;
    auto sum_ge = [&](uint32_t t) {
        double s = 0.0;
#pragma unroll
        for (int e = 0; e < KM; ++e) s += key[e] >= t ? (double)__uint_as_float(key[e]) : 0.0;
        return wave_sum_f64(s);
    };
    uint32_t lo = 0;
    for (int bit = 30; bit >= 0; --bit) {               // bit 31 (sign) is 0 for every mass
        const uint32_t cand = lo | (1u << bit);
        if (sum_ge(cand) >= target) lo = cand;
    }
    int gt = 0, eq = 0;
    double sgt = 0.0;
#pragma unroll
    for (int e = 0; e < KM; ++e) {
        const bool ok = lane + 64 * e < Nb;
        gt += (ok && key[e] > lo) ? 1 : 0;
        eq += (ok && key[e] == lo) ? 1 : 0;
        sgt += (ok && key[e] > lo) ? (double)__uint_as_float(key[e]) : 0.0;
    }
    gt = (int)wave_sum_f64((double)gt);
    eq = (int)wave_sum_f64((double)eq);
    sgt = wave_sum_f64(sgt);
    const double t = (double)__uint_as_float(lo);
    int need = gt;
    for (double s = sgt; need < gt + eq && s < target; ++need) s += t;
    if (lane == 0) {
        float *o = stats + row * 4;
        o[0] = (float)cls[2];
        o[1] = (float)cls[1];
        o[2] = (float)cls[0];
        o[3] = (float)need / (float)Nb;
    }
}

template <int D>
static hipError_t launch_mass_t(const MassArgs &a, hipStream_t st) {
    const int tiles_i = (a.Nb + 3) / 4;
    const size_t lds = sizeof(float) * 8 * (size_t)a.Nb;
    auto kern = block_mass16_kernel<D>;
    hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const float sl2 = 1.4426950408889634f / sqrtf((float)D);
    kern<<<(unsigned)(a.BH * tiles_i), 512, lds, st>>>((const bf16 *)a.q, (const bf16 *)a.k, a.N, a.Nb, tiles_i, sl2,
                                                       a.mass);
    return hipGetLastError();
}

hipError_t launch_block_mass(const MassArgs &a, hipStream_t st) {
    return a.D == 64 ? launch_mass_t<64>(a, st) : launch_mass_t<128>(a, st);
}

hipError_t launch_mask_stats(const float *mass, const int8_t *mask, long rows, int Nb, float *stats, hipStream_t st) {
    const unsigned grid = (unsigned)((rows + 3) / 4);
    const int ne = (Nb + 63) / 64;
    if (ne <= 8) mask_stats_kernel<8><<<grid, 256, 0, st>>>(mass, mask, rows, Nb, stats);
    else if (ne <= 16) mask_stats_kernel<16><<<grid, 256, 0, st>>>(mass, mask, rows, Nb, stats);
    else mask_stats_kernel<38><<<grid, 256, 0, st>>>(mass, mask, rows, Nb, stats);
    return hipGetLastError();
}

}  // namespace sla
