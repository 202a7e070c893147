// pool.hip -- block means of Q and K (SLA article, section 3: the compressed
// attention map is scored on mean-pooled Q and K).
//
// One thread owns 16 bytes of channels (8 bf16 or 4 float) of one block of one
// tensor and walks the block's valid tokens in ascending order, accumulating
// in fp64; the sum divided by the valid count (IEEE fp64 division) is rounded
// once to float32.  For bf16 inputs the fp64 sum of <= 64 values is exact; for
// float inputs the fixed ascending order makes the result reproducible.
// HBM-bound: each token row is read once, 16 rows in flight per thread.
#include "sla_device.h"
#include "sla_launch.h"

namespace sla {

template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                   float *__restrict__ qp, float *__restrict__ kp,
                                                   float *__restrict__ kpack, int Nb2, long BH, int N, int Nb,
                                                   int blk) {
    constexpr int CG = 16 / sizeof(T);   // channels per thread
    constexpr int TPB = D / CG;          // threads per (tensor, head, block)
    constexpr int BATCH = 16;            // rows loaded before they are summed
    const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long per_tensor = BH * Nb * TPB;
    if (gid >= 2 * per_tensor) return;
    const int which = gid >= per_tensor;
    const long r = gid - which * per_tensor;
    const int cg = (int)(r % TPB);
    const long rb = r / TPB;
    const int i = (int)(rb % Nb);
    const long bh = rb / Nb;
    const T *x = (which ? k : q) + (bh * N + (long)i * blk) * D + cg * CG;
    const int n = min(blk, N - i * blk);

    double s[CG];
#pragma unroll
    for (int e = 0; e < CG; ++e) s[e] = 0.0;
    for (int t0 = 0; t0 < n; t0 += BATCH) {
        Chunk c[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) c[u] = (t0 + u < n) ? ld_chunk(x + (long)(t0 + u) * D) : zero_chunk();
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            if (t0 + u < n) {
                const T *v = reinterpret_cast<const T *>(&c[u]);
#pragma unroll
                for (int e = 0; e < CG; ++e) s[e] += (double)to_f32<T>(v[e]);
            }
        }
    }
    float res[CG];
#pragma unroll
    for (int e = 0; e < CG; ++e) res[e] = (float)(s[e] / (double)n);
    float *o = (which ? kp : qp) + (bh * Nb + i) * D + cg * CG;
#pragma unroll
    for (int e = 0; e < CG; e += 4) st_chunk(o + e, *reinterpret_cast<const Chunk *>(&res[e]));
    if (which && kpack) {   // channels 4 c4 .. +3 of key block i at [bh][c4][i][0..3]
#pragma unroll
        for (int e = 0; e < CG; e += 4) {
            const long c4 = (cg * CG + e) / 4;
            st_chunk(kpack + ((bh * (D / 4) + c4) * Nb2 + i) * 4, *reinterpret_cast<const Chunk *>(&res[e]));
        }
    }
}

template <typename T, int D>
hipError_t launch_pool_t(const void *q, const void *k, float *qp, float *kp, float *kpack, long BH, int N,
                         int Nb, int blk, hipStream_t st) {
    constexpr int TPB = D / (16 / sizeof(T));
    const long threads = 2 * BH * (long)Nb * TPB;
    const unsigned grid = (unsigned)((threads + 255) / 256);
    pool_kernel<T, D><<<grid, 256, 0, st>>>((const T *)q, (const T *)k, qp, kp, kpack, classify_packed_keys(Nb), BH,
                                            N, Nb, blk);
    return hipGetLastError();
}

hipError_t launch_pool(bool bf16_in, int D, const void *q, const void *k, float *qp, float *kp, float *kpack,
                       long BH, int N, int Nb, int blk, hipStream_t st) {
    if (bf16_in) {
        return D == 64 ? launch_pool_t<bf16, 64>(q, k, qp, kp, kpack, BH, N, Nb, blk, st)
                       : launch_pool_t<bf16, 128>(q, k, qp, kp, kpack, BH, N, Nb, blk, st);
    }
    return D == 64 ? launch_pool_t<float, 64>(q, k, qp, kp, kpack, BH, N, Nb, blk, st)
                   : launch_pool_t<float, 128>(q, k, qp, kp, kpack, BH, N, Nb, blk, st);
}

}  // namespace sla
