// assemble.hip -- marginal linear-attention states per query-block row.
//
// For each row i the linear branch needs H_i = sum over the marginal key
// blocks of h_j (and Z_i likewise).  They are formed as the total over all
// key blocks minus the excluded (critical and negligible) ones:
//     H_i = H_tot - sum_j E_ij h_j,   E_ij = 1 if block j is critical or negligible.
// The excluded sums for all rows of a head are one dense GEMM E * Hs
// ([Nb x Nb] 0/1 times [Nb x (d*d+d)]) on fp16 MFMA with fp32 accumulation
// (float MFMA for float inputs); the 0/1 matrix is exact in fp16.  The
// totals are summed by the same workgroup from the very Hs values it streams,
// so H_tot and the excluded sums subtract consistently.
// Output row i is (H_tot - E_i Hs) * 64 / m_i with m_i the row's marginal
// token count: the linear output phi(q) H / (phi(q).Z) does not depend on a
// common scale of H and Z, and this one keeps |values| <= max|V W^T|.
//
// Tile: 128 rows x 128 columns per workgroup, 4 waves of 64 x 64, K-steps of
// 32 key blocks double-buffered through LDS; Hs arrives row-major (columns
// contiguous) and is transposed on its way into LDS so that each lane reads
// 8 consecutive key blocks of one column as its B fragment.
#include "sla_device.h"
#include "sla_launch.h"

namespace sla {

template <typename S>
__global__ __launch_bounds__(256) void assemble_kernel(const S *__restrict__ E, const S *__restrict__ hs,
                                                       const int32_t *__restrict__ mcount,
                                                       S *__restrict__ hhat, int Nb, int Nbc, int Lp,
                                                       int tiles_m, int tiles_n) {
    constexpr int EPC = 16 / sizeof(S);     // elements per 16-byte chunk
    constexpr int CPR = 128 / EPC;          // chunks per 128-column row
    constexpr int TPC = 256 / CPR;          // threads sharing one column group
    constexpr int NCH = 32 * CPR / 256;     // chunks per thread per stage
    constexpr int BSTR = 32 + EPC;          // transposed tile row stride
    __shared__ S Bs[2][128 * BSTR];
    __shared__ float red[TPC][128];
    __shared__ float totc[128];

    const int bid = blockIdx.x;
    const int tm = bid % tiles_m;
    const int rest = bid / tiles_m;
    const int tn = rest % tiles_n;
    const long bh = rest / tiles_n;
    const int row0 = 128 * tm, col0 = 128 * tn;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int wr = wave >> 1, wc = wave & 1;
    const S *Eh = E + bh * Nb * (long)Nbc;
    const S *Hh = hs + bh * Nb * (long)Lp;

    const int cg = tid % CPR, jr = tid / CPR;
    float tot[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) tot[e] = 0.f;
    Chunk pre[NCH];
    auto gload = [&](int j0) {
#pragma unroll
        for (int u = 0; u < NCH; ++u) {
            const int j = j0 + jr + TPC * u;
            pre[u] = (j < Nb) ? ld_chunk(Hh + (long)j * Lp + col0 + cg * EPC) : zero_chunk();
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int u = 0; u < NCH; ++u) {
            const int jj = jr + TPC * u;
            const S *x = reinterpret_cast<const S *>(&pre[u]);
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                Bs[buf][(cg * EPC + e) * BSTR + jj] = x[e];
                tot[e] += to_f32<S>(x[e]);
            }
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mt][nt][r] = 0.f;

    const int nst = Nbc / 32;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
        if (st + 1 < nst) gload(32 * (st + 1));
        const int buf = st & 1;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            v8<S> a[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const int i = row0 + 64 * wr + 32 * mt + l32;
                a[mt] = (i < Nb) ? ld8<S>(Eh + (long)i * Nbc + 32 * st + 16 * ks + 8 * hh) : zero8<S>();
            }
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const v8<S> b = ld8<S>(&Bs[buf][(64 * wc + 32 * nt + l32) * BSTR + 16 * ks + 8 * hh]);
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) mma16(acc[mt][nt], a[mt], b);
            }
        }
        if (st + 1 < nst) lstore(buf ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int e = 0; e < EPC; ++e) red[jr][cg * EPC + e] = tot[e];
    __syncthreads();
    if (tid < 128) {
        float t = 0.f;
#pragma unroll
        for (int x = 0; x < TPC; ++x) t += red[x][tid];
        totc[tid] = t;
    }
    __syncthreads();

#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = row0 + 64 * wr + 32 * mt + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (i >= Nb) continue;
            const int mc = mcount[bh * Nb + i];
            const float sc = mc > 0 ? 64.f / (float)mc : 0.f;
            S *orow = hhat + (bh * Nb + i) * (long)Lp + col0;
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int col = 64 * wc + 32 * nt + l32;
                orow[col] = from_f32<S>((totc[col] - acc[mt][nt][r]) * sc);
            }
        }
    }
}

template <typename S>
static hipError_t launch_assemble_t(const AssembleArgs &a, hipStream_t st) {
    const int tiles_m = (a.Nb + 127) / 128;
    const int tiles_n = a.Lp / 128;
    const unsigned grid = (unsigned)(a.BH * tiles_m * tiles_n);
    assemble_kernel<S><<<grid, 256, 0, st>>>((const S *)a.E, (const S *)a.hs, a.mcount, (S *)a.hhat,
                                             a.Nb, a.Nbc, a.Lp, tiles_m, tiles_n);
    return hipGetLastError();
}

hipError_t launch_assemble(const AssembleArgs &a, hipStream_t st) {
    return a.f32 ? launch_assemble_t<float>(a, st) : launch_assemble_t<f16>(a, st);
}

}  // namespace sla
