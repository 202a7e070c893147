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
// The product is computed transposed, D^T = Hs^T E^T (M = state column, N =
// query-block row, K = key block), so that each lane ends with 4 consecutive
// columns of one output row.  Tile: 256 columns x 128 rows per workgroup, 4
// waves of 128 x 64, K-steps of 32 key blocks double-buffered through LDS.
// Hs rows (one per key block, columns contiguous) are staged as they are and
// the A fragments (8 consecutive blocks of one column) come out of LDS with
// transposing reads; E rows are staged with a padded stride that keeps the B
// fragment reads free of bank conflicts.  The totals are summed from the very
// chunks each thread stages, then reduced across the 8 threads of a column
// group.  Workgroups are ordered so that the row tiles of one column slice run
// together on one XCD and share its L2.
#include "sla_device.h"
#include "sla_launch.h"

namespace sla {

template <typename S>
__global__ __launch_bounds__(256, 2) void assemble_kernel(const S *__restrict__ E, const S *__restrict__ hs,
                                                          const int32_t *__restrict__ mcount,
                                                          S *__restrict__ hhat, int Nb, int Nbc, int Lp,
                                                          int tiles_m, int tiles_n, long G, int per_xcd) {
    constexpr int TM = 256, TN = 128, TK = 32;
    constexpr int EPC = 16 / sizeof(S);                  // elements per 16-byte chunk
    constexpr int ACPR = TM / EPC;                       // chunks per staged Hs row
    constexpr int NA = TK * ACPR / 256;                  // A chunks per thread
    constexpr int TPA = 256 / ACPR;                      // threads sharing one A column group
    constexpr int ASTR = TM + (sizeof(S) == 2 ? 16 : 8); // staged Hs row stride
    constexpr int BCPR = TK / EPC;                       // chunks per staged E row
    constexpr int NB = TN * BCPR / 256;                  // B chunks per thread
    constexpr int BSTR = TK + EPC;                       // padded E row stride
    __shared__ __attribute__((aligned(16))) S As[2][TK * ASTR];
    __shared__ __attribute__((aligned(16))) S Bs[2][TN * BSTR];
    __shared__ float red[TPA][TM];
    __shared__ float scale_s[TN];

    const long logical = (long)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (logical >= G) return;
    const int tn = (int)(logical % tiles_n);
    const long rest = logical / tiles_n;
    const int tm = (int)(rest % tiles_m);
    const long bh = rest / tiles_m;
    const int col0 = TM * tm, row0 = TN * tn;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5, grp = lane >> 4;
    const int wm = wave & 1, wn = wave >> 1;
    const S *Eh = E + bh * Nb * (long)Nbc;
    const S *Hh = hs + bh * (long)Nbc * Lp;

    const int acg = tid % ACPR, ajr = tid / ACPR;        // this thread's A column group and first row
    float tot[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) tot[e] = 0.f;
    Chunk pa[NA], pb[NB];
    auto gload = [&](int j0) {
#pragma unroll
        for (int u = 0; u < NA; ++u)
            pa[u] = ld_chunk(Hh + (long)(j0 + ajr + TPA * u) * Lp + col0 + acg * EPC);
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int idx = tid + 256 * u, row = idx / BCPR, q = idx % BCPR;
            pb[u] = (row0 + row < Nb) ? ld_chunk(Eh + (long)(row0 + row) * Nbc + j0 + q * EPC) : zero_chunk();
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int u = 0; u < NA; ++u) {
            st_chunk(&As[buf][(ajr + TPA * u) * ASTR + acg * EPC], pa[u]);
            const S *x = reinterpret_cast<const S *>(&pa[u]);
#pragma unroll
            for (int e = 0; e < EPC; ++e) tot[e] += to_f32<S>(x[e]);
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int idx = tid + 256 * u, row = idx / BCPR, q = idx % BCPR;
            st_chunk(&Bs[buf][row * BSTR + q * EPC], pb[u]);
        }
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mt][nt][r] = 0.f;

    const int nst = Nbc / TK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
        if (st + 1 < nst) gload(TK * (st + 1));
        const int buf = st & 1;
#pragma unroll
        for (int s = 0; s < TK / 16; ++s) {
            v8<S> b[2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
                b[nt] = ld8<S>(&Bs[buf][(64 * wn + 32 * nt + l32) * BSTR + 16 * s + 8 * hh]);
            const int k0 = 16 * s + 8 * (grp >> 1);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int n0 = 128 * wm + 32 * mt + 16 * (grp & 1);
                const v8<S> a = cat8<S>(lds_col4<S>(As[buf], ASTR, k0, n0, lane),
                                        lds_col4<S>(As[buf], ASTR, k0 + 4, n0, lane));
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) mma16(acc[mt][nt], a, b[nt]);
            }
        }
        if (st + 1 < nst) lstore(buf ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int e = 0; e < EPC; ++e) red[ajr][acg * EPC + e] = tot[e];
    if (tid < TN) {
        const int i = row0 + tid;
        const int mc = (i < Nb) ? mcount[bh * Nb + i] : 0;
        scale_s[tid] = mc > 0 ? 64.f / (float)mc : 0.f;
    }
    __syncthreads();
    // column totals in LDS (reuse the A staging area)
    float *tot_s = reinterpret_cast<float *>(&As[0][0]);
    {
        float t = 0.f;
#pragma unroll
        for (int x = 0; x < TPA; ++x) t += red[x][tid];
        tot_s[tid] = t;
    }
    __syncthreads();

#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int il = 64 * wn + 32 * nt + l32;
        const int i = row0 + il;
        if (i >= Nb) continue;
        const float sc = scale_s[il];
        S *orow = hhat + (bh * Nb + i) * (long)Lp + col0;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int cl = 128 * wm + 32 * mt + 8 * g + 4 * hh;
                v4<S> y;
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = from_f32<S>((tot_s[cl + e] - acc[mt][nt][4 * g + e]) * sc);
                __builtin_memcpy(orow + cl, &y, sizeof(y));
            }
    }
}

template <typename S>
static hipError_t launch_assemble_t(const AssembleArgs &a, hipStream_t st) {
    const int tiles_m = a.Lp / 256;             // column tiles (Lp is a multiple of 256)
    const int tiles_n = (a.Nb + 127) / 128;     // row tiles
    const long G = a.BH * tiles_m * tiles_n;
    const int per = (int)((G + 7) / 8);
    assemble_kernel<S><<<(unsigned)(8L * per), 256, 0, st>>>((const S *)a.E, (const S *)a.hs, a.mcount,
                                                            (S *)a.hhat, a.Nb, a.Nbc, a.Lp, tiles_m,
                                                            tiles_n, G, per);
    return hipGetLastError();
}

hipError_t launch_assemble(const AssembleArgs &a, hipStream_t st) {
    return a.f32 ? launch_assemble_t<float>(a, st) : launch_assemble_t<f16>(a, st);
}

}  // namespace sla
