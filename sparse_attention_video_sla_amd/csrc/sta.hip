// sta.hip -- sliding tile attention (the VORTA page, "Key designs", item 1:
// a 3D sliding window whose mask is made block-dense by tiles) as a block
// schedule of the 16-bit fused kernel.
//
// Tokens are tile-major: the grid (F, Hh, Ww) is cut into tiles (tf, th, tw),
// tiles in raster order over the tile grid, tokens in raster order inside a
// tile; a tile of V = tf*th*tw tokens (a multiple of 64) is V/64 whole key or
// query blocks.  On every axis a query tile keeps the key tiles whose centre
// lies in (centre - W/2, centre + W/2] of its own centre for the axis window
// W; the centres of tiles g and g + delta differ by delta*t, so the test is
// 2*delta*t in (-W, W], and tiles past the grid do not exist.  The schedule
// depends on the tile only, so one schedule serves every head.
#include "sla_device.h"
#include "sla_launch.h"
#include "slot_merge.h"

namespace sla {

// one wave per pair of query-block rows
template <int KM>
__global__ __launch_bounds__(256) void sta_slots_kernel(StaParams p, int Nb, int kmax, uint32_t *__restrict__ slots,
                                                        int32_t *__restrict__ pcount) {
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
    const int bpt = p.vol / 64;                          // blocks per tile
    const int nd[3] = {2 * p.rf + 1, 2 * p.rh + 1, 2 * p.rw + 1};
    const int ncomb = nd[0] * nd[1] * nd[2];
    for (int r = 0; r < 2; ++r) {
        if (r == 1 && !has_b) break;
        uint32_t *bm = r == 0 ? ba : bb;
        const int g = (2 * pair + r) / bpt;              // query tile
        const int gf = g / (p.gh * p.gw), gh = (g / p.gw) % p.gh, gw = g % p.gw;
        for (int c = lane; c < ncomb; c += 64) {
            const int df = c / (nd[1] * nd[2]) - p.rf, dh = (c / nd[2]) % nd[1] - p.rh, dw = c % nd[2] - p.rw;
            const bool keep = 2 * df * p.tf > -p.wf && 2 * df * p.tf <= p.wf && 2 * dh * p.th > -p.wh &&
                              2 * dh * p.th <= p.wh && 2 * dw * p.tw > -p.ww && 2 * dw * p.tw <= p.ww;
            const int kf = gf + df, kh_ = gh + dh, kw = gw + dw;
            if (!keep || kf < 0 || kf >= p.gf || kh_ < 0 || kh_ >= p.gh || kw < 0 || kw >= p.gw) continue;
            const int b0 = ((kf * p.gh + kh_) * p.gw + kw) * bpt, b1 = b0 + bpt - 1;
            for (int w = b0 >> 5; w <= (b1 >> 5); ++w) {
                const int lo = max(b0, 32 * w) - 32 * w, hi = min(b1, 32 * w + 31) - 32 * w;
                const uint32_t m = (hi == 31 ? 0xFFFFFFFFu : ((1u << (hi + 1)) - 1u)) & ~((1u << lo) - 1u);
                atomicOr(&bm[w], m);
            }
        }
    }
    wave_lds_fence();
    uint16_t *sl = reinterpret_cast<uint16_t *>(slots + (long)pair * kmax);
    const int n = merge_pair<KM>(ba, bb, has_b, Nb, kmax, sl, [](int, int) { return 0u; });
    if (lane == 0) pcount[pair] = n;
}

hipError_t launch_sta_slots(const StaParams &p, int Nb, int kmax, uint32_t *slots, int32_t *pcount, hipStream_t st) {
    const int Np = (Nb + 1) / 2;
    const unsigned grid = (unsigned)((Np + 3) / 4);
    const size_t lds = sizeof(uint32_t) * 4 * 2 * ((Nb + 31) / 32);
    const int ne = (Nb + 63) / 64;
    if (ne <= 8) sta_slots_kernel<8><<<grid, 256, lds, st>>>(p, Nb, kmax, slots, pcount);
    else if (ne <= 16) sta_slots_kernel<16><<<grid, 256, lds, st>>>(p, Nb, kmax, slots, pcount);
    else if (ne <= 32) sta_slots_kernel<32><<<grid, 256, lds, st>>>(p, Nb, kmax, slots, pcount);
    else sta_slots_kernel<64><<<grid, 256, lds, st>>>(p, Nb, kmax, slots, pcount);
    return hipGetLastError();
}

}  // namespace sla
