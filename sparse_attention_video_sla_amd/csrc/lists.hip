// lists.hip -- the slot schedule of the 16-bit fused kernel built from block
// lists given by the caller (another mask source than the scores), for
// sparse attention over those lists with the linear branch off.
//
// One wave per pair of query-block rows (2p, 2p+1) sets the rows' membership
// bits from their lists and merges them (slot_merge.h).  The rows may list
// different numbers of blocks; entries outside [0, Nb) and entries past a
// row's count are ignored, and a repeated index counts once.
#include "sla_device.h"
#include "sla_launch.h"
#include "slot_merge.h"

namespace sla {

template <int KM>
__global__ __launch_bounds__(256) void lists_to_slots_kernel(const int32_t *__restrict__ lists,
                                                             const int32_t *__restrict__ counts, int kmax,
                                                             long BH, int Nb, uint32_t *__restrict__ slots,
                                                             int32_t *__restrict__ pcount) {
    extern __shared__ uint32_t bits[];      // per wave: two rows of Nb bits (words of 32 blocks)
    const int Np = (Nb + 1) / 2;
    const int W = (Nb + 31) / 32;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long pair = (long)blockIdx.x * 4 + wave;
    if (pair >= BH * Np) return;
    const long bh = pair / Np;
    const int p = (int)(pair % Np);
    const bool has_b = 2 * p + 1 < Nb;
    uint32_t *ba = bits + wave * 2 * W, *bb = ba + W;
    for (int x = lane; x < 2 * W; x += 64) ba[x] = 0u;
    wave_lds_fence();
    for (int r = 0; r < 2; ++r) {
        if (r == 1 && !has_b) break;
        const long row = bh * Nb + 2 * p + r;
        const int cnt = min(max(counts[row], 0), kmax);
        uint32_t *bm = r == 0 ? ba : bb;
        for (int x = lane; x < cnt; x += 64) {
            const int j = lists[row * kmax + x];
            if (j >= 0 && j < Nb) atomicOr(&bm[j >> 5], 1u << (j & 31));
        }
    }
    wave_lds_fence();
    uint16_t *sl = reinterpret_cast<uint16_t *>(slots + pair * (long)kmax);
    const int n = merge_pair<KM>(ba, bb, has_b, Nb, kmax, sl, [](int, int) { return 0u; });
    if (lane == 0) pcount[pair] = n;
}

hipError_t launch_lists_to_slots(const int32_t *lists, const int32_t *counts, int kmax, long BH, int Nb,
                                 uint32_t *slots, int32_t *pcount, hipStream_t st) {
    const long pairs = BH * ((Nb + 1) / 2);
    const unsigned grid = (unsigned)((pairs + 3) / 4);
    const size_t lds = sizeof(uint32_t) * 4 * 2 * ((Nb + 31) / 32);
    const int ne = (Nb + 63) / 64;
    if (ne <= 8) lists_to_slots_kernel<8><<<grid, 256, lds, st>>>(lists, counts, kmax, BH, Nb, slots, pcount);
    else if (ne <= 16) lists_to_slots_kernel<16><<<grid, 256, lds, st>>>(lists, counts, kmax, BH, Nb, slots, pcount);
    else if (ne <= 32) lists_to_slots_kernel<32><<<grid, 256, lds, st>>>(lists, counts, kmax, BH, Nb, slots, pcount);
    else lists_to_slots_kernel<64><<<grid, 256, lds, st>>>(lists, counts, kmax, BH, Nb, slots, pcount);
    return hipGetLastError();
}

}  // namespace sla
