// lists.hip -- the slot schedule of the 16-bit fused kernel built from block
// lists given by the caller (another mask source than the scores: the LVSA
// page's frame-level sets, or any other block-sparse pattern), for sparse
// attention over those lists with the linear branch off.
//
// For each pair of query-block rows (2p, 2p+1) one wave merges the two
// ascending lists into kmax slots: first the blocks both rows list (one tile
// serves both), ascending, then the i-th block only row 2p lists beside the
// i-th only row 2p+1 lists.  The rows may list different numbers of blocks:
// a row that has no block left in a slot gets NO_TILE there (the fused kernel
// masks its keys), and a pair without row 2p+1 gets 0xFFFF in the high half.
// Entries outside [0, Nb) and entries past a row's count are ignored; a
// repeated index counts once.
#include "sla_device.h"
#include "sla_launch.h"

namespace sla {

namespace {
constexpr uint32_t NO_TILE16 = 0xFFFEu;
}

template <int KM>
__global__ __launch_bounds__(256) void lists_to_slots_kernel(const int32_t *__restrict__ lists,
                                                             const int32_t *__restrict__ counts, int kmax,
                                                             long BH, int Nb, uint32_t *__restrict__ slots) {
    extern __shared__ uint32_t bits[];      // per wave: two rows of Nb bits (words of 32 blocks)
    const int Np = (Nb + 1) / 2;
    const int W = (Nb + 31) / 32;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long pair = (long)blockIdx.x * 4 + wave;
    if (pair >= BH * Np) return;
    const long bh = pair / Np;
    const int p = (int)(pair % Np);
    const int ra = 2 * p, rb = 2 * p + 1;
    const bool has_b = rb < Nb;
    uint32_t *ba = bits + wave * 2 * W, *bb = ba + W;
    // One wave per pair: the LDS runs a wave's accesses in issue order, so
    // waiting for them to complete (and keeping the compiler from moving
    // accesses across the wait) orders the lanes' writes before the reads.
    auto lds_fence = [] { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); };
    for (int x = lane; x < 2 * W; x += 64) ba[x] = 0u;
    lds_fence();
    // membership bits of the two rows
    for (int r = 0; r < 2; ++r) {
        if (r == 1 && !has_b) break;
        const long row = bh * Nb + (r == 0 ? ra : rb);
        const int cnt = min(max(counts[row], 0), kmax);
        uint32_t *bm = r == 0 ? ba : bb;
        for (int x = lane; x < cnt; x += 64) {
            const int j = lists[row * kmax + x];
            if (j >= 0 && j < Nb) atomicOr(&bm[j >> 5], 1u << (j & 31));
        }
    }
    lds_fence();
    const uint64_t lt = (1ull << lane) - 1ull;
    uint16_t *sl = reinterpret_cast<uint16_t *>(slots + pair * (long)kmax);   // (row 2p, row 2p+1) halves
    int ns = 0;
#pragma unroll
    for (int e = 0; e < KM; ++e) {
        const int j = lane + 64 * e;
        const bool a = j < Nb && ((ba[j >> 5] >> (j & 31)) & 1u);
        const bool b = j < Nb && ((bb[j >> 5] >> (j & 31)) & 1u);
        ns += __popcll(__ballot(a && b));
    }
    int rs = 0, rA = 0, rB = 0;
#pragma unroll
    for (int e = 0; e < KM; ++e) {
        const int j = lane + 64 * e;
        const bool a = j < Nb && ((ba[j >> 5] >> (j & 31)) & 1u);
        const bool b = j < Nb && ((bb[j >> 5] >> (j & 31)) & 1u);
        const uint64_t bs = __ballot(a && b), bA = __ballot(a && !b), bB = __ballot(b && !a);
        if (a && b) {
            const int q = rs + __popcll(bs & lt);
            if (q < kmax) { sl[2 * q] = (uint16_t)j; sl[2 * q + 1] = (uint16_t)j; }
        } else if (a) {
            const int q = ns + rA + __popcll(bA & lt);
            if (q < kmax) sl[2 * q] = (uint16_t)j;
        } else if (b) {
            const int q = ns + rB + __popcll(bB & lt);
            if (q < kmax) sl[2 * q + 1] = (uint16_t)j;
        }
        rs += __popcll(bs); rA += __popcll(bA); rB += __popcll(bB);
    }
    // the rest of each half: no block (or no second row)
    for (int q = ns + rA + lane; q < kmax; q += 64) sl[2 * q] = (uint16_t)NO_TILE16;
    for (int q = ns + rB + lane; q < kmax; q += 64) sl[2 * q + 1] = (uint16_t)(has_b ? NO_TILE16 : 0xFFFFu);
}

hipError_t launch_lists_to_slots(const int32_t *lists, const int32_t *counts, int kmax, long BH, int Nb,
                                 uint32_t *slots, hipStream_t st) {
    const long pairs = BH * ((Nb + 1) / 2);
    const unsigned grid = (unsigned)((pairs + 3) / 4);
    const size_t lds = sizeof(uint32_t) * 4 * 2 * ((Nb + 31) / 32);
    const int ne = (Nb + 63) / 64;
    if (ne <= 8) lists_to_slots_kernel<8><<<grid, 256, lds, st>>>(lists, counts, kmax, BH, Nb, slots);
    else if (ne <= 16) lists_to_slots_kernel<16><<<grid, 256, lds, st>>>(lists, counts, kmax, BH, Nb, slots);
    else lists_to_slots_kernel<38><<<grid, 256, lds, st>>>(lists, counts, kmax, BH, Nb, slots);
    return hipGetLastError();
}

}  // namespace sla
