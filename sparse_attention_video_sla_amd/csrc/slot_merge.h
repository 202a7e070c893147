// slot_merge.h -- one wave merges the key-block sets of a pair of query-block
// rows (2p, 2p+1) into the pair's slots of the 16-bit fused kernel: first the
// blocks both rows hold (one tile serves both), ascending, then the i-th block
// only row 2p holds beside the i-th only row 2p+1 holds.  A row with no block
// left in a slot gets the padding half 0xFFFE there (marks 0xF: no key seen);
// a pair without row 2p+1 gets 0xFFFF in the high half.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sla {

constexpr uint16_t SLOT_PAD = 0xFFFEu;
constexpr uint16_t SLOT_NO_ROW = 0xFFFFu;

// ba, bb: the rows' membership bits (word w holds blocks 32w .. 32w + 31),
// written by this wave; mark(r, j) gives the 4 frame-mark bits of block j in
// row r (0 when every key of the block is seen).  Writes kmax slots and
// returns the number the pair uses (<= kmax).
template <int KM, typename Mark>
__device__ __forceinline__ int merge_pair(const uint32_t *ba, const uint32_t *bb, bool has_b, int Nb, int kmax,
                                          uint16_t *sl, Mark mark) {
    const int lane = threadIdx.x & 63;
    const uint64_t lt = (1ull << lane) - 1ull;
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
            if (q < kmax) {
                sl[2 * q] = (uint16_t)(j | (mark(0, j) << 12));
                sl[2 * q + 1] = (uint16_t)(j | (mark(1, j) << 12));
            }
        } else if (a) {
            const int q = ns + rA + __popcll(bA & lt);
            if (q < kmax) sl[2 * q] = (uint16_t)(j | (mark(0, j) << 12));
        } else if (b) {
            const int q = ns + rB + __popcll(bB & lt);
            if (q < kmax) sl[2 * q + 1] = (uint16_t)(j | (mark(1, j) << 12));
        }
        rs += __popcll(bs); rA += __popcll(bA); rB += __popcll(bB);
    }
    for (int q = ns + rA + lane; q < kmax; q += 64) sl[2 * q] = SLOT_PAD;
    for (int q = ns + rB + lane; q < kmax; q += 64) sl[2 * q + 1] = has_b ? SLOT_PAD : SLOT_NO_ROW;
    return min(ns + max(rA, rB), kmax);
}

// LDS accesses of one wave complete in issue order: waiting for them (and
// keeping the compiler from moving accesses across the wait) orders the
// lanes' writes before the other lanes' reads
__device__ __forceinline__ void wave_lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

}  // namespace sla
