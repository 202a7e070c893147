// fused16.hip -- the three SLA branches in one kernel for bf16 inputs (SLA
// article, section 3: exact block-sparse FlashAttention over the critical
// blocks, linear attention over the marginal ones, negligible ones skipped,
// in one GPU kernel, with the learnable projection on the linear output).
//
// One workgroup of 8 waves per pair of consecutive query blocks (A = 2p,
// B = 2p+1) of one head.  Wave w: key half kh = w >> 2, block b = (w >> 1) & 1,
// query rows 32qh .. 32qh+31 with qh = w & 1.
//
// Slot schedule.  Both rows select exactly k_c key blocks, so the classifier
// pairs them into k_c slots: a block both rows selected is one shared tile,
// and otherwise the i-th block only A selected sits beside the i-th only B
// selected.  Every wave therefore has one tile in every slot and none idles.
//
// Key halves.  The waves with kh = 0 take keys 0..31 of every tile and those
// with kh = 1 keys 32..63, each with its own online softmax (running max m,
// sum l, output O over its keys); the two partial results of a query row
// merge at the end.  The normalisation runs over the union of all critical
// keys of the row (block-sparse softmax of the LVSA page, method steps).
//
// Two phases per slot n, separated by workgroup barriers:
//   MFMA(n):  O^T += V^T P^T for slot n-1 on V^T fragments already in
//             registers (P^T straight from the previous softmax), then
//             S^T = K Q^T for slot n (K rows from LDS, Q held in registers):
//             16 MFMAs, the K reads landing while the first 8 run;
//   VALU(n):  the transposing V reads of slot n for the next PV (landing
//             while the softmax runs), then row max with a cross-half lane
//             swap, lazy rescale of O, P in the log2 domain with the
//             1/sqrt(d) scale folded into one fma, converted to bf16 in the
//             MFMA operand layout.
// The kh = 1 waves run one phase behind the kh = 0 waves, so on every SIMD
// (which holds one wave of each) one wave's MFMAs overlap the other's
// softmax.
//
// Data movement.  K and V tiles go from global memory straight into LDS
// (buffer loads with the LDS destination, no registers in between): on
// gfx950 those writes do not slow the concurrent LDS reads the way
// ds_write does.  Each tensor has a two-slot ring (a slot holds the A and the
// B tile), four separate LDS arrays, and the loop is unrolled by two so that
// every access names its array: the compiler then waits for a load only
// before reads of the array it fills.  Loads are issued only by waves in
// their VALU phase (a wave streaming MFMAs would stall on them): in VALU(n)
// the kh = 0 group loads V of slot n+1 and the kh = 1 group K of slot n+2;
// each waits for its loads after its next MFMA phase.
//   K tile: rows of d elements, 16-byte chunk c of row r at chunk c ^ f(r),
//     so the 16-byte A-operand reads of 16 consecutive rows are conflict-free.
//   V tile: groups of 4 rows; inside a group chunk c of row 4g + m at
//     position 4c + m, so the transposing reads (4 rows x 16 columns per 16
//     lanes) are conflict-free and their offsets are compile-time constants.
//
// After the sparse part the two halves merge through LDS, each wave keeping
// half of the output channels, and add the linear branch for them:
// y = phi(q) Hhat_i^T / (phi(q).Zhat_i), phi = softmax over channels, Hhat_i
// already projected by W.  Workgroups are ordered so that each XCD (own L2)
// takes a contiguous run of (head, pair).
#include "sla_device.h"
#include "sla_launch.h"
#include "tile_common.h"

#include <type_traits>

namespace sla {

namespace {

template <typename TO> __device__ __forceinline__ void store4(TO *p, float a, float b, float c, float d);
template <> __device__ __forceinline__ void store4<float>(float *p, float a, float b, float c, float d) {
    f32x4 v = {a, b, c, d};
    *reinterpret_cast<f32x4 *>(p) = v;
}
template <> __device__ __forceinline__ void store4<bf16>(bf16 *p, float a, float b, float c, float d) {
    v4<bf16> v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
    __builtin_memcpy(p, &v, sizeof(v));
}

// slot entry: the half of row 2p in the low 16 bits, of row 2p+1 in the
// high 16 bits.  A half holds a key block index in its low 12 bits (clamped
// to Nb - 1 when used) and, in its top 4 bits, the pairs of frame parts it
// must not score: bit 2a + c set means that the query rows of part a of the
// query block do not see the keys of part c of the key block, where part 1
// of a block is what follows the frame boundary inside it (blocks of tokens
// from one frame have only part 0).  0 (the usual case): every key is seen;
// 0xF: none, the slot is padding for this row; 0xFFFF: the pair has no
// second row.
constexpr uint32_t IDX_BITS = 0xFFFu;
__device__ __forceinline__ int slot_tile(uint32_t e, int which, int Nb) {
    return min((int)((which ? (e >> 16) : e) & IDX_BITS), Nb - 1);
}
// one tile serves the slot: both rows name the same block, or the second row
// has none (no row, or padding in this slot)
__device__ __forceinline__ bool slot_single(uint32_t e) {
    return ((e >> 16) & IDX_BITS) == (e & IDX_BITS) || (e >> 28) == 0xFu;
}
// offset of the first token of the block's part 1 (a frame boundary inside
// the block), 64 when the block lies in one frame; frames of fp >= 64 tokens
__device__ __forceinline__ int frame_split(int blk, int fp) {
    const int start = 64 * blk;
    const int bnd = (start / fp + 1) * fp - start;
    return bnd < 64 ? bnd : 64;
}

}  // namespace

// MARKS: the slots may carry frame marks (schedules from frame sets); without
// it a half's top bits are 0 or 0xF only.
template <typename T, typename S, int D, typename TO, bool MARKS>
__global__ __launch_bounds__(512, 1) void fused16_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                         const T *__restrict__ v,
                                                         const uint32_t *__restrict__ slots, int kc_max,
                                                         const int32_t *__restrict__ pcount, int bcast, int fp,
                                                         const S *__restrict__ hhat,
                                                         const int32_t *__restrict__ mcount, int Lp,
                                                         TO *__restrict__ out, float *__restrict__ lse, long G,
                                                         int per_xcd, int N, int Nb, float sl2) {
    static_assert(__is_same(T, bf16), "bf16 inputs");
    constexpr int TILE = 64 * D;                         // elements of one tile (no padding)
    constexpr int NB1 = D / 32;                          // 1 KB loads per kh = 0 wave per tile
    constexpr int NS = D / 16;                           // k-steps over channels
    constexpr int NCT = D / 32;                          // 32-channel tiles of O
    constexpr int NCH = NCT / 2;                         // channel tiles each wave finishes
    constexpr float NEG_INF = -__builtin_inff();
    // Lazy rescale: the running max moves only when a tile exceeds it by TAU
    // (log2 units), so P may reach 2^TAU.  P is bf16 (the float exponent
    // range) and O and the row sums accumulate in fp32 over at most 64 * Nb
    // < 2^18 keys, so with TAU = 64 every value stays below 2^90: the rescale
    // (80 multiplies per wave) runs about once per row instead of on every
    // tile that raises the max.
    constexpr float TAU = 64.f;
    // rings: [tile A][tile B] per slot
    __shared__ __attribute__((aligned(1024))) T Kb0[2 * TILE];
    __shared__ __attribute__((aligned(1024))) T Kb1[2 * TILE];
    __shared__ __attribute__((aligned(1024))) T Vb0[2 * TILE];
    __shared__ __attribute__((aligned(1024))) T Vb1[2 * TILE];

    const long logical = (long)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (logical >= G) return;
    const int Np = (Nb + 1) / 2;
    const long bh = logical / Np;
    const int pr = (int)(logical % Np);
    const int tid = threadIdx.x, lane = tid & 63;
    // the wave index in a scalar register: every branch on kh and b below is
    // uniform across the wave (the barriers inside them rely on that)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hh = lane >> 5, grp = lane >> 4, L = lane & 15;
    const int kh = wave >> 2, b = (wave >> 1) & 1, qh = wave & 1, w4 = wave & 3;
    const int i = 2 * pr + b;                            // this wave's query block
    const bool bvalid = i < Nb;

    // Q rows of this wave as B fragments: lane (q, h) holds channels 16s + 8h .. +7.
    // Their loads, the row's marginal count and the first slot entries are
    // all issued before anything waits, so that their latencies overlap.
    const int qrow = 64 * i + 32 * qh + l32;
    const bool qvalid = bvalid && qrow < N;
    const long rid = bh * Nb + i;
    const bool lin = bvalid && mcount != nullptr && mcount[rid] > 0;
    v8<T> qf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s)
        qf[s] = qvalid ? ld8<T>(q + (bh * N + qrow) * (long)D + 16 * s + 8 * hh) : zero8<T>();

    float m = NEG_INF, l = 0.f;
    // row sums of P on the matrix core: lsum = 1^T P^T, every row of the
    // accumulator holds the sum of its query column (same layout as O^T)
    f32x16 lsum;
#pragma unroll
    for (int r = 0; r < 16; ++r) lsum[r] = 0.f;
    v8<T> ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = from_f32<T>(1.f);
    f32x16 o[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[ct][r] = 0.f;

    // this pair's slots: a schedule per head, or one shared by all heads (bcast)
    const long pair = bcast ? pr : bh * Np + pr;
    const uint32_t *sl = slots + pair * (long)kc_max;
    const int kc = pcount ? __builtin_amdgcn_readfirstlane(min(max(pcount[pair], 0), kc_max)) : kc_max;
    // part (0 or 1) of this lane's query row within its block, for the frame marks
    const int qpart = (MARKS && fp > 0 && 32 * qh + l32 >= frame_split(i, fp)) ? 1 : 0;
    // slot entry: tile of block A in the low half, of block B in the high half (0xFFFF: no block B)
    auto tile_a = [Nb](uint32_t e) { return slot_tile(e, 0, Nb); };
    auto tile_b = [Nb](uint32_t e) { return slot_tile(e, 1, Nb); };
    auto single = [](uint32_t e) { return slot_single(e); };
    // this wave's tile in a slot: element offset in the slot buffer, and its key block
    auto my_off = [b](uint32_t e) { return (b == 1 && !slot_single(e)) ? TILE : 0; };
    auto my_blk = [b, Nb](uint32_t e) { return slot_tile(e, b, Nb); };

    // one buffer resource per head and tensor: loads past the head's end come back as zeros
    const uint32_t head_bytes = (uint32_t)((long)N * D * sizeof(T));
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + bh * N * (long)D, head_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + bh * N * (long)D, head_bytes);

    // per-lane offsets, fixed for the whole kernel
    int koff[NS];                                        // K operand reads (elements within a tile)
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int r = 32 * kh + l32;
        koff[s] = r * D + ((2 * s + hh) ^ kswz<D>(r)) * 8;
    }
    // V transposing reads: byte offset of (ks, e2, ct) = vbase + ks * 32D + e2 * 16D + ct * 256
    const int vbase = ((8 * kh + (grp >> 1)) * 8 * D + ((2 * (grp & 1) + ((L & 3) >> 1)) * 4 + (L >> 2)) * 16 +
                       (L & 1) * 8) / 2;
    // loads into LDS by the kh = 0 waves: 1 KB block w4 * NB1 + u of a tile, lane at 16 * lane
    // This wave loads K (kh = 1) or V (kh = 0): its buffer resource and, per
    // block, the source offset of its lane, chosen once here so that the
    // loop's loads carry no per-tensor selects.
    const __amdgpu_buffer_rsrc_t rmy = kh == 1 ? rk : rv;
    uint32_t dvm[NB1];
#pragma unroll
    for (int u = 0; u < NB1; ++u) {
        const int byte = (w4 * NB1 + u) * 1024 + 16 * lane;
        if (kh == 1) {
            const int rk_ = byte / (2 * D), pk = (byte % (2 * D)) / 16;
            dvm[u] = (uint32_t)(rk_ * 2 * D + (pk ^ kswz<D>(rk_)) * 16);
        } else {
            const int g = byte / (8 * D), qv = (byte % (8 * D)) / 16;
            dvm[u] = (uint32_t)((4 * g + (qv & 3)) * 2 * D + (qv >> 2) * 16);
        }
    }

    f32x16 sacc;
    v8<T> pb[2];
    v8<T> av[NCT][2];                                    // V^T fragments of the next PV, read in the VALU phase
    // V^T operand of PV over this wave's 32 keys of a slot (V tile at Vt):
    // slots 0-3 of k-step ks hold keys 32kh + 16ks + 4h + 0..3, slots 4-7 keys
    // 32kh + 16ks + 8 + 4h + 0..3 (the S accumulator's order), each run read
    // as a column of the V tile by a transposing read
    auto read_v = [&](const T *Vt) {
        const T *Vs = Vt + vbase;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                av[ct][ks] = cat8<T>(lds_tr_raw<T>(Vs + ks * 16 * D + ct * 128),
                                     lds_tr_raw<T>(Vs + ks * 16 * D + 8 * D + ct * 128));
    };
    // MFMA phase of slot n: K operand reads of slot n (from Kt), then
    // O^T += V^T P^T for slot n-1 on the fragments already in registers while
    // they land (with the row sums 1^T P^T), then S^T = K Q^T for slot n.
    auto mfma_phase = [&](int n, uint32_t e1, const T *Kt) {
        const bool pv = bvalid && n > 0, sk = bvalid && n < kc;
        v8<T> ak[NS];
        if (sk) {
            const T *Ks = Kt + my_off(e1);
#pragma unroll
            for (int s = 0; s < NS; ++s) ak[s] = ld8<T>(Ks + koff[s]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (pv) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) mma16(o[ct], av[ct][ks], pb[ks]);
            mma16(lsum, ones, pb[0]);
            mma16(lsum, ones, pb[1]);
        }
        if (sk) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
            for (int s = 0; s < NS; ++s) mma16(sacc, ak[s], qf[s]);
        }
    };
    // loads into LDS of the tiles of slot entry e: K (kh = 1 waves) or V
    // (kh = 0 waves) into the ring slot dst; NB1 1 KB blocks per tile and
    // wave.  The tile's offset goes into the per-lane offset, which the
    // buffer's bounds check covers, so a ragged last tile reads zeros past
    // the head's end.
    auto load_tiles = [&](uint32_t e, const T *dst) {
        const uint32_t sa = (uint32_t)(64L * tile_a(e) * D * sizeof(T));
        const uint32_t sb = (uint32_t)(64L * tile_b(e) * D * sizeof(T));
        const bool two = !single(e);
#pragma unroll
        for (int u = 0; u < NB1; ++u) dma16(rmy, dst + (w4 * NB1 + u) * 512, dvm[u] + sa, 0);
        if (two) {
#pragma unroll
            for (int u = 0; u < NB1; ++u) dma16(rmy, dst + TILE + (w4 * NB1 + u) * 512, dvm[u] + sb, 0);
        }
    };
    auto softmax = [&](uint32_t e1) {
        const uint32_t marks = ((b ? (e1 >> 16) : e1) >> 12) & 0xFu;
        const int j = my_blk(e1);
        if (marks == 0xFu) [[unlikely]] {               // padding: no key of the slot for this row
            __builtin_amdgcn_sched_barrier(0);           // (a branch, not 16 selects on every slot)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[r] = NEG_INF;
        } else if (MARKS && marks != 0u) {               // a frame boundary hides some keys
            const int ks = fp > 0 ? frame_split(j, fp) : 64;
            const uint32_t hide = marks >> (2 * qpart);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 32 * kh + 8 * (r >> 2) + 4 * hh + (r & 3);
                if ((hide >> (key >= ks ? 1 : 0)) & 1u) sacc[r] = NEG_INF;
            }
        }
        if (64 * j + 64 > N) {                           // ragged last block: keys past N score -inf
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 64 * j + 32 * kh + 8 * (r >> 2) + 4 * hh + (r & 3);
                if (key >= N) sacc[r] = NEG_INF;
            }
        }
        float mx = vmax(sacc[0], sacc[1]);
#pragma unroll
        for (int r = 2; r < 16; ++r) mx = vmax(mx, sacc[r]);
        mx = half_swap_max(mx) * sl2;
        // lazy rescale: move the running max only when the tile exceeds it by TAU
        if (__ballot(mx > m + TAU)) {
            const float mnew = fmaxf(m, mx);
            const float alpha = (mnew == NEG_INF) ? 1.f : fast_exp2(m - mnew);
#pragma unroll
            for (int r = 0; r < 16; ++r) lsum[r] *= alpha;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[ct][r] *= alpha;
            m = mnew;
        }
        const float msub = (m == NEG_INF) ? 0.f : m;
#pragma unroll
        for (int r = 0; r < 16; ++r) pb[r >> 3][r & 7] = from_f32<T>(fast_exp2(__builtin_fmaf(sacc[r], sl2, -msub)));
    };
    // One slot n with the ring arrays of its parity: MFMA phase, wait for the
    // loads this group issued in its last VALU phase, barrier, VALU phase (V
    // reads of slot n for the next PV, this group's loads, softmax of S(n)),
    // barrier.  Loads are issued only in VALU phases: a load issued by a wave
    // that is streaming MFMAs stalls them.
    //   K(n) is read in the MFMA phases (kh = 0: phase 2n, kh = 1: 2n+1), V(n)
    //   in the VALU phases (2n+1, 2n+2).  kh = 1 loads K(n+2) in its VALU(n)
    //   (phase 2n+2) into the ring slot of n, free since phase 2n+1; kh = 0
    //   loads V(n+1) in its VALU(n) (phase 2n+1) into the ring slot of n-1,
    //   free since phase 2n.  Each waits after its next MFMA phase, before
    //   the barrier that ends it: one phase before the first read.
    // ea1, ea2: entries of slots n, n+1; ea3 (slot n+2) is read here.
    uint32_t ea1 = 0, ea2 = 0;
    auto slot = [&](int n, const T *Kt, const T *Vt, const T *Vnext) {
        mfma_phase(n, ea1, Kt);
        const uint32_t ea3 = (n + 2 < kc) ? sl[n + 2] : 0u;
        wait_vm0();                                      // this group's loads of the last VALU phase
        lds_barrier();
        if (bvalid) read_v(Vt + my_off(ea1));
        if (kh == 0 && n + 1 < kc) load_tiles(ea2, Vnext);   // V of slot n+1
        if (kh == 1 && n + 2 < kc) load_tiles(ea3, Kt);      // K of slot n+2, into the ring slot of n
        if (bvalid) softmax(ea1);
        lds_barrier();
        ea1 = ea2; ea2 = ea3;
    };

    if (kc > 0) {
        // prologue: K (kh = 1 waves) and V (kh = 0 waves) of slot 0 into their
        // ring slots; the kh = 1 group then takes the extra phase that puts
        // it one behind, in which it loads K of slot 1
        ea1 = sl[0];
        ea2 = kc > 1 ? sl[1] : 0u;
        load_tiles(ea1, kh == 1 ? Kb0 : Vb0);
        wait_vm0();
        lds_barrier();
        if (kh == 1) {
            if (kc > 1) load_tiles(ea2, Kb1);
            lds_barrier();
        }
        int n = 0;
        for (; n + 1 < kc; n += 2) {
            slot(n, Kb0, Vb0, Vb1);
            slot(n + 1, Kb1, Vb1, Vb0);
        }
        if (n < kc) {
            slot(n, Kb0, Vb0, Vb1);
            ++n;
        }
        // PV of the last slot (n == kc here: no K reads, no loads outstanding)
        mfma_phase(n, ea1, Kb0);
        if (kh == 0) lds_barrier();
        lds_barrier();
    }
    wait_vm0();                                          // no load into LDS outlives the loop

    // merge the two key halves: wave kh keeps channel tiles NCH*kh .. NCH*kh+NCH-1.
    // Exchange area: waves 0-3 in Kb0, 4-7 in Kb1 (4*NCH f32x4 per lane), m and l in Vb0.
    l = lsum[0];                                         // every row holds the column sum
    float *xo_mine = reinterpret_cast<float *>(kh == 0 ? Kb0 : Kb1) + w4 * (4 * NCH * 64 * 4);
    const float *xo_part = reinterpret_cast<const float *>(kh == 0 ? Kb1 : Kb0) + w4 * (4 * NCH * 64 * 4);
    float *xm = reinterpret_cast<float *>(Vb0);          // [8 waves][64]
    float *xl = xm + 8 * 64;
    const int partner = wave ^ 4;
    f32x16 mine[NCH], give[NCH];
#pragma unroll
    for (int t = 0; t < NCH; ++t) {
        mine[t] = kh == 0 ? o[t] : o[NCH + t];
        give[t] = kh == 0 ? o[NCH + t] : o[t];
    }
    if (kc > 0) {
#pragma unroll
        for (int t = 0; t < NCH; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 y = {give[t][4 * g], give[t][4 * g + 1], give[t][4 * g + 2], give[t][4 * g + 3]};
                *reinterpret_cast<f32x4 *>(xo_mine + ((4 * t + g) * 64 + lane) * 4) = y;
            }
        xm[wave * 64 + lane] = m;
        xl[wave * 64 + lane] = l;
    }

    // linear part: issue its loads before the exchange completes
    const S *hr = hhat + rid * (long)Lp;
    v8<S> hz[NS], hv[NCH][NS];
    if (lin) {
#pragma unroll
        for (int s = 0; s < NS; ++s) hz[s] = ld8<S>(hr + D * D + 16 * s + 8 * hh);
#pragma unroll
        for (int t = 0; t < NCH; ++t)
#pragma unroll
            for (int s = 0; s < NS; ++s)
                hv[t][s] = ld8<S>(hr + (32 * (NCH * kh + t) + l32) * D + 16 * s + 8 * hh);
    }
    if (kc > 0) {
        lds_barrier();
        const float mo = xm[partner * 64 + lane], lo = xl[partner * 64 + lane];
        const float mm = fmaxf(m, mo);
        const float as = (mm == NEG_INF) ? 0.f : fast_exp2(m - mm);
        const float ao = (mm == NEG_INF) ? 0.f : fast_exp2(mo - mm);
        const float lt = l * as + lo * ao;
        const float inv = (lt > 0.f) ? 1.f / lt : 0.f;
        // log-sum-exp of the row's sparse softmax in the kernel's log2 units
        // (P = exp2(s * log2(e) / sqrt(d) - lse)), +inf for a row with no key
        if (lse && kh == 0 && hh == 0 && qvalid) lse[bh * N + qrow] = lt > 0.f ? mm + __log2f(lt) : __builtin_inff();
#pragma unroll
        for (int t = 0; t < NCH; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 y = *reinterpret_cast<const f32x4 *>(xo_part + ((4 * t + g) * 64 + lane) * 4);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    mine[t][4 * g + e] = (mine[t][4 * g + e] * as + y[e] * ao) * inv;
            }
    }
    if (kc == 0 && lse && kh == 0 && hh == 0 && qvalid) lse[bh * N + qrow] = __builtin_inff();
    if (!bvalid) return;

    if (lin) {
        constexpr float LOG2E = 1.4426950408889634f;
        float mq = NEG_INF;
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) mq = fmaxf(mq, to_f32<T>(qf[s][e]));
        mq = half_swap_max(mq);
        float ex[NS][8];
        float se = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                ex[s][e] = fast_exp2((to_f32<T>(qf[s][e]) - mq) * LOG2E);
                se += ex[s][e];
            }
        se = half_swap_sum(se);
        const float inv_se = 1.f / se;
        v8<S> ph[NS];
        float den = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                ph[s][e] = from_f32<S>(ex[s][e] * inv_se);
                den += to_f32<S>(ph[s][e]) * to_f32<S>(hz[s][e]);
            }
        den = half_swap_sum(den);
        const float rden = 1.f / den;
#pragma unroll
        for (int t = 0; t < NCH; ++t) {
            f32x16 y;
#pragma unroll
            for (int r = 0; r < 16; ++r) y[r] = 0.f;
#pragma unroll
            for (int s = 0; s < NS; ++s) mma16(y, hv[t][s], ph[s]);
#pragma unroll
            for (int r = 0; r < 16; ++r) mine[t][r] += y[r] * rden;
        }
    }

    if (qvalid) {
        TO *orow = out + (bh * N + qrow) * (long)D;
#pragma unroll
        for (int t = 0; t < NCH; ++t) {
            const int c0 = 32 * (NCH * kh + t);
#pragma unroll
            for (int g = 0; g < 4; ++g)
                store4<TO>(orow + c0 + 8 * g + 4 * hh, mine[t][4 * g], mine[t][4 * g + 1], mine[t][4 * g + 2],
                           mine[t][4 * g + 3]);
        }
    }
}

template <typename T, typename S, int D, typename TO, bool MARKS>
static hipError_t launch_fused16_t(const FusedArgs &a, hipStream_t st) {
    const long G = a.BH * ((a.Nb + 1) / 2);
    const int per = (int)((G + 7) / 8);
    const float sl2 = 1.4426950408889634f / sqrtf((float)D);
    fused16_kernel<T, S, D, TO, MARKS><<<(unsigned)(8L * per), 512, 0, st>>>(
        (const T *)a.q, (const T *)a.k, (const T *)a.v, a.slots, a.kc, a.pcount, a.bcast ? 1 : 0, a.fp,
        (const S *)a.hhat, a.mcount, a.Lp, (TO *)a.out, a.lse, G, per, a.N, a.Nb, sl2);
    return hipGetLastError();
}

template <bool MARKS>
static hipError_t launch_fused16_m(const FusedArgs &a, hipStream_t st) {
    if (a.bf16_out)
        return a.D == 64 ? launch_fused16_t<bf16, f16, 64, bf16, MARKS>(a, st)
                         : launch_fused16_t<bf16, f16, 128, bf16, MARKS>(a, st);
    return a.D == 64 ? launch_fused16_t<bf16, f16, 64, float, MARKS>(a, st)
                     : launch_fused16_t<bf16, f16, 128, float, MARKS>(a, st);
}

hipError_t launch_fused16(const FusedArgs &a, hipStream_t st) {
    return a.fp > 0 ? launch_fused16_m<true>(a, st) : launch_fused16_m<false>(a, st);
}

}  // namespace sla
