// fused16s.hip -- the SLA forward's fused kernel with one query block per
// workgroup, for bf16 inputs (SLA article, section 3: exact block-sparse
// FlashAttention over the critical blocks and the linear read-out of the
// marginal states, with the learnable projection folded into them).
//
// One workgroup of 4 waves per query block i of one head, three workgroups
// per compute unit (50 KB of LDS and at most 168 registers per lane each, so
// every SIMD runs three independent waves).  Wave (qh, kh): query rows
// 32qh .. +31 against keys 32kh .. +31 of every critical block of row i, with
// its own online softmax (running max m, output O, row sum l); the two key
// halves of a row merge at the end, each wave keeping half of the output
// channels.  Per critical block:
//   S^T = K Q^T on the matrix core (K rows from LDS, Q held in registers);
//   the softmax in the VALU: the tile's row max (a lane holds 16 keys of one
//   query column, the other 16 of the half sit in the partner lane 32
//   away), a lazy rescale of O and l when the tile exceeds the running max
//   by TAU (log2 units), P = exp2(S log2(e)/sqrt(d) - m) added to l and
//   converted to bf16 in the MFMA operand layout;
//   O^T += V^T P^T on the matrix core, V^T by transposing reads of the V
//   tile.
// K and V tiles go from global memory straight into LDS: K through a
// two-slot ring, V through one slot, with two barriers per block (after the
// scores: V(c) and K(c+1) visible, K(c)'s slot free for K(c+2); after the
// accumulation: V's slot free for V(c+1)), so each load has a phase or two
// to land.  K rows are padded by one 16-byte chunk (its row reads touch
// every bank once, and one register holds a lane's read offset for every
// channel step: the steps differ by constants); V rows have their 16-byte
// chunks swizzled by vswz (its transposing reads, 8 rows x 4 chunks per
// instruction, touch every bank twice, the minimum); the loads into LDS read
// whole rows, through a buffer resource per key block.  (A V layout of
// 4-row groups stored chunk-major, also free of conflicts, was 12 % slower
// here: each of its loads gathers 16-byte pieces of four rows.)
// Every
// workgroup reads its own tiles; with three workgroups per compute unit the
// softmax of one overlaps the matrix work of another without any schedule
// between them.  Workgroups are ordered so that each XCD (own L2) takes a
// contiguous run of (head, query block).
#include "sla_device.h"
#include "sla_launch.h"
#include "tile_common.h"

namespace sla {

namespace {

template <typename TO> __device__ __forceinline__ void store4s(TO *p, float a, float b, float c, float d);
template <> __device__ __forceinline__ void store4s<float>(float *p, float a, float b, float c, float d) {
    f32x4 v = {a, b, c, d};
    *reinterpret_cast<f32x4 *>(p) = v;
}
template <> __device__ __forceinline__ void store4s<bf16>(bf16 *p, float a, float b, float c, float d) {
    v4<bf16> v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
    __builtin_memcpy(p, &v, sizeof(v));
}
template <> __device__ __forceinline__ void store4s<f16>(f16 *p, float a, float b, float c, float d) {
    v4<f16> v = {(f16)a, (f16)b, (f16)c, (f16)d};
    __builtin_memcpy(p, &v, sizeof(v));
}

}  // namespace

// SLOTS: the blocks come from a slot schedule of row pairs (the workgroup
// takes its row's half of each slot: a key block index in the low 12 bits,
// frame marks or 0xF for padding in the top 4; a padding half costs two
// barriers and nothing else) instead of critical lists;
// MARKS: those halves may carry frame marks (bit 2a + c set: query part a
// does not see key part c, part 1 being what follows a frame boundary inside
// the block).
template <typename T, typename S, int D, typename TO, bool SLOTS, bool MARKS>
__global__ __launch_bounds__(256, 3) void fused16s_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                          const T *__restrict__ v, const int32_t *__restrict__ crit,
                                                          int kc, const uint32_t *__restrict__ slots,
                                                          const int32_t *__restrict__ pcount, int bcast, int fp,
                                                          const S *__restrict__ hhat,
                                                          const int32_t *__restrict__ mcount, int Lp,
                                                          TO *__restrict__ out, float *__restrict__ lse,
                                                          float *__restrict__ os, long G,
                                                          int per_xcd, int N, int Nb, float sl2, int nchunk) {
    static_assert(__is_same(T, bf16), "bf16 inputs");
    constexpr int TILE = 64 * D, NS = D / 16, NCT = D / 32, NCH = NCT / 2, NBW = D / 32;
    // K tiles: rows padded by one 16-byte chunk (KRS elements), so that the
    // 16 lanes of a row read touch all banks and the read offsets of the 8
    // (4) channel steps differ by constants
    constexpr int KRS = D + 8, KCPR = D / 8 + 1, KTILE = 64 * KRS;
    constexpr int KDMA = 64 * KCPR / 64;                 // 1 KB loads into LDS per K tile (17, or 9 for d = 64)
    constexpr int KPW = (KDMA + 3) / 4;                  // per wave, at most
    constexpr float NEG_INF = -__builtin_inff();
    // Lazy rescale threshold: P may reach 2^TAU; P is bf16 (the float exponent
    // range) and O and l accumulate in fp32 over at most 64 * Nb < 2^18 keys,
    // so every value stays below 2^90.
    constexpr float TAU = 64.f;
    static_assert(KTILE * 2 >= D * KRS, "the marginal state fits the K ring");
    static_assert(2 * 4 * (D / 64) * 64 * 16 <= KTILE * 2, "two waves' exchange fits a K slot");
    // the two K slots are separate arrays, so that the reads of one slot do
    // not wait for loads still landing in the other or in the V tile
    __shared__ __attribute__((aligned(1024))) T Kk0[KTILE];
    __shared__ __attribute__((aligned(1024))) T Kk1[KTILE];
    __shared__ __attribute__((aligned(1024))) T Vk[TILE];
    __shared__ __attribute__((aligned(16))) S Zl[D];        // the row's Ẑ_i

    long logical = (long)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (logical >= G) return;
    // chunked schedules: workgroup order chunk-major, then (head, query
    // block); chunk ch takes the ch-th of nchunk equal shares of its row
    // pair's slots and writes its own normalized output and log-sum-exp
    // (merged afterwards)
    int chunk = 0;
    if (SLOTS && nchunk > 1) {
        const long rows = G / nchunk;
        chunk = (int)(logical / rows);
        logical -= (long)chunk * rows;
        out += (long)chunk * rows * 64 * D;              // [chunk][BH][64 Nb][D] (whole blocks of rows)
        lse += (long)chunk * rows * 64;
    }
    const long bh = logical / Nb;
    const int i = (int)(logical % Nb);
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, hh = lane >> 5;
    const int qh = wave >> 1, kh = wave & 1;
    const int qrow = 64 * i + 32 * qh + l32;
    const bool qvalid = qrow < N;
    const long rid = bh * Nb + i;
    const bool lin = mcount != nullptr && mcount[rid] > 0;
    v8<T> qf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s)
        qf[s] = qvalid ? ld8<T>(q + (bh * N + qrow) * (long)D + 16 * s + 8 * hh) : zero8<T>();

    float m = NEG_INF, l = 0.f;                          // l: this lane's share of the row sum
    f32x16 o[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[ct][r] = 0.f;

    const int32_t *cl = crit + rid * (long)kc;
    const uint32_t *sl = nullptr;
    int hb = 0;                                          // which half of a slot entry is this row's
    if constexpr (SLOTS) {
        const int Np = (Nb + 1) / 2, pr = i >> 1;
        const long pair = bcast ? pr : bh * Np + pr;
        sl = slots + pair * (long)kc;
        hb = 16 * (i & 1);
        if (pcount) kc = __builtin_amdgcn_readfirstlane(min(max(pcount[pair], 0), kc));
        if (nchunk > 1) {                                // equal shares of this row pair's slots
            const int share = (kc + nchunk - 1) / nchunk, c0 = chunk * share;
            sl += c0;
            kc = max(0, min(kc, c0 + share) - c0);
        }
    }
    // list entry c as a word (read once, where no LDS read is in flight: a
    // scalar load's wait also drains those), its key block and its frame
    // marks (0xF: padding)
    auto ent = [&](int c) __attribute__((always_inline)) {
        if constexpr (SLOTS) return sl[c];
        else return (uint32_t)cl[c];
    };
    auto blk_of = [&](uint32_t w) __attribute__((always_inline)) {
        if constexpr (SLOTS) return min((int)((w >> hb) & 0xFFFu), Nb - 1);
        else return (int)w;
    };
    auto marks_of = [&](uint32_t w) __attribute__((always_inline)) {
        if constexpr (SLOTS) return (w >> (hb + 12)) & 0xFu;
        else return 0u;
    };
    // a padding half: this row has no block in the slot (no load, no work)
    auto pad = [&](uint32_t w) __attribute__((always_inline)) { return SLOTS && marks_of(w) == 0xFu; };
    const int qpart = (MARKS && fp > 0 && 32 * qh + l32 >= frame_split(i, fp)) ? 1 : 0;
    // A buffer resource per key block: a ragged last block, and the pad
    // chunks of the K tile (offsets past the resource), read zeros.
    auto blk_rsrc = [&](const T *base, int j) __attribute__((always_inline)) {
        const int rows = min(64, N - 64 * j);
        return make_rsrc(base + (bh * N + 64L * j) * D, (uint32_t)(rows * D * sizeof(T)));
    };
    // K operand reads: key row 32kh + l32, channels 16 s + 8 hh .. +7 at +16 s
    const int kbase = (32 * kh + l32) * KRS + 8 * hh;
    // V transposing reads (V-swizzled rows): the second run of a step lies
    // 8 rows below the first at the same swizzle, 8D elements further on
    int toff[NCT][2];
    tr_offsets<D, true>(lane, toff);
    // accumulator ct holds output channel tile ct ^ (NCH kh): tiles 0 .. NCH-1
    // are the channels this wave keeps after the merge, the others its partner's
    int tv[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) tv[ct] = kh ? toff[ct ^ NCH][0] : toff[ct][0];
    // loads of a K tile into LDS: wave w takes the 1 KB pieces w, w + 4, ...;
    // lane l of piece t fills chunk 64 t + l of the padded tile, which is row
    // (64 t + l) / KCPR, chunk (64 t + l) % KCPR of the block (the last chunk
    // of a row is the pad: an offset past the tile, which reads zero)
    uint32_t kdo[KPW];
#pragma unroll
    for (int u = 0; u < KPW; ++u) {
        const int pos = 64 * (wave + 4 * u) + lane, row = pos / KCPR, ch = pos % KCPR;
        kdo[u] = ch < D / 8 ? (uint32_t)(row * D * 2 + ch * 16) : 0x40000000u;
    }
    // V: the swizzle only depends on the row modulo 4 (d = 128) or 8 (d = 64),
    // which a 1 KB piece (4 or 8 rows) does not change: piece u is piece 0
    // plus u KB
    const uint32_t ov0 = off_klayout<D, true>(wave * NBW * 1024 + 16 * lane);
    auto load_k = [&](uint32_t w, int slot) __attribute__((always_inline)) {
        if (pad(w)) return;
        const __amdgpu_buffer_rsrc_t r = blk_rsrc(k, blk_of(w));
#pragma unroll
        for (int u = 0; u < KPW; ++u)
            if (wave + 4 * u < KDMA) dma16(r, (slot ? Kk1 : Kk0) + (wave + 4 * u) * 512, kdo[u], 0);
    };
    auto load_v = [&](uint32_t w) __attribute__((always_inline)) {
        if (pad(w)) return;
        const __amdgpu_buffer_rsrc_t r = blk_rsrc(v, blk_of(w));
#pragma unroll
        for (int u = 0; u < NBW; ++u) dma16(r, &Vk[(wave * NBW + u) * 512], ov0 + 1024 * u, 0);
    };
    // the row's marginal state Ĥ_i^T ([c][a], D rows of 2D bytes, stored in
    // the K ring with the K layout's chunk swizzle once the loop is done) and
    // Ẑ_i, straight into LDS: one round trip for the whole read-out (issuing
    // it inside the last block instead spills registers in the loop)
    const S *hr = hhat + rid * (long)Lp;
    auto load_hhat = [&]() __attribute__((always_inline)) {
        constexpr int HDMA = D * KCPR / 64;              // 1 KB pieces of the padded D x D state (34 or 9)
        const __amdgpu_buffer_rsrc_t rh = make_rsrc(hr, (uint32_t)(D * D * sizeof(S)));
        // rows 0..63 (KCPR pieces of 1 KB) in the first slot, the rest in the second
        for (int t = wave; t < HDMA; t += 4) {
            const int pos = 64 * t + lane, row = pos / KCPR, ch = pos % KCPR;
            T *dst = t < KCPR ? Kk0 + t * 512 : Kk1 + (t - KCPR) * 512;
            dma16(rh, dst, ch < D / 8 ? (uint32_t)(row * D * 2 + ch * 16) : 0x40000000u, 0);
        }
        if (wave == 0 && lane < D / 8)
            dma16(make_rsrc(hr, (uint32_t)((D * D + D) * sizeof(S))), Zl, (uint32_t)(D * D * sizeof(S)) + 16 * lane, 0);
    };
    v8<T> pb[2];
    // S^T = K Q^T of block c and its softmax: P^T in pb
    // (last: entry c is the list's last, the only one a critical list can
    // have on the ragged last key block, the lists being ascending)
    auto score = [&](uint32_t w, int slot, bool last) __attribute__((always_inline)) {
        const int j = blk_of(w);
        v8<T> ak[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) ak[s] = ld8<T>((slot ? Kk1 : Kk0) + kbase + 16 * s);
        f32x16 sacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s) mma16(sacc, ak[s], qf[s]);
        if constexpr (MARKS) {
            const uint32_t marks = marks_of(w);
            if (marks != 0u) {                           // a frame boundary hides some keys
                const int ks = fp > 0 ? frame_split(j, fp) : 64;
                const uint32_t hide = marks >> (2 * qpart);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = 32 * kh + 8 * (r >> 2) + 4 * hh + (r & 3);
                    if ((hide >> (key >= ks ? 1 : 0)) & 1u) sacc[r] = NEG_INF;
                }
            }
        }
        if ((SLOTS || last) && 64 * j + 64 > N) {        // ragged last block: keys past N score -inf
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
        if (__ballot(mx > m + TAU)) {
            const float mnew = fmaxf(m, mx);
            const float alpha = (mnew == NEG_INF) ? 1.f : fast_exp2(m - mnew);
            l *= alpha;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[ct][r] *= alpha;
            m = mnew;
        }
        const float msub = (m == NEG_INF) ? 0.f : m;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = fast_exp2(__builtin_fmaf(sacc[r], sl2, -msub));
            l += p;
            pb[r >> 3][r & 7] = from_f32<T>(p);
        }
    };
    // O^T += V^T P^T
    auto accumulate = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const T *base = &Vk[(32 * kh + 16 * ks) * D];
                mma16(o[ct], cat8<T>(lds_tr_raw<T>(base + tv[ct]), lds_tr_raw<T>(base + tv[ct] + 8 * D)), pb[ks]);
            }
    };
    // Block c: score (K(c) visible; V(c) and K(c+1) in flight), wait for
    // both and barrier (V(c) visible, the K slot of c free), load K(c+2)
    // into it, accumulate, barrier (the V tile free), load V(c+1).  Each
    // load has a whole phase or two to land.
    // w0, w1: the words of entries c and c + 1; returns that of c + 2, read
    // after the first barrier, where no LDS read is in flight
    auto block = [&](int c, int slot, uint32_t w0, uint32_t w1) __attribute__((always_inline)) {
        const bool work = !pad(w0);                      // uniform across the workgroup
        if (work) score(w0, slot, c == kc - 1);
        wait_vm0();
        lds_barrier();
        const uint32_t w2 = c + 2 < kc ? ent(c + 2) : 0u;
        if (c + 2 < kc) load_k(w2, slot);
        if (work) accumulate();
        lds_barrier();
        if (c + 1 < kc) load_v(w1);
        return w2;
    };
    if (kc > 0) {
        uint32_t w0 = ent(0), w1 = kc > 1 ? ent(1) : 0u;
        load_k(w0, 0);
        if (kc > 1) load_k(w1, 1);
        wait_vm0();
        load_v(w0);
        lds_barrier();
        int c = 0;
        for (; c + 1 < kc; c += 2) {
            const uint32_t w2 = block(c, 0, w0, w1);
            const uint32_t w3 = block(c + 1, 1, w1, w2);
            w0 = w2;
            w1 = w3;
        }
        if (c < kc) block(c, 0, w0, w1);
    }
    if (lin) load_hhat();                                // the K ring is free once the loop is done
    wait_vm0();                                          // no load into LDS outlives the loop
    lds_barrier();                                       // Ĥ_i and Ẑ_i visible

    // linear read-out for this wave's output channels (tiles NCH*kh ..):
    // y = Ĥ_i phi(q) / (phi(q).Ẑ_i), Ĥ_i rows from LDS.  phi(q) = x / sum(x)
    // with x = exp(q - max q); the sum cancels between the two, so x itself
    // (in (0, 1], as fp16) takes phi's place.
    f32x16 yl[NCH];
    float rden = 0.f;
    if (lin) {
        constexpr float LOG2E = 1.4426950408889634f;
        float mq = NEG_INF;
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) mq = fmaxf(mq, to_f32<T>(qf[s][e]));
        mq = half_swap_max(mq) * LOG2E;
        v8<S> ph[NS];
        float den = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const v8<S> hz = ld8<S>(&Zl[16 * s + 8 * hh]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                ph[s][e] = from_f32<S>(fast_exp2(__builtin_fmaf(to_f32<T>(qf[s][e]), LOG2E, -mq)));
                den += to_f32<S>(ph[s][e]) * to_f32<S>(hz[e]);
            }
        }
        den = half_swap_sum(den);
        rden = 1.f / den;
#pragma unroll
        for (int t = 0; t < NCH; ++t) {
            const int c = 32 * (NCH * kh + t) + l32;
            const S *Hs = reinterpret_cast<const S *>(c < 64 ? Kk0 : Kk1) + (c & 63) * KRS;
#pragma unroll
            for (int r = 0; r < 16; ++r) yl[t][r] = 0.f;
#pragma unroll
            for (int s = 0; s < NS; ++s) mma16(yl[t], ld8<S>(&Hs[16 * s + 8 * hh]), ph[s]);
        }
    }
    lds_barrier();                                       // the ring is free for the exchange

    // merge the two key halves: wave kh keeps channel tiles NCH*kh .. +NCH-1.
    // Exchange area: 4*NCH f32x4 per lane and wave in Kk, m and l in Vk.
    l = half_swap_sum(l);                                // the row sum over the wave's 32 keys
    // waves 0, 1 exchange through the first slot, waves 2, 3 through the second
    float *xo = reinterpret_cast<float *>(wave < 2 ? Kk0 : Kk1);
    float *xm = reinterpret_cast<float *>(&Vk[0]);       // [4 waves][64]
    float *xl = xm + 4 * 64;
    const int partner = wave ^ 1;
    f32x16 mine[NCH], give[NCH];
#pragma unroll
    for (int t = 0; t < NCH; ++t) {
        mine[t] = o[t];
        give[t] = o[NCH + t];
    }
    if (kc > 0) {
#pragma unroll
        for (int t = 0; t < NCH; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 y = {give[t][4 * g], give[t][4 * g + 1], give[t][4 * g + 2], give[t][4 * g + 3]};
                *reinterpret_cast<f32x4 *>(xo + (((wave & 1) * 4 * NCH + 4 * t + g) * 64 + lane) * 4) = y;
            }
        xm[wave * 64 + lane] = m;
        xl[wave * 64 + lane] = l;
    }

    if (kc > 0) {
        lds_barrier();
        const float mo = xm[partner * 64 + lane], lo = xl[partner * 64 + lane];
        const float mm = fmaxf(m, mo);
        const float as = (mm == NEG_INF) ? 0.f : fast_exp2(m - mm);
        const float ao = (mm == NEG_INF) ? 0.f : fast_exp2(mo - mm);
        const float lt = l * as + lo * ao;
        const float inv = (lt > 0.f) ? 1.f / lt : 0.f;
        const float sa = as * inv, so = ao * inv;
        // log-sum-exp of the row's sparse softmax in the kernel's log2 units
        // (P = exp2(s * log2(e) / sqrt(d) - lse)), +inf for a row with no key
        if (lse && kh == 0 && hh == 0 && qvalid) lse[bh * (64L * Nb) + qrow] = lt > 0.f ? mm + __log2f(lt) : __builtin_inff();
#pragma unroll
        for (int t = 0; t < NCH; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 y = *reinterpret_cast<const f32x4 *>(xo + (((partner & 1) * 4 * NCH + 4 * t + g) * 64 + lane) * 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) mine[t][4 * g + e] = __builtin_fmaf(mine[t][4 * g + e], sa, y[e] * so);
            }
    }
    if (kc == 0 && lse && kh == 0 && hh == 0 && qvalid) lse[bh * (64L * Nb) + qrow] = __builtin_inff();

    // the output row's offset, formed again here (the empty asm hides the
    // lane index's origin) rather than kept in registers through the loop
    int lane_e = threadIdx.x & 63;
    asm volatile("" : "+v"(lane_e));
    const int hh_e = lane_e >> 5;
    const long orow_at = (bh * N + 64 * i + 32 * qh + (lane_e & 31)) * (long)D;

    // the sparse part alone, for a backward pass that reuses this forward
    // (critical lists only)
    if (!SLOTS && os && qvalid) {
        float *srow = os + orow_at;
#pragma unroll
        for (int t = 0; t < NCH; ++t) {
            const int c0 = 32 * (NCH * kh + t);
#pragma unroll
            for (int g = 0; g < 4; ++g)
                store4s<float>(srow + c0 + 8 * g + 4 * hh_e, mine[t][4 * g], mine[t][4 * g + 1], mine[t][4 * g + 2],
                               mine[t][4 * g + 3]);
        }
    }

    if (lin) {
#pragma unroll
        for (int t = 0; t < NCH; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) mine[t][r] += yl[t][r] * rden;
    }

    if (qvalid) {
        TO *orow = out + orow_at;
#pragma unroll
        for (int t = 0; t < NCH; ++t) {
            const int c0 = 32 * (NCH * kh + t);
#pragma unroll
            for (int g = 0; g < 4; ++g)
                store4s<TO>(orow + c0 + 8 * g + 4 * hh_e, mine[t][4 * g], mine[t][4 * g + 1], mine[t][4 * g + 2],
                            mine[t][4 * g + 3]);
        }
    }
}

template <int D, typename TO, bool SLOTS, bool MARKS>
static hipError_t launch_fused16s_t(const FusedArgs &a, hipStream_t st) {
    const int nchunk = a.nchunk > 1 ? a.nchunk : 1;
    const long G = nchunk * a.BH * a.Nb;
    const int per = (int)((G + 7) / 8);
    const float sl2 = 1.4426950408889634f / sqrtf((float)D);
    fused16s_kernel<bf16, f16, D, TO, SLOTS, MARKS><<<(unsigned)(8L * per), 256, 0, st>>>(
        (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v, a.crit, a.kc, a.slots, a.pcount, a.bcast ? 1 : 0,
        a.fp, (const f16 *)a.hhat, a.mcount, a.Lp, (TO *)a.out, a.lse, a.os, G, per, a.N, a.Nb, sl2, nchunk);
    return hipGetLastError();
}

template <bool SLOTS, bool MARKS>
static hipError_t launch_fused16s_m(const FusedArgs &a, hipStream_t st) {
    if constexpr (SLOTS) {                               // the shares' normalized partial outputs, fp16
        if (a.nchunk > 1)
            return a.D == 64 ? launch_fused16s_t<64, f16, SLOTS, MARKS>(a, st)
                             : launch_fused16s_t<128, f16, SLOTS, MARKS>(a, st);
    }
    if (a.bf16_out)
        return a.D == 64 ? launch_fused16s_t<64, bf16, SLOTS, MARKS>(a, st)
                         : launch_fused16s_t<128, bf16, SLOTS, MARKS>(a, st);
    return a.D == 64 ? launch_fused16s_t<64, float, SLOTS, MARKS>(a, st)
                     : launch_fused16s_t<128, float, SLOTS, MARKS>(a, st);
}

// critical lists (crit), or the slot schedule (slots) when crit is null
hipError_t launch_fused16s(const FusedArgs &a, hipStream_t st) {
    if (a.crit) return launch_fused16s_m<false, false>(a, st);
    return a.fp > 0 ? launch_fused16s_m<true, true>(a, st) : launch_fused16s_m<true, false>(a, st);
}

}  // namespace sla
