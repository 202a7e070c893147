// assemble.hip -- marginal linear-attention states per query-block row.
//
// For each row i the linear branch needs H_i = sum of h_j over the marginal
// key blocks j of that row (and Z_i likewise; SLA article, section 3).  For all
// rows of a head at once this is one dense GEMM M * Hs with M the [Nb x Nbc]
// 0/1 marginal indicator (M_ij = 1 iff block j is marginal for row i; padding
// columns 0) and Hs the [Nbc x Lp] block states, on fp16 MFMA with fp32
// accumulation (float MFMA for float inputs); the 0/1 matrix is exact in
// fp16.
// Output row i is (M_i Hs) * 64 / m_i with m_i the row's marginal token
// count: the linear output phi(q) H / (phi(q).Z) does not depend on a common
// scale of H and Z, and this one keeps |values| <= max|V W^T|.
//
// The product is computed transposed, D^T = Hs^T M^T (M = state column, N =
// query-block row, K = key block), so that each lane ends with 4 consecutive
// columns of one output row.  Workgroups are ordered so that the row tiles
// of one column slice run together on one XCD and share its L2.
//
// float path: the indicator as float rows; tile 256 columns x 128 rows per
// workgroup, 4 waves of 128 x 64, K-steps of 32 key blocks double-buffered
// through registers and LDS.
//
// fp16 path: one workgroup of 4 waves owns 128 state columns and up to 256
// query-block rows (64 per wave); two workgroups share a CU (72 KB of LDS
// and up to 256 registers per lane each), so one's barrier waits, prologue
// and epilogue run under the other's products.  The two row tiles of a
// column slice are neighbours in the launch order and read the slice's
// states through the same L2.  The K-steps (64 key blocks, 16 KB of Hs) go through
// a ring of four LDS stages filled by loads that go straight from memory into
// LDS: three steps are in flight while the fourth is multiplied, with one
// barrier per step.  A stage also holds the step's indicator words of the
// tile's rows.  The step loop is unrolled by four so that every stage is
// a fixed LDS array.  Hs rows are stored as they are with 16-byte chunks
// XOR-swizzled by row, so that the A fragments (8 consecutive blocks of one
// column) come out with conflict-free transposing reads.  The indicator comes
// as bits (32 key blocks per word); each lane reads the words of its own
// rows from the stage and expands them into the fp16 B operand in registers.  The output tile of a wave is
// scaled, staged through LDS (8-byte units swizzled by row) and written as
// whole contiguous row segments.
// Scaled mode (the backward pass sums its per-row state gradients this
// way): input row k is stored as fp16 values x times 2^-E_k (|x| < 1), and
// the B operand of (j, k) is 2^(E_k - R + 14) instead of 1 (R the largest
// E_k of the head; rows more than 28 below it count as zero), given as the
// fp16 exponent byte of each row; output row j is the sum times
// 2^-(14 + c), c = ceil(log2 Nbc), which keeps it below 1 in magnitude: its
// true value is that times 2^(R + c).
#include "sla_device.h"
#include "sla_launch.h"

namespace sla {

namespace {

// workgroup barrier that leaves global loads (and loads into LDS) in flight
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);                  // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
}
// 16 (4) bytes per lane from a buffer into LDS at lds + 16 (4) * lane (lds is wave-uniform)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, const void *lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, const void *lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 4, voff, 0, 0, 0);
}

constexpr int AT_W = 4;                                  // waves per workgroup, 64 rows each
constexpr int AT_TM = 128;                               // state columns per workgroup
constexpr int AT_TN = 64 * AT_W;                         // query-block rows per workgroup (256)
constexpr int AT_TK = 64;                                // key blocks per step
constexpr int AT_HS = AT_TK * AT_TM;                     // Hs elements of one step (16 KB)
constexpr int AT_STAGE = AT_HS + 2 * AT_TN * 2;          // one LDS stage in f16 units: Hs, then 2 x AT_TN words
constexpr int AT_NA = AT_HS * 2 / 1024 / AT_W;           // 1 KB Hs loads per wave per step (4)
constexpr int AT_NW = 2 * AT_TN * 4 / 256 / AT_W;        // 256-byte indicator loads per wave per step (2)
constexpr int AT_VM = AT_NA + AT_NW;                     // memory operations per wave per step
static_assert(2 * AT_VM < 16, "the stage wait's count fits the low vmcnt field");
static_assert(AT_STAGE >= 2 * 4096, "a stage holds the epilogue slices of two waves");
constexpr int AT_KB_MAX = 4096;                          // scaled mode: rows (Nbc) at most

// one K-step into a stage: this wave's AT_NA 1 KB pieces of the Hs rows (four
// 256-byte rows each) and its AT_NW 256-byte pieces of the indicator words
// (word h of rows 64 g .. 64 g + 63 of the tile at 64 (AT_W h + g))
template <typename T>
__device__ __forceinline__ void at_issue(__amdgpu_buffer_rsrc_t rh, __amdgpu_buffer_rsrc_t rb, T *S,
                                         const uint32_t (&va)[AT_NA], const uint32_t (&vw)[AT_NW], int w,
                                         uint32_t aoff, uint32_t woff) {
#pragma unroll
    for (int u = 0; u < AT_NA; ++u) dma16(rh, S + (AT_NA * w + u) * 512, va[u] + aoff);
    uint32_t *W = reinterpret_cast<uint32_t *>(S + AT_HS);
#pragma unroll
    for (int u = 0; u < AT_NW; ++u) dma4(rb, W + 64 * (AT_NW * w + u), vw[u] + woff);
}

// 8 indicator bits -> 8 fp16 B values, 0 or ONE = 2^-14 (0x0400, the
// smallest normal: high byte 0x04, low byte 0), so a value is a byte: each
// nibble spreads to bit 2 of four bytes by one multiply (bit i of n lands at
// i + 2 + 7k for k = 0..3, distinct positions, so no carries; byte k keeps
// bit k), and byte permutes put byte e in the high byte of half e: ten
// operations for the eight values.  The products h * 2^-14 and their fp32
// sums are those of ONE = 1 scaled by 2^-14 exactly (no value comes near the
// bottom of the fp32 range), and the output scale takes the 2^14 back.
constexpr float kOneInv = 16384.f;                       // 1 / ONE
__device__ __forceinline__ v8<f16> expand_bits(uint32_t x) {
    const uint32_t wa = __umul24(x & 0xFu, 0x810204u) & 0x04040404u;          // bits 0..3 -> bytes 0..3
    const uint32_t wb = __umul24((x >> 4) & 0xFu, 0x810204u) & 0x04040404u;   // bits 4..7 -> bytes 4..7
    uint32_t d[4];
    d[0] = __builtin_amdgcn_perm(wb, wa, 0x010C000Cu);   // byte sel 12 reads as 0x00
    d[1] = __builtin_amdgcn_perm(wb, wa, 0x030C020Cu);
    d[2] = __builtin_amdgcn_perm(wb, wa, 0x050C040Cu);
    d[3] = __builtin_amdgcn_perm(wb, wa, 0x070C060Cu);
    v8<f16> r;
    __builtin_memcpy(&r, d, sizeof(r));
    return r;
}
// Scaled mode: 8 indicator bits -> 8 fp16 B values, the row's exponent byte
// (elo: rows 0..3, ehi: rows 4..7, one byte each, low two bits zero) or 0:
// the spread bits (0x04 per byte) times 63 give a 0xFC mask per set byte
// (no carry between bytes; the top byte's borrow leaves the word).
__device__ __forceinline__ v8<f16> expand_bits_scaled(uint32_t x, uint32_t elo, uint32_t ehi) {
    uint32_t wa = __umul24(x & 0xFu, 0x810204u) & 0x04040404u;
    uint32_t wb = __umul24((x >> 4) & 0xFu, 0x810204u) & 0x04040404u;
    wa = ((wa << 6) - wa) & elo;
    wb = ((wb << 6) - wb) & ehi;
    uint32_t d[4];
    d[0] = __builtin_amdgcn_perm(wb, wa, 0x010C000Cu);
    d[1] = __builtin_amdgcn_perm(wb, wa, 0x030C020Cu);
    d[2] = __builtin_amdgcn_perm(wb, wa, 0x050C040Cu);
    d[3] = __builtin_amdgcn_perm(wb, wa, 0x070C060Cu);
    v8<f16> r;
    __builtin_memcpy(&r, d, sizeof(r));
    return r;
}
// per-lane LDS element offsets of the A fragment reads: abase[mt] is the
// first of the 4 consecutive state columns n = 32 mt + 16 (grp & 1) +
// 4 (L & 3) in key block 8 (grp >> 1) + (L >> 2) of a stage; the block's two
// low bits (L >> 2) pick the chunk swizzle, which the further blocks 16 s +
// 4 x of the same lane keep, so those reads sit at constant offsets
__device__ __forceinline__ void at_abase(int lane, int (&abase)[4]) {
    const int grp = lane >> 4, L = lane & 15, kb = 8 * (grp >> 1) + (L >> 2), sw = 4 * (kb & 3);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const int n = 32 * mt + 16 * (grp & 1) + 4 * (L & 3);
        abase[mt] = kb * AT_TM + 8 * ((n >> 3) ^ sw) + (n & 7);
    }
}
// the 32 MFMAs of one K-step for a wave's 128 x 64 tile (rows 64 w .. 64 w + 63);
// kb: scaled mode's exponent bytes of the step's 64 rows (else null).  The A
// fragment of the next (s, mt) is read before the two MFMAs of the current
// one, so each read has two MFMAs to land.
template <typename T, bool SCALED>
__device__ __forceinline__ void at_compute(const T *S, f32x16 (&acc)[4][2], int w, int lane, const uint32_t *kb,
                                           const int (&abase)[4]) {
    const int l32 = lane & 31, hh = lane >> 5;
    const T *A = S;
    const uint32_t *W = reinterpret_cast<const uint32_t *>(S + AT_HS);
    uint32_t bw[2][2];                                   // word h of row nt: key blocks 32 h .. 32 h + 31
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int h = 0; h < 2; ++h) bw[nt][h] = W[AT_TN * h + 64 * w + 32 * nt + l32];
    // key blocks 16 s + 8 hh .. + 7 of the lane's row nt as the B operand
    auto bop = [&](int s, v8<T> (&b)[2]) __attribute__((always_inline)) {
        if constexpr (SCALED) {
            const uint32_t elo = kb[4 * s + 2 * hh], ehi = kb[4 * s + 2 * hh + 1];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
                b[nt] = expand_bits_scaled(bw[nt][s >> 1] >> (8 * (2 * (s & 1) + hh)), elo, ehi);
        } else {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) b[nt] = expand_bits(bw[nt][s >> 1] >> (8 * (2 * (s & 1) + hh)));
        }
    };
    auto aop = [&](int s, int mt) __attribute__((always_inline)) {
        const T *p = A + abase[mt] + 16 * s * AT_TM;
        return cat8<T>(lds_tr_raw<T>(p), lds_tr_raw<T>(p + 4 * AT_TM));
    };
    v8<T> b[2];
    bop(0, b);
    v8<T> a = aop(0, 0);
#pragma unroll
    for (int s = 0; s < AT_TK / 16; ++s) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            v8<T> an = a;
            if (mt < 3) an = aop(s, mt + 1);
            else if (s + 1 < AT_TK / 16) an = aop(s + 1, 0);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) mma16(acc[mt][nt], a, b[nt]);
            if (mt == 3 && s + 1 < AT_TK / 16) bop(s + 1, b);
            a = an;
        }
    }
}

}  // namespace

// T: the 16-bit type of the states; O: f16 (rows scaled by 64 / m_i, or in
// scaled mode by 2^-oshift; staged through LDS) or float (written from the
// accumulators as they are, 16 bytes per lane)
template <typename T, typename O, bool SCALED>
__global__ __launch_bounds__(64 * AT_W, 2) void assemble16_kernel(const uint32_t *__restrict__ mbits,
                                                         const T *__restrict__ hs,
                                                         const int32_t *__restrict__ mcount,
                                                         const uint8_t *__restrict__ kbyte, int oshift,
                                                         O *__restrict__ hhat, int Nb, int Nbc, int Nbp, int Lp,
                                                         int tiles_m, int tiles_n, long G, int per_xcd) {
    // four stages; separate arrays so that reads of one stage never wait for
    // loads still landing in another
    __shared__ __attribute__((aligned(1024))) T S0[AT_STAGE], S1[AT_STAGE], S2[AT_STAGE], S3[AT_STAGE];
    // scaled mode: the exponent bytes of the head's Nbc rows
    __shared__ __attribute__((aligned(16))) uint32_t Kb[SCALED ? AT_KB_MAX / 4 : 1];

    const long logical = (long)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (logical >= G) return;
    const int tn = (int)(logical % tiles_n);
    const long rest = logical / tiles_n;
    const int tm = (int)(rest % tiles_m);
    const long bh = rest / tiles_m;
    const int col0 = AT_TM * tm, row0 = AT_TN * tn;
    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wrow = row0 + 64 * wave;                   // first row of this wave
    if constexpr (SCALED) {
        // before the first loads into LDS, so that this wait covers only these;
        // visible after the first barrier of the step loop
        const uint8_t *kr = kbyte + bh * (long)Nbc;
        for (int x = tid; x < Nbc / 16; x += 64 * AT_W)
            *reinterpret_cast<Chunk *>(&Kb[4 * x]) = *reinterpret_cast<const Chunk *>(kr + 16 * x);
    }

    // buffer resources over one head: Hs rows and indicator words past the
    // end read as zeros
    const int nw = Nbc / 32;
    const auto rh = make_rsrc(hs + bh * (long)Nbc * Lp, (uint32_t)((long)Nbc * Lp * 2));
    const auto rb = make_rsrc(mbits + bh * (long)nw * Nbp, (uint32_t)((long)nw * Nbp * 4));
    uint32_t va[AT_NA], vw[AT_NW];
#pragma unroll
    for (int u = 0; u < AT_NA; ++u) {
        const int r = 4 * (AT_NA * wave + u) + (lane >> 4), p = lane & 15;   // LDS row and chunk of this lane
        va[u] = (uint32_t)(((long)r * Lp + col0 + 8 * (p ^ (4 * (r & 3)))) * 2);
    }
#pragma unroll
    for (int u = 0; u < AT_NW; ++u) {
        const int i = AT_NW * wave + u;                  // word i / AT_W of rows 64 (i % AT_W) + lane
        vw[u] = (uint32_t)(((long)(i / AT_W) * Nbp + row0 + 64 * (i % AT_W) + lane) * 4);
    }
    const uint32_t astep = (uint32_t)AT_TK * Lp * 2, wstep = (uint32_t)Nbp * 8;
    int abase[4];
    at_abase(lane, abase);

    f32x16 acc[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mt][nt][r] = 0.f;

    const int nst = Nbc / AT_TK;
    const bool active = wrow < Nb;                       // the wave has rows to compute
    at_issue(rh, rb, S0, va, vw, wave, 0, 0);
    at_issue(rh, rb, S1, va, vw, wave, astep, wstep);
    at_issue(rh, rb, S2, va, vw, wave, 2 * astep, 2 * wstep);
    // step st: wait for its loads (the next two steps' stay in flight),
    // barrier, refill the stage freed by step st - 1 with step st + 3,
    // multiply.  The loads are issued on every path, also for the steps past
    // the end (they read zeros): every step then issues the same number of
    // memory operations, which the wait counts, and the compiler tells the
    // stages apart and adds no waits of its own before the reads of a stage.
    auto stage = [&](int st, const T *S, T *Sn) {
        __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * AT_VM));   // vmcnt(8)
        lds_barrier();
        at_issue(rh, rb, Sn, va, vw, wave, (uint32_t)(st + 3) * astep, (uint32_t)(st + 3) * wstep);
        if (active && st < nst) at_compute<T, SCALED>(S, acc, wave, lane, SCALED ? &Kb[16 * st] : nullptr, abase);
    };
    for (int st = 0; st < nst; st += 4) {
        stage(st, S0, S3);
        stage(st + 1, S1, S0);
        stage(st + 2, S2, S1);
        stage(st + 3, S3, S2);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);                  // vmcnt(0)
    lds_barrier();                                       // every wave is done with the stages
    if (!active) return;
    // epilogue: the wave's 32-row halves go through a private 8 KB LDS slice,
    // 8-byte unit u of row r at unit u ^ r (conflict-free both ways)
    static_assert(AT_W <= 8, "four stages hold the slices of up to eight waves");
    T *stg0 = (wave < 2 ? S0 : wave < 4 ? S1 : wave < 6 ? S2 : S3) + (wave & 1) * 4096;
    O *stg = reinterpret_cast<O *>(stg0);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int i = wrow + 32 * nt + l32;
        float sc;
        if constexpr (SCALED) {
            sc = ldexpf(1.f, -oshift);
        } else {
            const int mc = (i < Nb) ? mcount[bh * Nb + i] : 0;
            sc = mc > 0 ? 64.f / (float)mc * kOneInv : 0.f;
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int u = 8 * mt + 2 * g + hh;       // 8-byte unit: columns 4u .. 4u + 3 of the tile
                v4<O> y;
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = (O)(acc[mt][nt][4 * g + e] * sc);
                __builtin_memcpy(&stg[l32 * AT_TM + 4 * (u ^ l32)], &y, sizeof(y));
            }
        // row 2 x + hh of the staged half, unit l32; one running pointer over
        // the rows (no 64-bit products per store)
        const int r0 = wrow + 32 * nt + hh;
        O *orow = hhat + (bh * Nb + r0) * (long)Lp + col0 + 4 * l32;
        const long rstep = 2L * Lp;
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            const int r = 2 * x + hh;
            const v4<O> y = ld4<O>(&stg[r * AT_TM + 4 * (l32 ^ r)]);
            if (r0 + 2 * x < Nb) __builtin_memcpy(orow, &y, sizeof(y));
            orow += rstep;
        }
    }
}

template <typename S>
__global__ __launch_bounds__(256, 2) void assemble_kernel(const S *__restrict__ marg, const S *__restrict__ hs,
                                                          const int32_t *__restrict__ mcount,
                                                          S *__restrict__ hhat, int Nb, int Nbc, int Lp,
                                                          int tiles_m, int tiles_n, long G, int per_xcd) {
    // register-staged double buffering (float states)
    constexpr int TM = 256, TN = 128, TK = 32;
    constexpr int EPC = 16 / sizeof(S);                  // elements per 16-byte chunk
    constexpr int ACPR = TM / EPC;                       // chunks per staged Hs row
    constexpr int NA = TK * ACPR / 256;                  // A chunks per thread
    constexpr int TPA = 256 / ACPR;                      // threads sharing one A column group
    constexpr int ASTR = TM + (sizeof(S) == 2 ? 16 : 8); // staged Hs row stride
    constexpr int BCPR = TK / EPC;                       // chunks per staged M row
    constexpr int NB = TN * BCPR / 256;                  // B chunks per thread
    constexpr int BSTR = TK + EPC;                       // padded M row stride
    __shared__ __attribute__((aligned(16))) S As[2][TK * ASTR];
    __shared__ __attribute__((aligned(16))) S Bs[2][TN * BSTR];

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
    const S *Mh = marg + bh * Nb * (long)Nbc;
    const S *Hh = hs + bh * (long)Nbc * Lp;

    const int acg = tid % ACPR, ajr = tid / ACPR;        // this thread's A column group and first row
    Chunk pa[NA], pb[NB];
    auto gload = [&](int j0) {
#pragma unroll
        for (int u = 0; u < NA; ++u)
            pa[u] = ld_chunk(Hh + (long)(j0 + ajr + TPA * u) * Lp + col0 + acg * EPC);
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int idx = tid + 256 * u, row = idx / BCPR, q = idx % BCPR;
            pb[u] = (row0 + row < Nb) ? ld_chunk(Mh + (long)(row0 + row) * Nbc + j0 + q * EPC) : zero_chunk();
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int u = 0; u < NA; ++u) st_chunk(&As[buf][(ajr + TPA * u) * ASTR + acg * EPC], pa[u]);
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
    for (int nt = 0; nt < 2; ++nt) {
        const int i = row0 + 64 * wn + 32 * nt + l32;
        if (i >= Nb) continue;
        const int mc = mcount[bh * Nb + i];
        const float sc = mc > 0 ? 64.f / (float)mc : 0.f;
        S *orow = hhat + (bh * Nb + i) * (long)Lp + col0;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int cl = 128 * wm + 32 * mt + 8 * g + 4 * hh;
                v4<S> y;
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = from_f32<S>(acc[mt][nt][4 * g + e] * sc);
                __builtin_memcpy(orow + cl, &y, sizeof(y));
            }
    }
}

hipError_t launch_assemble(const AssembleArgs &a, hipStream_t st) {
    if (a.Nbc % 64 != 0 || a.Nbc < a.Nb || (long)(a.Nbc + 256) * a.Lp * 4 >= (1L << 32)) return hipErrorInvalidValue;
    if (a.f32) {
        const int tiles_m = a.Lp / 256;             // column tiles (Lp is a multiple of 256)
        const int tiles_n = (a.Nb + 127) / 128;     // row tiles
        const long G = a.BH * tiles_m * tiles_n;
        const int per = (int)((G + 7) / 8);
        assemble_kernel<float><<<(unsigned)(8L * per), 256, 0, st>>>((const float *)a.marg, (const float *)a.hs,
                                                                    a.mcount, (float *)a.hhat, a.Nb, a.Nbc, a.Lp,
                                                                    tiles_m, tiles_n, G, per);
    } else {
        if (a.Nbp % AT_TN != 0 || a.Nbp < a.Nb) return hipErrorInvalidValue;
        const int tiles_m = a.Lp / AT_TM;
        const int tiles_n = (a.Nb + AT_TN - 1) / AT_TN;
        const long G = a.BH * tiles_m * tiles_n;
        const int per = (int)((G + 7) / 8);
        if (a.kbyte) {
            if (a.Nbc > AT_KB_MAX) return hipErrorInvalidValue;
            assemble16_kernel<f16, f16, true><<<(unsigned)(8L * per), 64 * AT_W, 0, st>>>(
                a.mbits, (const f16 *)a.hs, nullptr, a.kbyte, a.oshift, (f16 *)a.hhat, a.Nb, a.Nbc, a.Nbp, a.Lp,
                tiles_m, tiles_n, G, per);
        } else {
            assemble16_kernel<f16, f16, false><<<(unsigned)(8L * per), 64 * AT_W, 0, st>>>(
                a.mbits, (const f16 *)a.hs, a.mcount, nullptr, 0, (f16 *)a.hhat, a.Nb, a.Nbc, a.Nbp, a.Lp, tiles_m,
                tiles_n, G, per);
        }
    }
    return hipGetLastError();
}

}  // namespace sla
