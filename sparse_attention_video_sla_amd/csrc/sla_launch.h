// sla_launch.h -- host-side launchers of the gfx950 kernels (internal to libsla).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sla.h"

namespace sla {

struct ClassifyArgs {
    const float *qp, *kp;
    const float *kpack; // nullable: the key means packed by channel quads, [BH][D/4][classify_packed_keys(Nb)][4]
    long BH;
    int Nb, D, kc, kn;
    int8_t *mask;
    int32_t *crit, *excl;
    float *pc;
    float *marg;      // nullable [BH][Nb][Nbc] 0/1 marginal indicator rows (float inputs)
    uint32_t *mbits;  // nullable [BH][Nbc/32][Nbp] the same as bits: word w of row i holds blocks 32w..32w+31
    int Nbc, Nbp;     // key blocks rounded up to 64, rows of the bit array
    int32_t *mcount;  // nullable [BH][Nb] marginal token count per row
    int n_last;       // valid tokens of the last block
    uint32_t *ulist;  // nullable [BH][ceil(Nb/2)][2*kc] union of each row pair's critical lists
    int32_t *ucount;  // [BH][ceil(Nb/2)] union lengths
    double inv_sqrt_d;
};

struct StateArgs {
    const void *k, *v;
    const float *w;
    long BH;
    int N, Nb, D, Lp;
    int Nbc;          // rows of hs per head (Nb rounded up to 64; the extra rows are zero)
    void *hs;         // [BH][Nbc][Lp] per-block states (h'^T then z), scaled by 1/64
    void *wstate;     // [d][d] W converted to the state type (scratch)
    bool bf16_in;
};

struct AssembleArgs {
    const void *marg;        // [BH][Nb][Nbc] float marginal indicator (float inputs)
    const uint32_t *mbits;   // [BH][Nbc/32][Nbp] marginal indicator bits (16-bit inputs)
    const void *hs;          // [BH][Nbc][Lp] block states
    const int32_t *mcount;
    void *hhat;       // [BH][Nb][Lp] marginal states per query-block row
    long BH;
    int Nb, Nbc, Nbp, Lp;
    bool f32;
    const uint8_t *kbyte;    // nullable: scaled mode, [BH][Nbc] fp16 exponent byte of each input row (0: zero row)
    int oshift;              // scaled mode: output rows are the sums times 2^-oshift
};

struct FusedArgs {
    const void *q, *k, *v;
    const uint32_t *ulist;   // [BH][ceil(Nb/2)][2*kc] union of each row pair's critical lists
    const int32_t *ucount;   // [BH][ceil(Nb/2)]
    const uint32_t *slots;   // [BH][ceil(Nb/2)][kc] slot schedule (16-bit inputs), [ceil(Nb/2)][kc] with bcast
    const int32_t *crit;     // [BH][Nb][kc] critical lists (null: the slot schedule gives the blocks)
    int kc;
    const int32_t *pcount;   // nullable: slots used per pair ([BH][ceil(Nb/2)], or [ceil(Nb/2)] with bcast)
    bool bcast;              // one schedule shared by every head
    int fp;                  // tokens per frame for the frame marks in the slots (0: no marks)
    float *lse;              // nullable: [BH][64 Nb] log-sum-exp of each row's sparse softmax (log2 units)
    float *os;               // nullable: [BH][N][D] float32 sparse part of the output (before the linear read-out)
    int nchunk;              // slot schedules: nchunk > 1 splits each row pair's slots into nchunk equal shares;
                             // out and lse are then [nchunk][BH][64 Nb][D] fp16, [nchunk][BH][64 Nb] float32
    const void *hhat;
    const int32_t *mcount;   // nullable: no marginal blocks anywhere
    int Lp;
    void *out;
    long BH;
    int N, Nb, D;
    bool bf16_in, bf16_out;
};

struct MassArgs {
    const void *q, *k;       // [BH][N][D] bf16
    long BH;
    int N, Nb, D;
    float *mass;             // [BH][Nb][Nb]
};

// kpack (nullable): the key means also packed as classify reads them in the
// forward pass
hipError_t launch_pool(bool bf16_in, int D, const void *q, const void *k, float *qp, float *kp, float *kpack,
                       long BH, int N, int Nb, int blk, hipStream_t st);
int classify_packed_keys(int Nb);   // key blocks of the packed key means (Nb rounded up to even)
int classify_rows_per_group(int Nb, int D);
size_t classify_lds_bytes(int R, int D, int Nb);
hipError_t launch_classify(const ClassifyArgs &a, hipStream_t st);
hipError_t launch_state(const StateArgs &a, hipStream_t st);
hipError_t launch_assemble(const AssembleArgs &a, hipStream_t st);
hipError_t launch_fused(const FusedArgs &a, hipStream_t st);     // float inputs
hipError_t launch_fused16s(const FusedArgs &a, hipStream_t st);
// out[t] = the chunks' normalized outputs weighted by 2^lse (the chunks' log2
// masses; +inf: an empty chunk), over the rows t of [BH][N]
hipError_t launch_chunk_merge(const _Float16 *part, const float *plse, int nchunk, long BH, int N, int Nb, int D,
                              void *out, bool bf16_out, hipStream_t st);  // bf16 inputs: critical lists, or a slot schedule
hipError_t launch_block_mass(const MassArgs &a, hipStream_t st);
hipError_t launch_lists_to_slots(const int32_t *lists, const int32_t *counts, int kmax, long BH, int Nb,
                                 uint32_t *slots, int32_t *pcount, hipStream_t st);

// LVSA frame sets: T frames, half window W, step s, T_per, m = |G_s| = ceil(T / T_per)
struct LvsaParams {
    int T, W, s, Tper, m;
};
hipError_t launch_lvsa_frames(const LvsaParams &p, int32_t *lohi, int32_t *sets, int32_t *counts, int max_frames,
                              hipStream_t st);
// backward: inputs, the forward's recomputed pieces, outputs and scratch
struct BackwardArgs {
    const void *q, *k, *v, *dout;     // [BH][N][D] bf16
    const float *w;                   // [D][D]
    const float *o_s, *lse;           // sparse output [BH][N][D] and its log-sum-exp [BH][64 Nb] (log2 units)
    const int32_t *crit;              // [BH][Nb][kc]
    int kc;
    const int8_t *mask;               // [BH][Nb][Nb] labels
    const void *hhat;                 // [BH][Nb][Lp] f16 marginal states (Ĥ'^T, Ẑ; / m_i)
    const int32_t *mcount;            // [BH][Nb] marginal tokens per row
    float *dq, *dk, *dv, *dw;         // gradients
    float *dbuf;                      // [BH][64 Nb] D_r = dO_r . O_s,r
    int32_t *tlist;                   // [BH][Nb][Nb] transposed critical lists
    int32_t *tcnt;                    // [BH][Nb]
    uint32_t *mbitsT;                 // [BH][Nbc / 32][Nbp] transposed marginal indicator bits
    void *dhr;                        // [BH][Nbc][Lp] f16 per-row state gradients x 2^-dexp
    int32_t *dexp;                    // [BH][Nbc] their exponents
    uint8_t *kbyte;                   // [BH][Nbc] fp16 exponent bytes of the rows for the transposed sum
    int32_t *hexp;                    // [BH] output exponent Q of the transposed sum
    void *dhs;                        // [BH][Nb][Lp] f16 per-key-block state gradients x 2^-Q
    float *dwp;                       // [backward_key_groups][D][D] per-workgroup partial sums of dW
    long BH;
    int N, Nb, Nbc, Nbp, Lp, D;
};
// workgroups of the linear-keys kernel (a fixed count, so that dW sums its
// per-workgroup partials in the same order on every device and every run)
long backward_key_groups(long BH, int Nb, int D);
hipError_t launch_backward_dq(const BackwardArgs &a, hipStream_t st);        // transposed lists + dQ (sparse)
hipError_t launch_backward_dkv(const BackwardArgs &a, hipStream_t st);       // dK, dV (sparse)
hipError_t launch_backward_lin_rows(const BackwardArgs &a, hipStream_t st);  // linear rows + transposed sums
hipError_t launch_backward_lin_keys(const BackwardArgs &a, hipStream_t st);  // linear keys + dW
hipError_t launch_zero(float *p, long n, hipStream_t st);

// Sets the thread's error text (sla_last_error); returns st.
sla_status set_error(sla_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

// STA tiles: tile sizes, windows, tile grid, tile volume and the largest
// |delta| per axis worth testing (2*delta*t <= W)
struct StaParams {
    int tf, th, tw, wf, wh, ww, gf, gh, gw, vol, rf, rh, rw;
};
hipError_t launch_sta_slots(const StaParams &p, int Nb, int kmax, uint32_t *slots, int32_t *pcount, hipStream_t st);
hipError_t launch_lvsa_slots(const LvsaParams &p, int P, int N, int Nb, const int32_t *lohi, int kmax,
                             uint32_t *slots, int32_t *pcount, hipStream_t st);
hipError_t launch_mask_stats(const float *mass, const int8_t *mask, long rows, int Nb, float *stats, hipStream_t st);

}  // namespace sla
