/*
 * sla.h -- C ABI of the MI355X (gfx950) SLA sparse-linear attention forward.
 *
 * The operation is the forward pass of SLA as described by the SLA article
 * ("Tsinghua cracks the video generation stall ...", techwalker.com,
 * section 3 "SLA's core mechanism"):
 *   pool Q and K per block; score the compressed map P_c = softmax(Qbar Kbar^T/sqrt(d));
 *   per query-block row label the key blocks critical (top crit_frac), negligible
 *   (bottom negl_frac) or marginal (the rest); exact softmax attention over the
 *   critical blocks; linear attention phi(Q)(phi(K)^T V) over the marginal blocks
 *   followed by a d x d projection; negligible blocks skipped.
 * The sparse part is one softmax over every attended key of the row (the
 * normalisation of the block-sparse formula on the LVSA page, "method steps").
 *
 * Conventions shared by every entry point:
 *   - Tensors Q, K, V, O are row-major [B, H, N, d] (d fastest), contiguous,
 *     16-byte aligned DEVICE pointers owned by the caller.  The library never
 *     allocates, frees or synchronises; scratch memory comes only from the
 *     caller's workspace.  Work is enqueued on `stream` (a hipStream_t; NULL
 *     means the default stream) and runs asynchronously.
 *   - N is the number of valid tokens.  Blocks are `block` consecutive tokens;
 *     Nb = ceil(N / block); the last block may be ragged (n = N - (Nb-1)*block
 *     tokens) and the library masks its pad positions itself.
 *   - Supported: d in {64, 128}; block = 64; in_dtype F32 or BF16; out_dtype F32
 *     or equal to in_dtype; 0 <= crit_frac, negl_frac <= 1, crit_frac +
 *     negl_frac <= 1; B, H, N >= 1; Nb <= 2432 (N <= 155648).
 *   - Counts per row: k_c = min(Nb, ceil(crit_frac*Nb - 1e-9)),
 *     k_n = min(Nb - k_c, floor(negl_frac*Nb + 1e-9)).
 *   - Ranking: one total order per row, score descending then block index
 *     ascending; the first k_c blocks are critical, the last k_n negligible.
 *     Scores are fp64 dot products (ascending channel order) of the float32
 *     block means (fp64 sums in ascending token order / n, rounded once).
 *   - Errors: invalid or unsupported arguments return a status before anything
 *     is launched; a failed launch returns SLA_ERR_DEVICE.  sla_last_error()
 *     gives a thread-local message for the last non-OK status of the thread.
 *   - Inputs must be finite.  BF16 inputs: the linear branch stages values in
 *     fp16, so |V| and |V W^T| must stay below 65504; so does |V| for the
 *     slot-schedule entry points (lists, LVSA, sliding tiles) when a row
 *     pair's schedule has 256 or more slots, whose shares' normalized
 *     outputs are staged in fp16.
 *   - Reentrant.  Mutable state: per thread, the error message and the
 *     optional stage-timing events.  Every kernel of a call runs on the
 *     caller's stream, in order.  Results are
 *     bitwise deterministic run to run: no kernel adds floating-point values
 *     with atomics (the only atomics are ORs into bit sets, whose result
 *     does not depend on their order), and every sum over workgroups (dW in
 *     sla_backward) adds per-workgroup partials in a fixed order over a
 *     fixed number of workgroups.
 */
#ifndef SLA_H
#define SLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SLA_OK = 0,
    SLA_ERR_INVALID_ARG = 1,   /* null pointer, non-positive size, fraction out of range */
    SLA_ERR_UNSUPPORTED = 2,   /* valid but not implemented: d, block, dtype, Nb limit */
    SLA_ERR_WORKSPACE = 3,     /* workspace_bytes smaller than sla_workspace_size() */
    SLA_ERR_DEVICE = 4         /* HIP launch / runtime failure */
} sla_status;

/* Element types.  A C caller may pass any int for an enum argument; C++
 * gives these enums int as their underlying type so that the library can
 * read such a value and reject it (SLA_ERR_UNSUPPORTED) instead of holding
 * an enum value outside its range.  Both spellings have the size and the
 * calling convention of int. */
#ifdef __cplusplus
typedef enum : int { SLA_F32 = 0, SLA_BF16 = 1 } sla_dtype;
#else
typedef enum { SLA_F32 = 0, SLA_BF16 = 1 } sla_dtype;
#endif

/* Feature map of the linear branch: softmax over the d channels of each token
 * (the SLA article, section 5, reports softmax beating ELU+1 and ReLU). */
#ifdef __cplusplus
typedef enum : int { SLA_PHI_SOFTMAX = 0 } sla_phi;
#else
typedef enum { SLA_PHI_SOFTMAX = 0 } sla_phi;
#endif

/* Library version (major*10000 + minor*100 + patch). */
int sla_version(void);

/* Per-row counts k_c (critical) and k_n (negligible) for Nb key blocks and
 * the given shares (SLA article, section 3: top 5% critical, bottom 10%
 * negligible by default in the article).  Host only. */
sla_status sla_counts(int Nb, double crit_frac, double negl_frac, int *k_c, int *k_n);

/* Bytes of device workspace sla_forward needs for these arguments.  Host only. */
sla_status sla_workspace_size(int B, int H, int N, int d, int block, sla_dtype in_dtype,
                              double crit_frac, double negl_frac, size_t *bytes);

/* Step 1 (SLA article, section 3: mean pooling of Q and K).
 * q, k: [B,H,N,d] of in_dtype.  q_pool, k_pool: [B,H,Nb,d] float32 outputs,
 * each the fp64 sum of the block's valid tokens in ascending order divided by
 * their count, rounded once to float32. */
sla_status sla_pool(const void *q, const void *k, sla_dtype in_dtype,
                    int B, int H, int N, int d, int block,
                    float *q_pool, float *k_pool, void *stream);

/* Steps 2-3 (SLA article, section 3: compressed map and three-way labels).
 * q_pool, k_pool: [B,H,Nb,d] float32 (from sla_pool).
 * mask: [B,H,Nb,Nb] int8 output, +1 critical, 0 marginal, -1 negligible.
 * crit_idx: [B,H,Nb,k_c] int32 output, critical block indices ascending
 *   (may be NULL only when k_c == 0).
 * excl_idx: nullable [B,H,Nb,k_c+k_n] int32 output, critical and negligible
 *   indices together, ascending.
 * p_c: nullable [B,H,Nb,Nb] float32 output, softmax_j(s_ij / sqrt(d)). */
sla_status sla_classify(const float *q_pool, const float *k_pool,
                        int B, int H, int Nb, int d, double crit_frac, double negl_frac,
                        int8_t *mask, int32_t *crit_idx, int32_t *excl_idx, float *p_c,
                        void *stream);

/* The whole forward pass (SLA article, section 3; one fused attention kernel
 * covers the three branches, with the learnable projection on the linear
 * output).
 * q, k, v: [B,H,N,d] of in_dtype.  w_proj: [d,d] float32, applied as x W^T
 *   (row c of W produces output channel c), shared by all heads.
 * out: [B,H,N,d] of out_dtype: O = O_sparse + O_linear W^T.
 * mask_out: nullable [B,H,Nb,Nb] int8 copy of the labels.
 * workspace: device memory of at least sla_workspace_size() bytes, 256-byte
 *   aligned; its contents on entry do not matter and are clobbered. */
sla_status sla_forward(const void *q, const void *k, const void *v, const float *w_proj,
                       sla_dtype in_dtype, sla_dtype out_dtype,
                       int B, int H, int N, int d, int block,
                       double crit_frac, double negl_frac, sla_phi phi,
                       void *out, int8_t *mask_out,
                       void *workspace, size_t workspace_bytes, void *stream);

/* sla_forward without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops or harnesses that forbid hipMalloc).  Arguments and results
 * are those of sla_forward.  The scratch memory is a static device array of
 * SLA_NOALLOC_SCRATCH_BYTES inside the library: each GPU holds its own copy
 * from the first call on it (its address is looked up then, with that
 * device current) until the process ends.  A call whose sla_workspace_size()
 * exceeds SLA_NOALLOC_SCRATCH_BYTES returns SLA_ERR_WORKSPACE before any
 * launch (512 MiB holds B=1, H=12, N=32760, d=128 at the default shares:
 * 403 MiB).  Every call on one GPU uses the same array: calls that overlap
 * on one GPU (other streams, other host threads) race and must be
 * serialised by the caller; nothing needs clearing between calls. */
#define SLA_NOALLOC_SCRATCH_BYTES ((size_t)512 << 20)
sla_status sla_forward_noalloc(const void *q, const void *k, const void *v, const float *w_proj,
                               sla_dtype in_dtype, sla_dtype out_dtype,
                               int B, int H, int N, int d, int block,
                               double crit_frac, double negl_frac, sla_phi phi,
                               void *out, int8_t *mask_out, void *stream);

/* Gradients of sla_forward (SLA article, section 三: FlashAttention
 * gradients for the sparse part, linear-attention gradients for the linear
 * part).  The block labels are those sla_forward forms from the same q, k
 * and fractions and are held fixed (no gradient flows through the
 * selection).  q, k, v, dout: [B,H,N,d] bf16 (float32: SLA_ERR_UNSUPPORTED);
 * w_proj [d,d] float32 as in sla_forward; dq, dk, dv: [B,H,N,d] float32
 * outputs, dw: [d,d] float32 output (summed over batch and heads).  The call
 * runs the forward pass again inside (labels, lists, marginal states, the
 * sparse output and its log-sum-exp), then the gradient kernels.  Workspace:
 * sla_backward_workspace_size() bytes, 256-byte aligned, clobbered. */
sla_status sla_backward_workspace_size(int B, int H, int N, int d, int block, double crit_frac, double negl_frac,
                                       size_t *bytes);
sla_status sla_backward(const void *q, const void *k, const void *v, const float *w_proj, const void *dout,
                        sla_dtype in_dtype, int B, int H, int N, int d, int block, double crit_frac,
                        double negl_frac, sla_phi phi, float *dq, float *dk, float *dv, float *dw, void *workspace,
                        size_t workspace_bytes, void *stream);

/* The same gradients without running the forward pass again, for training
 * loops that run the forward anyway (SLA article, section 三: the forward
 * keeps what the backward's split needs).
 * sla_forward_save is sla_forward for bf16 inputs (same arguments, same
 * output bits, the same kernels) that also leaves in `saved` everything the
 * backward reads: the labels, critical lists, marginal-state products and
 * counts, the sparse part of the output alone (float32) and its rows'
 * log-sum-exp.  `saved`: sla_backward_workspace_size() bytes, 256-byte
 * aligned, owned by the caller; mask_out, if not NULL, gets a copy of the
 * labels.
 * sla_backward_saved takes the arguments of sla_backward, with `saved` as its
 * workspace; it must hold what sla_forward_save wrote for the same q, k, v,
 * w_proj, shapes and fractions, untouched since (nothing checks this: other
 * contents give wrong gradients, not an error).  Its gradients are those of
 * sla_backward bit for bit.  It overwrites the gradient scratch parts of
 * `saved` and keeps the forward's parts, so it can run again on the same
 * saved state (with another dout). */
sla_status sla_forward_save(const void *q, const void *k, const void *v, const float *w_proj, sla_dtype in_dtype,
                            sla_dtype out_dtype, int B, int H, int N, int d, int block, double crit_frac,
                            double negl_frac, sla_phi phi, void *out, int8_t *mask_out, void *saved,
                            size_t saved_bytes, void *stream);
sla_status sla_backward_saved(const void *q, const void *k, const void *v, const float *w_proj, const void *dout,
                              sla_dtype in_dtype, int B, int H, int N, int d, int block, double crit_frac,
                              double negl_frac, sla_phi phi, float *dq, float *dk, float *dv, float *dw, void *saved,
                              size_t saved_bytes, void *stream);

/* Sparse attention over block lists given by the caller, with the linear
 * branch off (a mask source other than the scores, e.g. the LVSA page's
 * frame-level sets A(t) = G_s U W(t) turned into key blocks; block-sparse
 * softmax over the union of the listed blocks as in the LVSA page's method
 * steps).
 * lists: [B,H,Nb,kmax] int32 device array: for every query-block row, its key
 *   blocks in ascending order in the first counts[row] entries (the rest is
 *   ignored; entries outside [0, Nb) are ignored, a repeated index counts
 *   once).  counts: [B,H,Nb] int32, each in [0, kmax].  A row with no block
 *   gives zeros.  kmax in [1, Nb]; Nb = ceil(N/64) <= 4095.
 * q, k, v: [B,H,N,d] bf16 (float32: SLA_ERR_UNSUPPORTED); out: [B,H,N,d] of
 *   out_dtype (F32 or BF16).  workspace: sla_lists_workspace_size() bytes,
 *   256-byte aligned.  Rows 2p and 2p+1 share a schedule of slots (blocks
 *   both list, then their other blocks side by side); each row's cost
 *   follows the number of slots of its pair.  With kmax >= 256 each pair's
 *   slots run in four shares whose normalized outputs (fp16) and
 *   log-sum-exps are merged afterwards (the workspace holds them). */
sla_status sla_lists_workspace_size(int B, int H, int N, int kmax, size_t *bytes);
sla_status sla_forward_lists(const void *q, const void *k, const void *v, sla_dtype in_dtype, sla_dtype out_dtype,
                             int B, int H, int N, int d, int block, const int32_t *lists, const int32_t *counts,
                             int kmax, void *out, void *workspace, size_t workspace_bytes, void *stream);

/* LVSA frame-level sparse attention (the LVSA page, training-free sparse
 * attention for long-video diffusion: "Core method", "Method steps in
 * detail"; linear branch off).  The sequence is T frames of P = N / T tokens
 * each (token n in frame n / P), P >= 64.  At denoising step `step` every
 * query token of frame t attends, in one softmax with scale 1/sqrt(d), every
 * token of the frames in A(t) = G_s U W(t):
 *   T_per = ceil(T / (C - (2W + 1)))  (C > 2W + 1, else SLA_ERR_INVALID_ARG);
 *   G_s = {(step mod T_per + i T_per) mod T : 0 <= i < ceil(T / T_per)};
 *   W(t): the window [w_lo, w_lo + 2W] clipped to frame T - 1, with
 *   w_lo = max(0, min(t - W, T - 1 - 2W)), grown one frame at a time on the
 *   side with more frames left outside it (the earlier side on a tie) until
 *   it holds min(2W + 1, T - |G_s|) frames not in G_s.
 * Every set then has |G_s| + min(2W + 1, T - |G_s|) frames.
 *
 * sla_lvsa_plan: host arithmetic only: T_per, |G_s| and the set size.
 * sla_lvsa_sets: the sets on the device: sets [T][max_frames] int32, frame
 *   t's set ascending in its first counts[t] entries; max_frames >= the set
 *   size.
 * sla_forward_lvsa: q, k, v: [B,H,N,d] bf16; out: [B,H,N,d] of out_dtype (F32
 *   or BF16); N = T * P, Nb = ceil(N/64) <= 4095; workspace of
 *   sla_lvsa_workspace_size() bytes, 256-byte aligned, clobbered.  The sets
 *   and the block schedule are built in the stream by the library's own
 *   kernels before the attention kernel (no host round trip). */
sla_status sla_lvsa_plan(int T, int C, int W, int *t_per, int *n_global, int *frames_per_set);
sla_status sla_lvsa_sets(int T, int C, int W, int step, int32_t *sets, int32_t *counts, int max_frames,
                         void *stream);
sla_status sla_lvsa_workspace_size(int B, int H, int N, int T, int C, int W, size_t *bytes);
sla_status sla_forward_lvsa(const void *q, const void *k, const void *v, sla_dtype in_dtype, sla_dtype out_dtype,
                            int B, int H, int N, int d, int block, int T, int C, int W, int step, void *out,
                            void *workspace, size_t workspace_bytes, void *stream);

/* Sliding tile attention (the VORTA page, "Key designs", item 1: a 3D
 * sliding window made block-dense by tiles; linear branch off).  The grid
 * (F, Hh, Ww) of N = F*Hh*Ww tokens is cut into tiles (tf, th, tw) that
 * divide it, of tf*th*tw tokens, a multiple of 64; tokens are TILE-MAJOR:
 * tiles in raster order over the tile grid, tokens in raster order inside a
 * tile (sla_sta_tile_order gives the permutation).  On every axis a query
 * tile keeps the key tiles whose centre (floor(i/t)*t + ceil(t/2)) lies in
 * (c - W/2, c + W/2] of its own centre c, for the axis window W (wf, wh,
 * ww); tiles past the grid do not exist.  Every query token of a tile
 * attends every token of the kept tiles, one softmax, scale 1/sqrt(d).
 *
 * sla_sta_tile_order: host only: perm[m] = raster index (frames slowest) of
 *   the m-th token in tile-major order; perm holds N entries.
 * sla_forward_sta: q, k, v: [B,H,N,d] bf16, tile-major; out: [B,H,N,d] of
 *   out_dtype (F32 or BF16), tile-major; N/64 <= 4095; workspace of
 *   sla_sta_workspace_size() bytes, 256-byte aligned, clobbered.  The block
 *   schedule is built in the stream and shared by every head. */
sla_status sla_sta_tile_order(int F, int Hh, int Ww, int tf, int th, int tw, int32_t *perm);
sla_status sla_sta_workspace_size(int B, int H, int F, int Hh, int Ww, int tf, int th, int tw, int wf, int wh, int ww,
                                  size_t *bytes);
sla_status sla_forward_sta(const void *q, const void *k, const void *v, sla_dtype in_dtype, sla_dtype out_dtype,
                           int B, int H, int d, int block, int F, int Hh, int Ww, int tf, int th, int tw, int wf,
                           int wh, int ww, void *out, void *workspace, size_t workspace_bytes, void *stream);

/* Mask-quality diagnostics (SLA article, section 2: a few attention weights
 * carry most of the mass; SVOO page: attention density as the share of
 * entries that covers 95 % of the cumulative attention mass).  Not part of
 * the forward pass; dense work, O(N^2 d) per head.
 *
 * sla_block_mass: the exact block attention mass.
 *   q, k: [B,H,N,d] bf16 (float32 inputs: SLA_ERR_UNSUPPORTED); block 64;
 *   d in {64, 128}; Nb = ceil(N/64) <= 2432.
 *   mass: [B,H,Nb,Nb] float32 output: mass[i][j] = the mean over the valid
 *   rows r of query block i of the sum over the valid keys u of key block j
 *   of softmax_u(q_r . k_u / sqrt(d)), the softmax over all N keys; each row
 *   sums to 1 (fp32 accumulation).  Deterministic.
 *
 * sla_mask_stats: per row of blocks, from a mass matrix and the labels of
 *   sla_classify / sla_forward (mask [rows][Nb] int8, rows = B*H*Nb):
 *   stats [rows][4] float32 = mass on the critical, marginal and negligible
 *   blocks, and the 95 % block density: the smallest number of key blocks,
 *   taken by decreasing mass, whose mass reaches 0.95 of the row's total,
 *   divided by Nb.  Sums in fp64 (class masses rounded once to float32), so
 *   the count equals that of an fp64 cumulative sum over the sorted masses
 *   unless a row's cumulative mass lies within fp64 rounding of 0.95 of its
 *   total.  Nb <= 2432. */
sla_status sla_block_mass(const void *q, const void *k, sla_dtype in_dtype, int B, int H, int N, int d, int block,
                          float *mass, void *stream);
sla_status sla_mask_stats(const float *mass, const int8_t *mask, long rows, int Nb, float *stats, void *stream);

/* Stage timing, for profiling.  While enabled on a thread, every sla_forward
 * call of that thread records HIP events around each of its kernels, on the
 * stream the kernel runs on: 0 pool, 1 classify, 2 state, 3 assemble, 4 fused
 * (a stage that does not run records zero time).  The stages run one
 * after another on the caller's stream, so with timing on their times add
 * up to about the time of a call.  sla_stage_times waits for the recorded
 * events, writes the summed milliseconds per stage to ms[0..4] and the number
 * of calls summed to *calls, and forgets them.  Events are created on first
 * use and kept per thread.  Disabled by default.  sla_forward_lists,
 * sla_forward_lvsa and sla_forward_sta calls are recorded too: stage 1 is
 * building their block schedule, stage 4 their attention kernel, stage 3
 * the merge of its shares (a schedule of 256 or more slots per row pair
 * runs in four shares; zero otherwise), the other stages zero.  sla_backward calls record: 0 the forward recomputed inside,
 * 1 the transposed lists and dQ of the sparse part, 2 dK and dV of the
 * sparse part, 3 the linear part's rows and transposed sums, 4 its keys and
 * dW; sla_backward_saved calls the same with stage 0 zero; sla_forward_save
 * calls are recorded as forward calls. */
#define SLA_NUM_STAGES 5
sla_status sla_set_stage_timing(int enable);
sla_status sla_stage_times(float *ms, int *calls);

/* Thread-local text for the last non-OK status returned on this thread. */
const char *sla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SLA_H */
