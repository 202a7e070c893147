/*
 * sla_oracle.c -- plain CPU oracle of the SLA sparse-linear attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or constant generator with the GPU library.
 *
 * What it computes follows the SLA article ("Tsinghua cracks the video
 * generation stall ..." on techwalker.com), section 3 ("SLA's core mechanism"):
 *   1. mean-pool Q and K per block of consecutive tokens;
 *   2. compressed attention map P_c = softmax(Qbar Kbar^T / sqrt(d));
 *   3. per query-block row, label each key block critical (top share, +1),
 *      negligible (bottom share, -1) or marginal (0);
 *   4. exact softmax attention over the critical blocks;
 *   5. linear attention phi(Q)(phi(K)^T V) over the marginal blocks, with
 *      phi = softmax (article section 5 reports softmax beating ELU+1/ReLU);
 *   6. negligible blocks are skipped;
 *   7. a d x d projection applied to the linear output, then added to the
 *      sparse output.
 * The normalisation of the sparse part (one softmax over the union of all
 * attended keys of the row, scale 1/sqrt(d)) is the block-sparse attention
 * formula of the LVSA page, "method steps" paragraph.
 *
 * Arithmetic: every input is a float32 value (bf16 inputs are exact in
 * float32); everything is float64.  Readings of points the pages leave open:
 *   - blocks are consecutive tokens; the last block may be ragged and holds
 *     n_i = min(b, N - i*b) tokens; pad positions take part in nothing;
 *   - pooled means are fp64 sums in ascending token order divided by n_i and
 *     rounded once to float32;
 *   - scores s_ij are fp64 dot products of the float32 means in ascending
 *     channel order (each product is exact, so contraction cannot change it);
 *   - the ranking is one total order: score descending, block index
 *     ascending.  The first k_c blocks are critical, the last k_n negligible;
 *     k_c = min(Nb, ceil(rho_c*Nb - 1e-9)), k_n = min(Nb-k_c, floor(rho_n*Nb + 1e-9));
 *   - an empty branch contributes zero; the linear normaliser has no epsilon;
 *   - the projection is y = x W^T (one W for all heads, no bias).
 * The linear branch forms H_i and Z_i as direct sums over the marginal blocks.
 *
 * Parity pins (tests/test_oracle_pins.py): dense attention at rho_c = 1,
 * quadratic linear attention at rho_c = rho_n = 0, softmax row sums, token
 * level brute force at tiny N, tie rules, invariants in V and W, exact means.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int sla_oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Number of critical and negligible blocks per row.  Returns 0 on success,
 * -1 for fractions outside [0,1] or summing above 1. */
int sla_oracle_counts(long Nb, double rho_c, double rho_n, int *k_c, int *k_n) {
    if (!(rho_c >= 0.0 && rho_c <= 1.0 && rho_n >= 0.0 && rho_n <= 1.0)) return -1;
    if (rho_c + rho_n > 1.0 + 1e-12) return -1;
    double c = ceil(rho_c * (double)Nb - 1e-9);
    double n = floor(rho_n * (double)Nb + 1e-9);
    if (c < 0) c = 0;
    if (c > Nb) c = (double)Nb;
    if (n < 0) n = 0;
    if (n > Nb - c) n = (double)Nb - c;
    *k_c = (int)c;
    *k_n = (int)n;
    return 0;
}

/* Step 1: block means.  x [BH, N, d] -> out [BH, Nb, d]. */
void sla_oracle_pool(const float *x, long BH, long N, long d, long blk, float *out) {
    long Nb = (N + blk - 1) / blk;
    #pragma omp parallel for collapse(2) schedule(static)
    for (long bh = 0; bh < BH; ++bh) {
        for (long i = 0; i < Nb; ++i) {
            long t0 = i * blk;
            long n_i = (N - t0 < blk) ? (N - t0) : blk;
            for (long c = 0; c < d; ++c) {
                double s = 0.0;
                for (long t = 0; t < n_i; ++t)
                    s += (double)x[(bh * N + t0 + t) * d + c];
                out[(bh * Nb + i) * d + c] = (float)(s / (double)n_i);
            }
        }
    }
}

typedef struct { double s; int j; } ranked;

/* Total order of the ranking: higher score first, then lower block index. */
static int rank_cmp(const void *a, const void *b) {
    const ranked *x = (const ranked *)a, *y = (const ranked *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->j < y->j) ? -1 : (x->j > y->j);
}

/* Steps 2 and 3: scores, optional P_c, and the three-way labels.
 * qp, kp [BH, Nb, d]; mask [BH, Nb, Nb] int8 (+1/0/-1); crit [BH, Nb, k_c] and
 * negl [BH, Nb, k_n] in ascending block order; scores/pc nullable [BH,Nb,Nb]. */
void sla_oracle_classify(const float *qp, const float *kp, long BH, long Nb, long d,
                         int k_c, int k_n, int8_t *mask, int32_t *crit, int32_t *negl,
                         double *scores, double *pc) {
    #pragma omp parallel
    {
        ranked *r = (ranked *)malloc(sizeof(ranked) * (size_t)Nb);
        double *s = (double *)malloc(sizeof(double) * (size_t)Nb);
        #pragma omp for collapse(2) schedule(dynamic, 4)
        for (long bh = 0; bh < BH; ++bh) {
            for (long i = 0; i < Nb; ++i) {
                const float *qi = qp + (bh * Nb + i) * d;
                for (long j = 0; j < Nb; ++j) {
                    const float *kj = kp + (bh * Nb + j) * d;
                    double acc = 0.0;
                    for (long c = 0; c < d; ++c) acc += (double)qi[c] * (double)kj[c];
                    s[j] = acc;
                    r[j].s = acc;
                    r[j].j = (int)j;
                }
                long row = bh * Nb + i;
                if (scores) memcpy(scores + row * Nb, s, sizeof(double) * (size_t)Nb);
                if (pc) {
                    double m = s[0];
                    for (long j = 1; j < Nb; ++j) if (s[j] > m) m = s[j];
                    double z = 0.0, inv = 1.0 / sqrt((double)d);
                    for (long j = 0; j < Nb; ++j) { pc[row * Nb + j] = exp((s[j] - m) * inv); z += pc[row * Nb + j]; }
                    for (long j = 0; j < Nb; ++j) pc[row * Nb + j] /= z;
                }
                qsort(r, (size_t)Nb, sizeof(ranked), rank_cmp);
                int8_t *mrow = mask + row * Nb;
                memset(mrow, 0, (size_t)Nb);
                for (long p = 0; p < k_c; ++p) mrow[r[p].j] = 1;
                for (long p = Nb - k_n; p < Nb; ++p) mrow[r[p].j] = -1;
                long nc = 0, nn = 0;
                for (long j = 0; j < Nb; ++j) {
                    if (mrow[j] == 1) crit[row * k_c + nc++] = (int32_t)j;
                    else if (mrow[j] == -1) negl[row * k_n + nn++] = (int32_t)j;
                }
            }
        }
        free(r);
        free(s);
    }
}

/* phi = softmax over the d channels of one token, with the maximum removed. */
static void phi_row(const float *x, long d, double *out) {
    double m = (double)x[0];
    for (long c = 1; c < d; ++c) if ((double)x[c] > m) m = (double)x[c];
    double z = 0.0;
    for (long c = 0; c < d; ++c) { out[c] = exp((double)x[c] - m); z += out[c]; }
    for (long c = 0; c < d; ++c) out[c] /= z;
}

/* phi of n tokens: x [n, d] -> out [n, d] (exposed for the row-sum pin). */
void sla_oracle_phi(const float *x, long n, long d, double *out) {
    for (long t = 0; t < n; ++t) phi_row(x + t * d, d, out + t * d);
}

/* Per key block j of one head: h_j = sum_u phi(k_u)^T v_u  [d x d, a-major]
 * and z_j = sum_u phi(k_u)  [d], over the valid tokens u of the block. */
static void head_states(const float *k, const float *v, long N, long d, long blk,
                        double *h, double *z) {
    long Nb = (N + blk - 1) / blk;
    #pragma omp parallel
    {
        double *ph = (double *)malloc(sizeof(double) * (size_t)d);
        #pragma omp for schedule(static)
        for (long j = 0; j < Nb; ++j) {
            double *hj = h + j * d * d, *zj = z + j * d;
            memset(hj, 0, sizeof(double) * (size_t)(d * d));
            memset(zj, 0, sizeof(double) * (size_t)d);
            long t0 = j * blk, t1 = (t0 + blk < N) ? t0 + blk : N;
            for (long u = t0; u < t1; ++u) {
                phi_row(k + u * d, d, ph);
                const float *vu = v + u * d;
                for (long a = 0; a < d; ++a) {
                    zj[a] += ph[a];
                    for (long e = 0; e < d; ++e) hj[a * d + e] += ph[a] * (double)vu[e];
                }
            }
        }
        free(ph);
    }
}

/* Steps 4-7 for chosen query blocks.
 * q, k, v [BH, N, d]; w [d, d]; mask [BH, Nb, Nb] from sla_oracle_classify.
 * rows [n_rows, 2] = (bh, i) pairs sorted by bh.  Outputs are [n_rows, blk, d]
 * doubles: out = o_s + o_l W^T, o_s (sparse part), o_l (linear part before the
 * projection).  Rows of a ragged last block beyond N are written as zero. */
void sla_oracle_forward_rows(const float *q, const float *k, const float *v, const float *w,
                             long BH, long N, long d, long blk, const int8_t *mask,
                             const int32_t *rows, long n_rows,
                             double *out, double *out_s, double *out_l) {
    long Nb = (N + blk - 1) / blk;
    double *h = NULL, *z = NULL;
    long cur = -1;
    double inv_sqrt_d = 1.0 / sqrt((double)d);
    memset(out, 0, sizeof(double) * (size_t)(n_rows * blk * d));
    memset(out_s, 0, sizeof(double) * (size_t)(n_rows * blk * d));
    memset(out_l, 0, sizeof(double) * (size_t)(n_rows * blk * d));
    long r0 = 0;
    while (r0 < n_rows) {
        long bh = rows[2 * r0];
        long r1 = r0;
        while (r1 < n_rows && rows[2 * r1] == bh) ++r1;
        const float *qh = q + bh * N * d, *kh = k + bh * N * d, *vh = v + bh * N * d;
        /* the linear states of this head are needed only if some row has a marginal block */
        int need_states = 0;
        for (long r = r0; r < r1 && !need_states; ++r) {
            const int8_t *mrow = mask + (bh * Nb + rows[2 * r + 1]) * Nb;
            for (long j = 0; j < Nb; ++j) if (mrow[j] == 0) { need_states = 1; break; }
        }
        if (need_states && cur != bh) {
            if (!h) {
                h = (double *)malloc(sizeof(double) * (size_t)(Nb * d * d));
                z = (double *)malloc(sizeof(double) * (size_t)(Nb * d));
            }
            head_states(kh, vh, N, d, blk, h, z);
            cur = bh;
        }
        #pragma omp parallel
        {
            double *logit = (double *)malloc(sizeof(double) * (size_t)(Nb * blk));
            double *Hi = (double *)malloc(sizeof(double) * (size_t)(d * d));
            double *Zi = (double *)malloc(sizeof(double) * (size_t)d);
            double *ph = (double *)malloc(sizeof(double) * (size_t)d);
            double *ol = (double *)malloc(sizeof(double) * (size_t)d);
            #pragma omp for schedule(dynamic, 1)
            for (long r = r0; r < r1; ++r) {
                long i = rows[2 * r + 1];
                const int8_t *mrow = mask + (bh * Nb + i) * Nb;
                long q0 = i * blk, q1 = (q0 + blk < N) ? q0 + blk : N;
                double *o = out + r * blk * d, *os = out_s + r * blk * d, *olin = out_l + r * blk * d;
                /* linear branch: direct sums over the marginal blocks */
                int n_marg = 0;
                memset(Hi, 0, sizeof(double) * (size_t)(d * d));
                memset(Zi, 0, sizeof(double) * (size_t)d);
                for (long j = 0; j < Nb; ++j) {
                    if (mrow[j] != 0) continue;
                    ++n_marg;
                    const double *hj = h + j * d * d, *zj = z + j * d;
                    for (long x = 0; x < d * d; ++x) Hi[x] += hj[x];
                    for (long a = 0; a < d; ++a) Zi[a] += zj[a];
                }
                for (long t = q0; t < q1; ++t) {
                    const float *qt = qh + t * d;
                    double *os_t = os + (t - q0) * d, *ol_t = olin + (t - q0) * d, *o_t = o + (t - q0) * d;
                    /* sparse branch: one softmax over every valid key of the critical blocks */
                    long nu = 0;
                    double m = -INFINITY;
                    for (long j = 0; j < Nb; ++j) {
                        if (mrow[j] != 1) continue;
                        long u0 = j * blk, u1 = (u0 + blk < N) ? u0 + blk : N;
                        for (long u = u0; u < u1; ++u) {
                            const float *ku = kh + u * d;
                            double acc = 0.0;
                            for (long c = 0; c < d; ++c) acc += (double)qt[c] * (double)ku[c];
                            acc *= inv_sqrt_d;
                            logit[nu++] = acc;
                            if (acc > m) m = acc;
                        }
                    }
                    if (nu > 0) {
                        double den = 0.0;
                        long p = 0;
                        for (long j = 0; j < Nb; ++j) {
                            if (mrow[j] != 1) continue;
                            long u0 = j * blk, u1 = (u0 + blk < N) ? u0 + blk : N;
                            for (long u = u0; u < u1; ++u, ++p) {
                                double e = exp(logit[p] - m);
                                den += e;
                                const float *vu = vh + u * d;
                                for (long c = 0; c < d; ++c) os_t[c] += e * (double)vu[c];
                            }
                        }
                        for (long c = 0; c < d; ++c) os_t[c] /= den;
                    }
                    /* linear branch: phi(q) H_i / (phi(q) . Z_i) */
                    if (n_marg > 0) {
                        phi_row(qt, d, ph);
                        double den = 0.0;
                        for (long a = 0; a < d; ++a) den += ph[a] * Zi[a];
                        for (long e = 0; e < d; ++e) {
                            double acc = 0.0;
                            for (long a = 0; a < d; ++a) acc += ph[a] * Hi[a * d + e];
                            ol[e] = acc / den;
                        }
                        memcpy(ol_t, ol, sizeof(double) * (size_t)d);
                    }
                    /* combine: O = O_s + O_l W^T */
                    for (long c = 0; c < d; ++c) {
                        double y = 0.0;
                        if (n_marg > 0)
                            for (long e = 0; e < d; ++e) y += ol_t[e] * (double)w[c * d + e];
                        o_t[c] = os_t[c] + y;
                    }
                }
            }
            free(logit); free(Hi); free(Zi); free(ph); free(ol);
        }
        r0 = r1;
    }
    free(h);
    free(z);
}
