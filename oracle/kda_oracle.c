/*
 * kda_oracle.c -- the fp64 CPU oracle for the Kimi Delta Attention (KDA) core.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg call this code.  It shares no source, header,
 * table or helper with the HIP library, and it is deliberately plain and slow:
 * one token at a time, in double precision, in the order the pages describe.
 *
 * What it computes (sources: page "每 4 层插 3 次线性注意力KDA 与 Gated
 * Attention 的混合账本" (AliceAI-Foundation-80B-A3B), section 二 -- the
 * depthwise causal conv of kernel 4 with padding 3 and no bias followed by
 * SiLU, the per-token delta-rule loop of `_torch_kda`, the gate formula and
 * the L2 normalisation of q and k; page "42层混合主干的长上下文秘诀
 * Ling-3.0-flash-VL ...", section "KDA 层的安全门", for the gate's lower
 * bound of -5.0):
 *
 *   per channel c of q, k, v:  y_t = sum_{j=0..3} w[c][j] * x_{t-3+j}
 *                              (x before the sequence = conv history or 0)
 *                              u_t = y_t * sigmoid(y_t)
 *   q_t = scale * u_q / sqrt(|u_q|^2 + eps),  k_t = u_k / sqrt(|u_k|^2 + eps),
 *   v_t = u_v
 *   g_t[i] = max(-exp(A_log[h]) * softplus(alpha_t[i] + dt_bias[h][i]), lb)
 *   beta_t = sigmoid(b_t)
 *   S <- Diag(exp(g_t)) S            (rows of S are key channels)
 *   p  = k_t^T S
 *   d  = beta_t (v_t - p)
 *   S <- S + k_t d^T
 *   o_t = q_t^T S                    (the output reads the updated state)
 *
 * The output epilogue (kda_oracle_output_gate below): the same AliceAI page,
 * section 三, puts KDA's output through `o_norm` and a sigmoid gate (the
 * full-attention layers' `output * sigmoid(output_gate)` is likened to it),
 * and its section 二 lists `output_gate` among the per-token control inputs:
 *   y_t[j] = o_t[j] / sqrt(mean_j' o_t[j']^2 + eps_o) * w[j] * sigmoid(gate_t[j])
 * per (token, head), the mean over the head's dv channels.
 *
 * Readings where the pages are silent (each one is a choice, listed in the
 * design notes): eps = 1e-6 inside the square root; scale defaults to 1;
 * o_norm is an RMS norm over one head's dv outputs with one weight per
 * channel shared by the heads, its epsilon a parameter (1e-6 by default);
 * the safe gate is a clamp applied after the product; the conv history holds
 * the last three raw (pre-conv) inputs per channel, oldest first, with the
 * channels ordered q | k | v.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_FLAG_SKIP_CONV   1u  /* u = raw input (no conv, no SiLU)        */
#define ORC_FLAG_SKIP_L2NORM 2u  /* q, k used as given                      */
#define ORC_FLAG_RAW_GATE    4u  /* alpha holds g itself (no softplus/clamp) */
#define ORC_FLAG_RAW_BETA    8u  /* b holds beta itself (no sigmoid)         */
#define ORC_FLAG_BETA_X2    16u  /* beta = 2*sigmoid(b): negative eigenvalues allowed */

static double orc_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* softplus(x) = log(1 + e^x), in a form that neither overflows nor loses the
 * small tail: max(x, 0) + log1p(e^{-|x|}). */
static double orc_softplus(double x) { return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x))); }

/*
 * Preprocess one head of one sequence.
 *   L          tokens in the sequence
 *   q_raw      [L][H*dk] raw q projections (row stride H*dk)
 *   k_raw      [L][H*dk]
 *   v_raw      [L][H*dv]
 *   alpha      [L][H][dk]
 *   b          [L][H]
 *   w_q, w_k   [H*dk][4];  w_v [H*dv][4]; tap 3 multiplies the current token
 *   A_log      [H];  dt_bias [H*dk]
 *   conv_in    [3][Ctot] history for this sequence (oldest first) or NULL
 * Outputs, dense per head: qh, kh [L][dk], vh [L][dv], g [L][dk], beta [L].
 */
void kda_oracle_preprocess_head(int L, int H, int dk, int dv, int h,
                                const double *q_raw, const double *k_raw, const double *v_raw,
                                const double *alpha, const double *b,
                                const double *w_q, const double *w_k, const double *w_v,
                                const double *A_log, const double *dt_bias,
                                const double *conv_in, double scale, double lb, double eps,
                                unsigned flags,
                                double *qh, double *kh, double *vh, double *g, double *beta)
{
    const int Ctot = H * (2 * dk + dv);
    /* three channel groups: q, k, v */
    for (int grp = 0; grp < 3; ++grp) {
        const int d = grp == 2 ? dv : dk;
        const int row = grp == 2 ? H * dv : H * dk;      /* row stride of the raw input */
        const int c0 = h * d;                             /* first channel of this head */
        const int ctot_off = grp == 0 ? 0 : (grp == 1 ? H * dk : 2 * H * dk);
        const double *x = grp == 0 ? q_raw : (grp == 1 ? k_raw : v_raw);
        const double *w = grp == 0 ? w_q : (grp == 1 ? w_k : w_v);
        double *u = grp == 0 ? qh : (grp == 1 ? kh : vh);
        for (int t = 0; t < L; ++t) {
            for (int i = 0; i < d; ++i) {
                const int c = c0 + i;
                double val;
                if (flags & ORC_FLAG_SKIP_CONV) {
                    val = x[(size_t)t * row + c];
                } else {
                    double y = 0.0;
                    for (int j = 0; j < 4; ++j) {
                        const int tt = t - 3 + j;     /* token that tap j sees */
                        double xv;
                        if (tt >= 0)
                            xv = x[(size_t)tt * row + c];
                        else if (conv_in)
                            xv = conv_in[(size_t)(3 + tt) * Ctot + ctot_off + c];
                        else
                            xv = 0.0;
                        y += w[(size_t)c * 4 + j] * xv;
                    }
                    val = y * orc_sigmoid(y);          /* SiLU */
                }
                u[(size_t)t * d + i] = val;
            }
        }
    }
    for (int t = 0; t < L; ++t) {
        if (!(flags & ORC_FLAG_SKIP_L2NORM)) {
            double sq = 0.0, sk = 0.0;
            for (int i = 0; i < dk; ++i) {
                sq += qh[(size_t)t * dk + i] * qh[(size_t)t * dk + i];
                sk += kh[(size_t)t * dk + i] * kh[(size_t)t * dk + i];
            }
            const double nq = sqrt(sq + eps), nk = sqrt(sk + eps);
            for (int i = 0; i < dk; ++i) {
                qh[(size_t)t * dk + i] /= nq;
                kh[(size_t)t * dk + i] /= nk;
            }
        }
        for (int i = 0; i < dk; ++i) qh[(size_t)t * dk + i] *= scale;
        const double a = exp(A_log[h]);
        for (int i = 0; i < dk; ++i) {
            const double al = alpha[((size_t)t * H + h) * dk + i];
            double gi;
            if (flags & ORC_FLAG_RAW_GATE) {
                gi = al;
            } else {
                gi = -a * orc_softplus(al + dt_bias[(size_t)h * dk + i]);
                if (gi < lb) gi = lb;                  /* safe gate: lower bound */
            }
            g[(size_t)t * dk + i] = gi;
        }
        const double bb = b[(size_t)t * H + h];
        double be = (flags & ORC_FLAG_RAW_BETA) ? bb : orc_sigmoid(bb);
        if (flags & ORC_FLAG_BETA_X2) be *= 2.0;
        beta[t] = be;
    }
}

/*
 * The token recurrence for one head.  S [dk][dv] holds the initial state on
 * entry and the final state on exit.  o is written with row stride o_stride.
 */
void kda_oracle_recurrence(int L, int dk, int dv,
                           const double *qh, const double *kh, const double *vh,
                           const double *g, const double *beta,
                           double *S, double *o, long o_stride)
{
    double *p = (double *)malloc(sizeof(double) * (size_t)dv);
    double *d = (double *)malloc(sizeof(double) * (size_t)dv);
    for (int t = 0; t < L; ++t) {
        const double *q = qh + (size_t)t * dk, *k = kh + (size_t)t * dk;
        const double *v = vh + (size_t)t * dv, *gt = g + (size_t)t * dk;
        /* decay: row i of S is key channel i */
        for (int i = 0; i < dk; ++i) {
            const double e = exp(gt[i]);
            for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= e;
        }
        /* prediction p = k^T S */
        for (int j = 0; j < dv; ++j) p[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) p[j] += k[i] * S[(size_t)i * dv + j];
        for (int j = 0; j < dv; ++j) d[j] = beta[t] * (v[j] - p[j]);
        /* write S += k d^T */
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += k[i] * d[j];
        /* read o = q^T S with the updated state */
        double *ot = o + (size_t)t * o_stride;
        for (int j = 0; j < dv; ++j) ot[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) ot[j] += q[i] * S[(size_t)i * dv + j];
    }
    free(p);
    free(d);
}

/* ---------------------------------------------------------------------- */
/* Whole packed batch, threads over (sequence, head).                       */
/* ---------------------------------------------------------------------- */
typedef struct {
    int nseq, H, dk, dv;
    const int64_t *cu;
    const double *q, *k, *v, *alpha, *b, *w_q, *w_k, *w_v, *A_log, *dt_bias;
    double scale, lb, eps;
    unsigned flags;
    const double *S0, *conv_in;
    double *o, *S_out;
    const int32_t *items;   /* optional list of (seq*H + head) items; NULL = all */
    int n_items;
    volatile int next;
} orc_job_t;

static void run_item(orc_job_t *J, int item)
{
    const int n = item / J->H, h = item % J->H;
    const int H = J->H, dk = J->dk, dv = J->dv, Ctot = H * (2 * dk + dv);
    const int64_t t0 = J->cu[n];
    const int L = (int)(J->cu[n + 1] - t0);
    double *S = J->S_out + ((size_t)n * H + h) * dk * dv;
    if (J->S0)
        memcpy(S, J->S0 + ((size_t)n * H + h) * dk * dv, sizeof(double) * (size_t)dk * dv);
    else
        memset(S, 0, sizeof(double) * (size_t)dk * dv);
    if (L <= 0) return;
    double *qh = (double *)malloc(sizeof(double) * (size_t)L * dk);
    double *kh = (double *)malloc(sizeof(double) * (size_t)L * dk);
    double *vh = (double *)malloc(sizeof(double) * (size_t)L * dv);
    double *g = (double *)malloc(sizeof(double) * (size_t)L * dk);
    double *be = (double *)malloc(sizeof(double) * (size_t)L);
    kda_oracle_preprocess_head(L, H, dk, dv, h,
                               J->q + (size_t)t0 * H * dk, J->k + (size_t)t0 * H * dk,
                               J->v + (size_t)t0 * H * dv, J->alpha + (size_t)t0 * H * dk,
                               J->b + (size_t)t0 * H, J->w_q, J->w_k, J->w_v, J->A_log, J->dt_bias,
                               J->conv_in ? J->conv_in + (size_t)n * 3 * Ctot : NULL,
                               J->scale, J->lb, J->eps, J->flags, qh, kh, vh, g, be);
    kda_oracle_recurrence(L, dk, dv, qh, kh, vh, g, be, S,
                          J->o + ((size_t)t0 * H + h) * dv, (long)H * dv);
    free(qh); free(kh); free(vh); free(g); free(be);
}

static void *worker(void *arg)
{
    orc_job_t *J = (orc_job_t *)arg;
    const int total = J->items ? J->n_items : J->nseq * J->H;
    for (;;) {
        const int i = __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED);
        if (i >= total) break;
        run_item(J, J->items ? J->items[i] : i);
    }
    return NULL;
}

/*
 * Full forward over nseq packed sequences (cu_seqlens [nseq+1] token offsets).
 *   q, k [total_T][H*dk], v [total_T][H*dv], alpha [total_T][H][dk], b [total_T][H]
 *   S0 [nseq][H][dk][dv] or NULL (zeros); conv_in [nseq][3][Ctot] or NULL (zeros)
 *   o [total_T][H][dv]; S_out [nseq][H][dk][dv]; conv_out [nseq][3][Ctot] or NULL
 *   items/n_items: optional subset of (seq*H + head) to compute (others untouched)
 * Returns the number of threads used.
 */
int kda_oracle_forward(int nseq, const int64_t *cu, int H, int dk, int dv,
                       const double *q, const double *k, const double *v,
                       const double *alpha, const double *b,
                       const double *w_q, const double *w_k, const double *w_v,
                       const double *A_log, const double *dt_bias,
                       double scale, double lb, double eps, unsigned flags,
                       const double *S0, const double *conv_in,
                       double *o, double *S_out, double *conv_out,
                       const int32_t *items, int n_items, int nthreads)
{
    orc_job_t J = {nseq, H, dk, dv, cu, q, k, v, alpha, b, w_q, w_k, w_v, A_log, dt_bias,
                   scale, lb, eps, flags, S0, conv_in, o, S_out, items, n_items, 0};
    const int total = items ? n_items : nseq * H;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > total) nthreads = total > 0 ? total : 1;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, &J);
    worker(&J);
    for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);

    /* conv history out: the last three raw inputs of each sequence, reaching
     * into the incoming history when the sequence is shorter than three. */
    if (conv_out) {
        const int Ctot = H * (2 * dk + dv);
        for (int n = 0; n < nseq; ++n) {
            const int64_t t0 = cu[n];
            const int L = (int)(cu[n + 1] - t0);
            for (int m = 0; m < 3; ++m) {
                const int tt = L - 3 + m;
                for (int c = 0; c < Ctot; ++c) {
                    double val;
                    if (tt >= 0) {
                        const int64_t tok = t0 + tt;
                        if (c < H * dk) val = q[(size_t)tok * H * dk + c];
                        else if (c < 2 * H * dk) val = k[(size_t)tok * H * dk + (c - H * dk)];
                        else val = v[(size_t)tok * H * dv + (c - 2 * H * dk)];
                    } else if (conv_in) {
                        val = conv_in[((size_t)n * 3 + (3 + tt)) * Ctot + c];
                    } else {
                        val = 0.0;
                    }
                    conv_out[((size_t)n * 3 + m) * Ctot + c] = val;
                }
            }
        }
    }
    return nthreads;
}

/*
 * The output epilogue over n_rows (token, head) rows of dv outputs each:
 * o, gate, y [n_rows][dv]; w [dv] (one weight per channel, shared by the
 * heads).  y may alias o.
 */
void kda_oracle_output_gate(long n_rows, int dv, const double *o, const double *gate, const double *w,
                            double eps, double *y)
{
    for (long r = 0; r < n_rows; ++r) {
        const double *orow = o + (size_t)r * dv;
        const double *grow = gate + (size_t)r * dv;
        double ss = 0.0;
        for (int j = 0; j < dv; ++j) ss += orow[j] * orow[j];
        const double rms = sqrt(ss / dv + eps);
        for (int j = 0; j < dv; ++j)
            y[(size_t)r * dv + j] = orow[j] / rms * w[j] * orc_sigmoid(grow[j]);
    }
}
