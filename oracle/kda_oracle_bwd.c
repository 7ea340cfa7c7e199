/*
 * kda_oracle_bwd.c -- the fp64 CPU oracle for the gradient of the KDA core.
 *
 * TEST INFRASTRUCTURE, like kda_oracle.c: only the test suite calls it, and
 * it shares nothing with the HIP library.
 *
 * The models the pages describe are trained natively with KDA layers (page
 * "Kimi Delta Attention与MLA交替堆叠：Ling-3.0-flash架构创新背后的技术原理",
 * section on the 5:1 hybrid stacking; page "Ling-3.0-flash vs 传统大模型",
 * the staged 8K -> 32K -> 256K training), so the core needs its vector-
 * Jacobian product.  The pages give only the forward computation (AliceAI
 * page, section 二); this file is its reverse-mode derivative, written out
 * step by step in the reverse order of the forward, in double precision:
 *
 * Forward, per token t (rows of S are key channels):
 *   S~_t = Diag(e^{g_t}) S_{t-1};  p_t = S~_t^T k_t;  d_t = beta_t (v_t - p_t)
 *   S_t = S~_t + k_t d_t^T;         o_t = S_t^T q_t
 * Reverse, with dS the adjoint of S_t (dS = dS_T after the last token):
 *   dS += q_t do_t^T;               dq_t = S_t do_t
 *   dd = dS^T k_t;                  dk_t = dS d_t
 *   dv_t = beta_t dd;               dbeta_t = dd . (v_t - p_t)
 *   dp = -beta_t dd;                dk_t += S~_t dp;   dS~ = dS + k_t dp^T
 *   dg_t[i] = sum_j dS~[i][j] S~_t[i][j];              dS = Diag(e^{g_t}) dS~
 * and dS_0 = dS at the end.  Then through the preprocess of every token:
 *   q = s u_q / n_q with n_q = sqrt(|u_q|^2 + eps):
 *       du_q = s (dq / n_q - u_q (u_q . dq) / n_q^3)     (k likewise, s = 1)
 *   u = y sigmoid(y):  dy = du sigmoid(y) (1 + y (1 - sigmoid(y)))
 *   y_t[c] = sum_j w[c][j] x_{t-3+j}[c]:
 *       dx_{t-3+j}[c] += w[c][j] dy_t[c]  (into the conv history for t-3+j < 0)
 *       dw[c][j] += dy_t[c] x_{t-3+j}[c]
 *   g = max(g_raw, lb), g_raw = -e^{A_log} softplus(alpha + dt_bias):
 *       where g_raw >= lb:  dalpha = -dg e^{A_log} sigmoid(alpha + dt_bias),
 *       ddt_bias += dalpha,  dA_log += dg g_raw;  where clamped: 0
 *   beta = sigmoid(b) (x2 with the flag):  db = dbeta beta (1 - sigmoid(b))
 * The test-hook flags of kda_oracle.c cut the matching links of the chain.
 *
 * The loss's gradients come in as do (w.r.t. every output) and dS_T (w.r.t.
 * the final state, may be absent); the conv history out is a copy of raw
 * inputs and takes no gradient here.  States are kept at every 64th token and
 * the 64 states of a segment are recomputed from its checkpoint by the same
 * forward loop, so memory stays at (L/64 + 65) dk dv doubles per head.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORB_FLAG_SKIP_CONV   1u
#define ORB_FLAG_SKIP_L2NORM 2u
#define ORB_FLAG_RAW_GATE    4u
#define ORB_FLAG_RAW_BETA    8u
#define ORB_FLAG_BETA_X2    16u

#define ORB_SEG 64

static double orb_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }
static double orb_softplus(double x) { return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x))); }

/* one forward token: S (in: S_{t-1}, out: S_t); also returns S~ and p, d */
static void orb_token(int dk, int dv, const double *q, const double *k, const double *v, const double *g,
                      double beta, double *S, double *Stil, double *p, double *d, double *o)
{
    (void)q;
    for (int i = 0; i < dk; ++i) {
        const double e = exp(g[i]);
        for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= e;
    }
    if (Stil) memcpy(Stil, S, sizeof(double) * (size_t)dk * dv);
    for (int j = 0; j < dv; ++j) p[j] = 0.0;
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) p[j] += k[i] * S[(size_t)i * dv + j];
    for (int j = 0; j < dv; ++j) d[j] = beta * (v[j] - p[j]);
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += k[i] * d[j];
    if (o) {
        for (int j = 0; j < dv; ++j) o[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) o[j] += q[i] * S[(size_t)i * dv + j];
    }
}

/*
 * Backward of the token recurrence for one head, on post-preprocess inputs.
 *   q, k, g [L][dk]; v [L][dv]; beta [L]; S0 [dk][dv] (NULL = zeros)
 *   dO [L][dv] (row stride do_stride); dST [dk][dv] or NULL
 * Outputs: dq, dk, dg [L][dk]; dv [L][dv]; dbeta [L]; dS0 [dk][dv].
 */
void kda_oracle_recurrence_bwd(int L, int dk, int dv, const double *q, const double *k, const double *v,
                               const double *g, const double *beta, const double *S0,
                               const double *dO, long do_stride, const double *dST,
                               double *dq, double *dkk, double *dvv, double *dg, double *dbeta, double *dS0)
{
    const size_t SZ = (size_t)dk * dv;
    const int nseg = (L + ORB_SEG - 1) / ORB_SEG;
    double *ckpt = (double *)malloc(sizeof(double) * SZ * (size_t)(nseg > 0 ? nseg : 1));
    double *seg = (double *)malloc(sizeof(double) * SZ * (ORB_SEG + 1));   /* S before each token, and after the last */
    double *Stil = (double *)malloc(sizeof(double) * SZ);
    double *dS = (double *)malloc(sizeof(double) * SZ);
    double *dSt = (double *)malloc(sizeof(double) * SZ);
    double *p = (double *)malloc(sizeof(double) * (size_t)dv);
    double *d = (double *)malloc(sizeof(double) * (size_t)dv);
    double *dd = (double *)malloc(sizeof(double) * (size_t)dv);
    double *dp = (double *)malloc(sizeof(double) * (size_t)dv);
    double *S = (double *)malloc(sizeof(double) * SZ);

    /* forward: the state at the start of every segment */
    if (S0) memcpy(S, S0, sizeof(double) * SZ); else memset(S, 0, sizeof(double) * SZ);
    for (int t = 0; t < L; ++t) {
        if (t % ORB_SEG == 0) memcpy(ckpt + (size_t)(t / ORB_SEG) * SZ, S, sizeof(double) * SZ);
        orb_token(dk, dv, q + (size_t)t * dk, k + (size_t)t * dk, v + (size_t)t * dv, g + (size_t)t * dk, beta[t],
                  S, NULL, p, d, NULL);
    }
    if (dST) memcpy(dS, dST, sizeof(double) * SZ); else memset(dS, 0, sizeof(double) * SZ);

    for (int sgi = nseg - 1; sgi >= 0; --sgi) {
        const int t0 = sgi * ORB_SEG, t1 = (t0 + ORB_SEG < L) ? t0 + ORB_SEG : L;
        /* recompute the segment's states: seg[m] = S_{t0+m-1} (state before token t0+m) */
        memcpy(seg, ckpt + (size_t)sgi * SZ, sizeof(double) * SZ);
        for (int t = t0; t < t1; ++t) {
            double *nxt = seg + (size_t)(t - t0 + 1) * SZ;
            memcpy(nxt, seg + (size_t)(t - t0) * SZ, sizeof(double) * SZ);
            orb_token(dk, dv, q + (size_t)t * dk, k + (size_t)t * dk, v + (size_t)t * dv, g + (size_t)t * dk,
                      beta[t], nxt, NULL, p, d, NULL);
        }
        for (int t = t1 - 1; t >= t0; --t) {
            const double *qt = q + (size_t)t * dk, *kt = k + (size_t)t * dk, *vt = v + (size_t)t * dv;
            const double *gt = g + (size_t)t * dk, *dot = dO + (size_t)t * do_stride;
            const double *Sprev = seg + (size_t)(t - t0) * SZ, *Snew = seg + (size_t)(t - t0 + 1) * SZ;
            /* S~_t, p_t, d_t of this token */
            for (int i = 0; i < dk; ++i) {
                const double e = exp(gt[i]);
                for (int j = 0; j < dv; ++j) Stil[(size_t)i * dv + j] = e * Sprev[(size_t)i * dv + j];
            }
            for (int j = 0; j < dv; ++j) p[j] = 0.0;
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) p[j] += kt[i] * Stil[(size_t)i * dv + j];
            for (int j = 0; j < dv; ++j) d[j] = beta[t] * (vt[j] - p[j]);
            /* o_t = S_t^T q_t */
            for (int i = 0; i < dk; ++i) {
                double s = 0.0;
                for (int j = 0; j < dv; ++j) {
                    dS[(size_t)i * dv + j] += qt[i] * dot[j];
                    s += Snew[(size_t)i * dv + j] * dot[j];
                }
                dq[(size_t)t * dk + i] = s;
            }
            /* S_t = S~_t + k_t d_t^T */
            for (int j = 0; j < dv; ++j) dd[j] = 0.0;
            for (int i = 0; i < dk; ++i) {
                double s = 0.0;
                for (int j = 0; j < dv; ++j) {
                    dd[j] += dS[(size_t)i * dv + j] * kt[i];
                    s += dS[(size_t)i * dv + j] * d[j];
                }
                dkk[(size_t)t * dk + i] = s;
            }
            /* d_t = beta_t (v_t - p_t) */
            double db = 0.0;
            for (int j = 0; j < dv; ++j) {
                dvv[(size_t)t * dv + j] = beta[t] * dd[j];
                db += dd[j] * (vt[j] - p[j]);
                dp[j] = -beta[t] * dd[j];
            }
            dbeta[t] = db;
            /* p_t = S~_t^T k_t */
            for (int i = 0; i < dk; ++i) {
                double s = 0.0;
                for (int j = 0; j < dv; ++j) {
                    s += Stil[(size_t)i * dv + j] * dp[j];
                    dSt[(size_t)i * dv + j] = dS[(size_t)i * dv + j] + kt[i] * dp[j];
                }
                dkk[(size_t)t * dk + i] += s;
            }
            /* S~_t = Diag(e^{g_t}) S_{t-1} */
            for (int i = 0; i < dk; ++i) {
                const double e = exp(gt[i]);
                double s = 0.0;
                for (int j = 0; j < dv; ++j) {
                    s += dSt[(size_t)i * dv + j] * Stil[(size_t)i * dv + j];
                    dS[(size_t)i * dv + j] = e * dSt[(size_t)i * dv + j];
                }
                dg[(size_t)t * dk + i] = s;
            }
        }
    }
    memcpy(dS0, dS, sizeof(double) * SZ);
    free(ckpt); free(seg); free(Stil); free(dS); free(dSt); free(p); free(d); free(dd); free(dp); free(S);
}

/*
 * Backward of the preprocess for one head of one sequence: from the
 * gradients of the post-preprocess tensors (dq, dk, dg [L][dk], dv [L][dv],
 * dbeta [L]) to those of the raw inputs and parameters.  Input layouts as in
 * kda_oracle_preprocess_head.  Outputs:
 *   dq_raw, dk_raw [L][H*dk] and dv_raw [L][H*dv] (this head's columns only),
 *   dalpha [L][H][dk] (this head), db [L][H] (this head),
 *   dconv_in [3][Ctot] (this head's channels; may be NULL),
 *   pw_q, pw_k [dk][4], pw_v [dv][4], pdtb [dk], *pAlog: this (sequence,
 *   head)'s contribution to the parameter gradients (overwritten).
 */
void kda_oracle_preprocess_bwd_head(int L, int H, int dk, int dv, int h,
                                    const double *q_raw, const double *k_raw, const double *v_raw,
                                    const double *alpha, const double *b,
                                    const double *w_q, const double *w_k, const double *w_v,
                                    const double *A_log, const double *dt_bias, const double *conv_in,
                                    double scale, double lb, double eps, unsigned flags,
                                    const double *dqh, const double *dkh, const double *dvh,
                                    const double *dg, const double *dbeta,
                                    double *dq_raw, double *dk_raw, double *dv_raw, double *dalpha, double *db,
                                    double *dconv_in, double *pw_q, double *pw_k, double *pw_v, double *pdtb,
                                    double *pAlog)
{
    const int Ctot = H * (2 * dk + dv);
    const int dmax = dk > dv ? dk : dv;
    double *y = (double *)malloc(sizeof(double) * (size_t)L * dmax);
    double *u = (double *)malloc(sizeof(double) * (size_t)L * dmax);
    double *du = (double *)malloc(sizeof(double) * (size_t)L * dmax);
    for (int grp = 0; grp < 3; ++grp) {
        const int d = grp == 2 ? dv : dk;
        const int row = grp == 2 ? H * dv : H * dk;
        const int c0 = h * d;
        const int ctot_off = grp == 0 ? 0 : (grp == 1 ? H * dk : 2 * H * dk);
        const double *x = grp == 0 ? q_raw : (grp == 1 ? k_raw : v_raw);
        const double *w = grp == 0 ? w_q : (grp == 1 ? w_k : w_v);
        const double *dpost = grp == 0 ? dqh : (grp == 1 ? dkh : dvh);
        double *dx = grp == 0 ? dq_raw : (grp == 1 ? dk_raw : dv_raw);
        double *pw = grp == 0 ? pw_q : (grp == 1 ? pw_k : pw_v);
        /* forward: conv output y and activation u */
        for (int t = 0; t < L; ++t)
            for (int i = 0; i < d; ++i) {
                const int c = c0 + i;
                double val, yy = 0.0;
                if (flags & ORB_FLAG_SKIP_CONV) {
                    val = x[(size_t)t * row + c];
                } else {
                    for (int j = 0; j < 4; ++j) {
                        const int tt = t - 3 + j;
                        double xv = 0.0;
                        if (tt >= 0) xv = x[(size_t)tt * row + c];
                        else if (conv_in) xv = conv_in[(size_t)(3 + tt) * Ctot + ctot_off + c];
                        yy += w[(size_t)c * 4 + j] * xv;
                    }
                    val = yy * orb_sigmoid(yy);
                }
                y[(size_t)t * d + i] = yy;
                u[(size_t)t * d + i] = val;
            }
        /* the L2 norm (q, k) and the scale (q) */
        for (int t = 0; t < L; ++t) {
            const double *ut = u + (size_t)t * d, *gt = dpost + (size_t)t * d;
            double *dut = du + (size_t)t * d;
            const double s = grp == 0 ? scale : 1.0;
            if (grp < 2 && !(flags & ORB_FLAG_SKIP_L2NORM)) {
                double ss = 0.0, dot = 0.0;
                for (int i = 0; i < d; ++i) { ss += ut[i] * ut[i]; dot += ut[i] * gt[i]; }
                const double n = sqrt(ss + eps);
                for (int i = 0; i < d; ++i) dut[i] = s * (gt[i] / n - ut[i] * dot / (n * n * n));
            } else {
                for (int i = 0; i < d; ++i) dut[i] = s * gt[i];
            }
        }
        /* SiLU and the conv */
        for (int i = 0; i < d; ++i) for (int j = 0; j < 4; ++j) pw[(size_t)i * 4 + j] = 0.0;
        for (int t = 0; t < L; ++t)
            for (int i = 0; i < d; ++i) dx[(size_t)t * row + c0 + i] = 0.0;
        if (dconv_in)
            for (int m = 0; m < 3; ++m)
                for (int i = 0; i < d; ++i) dconv_in[(size_t)m * Ctot + ctot_off + c0 + i] = 0.0;
        for (int t = 0; t < L; ++t)
            for (int i = 0; i < d; ++i) {
                const int c = c0 + i;
                const double dut = du[(size_t)t * d + i];
                if (flags & ORB_FLAG_SKIP_CONV) {
                    dx[(size_t)t * row + c] += dut;
                    continue;
                }
                const double yy = y[(size_t)t * d + i], sg = orb_sigmoid(yy);
                const double dy = dut * sg * (1.0 + yy * (1.0 - sg));
                for (int j = 0; j < 4; ++j) {
                    const int tt = t - 3 + j;
                    double xv = 0.0;
                    if (tt >= 0) {
                        xv = x[(size_t)tt * row + c];
                        dx[(size_t)tt * row + c] += w[(size_t)c * 4 + j] * dy;
                    } else {
                        /* a tap before the sequence reads the history (zeros without one) */
                        if (conv_in) xv = conv_in[(size_t)(3 + tt) * Ctot + ctot_off + c];
                        if (dconv_in) dconv_in[(size_t)(3 + tt) * Ctot + ctot_off + c] += w[(size_t)c * 4 + j] * dy;
                    }
                    pw[(size_t)i * 4 + j] += dy * xv;
                }
            }
    }
    /* gate and beta */
    const double a = exp(A_log[h]);
    double dAl = 0.0;
    for (int i = 0; i < dk; ++i) pdtb[i] = 0.0;
    for (int t = 0; t < L; ++t) {
        for (int i = 0; i < dk; ++i) {
            const double al = alpha[((size_t)t * H + h) * dk + i];
            const double dgi = dg[(size_t)t * dk + i];
            double da;
            if (flags & ORB_FLAG_RAW_GATE) {
                da = dgi;
            } else {
                const double z = al + dt_bias[(size_t)h * dk + i];
                const double graw = -a * orb_softplus(z);
                if (graw >= lb) {
                    da = -dgi * a * orb_sigmoid(z);
                    pdtb[i] += da;
                    dAl += dgi * graw;
                } else {
                    da = 0.0;
                }
            }
            dalpha[((size_t)t * H + h) * dk + i] = da;
        }
        const double bb = b[(size_t)t * H + h];
        double dbv;
        if (flags & ORB_FLAG_RAW_BETA) {
            dbv = dbeta[t];
        } else {
            const double sg = orb_sigmoid(bb);
            dbv = dbeta[t] * sg * (1.0 - sg);
        }
        if (flags & ORB_FLAG_BETA_X2) dbv *= 2.0;
        db[(size_t)t * H + h] = dbv;
    }
    *pAlog = dAl;
    free(y); free(u); free(du);
}

/* the forward preprocess of kda_oracle.c (same library) */
void kda_oracle_preprocess_head(int L, int H, int dk, int dv, int h,
                                const double *q_raw, const double *k_raw, const double *v_raw,
                                const double *alpha, const double *b,
                                const double *w_q, const double *w_k, const double *w_v,
                                const double *A_log, const double *dt_bias,
                                const double *conv_in, double scale, double lb, double eps,
                                unsigned flags,
                                double *qh, double *kh, double *vh, double *g, double *beta);

typedef struct {
    int nseq, H, dk, dv;
    const int64_t *cu;
    const double *q, *k, *v, *alpha, *b, *w_q, *w_k, *w_v, *A_log, *dt_bias;
    double scale, lb, eps;
    unsigned flags;
    const double *S0, *conv_in, *dO, *dST;
    double *dq, *dk_, *dv_, *dalpha, *db, *dS0, *dconv_in;
    double *pw_q, *pw_k, *pw_v, *pdtb, *pAlog;     /* per-item partials [nseq*H][...] */
    volatile int next;
} orb_job_t;

static void orb_item(orb_job_t *J, int item)
{
    const int n = item / J->H, h = item % J->H;
    const int H = J->H, dk = J->dk, dv = J->dv, Ctot = H * (2 * dk + dv);
    const size_t SZ = (size_t)dk * dv;
    const int64_t t0 = J->cu[n];
    const int L = (int)(J->cu[n + 1] - t0);
    const double *S0 = J->S0 ? J->S0 + ((size_t)n * H + h) * SZ : NULL;
    const double *dST = J->dST ? J->dST + ((size_t)n * H + h) * SZ : NULL;
    double *dS0 = J->dS0 + ((size_t)n * H + h) * SZ;
    double *pwq = J->pw_q + (size_t)item * dk * 4, *pwk = J->pw_k + (size_t)item * dk * 4;
    double *pwv = J->pw_v + (size_t)item * dv * 4, *pdtb = J->pdtb + (size_t)item * dk;
    if (L <= 0) {
        if (dST) memcpy(dS0, dST, sizeof(double) * SZ); else memset(dS0, 0, sizeof(double) * SZ);
        memset(pwq, 0, sizeof(double) * dk * 4); memset(pwk, 0, sizeof(double) * dk * 4);
        memset(pwv, 0, sizeof(double) * dv * 4); memset(pdtb, 0, sizeof(double) * dk);
        J->pAlog[item] = 0.0;
        if (J->dconv_in) {
            /* an empty sequence passes its history through untouched: no gradient */
            for (int m = 0; m < 3; ++m) {
                double *row = J->dconv_in + ((size_t)n * 3 + m) * Ctot;
                for (int i = 0; i < dk; ++i) { row[h * dk + i] = 0.0; row[H * dk + h * dk + i] = 0.0; }
                for (int i = 0; i < dv; ++i) row[2 * H * dk + h * dv + i] = 0.0;
            }
        }
        return;
    }
    double *qh = (double *)malloc(sizeof(double) * (size_t)L * dk);
    double *kh = (double *)malloc(sizeof(double) * (size_t)L * dk);
    double *vh = (double *)malloc(sizeof(double) * (size_t)L * dv);
    double *g = (double *)malloc(sizeof(double) * (size_t)L * dk);
    double *be = (double *)malloc(sizeof(double) * (size_t)L);
    double *dqh = (double *)malloc(sizeof(double) * (size_t)L * dk);
    double *dkh = (double *)malloc(sizeof(double) * (size_t)L * dk);
    double *dvh = (double *)malloc(sizeof(double) * (size_t)L * dv);
    double *dg = (double *)malloc(sizeof(double) * (size_t)L * dk);
    double *dbe = (double *)malloc(sizeof(double) * (size_t)L);
    const double *cin = J->conv_in ? J->conv_in + (size_t)n * 3 * Ctot : NULL;
    kda_oracle_preprocess_head(L, H, dk, dv, h, J->q + (size_t)t0 * H * dk, J->k + (size_t)t0 * H * dk,
                               J->v + (size_t)t0 * H * dv, J->alpha + (size_t)t0 * H * dk, J->b + (size_t)t0 * H,
                               J->w_q, J->w_k, J->w_v, J->A_log, J->dt_bias, cin, J->scale, J->lb, J->eps, J->flags,
                               qh, kh, vh, g, be);
    kda_oracle_recurrence_bwd(L, dk, dv, qh, kh, vh, g, be, S0, J->dO + ((size_t)t0 * H + h) * dv, (long)H * dv, dST,
                              dqh, dkh, dvh, dg, dbe, dS0);
    /* this head's columns of the raw gradients; the history gradient goes to a
     * per-item buffer first, then into its channels */
    double *dci = J->dconv_in ? (double *)calloc((size_t)3 * Ctot, sizeof(double)) : NULL;
    kda_oracle_preprocess_bwd_head(L, H, dk, dv, h, J->q + (size_t)t0 * H * dk, J->k + (size_t)t0 * H * dk,
                                   J->v + (size_t)t0 * H * dv, J->alpha + (size_t)t0 * H * dk, J->b + (size_t)t0 * H,
                                   J->w_q, J->w_k, J->w_v, J->A_log, J->dt_bias, cin, J->scale, J->lb, J->eps,
                                   J->flags, dqh, dkh, dvh, dg, dbe,
                                   J->dq + (size_t)t0 * H * dk, J->dk_ + (size_t)t0 * H * dk,
                                   J->dv_ + (size_t)t0 * H * dv, J->dalpha + (size_t)t0 * H * dk,
                                   J->db + (size_t)t0 * H, dci, pwq, pwk, pwv, pdtb, &J->pAlog[item]);
    if (dci) {
        for (int m = 0; m < 3; ++m) {
            double *row = J->dconv_in + ((size_t)n * 3 + m) * Ctot;
            const double *src = dci + (size_t)m * Ctot;
            for (int i = 0; i < dk; ++i) {
                row[h * dk + i] = src[h * dk + i];
                row[H * dk + h * dk + i] = src[H * dk + h * dk + i];
            }
            for (int i = 0; i < dv; ++i) row[2 * H * dk + h * dv + i] = src[2 * H * dk + h * dv + i];
        }
        free(dci);
    }
    free(qh); free(kh); free(vh); free(g); free(be); free(dqh); free(dkh); free(dvh); free(dg); free(dbe);
}

static void *orb_worker(void *arg)
{
    orb_job_t *J = (orb_job_t *)arg;
    const int total = J->nseq * J->H;
    for (;;) {
        const int i = __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED);
        if (i >= total) break;
        orb_item(J, i);
    }
    return NULL;
}

/*
 * Gradient of a packed batch (layouts of kda_oracle_forward).  Inputs: the
 * forward's inputs, dO [total_T][H][dv] and dST [nseq][H][dk][dv] (or NULL).
 * Outputs: dq, dk [total_T][H*dk]; dv [total_T][H*dv]; dalpha
 * [total_T][H][dk]; db [total_T][H]; dS0 [nseq][H][dk][dv]; dconv_in
 * [nseq][3][Ctot] (or NULL); dw_q, dw_k [H*dk][4]; dw_v [H*dv][4]; ddt_bias
 * [H*dk]; dA_log [H].  The parameter gradients are sums over the sequences,
 * added in sequence order.  Returns the number of threads used.
 */
int kda_oracle_backward(int nseq, const int64_t *cu, int H, int dk, int dv,
                        const double *q, const double *k, const double *v, const double *alpha, const double *b,
                        const double *w_q, const double *w_k, const double *w_v,
                        const double *A_log, const double *dt_bias,
                        double scale, double lb, double eps, unsigned flags,
                        const double *S0, const double *conv_in, const double *dO, const double *dST,
                        double *dq, double *dk_, double *dv_, double *dalpha, double *db, double *dS0,
                        double *dconv_in, double *dw_q, double *dw_k, double *dw_v, double *ddt_bias,
                        double *dA_log, int nthreads)
{
    const int items = nseq * H;
    orb_job_t J;
    memset(&J, 0, sizeof(J));
    J.nseq = nseq; J.H = H; J.dk = dk; J.dv = dv; J.cu = cu;
    J.q = q; J.k = k; J.v = v; J.alpha = alpha; J.b = b; J.w_q = w_q; J.w_k = w_k; J.w_v = w_v;
    J.A_log = A_log; J.dt_bias = dt_bias; J.scale = scale; J.lb = lb; J.eps = eps; J.flags = flags;
    J.S0 = S0; J.conv_in = conv_in; J.dO = dO; J.dST = dST;
    J.dq = dq; J.dk_ = dk_; J.dv_ = dv_; J.dalpha = dalpha; J.db = db; J.dS0 = dS0; J.dconv_in = dconv_in;
    const int ni = items > 0 ? items : 1;
    J.pw_q = (double *)calloc((size_t)ni * dk * 4, sizeof(double));
    J.pw_k = (double *)calloc((size_t)ni * dk * 4, sizeof(double));
    J.pw_v = (double *)calloc((size_t)ni * dv * 4, sizeof(double));
    J.pdtb = (double *)calloc((size_t)ni * dk, sizeof(double));
    J.pAlog = (double *)calloc((size_t)ni, sizeof(double));
    J.next = 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > items) nthreads = items > 0 ? items : 1;
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, orb_worker, &J);
    orb_worker(&J);
    for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
    /* parameter gradients: sums over the sequences, in sequence order */
    memset(dw_q, 0, sizeof(double) * (size_t)H * dk * 4);
    memset(dw_k, 0, sizeof(double) * (size_t)H * dk * 4);
    memset(dw_v, 0, sizeof(double) * (size_t)H * dv * 4);
    memset(ddt_bias, 0, sizeof(double) * (size_t)H * dk);
    memset(dA_log, 0, sizeof(double) * (size_t)H);
    for (int n = 0; n < nseq; ++n)
        for (int h = 0; h < H; ++h) {
            const int it = n * H + h;
            for (int e = 0; e < dk * 4; ++e) {
                dw_q[(size_t)h * dk * 4 + e] += J.pw_q[(size_t)it * dk * 4 + e];
                dw_k[(size_t)h * dk * 4 + e] += J.pw_k[(size_t)it * dk * 4 + e];
            }
            for (int e = 0; e < dv * 4; ++e) dw_v[(size_t)h * dv * 4 + e] += J.pw_v[(size_t)it * dv * 4 + e];
            for (int e = 0; e < dk; ++e) ddt_bias[(size_t)h * dk + e] += J.pdtb[(size_t)it * dk + e];
            dA_log[h] += J.pAlog[it];
        }
    free(J.pw_q); free(J.pw_k); free(J.pw_v); free(J.pdtb); free(J.pAlog);
    return nthreads;
}
