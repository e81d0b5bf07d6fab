/*
 * StreamKL oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, deliberately slow, fp64 CPU implementation of what the fused
 * attention-KL primitive computes.  It materialises full score rows and both
 * softmaxes and reduces them in the plainest order; it shares no code, header,
 * table or helper with the HIP path under attention_kl_divergence_amd/.
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
 * load it.  The product path never calls it.
 *
 * Source of the definitions (cited by page title, section and equation):
 *  - "StreamKL: Fast and Memory-Efficient KL Divergence for Boosting Attention
 *    Distillation" (abstract): the quantity is the KL divergence between two
 *    attention distributions, teacher against student, reduced per query row.
 *  - "Lecture 05 - Where It All Lands ..." section 3.1 (the distillation
 *    objective): forward KL with the teacher p in the first slot,
 *    sum_v p(v) [log p(v) - log q(v)], softmax of logits divided by a
 *    temperature, natural logarithm (nats, section 6 "mean_kld in nats").
 *  - same lecture, section 1: H(p,q) = H(p) + D_KL(p||q) (used by the tests
 *    as an independent cross-check, not here).
 *
 * Readings taken where the pages are silent (each also listed with the design notes):
 *  - scores are s = tau * (q . k), tau applied in fp64 after the dot product;
 *  - causal alignment is bottom-right: key j is allowed for query i iff
 *    j <= i + (n_k - n_q); causal with n_q > n_k is rejected by the caller;
 *  - the reduced scalar is the plain sum over all B*H*N_Q rows;
 *  - gradients are for L = sum_r g_r * KL_r with respect to the student
 *    queries and keys (the teacher is a fixed target); the *_teacher and
 *    *_dqt / *_dkt functions give the same loss's gradients with respect to the
 *    teacher (first-argument) queries and keys;
 *  - oracle_vocab_fwd / oracle_vocab_bwd apply the same definition to rows of
 *    vocabulary logits (section 3.1 at temperature T, scale = 1/T); the T^2
 *    factor of section 3.3 is left to the caller.
 *
 * Layout: every tensor is contiguous [B][H][N][d] of fp64 values (bf16 and
 * fp32 inputs are passed already widened, which is exact); outputs are fp64.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_ROWBLOCK 32

/* Number of keys query row i may attend to. */
static int allowed_keys(int i, int n_q, int n_k, int causal)
{
    if (!causal)
        return n_k;
    int last = i + (n_k - n_q); /* largest allowed key index */
    int n = last + 1;
    if (n > n_k) n = n_k;
    if (n < 0) n = 0;
    return n;
}

/* s[j] = tau * sum_c q[c] * k[j][c], for j < n (the scaled score row). */
static void score_row(const double *q, const double *k, int d, int n, double tau, double *s)
{
    for (int j = 0; j < n; ++j) {
        double acc = 0.0;
        const double *kj = k + (size_t)j * d;
        for (int c = 0; c < d; ++c)
            acc += q[c] * kj[c];
        s[j] = tau * acc;
    }
}

/* log sum_j exp(s[j]) computed as M + log sum exp(s - M), M = max s. */
static double log_sum_exp(const double *s, int n)
{
    double m = -INFINITY;
    for (int j = 0; j < n; ++j)
        if (s[j] > m) m = s[j];
    double z = 0.0;
    for (int j = 0; j < n; ++j)
        z += exp(s[j] - m);
    return m + log(z);
}

/*
 * One query row: both score rows, both log-normalisers, and
 * KL = sum_j P_t[j] (log P_t[j] - log P_s[j]) with the logs taken in the log
 * domain (log P = s - LSE), so an underflowing student probability cannot turn
 * a finite divergence into +inf.  Terms with P_t[j] == 0 contribute 0.
 */
static void row_kl(const double *qt, const double *kt, const double *qs, const double *ks,
                   int dt, int ds, int n, double tau_t, double tau_s,
                   double *st, double *ss, double *kl, double *lse_t, double *lse_s)
{
    score_row(qt, kt, dt, n, tau_t, st);
    score_row(qs, ks, ds, n, tau_s, ss);
    double lt = log_sum_exp(st, n);
    double ls = log_sum_exp(ss, n);
    double acc = 0.0;
    for (int j = 0; j < n; ++j) {
        double logpt = st[j] - lt;
        double logps = ss[j] - ls;
        double pt = exp(logpt);
        if (pt != 0.0)
            acc += pt * (logpt - logps);
    }
    *kl = acc;
    *lse_t = lt;
    *lse_s = ls;
}

static size_t head_off(int b, int h, int H, int n, int d)
{
    return (((size_t)b * H + h) * n) * (size_t)d;
}

/*
 * Forward over every row.  kl_rows, lse_t, lse_s: [B][H][n_q].  kl_sum: the
 * Neumaier-compensated sum of kl_rows in (b, h, i) order.
 */
void oracle_fwd(const double *q_t, const double *k_t, const double *q_s, const double *k_s,
                int B, int H, int n_q, int n_k, int d_t, int d_s,
                double tau_t, double tau_s, int causal,
                double *kl_rows, double *lse_t, double *lse_s, double *kl_sum)
{
    long long rows = (long long)B * H * n_q;
#pragma omp parallel
    {
        double *st = (double *)malloc(sizeof(double) * (size_t)(n_k > 0 ? n_k : 1));
        double *ss = (double *)malloc(sizeof(double) * (size_t)(n_k > 0 ? n_k : 1));
#pragma omp for schedule(dynamic, 16)
        for (long long r = 0; r < rows; ++r) {
            int i = (int)(r % n_q);
            long long bh = r / n_q;
            int h = (int)(bh % H), b = (int)(bh / H);
            int n = allowed_keys(i, n_q, n_k, causal);
            const double *qt = q_t + head_off(b, h, H, n_q, d_t) + (size_t)i * d_t;
            const double *qs = q_s + head_off(b, h, H, n_q, d_s) + (size_t)i * d_s;
            const double *kt = k_t + head_off(b, h, H, n_k, d_t);
            const double *ks = k_s + head_off(b, h, H, n_k, d_s);
            row_kl(qt, kt, qs, ks, d_t, d_s, n, tau_t, tau_s, st, ss,
                   &kl_rows[r], &lse_t[r], &lse_s[r]);
        }
        free(st);
        free(ss);
    }
    if (kl_sum) {
        double s = 0.0, c = 0.0;
        for (long long r = 0; r < rows; ++r) {
            double x = kl_rows[r], t = s + x;
            if (fabs(s) >= fabs(x)) c += (s - t) + x;
            else c += (x - t) + s;
            s = t;
        }
        *kl_sum = s + c;
    }
}

/*
 * Forward for a chosen set of rows only (flat row index r = (b*H + h)*n_q + i).
 * Used to sample outputs at sizes where the full forward is too slow.
 */
void oracle_fwd_rows(const double *q_t, const double *k_t, const double *q_s, const double *k_s,
                     int B, int H, int n_q, int n_k, int d_t, int d_s,
                     double tau_t, double tau_s, int causal,
                     int n_rows, const int64_t *rows,
                     double *kl, double *lse_t, double *lse_s)
{
    (void)B;
#pragma omp parallel
    {
        double *st = (double *)malloc(sizeof(double) * (size_t)(n_k > 0 ? n_k : 1));
        double *ss = (double *)malloc(sizeof(double) * (size_t)(n_k > 0 ? n_k : 1));
#pragma omp for schedule(dynamic, 1)
        for (int t = 0; t < n_rows; ++t) {
            long long r = rows[t];
            int i = (int)(r % n_q);
            long long bh = r / n_q;
            int h = (int)(bh % H), b = (int)(bh / H);
            int n = allowed_keys(i, n_q, n_k, causal);
            const double *qt = q_t + head_off(b, h, H, n_q, d_t) + (size_t)i * d_t;
            const double *qs = q_s + head_off(b, h, H, n_q, d_s) + (size_t)i * d_s;
            const double *kt = k_t + head_off(b, h, H, n_k, d_t);
            const double *ks = k_s + head_off(b, h, H, n_k, d_s);
            row_kl(qt, kt, qs, ks, d_t, d_s, n, tau_t, tau_s, st, ss, &kl[t], &lse_t[t], &lse_s[t]);
        }
        free(st);
        free(ss);
    }
}

/*
 * dS row for query i of one head:  dS[j] = g * tau_s * (P_s[j] - P_t[j]) for
 * allowed j, 0 otherwise.  This is the derivative of g * KL_i with respect to
 * the student score s_s[j] = tau_s * q_s . k_s[j]:
 *   d/ds_s[j] of sum_k P_t[k] (log P_t[k] - log P_s[k])
 *     = - sum_k P_t[k] d log P_s[k] / d s_s[j] = - P_t[j] + P_s[j],
 * times tau_s for the chain rule through the scaled score.
 */
static void row_dS(const double *qt, const double *kt, const double *qs, const double *ks,
                   int dt, int ds, int n, int n_k, double tau_t, double tau_s, double g,
                   double *st, double *ss, double *dS)
{
    score_row(qt, kt, dt, n, tau_t, st);
    score_row(qs, ks, ds, n, tau_s, ss);
    double lt = log_sum_exp(st, n);
    double ls = log_sum_exp(ss, n);
    for (int j = 0; j < n; ++j) {
        double pt = exp(st[j] - lt);
        double ps = exp(ss[j] - ls);
        dS[j] = g * tau_s * (ps - pt);
    }
    for (int j = n; j < n_k; ++j)
        dS[j] = 0.0;
}

/*
 * Backward over every row: dq_s [B][H][n_q][d_s] and dk_s [B][H][n_k][d_s]
 * (fp64, overwritten) for L = sum_r g_r KL_r.  g_rows may be NULL, in which
 * case every row uses g_scalar.
 *   dq_s[i] = sum_j dS[i][j] k_s[j],   dk_s[j] = sum_i dS[i][j] q_s[i].
 * For each head the dS rows of a block of queries are materialised, then the
 * block's contribution is added to dk_s key by key.
 */
void oracle_bwd(const double *q_t, const double *k_t, const double *q_s, const double *k_s,
                int B, int H, int n_q, int n_k, int d_t, int d_s,
                double tau_t, double tau_s, int causal,
                const double *g_rows, double g_scalar,
                double *dq_s, double *dk_s)
{
    const int R = ORACLE_ROWBLOCK;
    double *dS = (double *)malloc(sizeof(double) * (size_t)R * (size_t)(n_k > 0 ? n_k : 1));
    memset(dk_s, 0, sizeof(double) * (size_t)B * H * n_k * d_s);
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            const double *kt = k_t + head_off(b, h, H, n_k, d_t);
            const double *ks = k_s + head_off(b, h, H, n_k, d_s);
            double *dkh = dk_s + head_off(b, h, H, n_k, d_s);
            for (int i0 = 0; i0 < n_q; i0 += R) {
                int nr = (n_q - i0 < R) ? (n_q - i0) : R;
#pragma omp parallel
                {
                    double *st = (double *)malloc(sizeof(double) * (size_t)(n_k > 0 ? n_k : 1));
                    double *ss = (double *)malloc(sizeof(double) * (size_t)(n_k > 0 ? n_k : 1));
#pragma omp for schedule(static, 1)
                    for (int t = 0; t < nr; ++t) {
                        int i = i0 + t;
                        long long r = ((long long)b * H + h) * n_q + i;
                        double g = g_rows ? g_rows[r] : g_scalar;
                        int n = allowed_keys(i, n_q, n_k, causal);
                        const double *qt = q_t + head_off(b, h, H, n_q, d_t) + (size_t)i * d_t;
                        const double *qs = q_s + head_off(b, h, H, n_q, d_s) + (size_t)i * d_s;
                        double *dSi = dS + (size_t)t * n_k;
                        row_dS(qt, kt, qs, ks, d_t, d_s, n, n_k, tau_t, tau_s, g, st, ss, dSi);
                        double *dqi = dq_s + head_off(b, h, H, n_q, d_s) + (size_t)i * d_s;
                        for (int c = 0; c < d_s; ++c) {
                            double acc = 0.0;
                            for (int j = 0; j < n_k; ++j)
                                acc += dSi[j] * ks[(size_t)j * d_s + c];
                            dqi[c] = acc;
                        }
                    }
                    free(st);
                    free(ss);
#pragma omp for schedule(static)
                    for (int j = 0; j < n_k; ++j)
                        for (int t = 0; t < nr; ++t) {
                            double w = dS[(size_t)t * n_k + j];
                            if (w == 0.0) continue;
                            const double *qs = q_s + head_off(b, h, H, n_q, d_s) + (size_t)(i0 + t) * d_s;
                            for (int c = 0; c < d_s; ++c)
                                dkh[(size_t)j * d_s + c] += w * qs[c];
                        }
                }
            }
        }
    free(dS);
}

/*
 * dq_s for a chosen set of rows only (flat row index as in oracle_fwd_rows).
 * dq: [n_rows][d_s].
 */
void oracle_dq_rows(const double *q_t, const double *k_t, const double *q_s, const double *k_s,
                    int B, int H, int n_q, int n_k, int d_t, int d_s,
                    double tau_t, double tau_s, int causal,
                    const double *g_rows, double g_scalar,
                    int n_rows, const int64_t *rows, double *dq)
{
    (void)B;
#pragma omp parallel
    {
        double *st = (double *)malloc(sizeof(double) * (size_t)(n_k > 0 ? n_k : 1));
        double *ss = (double *)malloc(sizeof(double) * (size_t)(n_k > 0 ? n_k : 1));
        double *dS = (double *)malloc(sizeof(double) * (size_t)(n_k > 0 ? n_k : 1));
#pragma omp for schedule(dynamic, 1)
        for (int t = 0; t < n_rows; ++t) {
            long long r = rows[t];
            int i = (int)(r % n_q);
            long long bh = r / n_q;
            int h = (int)(bh % H), b = (int)(bh / H);
            double g = g_rows ? g_rows[r] : g_scalar;
            int n = allowed_keys(i, n_q, n_k, causal);
            const double *qt = q_t + head_off(b, h, H, n_q, d_t) + (size_t)i * d_t;
            const double *qs = q_s + head_off(b, h, H, n_q, d_s) + (size_t)i * d_s;
            const double *kt = k_t + head_off(b, h, H, n_k, d_t);
            const double *ks = k_s + head_off(b, h, H, n_k, d_s);
            row_dS(qt, kt, qs, ks, d_t, d_s, n, n_k, tau_t, tau_s, g, st, ss, dS);
            for (int c = 0; c < d_s; ++c) {
                double acc = 0.0;
                for (int j = 0; j < n_k; ++j)
                    acc += dS[j] * ks[(size_t)j * d_s + c];
                dq[(size_t)t * d_s + c] = acc;
            }
        }
        free(st);
        free(ss);
        free(dS);
    }
}

/*
 * dk_s for chosen keys of ONE head (b, h): dk[t][c] = sum_i dS[i][key_t] q_s[i][c].
 * Every query row of the head is visited (its full score rows are needed for
 * its normalisers), so the cost is that of the head's forward.
 */
void oracle_dk_keys(const double *q_t, const double *k_t, const double *q_s, const double *k_s,
                    int B, int H, int n_q, int n_k, int d_t, int d_s,
                    double tau_t, double tau_s, int causal,
                    const double *g_rows, double g_scalar,
                    int b, int h, int n_keys, const int64_t *keys, double *dk)
{
    (void)B;
    const double *kt = k_t + head_off(b, h, H, n_k, d_t);
    const double *ks = k_s + head_off(b, h, H, n_k, d_s);
    memset(dk, 0, sizeof(double) * (size_t)n_keys * d_s);
#pragma omp parallel
    {
        double *st = (double *)malloc(sizeof(double) * (size_t)(n_k > 0 ? n_k : 1));
        double *ss = (double *)malloc(sizeof(double) * (size_t)(n_k > 0 ? n_k : 1));
        double *dS = (double *)malloc(sizeof(double) * (size_t)(n_k > 0 ? n_k : 1));
        double *part = (double *)calloc((size_t)n_keys * d_s, sizeof(double));
#pragma omp for schedule(dynamic, 4)
        for (int i = 0; i < n_q; ++i) {
            long long r = ((long long)b * H + h) * n_q + i;
            double g = g_rows ? g_rows[r] : g_scalar;
            int n = allowed_keys(i, n_q, n_k, causal);
            const double *qt = q_t + head_off(b, h, H, n_q, d_t) + (size_t)i * d_t;
            const double *qs = q_s + head_off(b, h, H, n_q, d_s) + (size_t)i * d_s;
            row_dS(qt, kt, qs, ks, d_t, d_s, n, n_k, tau_t, tau_s, g, st, ss, dS);
            for (int t = 0; t < n_keys; ++t) {
                double w = dS[keys[t]];
                if (w == 0.0) continue;
                for (int c = 0; c < d_s; ++c)
                    part[(size_t)t * d_s + c] += w * qs[c];
            }
        }
#pragma omp critical
        for (size_t x = 0; x < (size_t)n_keys * d_s; ++x)
            dk[x] += part[x];
        free(st);
        free(ss);
        free(dS);
        free(part);
    }
}

/*
 * Gradients with respect to the FIRST (teacher) distribution.
 *
 * dS_t row for query i of one head:
 *   dS_t[j] = g * tau_t * P_t[j] * (log P_t[j] - log P_s[j] - KL_i)
 * for allowed j, 0 otherwise.  This is the derivative of g * KL_i with respect
 * to the teacher score s_t[j] = tau_t * q_t . k_t[j].  Writing
 * L[k] = log P_t[k] - log P_s[k] and dP_t[k]/ds_t[j] = P_t[k] (delta_kj - P_t[j]):
 *   d/ds_t[j] sum_k P_t[k] L[k]
 *     = sum_k P_t[k] (delta_kj - P_t[j]) L[k] + sum_k P_t[k] dL[k]/ds_t[j]
 *     = P_t[j] (L[j] - KL_i) + sum_k P_t[k] (delta_kj - P_t[j])
 *     = P_t[j] (L[j] - KL_i) + 0.
 * Swapping the two distributions (student first) gives the student gradient of
 * the reverse divergence KL(P_s || P_t) with the same formula.
 */
static void row_dS_teacher(const double *qt, const double *kt, const double *qs, const double *ks,
                           int dt, int ds, int n, int n_k, double tau_t, double tau_s, double g,
                           double *st, double *ss, double *dS)
{
    score_row(qt, kt, dt, n, tau_t, st);
    score_row(qs, ks, ds, n, tau_s, ss);
    double lt = log_sum_exp(st, n);
    double ls = log_sum_exp(ss, n);
    double kl = 0.0;
    for (int j = 0; j < n; ++j) {
        double logpt = st[j] - lt;
        double logps = ss[j] - ls;
        double pt = exp(logpt);
        if (pt != 0.0)
            kl += pt * (logpt - logps);
    }
    for (int j = 0; j < n; ++j) {
        double logpt = st[j] - lt;
        double logps = ss[j] - ls;
        double pt = exp(logpt);
        dS[j] = pt != 0.0 ? g * tau_t * pt * (logpt - logps - kl) : 0.0;
    }
    for (int j = n; j < n_k; ++j)
        dS[j] = 0.0;
}

/*
 * Teacher backward over every row: dq_t [B][H][n_q][d_t] and dk_t [B][H][n_k][d_t]
 * (fp64, overwritten) for L = sum_r g_r KL_r:
 *   dq_t[i] = sum_j dS_t[i][j] k_t[j],   dk_t[j] = sum_i dS_t[i][j] q_t[i].
 */
void oracle_bwd_teacher(const double *q_t, const double *k_t, const double *q_s, const double *k_s,
                        int B, int H, int n_q, int n_k, int d_t, int d_s,
                        double tau_t, double tau_s, int causal,
                        const double *g_rows, double g_scalar,
                        double *dq_t, double *dk_t)
{
    const int R = ORACLE_ROWBLOCK;
    double *dS = (double *)malloc(sizeof(double) * (size_t)R * (size_t)(n_k > 0 ? n_k : 1));
    memset(dk_t, 0, sizeof(double) * (size_t)B * H * n_k * d_t);
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            const double *kt = k_t + head_off(b, h, H, n_k, d_t);
            const double *ks = k_s + head_off(b, h, H, n_k, d_s);
            double *dkh = dk_t + head_off(b, h, H, n_k, d_t);
            for (int i0 = 0; i0 < n_q; i0 += R) {
                int nr = (n_q - i0 < R) ? (n_q - i0) : R;
#pragma omp parallel
                {
                    double *st = (double *)malloc(sizeof(double) * (size_t)(n_k > 0 ? n_k : 1));
                    double *ss = (double *)malloc(sizeof(double) * (size_t)(n_k > 0 ? n_k : 1));
#pragma omp for schedule(static, 1)
                    for (int t = 0; t < nr; ++t) {
                        int i = i0 + t;
                        long long r = ((long long)b * H + h) * n_q + i;
                        double g = g_rows ? g_rows[r] : g_scalar;
                        int n = allowed_keys(i, n_q, n_k, causal);
                        const double *qt = q_t + head_off(b, h, H, n_q, d_t) + (size_t)i * d_t;
                        const double *qs = q_s + head_off(b, h, H, n_q, d_s) + (size_t)i * d_s;
                        double *dSi = dS + (size_t)t * n_k;
                        row_dS_teacher(qt, kt, qs, ks, d_t, d_s, n, n_k, tau_t, tau_s, g, st, ss, dSi);
                        double *dqi = dq_t + head_off(b, h, H, n_q, d_t) + (size_t)i * d_t;
                        for (int c = 0; c < d_t; ++c) {
                            double acc = 0.0;
                            for (int j = 0; j < n_k; ++j)
                                acc += dSi[j] * kt[(size_t)j * d_t + c];
                            dqi[c] = acc;
                        }
                    }
                    free(st);
                    free(ss);
#pragma omp for schedule(static)
                    for (int j = 0; j < n_k; ++j)
                        for (int t = 0; t < nr; ++t) {
                            double w = dS[(size_t)t * n_k + j];
                            if (w == 0.0) continue;
                            const double *qt = q_t + head_off(b, h, H, n_q, d_t) + (size_t)(i0 + t) * d_t;
                            for (int c = 0; c < d_t; ++c)
                                dkh[(size_t)j * d_t + c] += w * qt[c];
                        }
                }
            }
        }
    free(dS);
}

/* dq_t for a chosen set of rows only (flat row index as in oracle_fwd_rows); dq: [n_rows][d_t]. */
void oracle_dqt_rows(const double *q_t, const double *k_t, const double *q_s, const double *k_s,
                     int B, int H, int n_q, int n_k, int d_t, int d_s,
                     double tau_t, double tau_s, int causal,
                     const double *g_rows, double g_scalar,
                     int n_rows, const int64_t *rows, double *dq)
{
    (void)B;
#pragma omp parallel
    {
        double *st = (double *)malloc(sizeof(double) * (size_t)(n_k > 0 ? n_k : 1));
        double *ss = (double *)malloc(sizeof(double) * (size_t)(n_k > 0 ? n_k : 1));
        double *dS = (double *)malloc(sizeof(double) * (size_t)(n_k > 0 ? n_k : 1));
#pragma omp for schedule(dynamic, 1)
        for (int t = 0; t < n_rows; ++t) {
            long long r = rows[t];
            int i = (int)(r % n_q);
            long long bh = r / n_q;
            int h = (int)(bh % H), b = (int)(bh / H);
            double g = g_rows ? g_rows[r] : g_scalar;
            int n = allowed_keys(i, n_q, n_k, causal);
            const double *qt = q_t + head_off(b, h, H, n_q, d_t) + (size_t)i * d_t;
            const double *qs = q_s + head_off(b, h, H, n_q, d_s) + (size_t)i * d_s;
            const double *kt = k_t + head_off(b, h, H, n_k, d_t);
            const double *ks = k_s + head_off(b, h, H, n_k, d_s);
            row_dS_teacher(qt, kt, qs, ks, d_t, d_s, n, n_k, tau_t, tau_s, g, st, ss, dS);
            for (int c = 0; c < d_t; ++c) {
                double acc = 0.0;
                for (int j = 0; j < n_k; ++j)
                    acc += dS[j] * kt[(size_t)j * d_t + c];
                dq[(size_t)t * d_t + c] = acc;
            }
        }
        free(st);
        free(ss);
        free(dS);
    }
}

/* dk_t for chosen keys of ONE head (b, h): dk[t][c] = sum_i dS_t[i][key_t] q_t[i][c]. */
void oracle_dkt_keys(const double *q_t, const double *k_t, const double *q_s, const double *k_s,
                     int B, int H, int n_q, int n_k, int d_t, int d_s,
                     double tau_t, double tau_s, int causal,
                     const double *g_rows, double g_scalar,
                     int b, int h, int n_keys, const int64_t *keys, double *dk)
{
    (void)B;
    const double *kt = k_t + head_off(b, h, H, n_k, d_t);
    const double *ks = k_s + head_off(b, h, H, n_k, d_s);
    memset(dk, 0, sizeof(double) * (size_t)n_keys * d_t);
#pragma omp parallel
    {
        double *st = (double *)malloc(sizeof(double) * (size_t)(n_k > 0 ? n_k : 1));
        double *ss = (double *)malloc(sizeof(double) * (size_t)(n_k > 0 ? n_k : 1));
        double *dS = (double *)malloc(sizeof(double) * (size_t)(n_k > 0 ? n_k : 1));
        double *part = (double *)calloc((size_t)n_keys * d_t, sizeof(double));
#pragma omp for schedule(dynamic, 4)
        for (int i = 0; i < n_q; ++i) {
            long long r = ((long long)b * H + h) * n_q + i;
            double g = g_rows ? g_rows[r] : g_scalar;
            int n = allowed_keys(i, n_q, n_k, causal);
            const double *qt = q_t + head_off(b, h, H, n_q, d_t) + (size_t)i * d_t;
            const double *qs = q_s + head_off(b, h, H, n_q, d_s) + (size_t)i * d_s;
            row_dS_teacher(qt, kt, qs, ks, d_t, d_s, n, n_k, tau_t, tau_s, g, st, ss, dS);
            for (int t = 0; t < n_keys; ++t) {
                double w = dS[keys[t]];
                if (w == 0.0) continue;
                for (int c = 0; c < d_t; ++c)
                    part[(size_t)t * d_t + c] += w * qt[c];
            }
        }
#pragma omp critical
        for (size_t x = 0; x < (size_t)n_keys * d_t; ++x)
            dk[x] += part[x];
        free(st);
        free(ss);
        free(dS);
        free(part);
    }
}

/*
 * Vocabulary-logit KL ("Lecture 05 - Where It All Lands", section 3.1: the
 * distillation loss at temperature T between the teacher and student output
 * distributions over the vocabulary; section 3.3: any T^2 factor is the
 * caller's).  Per row r of zt, zs ([rows][V]):
 *   p = softmax(scale * zt[r]),  q = softmax(scale * zs[r]),  scale = 1 / T
 *   KL_r = sum_v p[v] (log p[v] - log q[v])   (log domain, as row_kl)
 * kl_sum: Neumaier-compensated sum of the rows.
 */
void oracle_vocab_fwd(const double *zt, const double *zs, int rows, int V, double scale,
                      double *kl_rows, double *lse_t, double *lse_s, double *kl_sum)
{
#pragma omp parallel
    {
        double *st = (double *)malloc(sizeof(double) * (size_t)V);
        double *ss = (double *)malloc(sizeof(double) * (size_t)V);
#pragma omp for schedule(dynamic, 4)
        for (int r = 0; r < rows; ++r) {
            for (int v = 0; v < V; ++v) {
                st[v] = scale * zt[(size_t)r * V + v];
                ss[v] = scale * zs[(size_t)r * V + v];
            }
            double lt = log_sum_exp(st, V), ls = log_sum_exp(ss, V), acc = 0.0;
            for (int v = 0; v < V; ++v) {
                double lp = st[v] - lt, lq = ss[v] - ls, p = exp(lp);
                if (p != 0.0)
                    acc += p * (lp - lq);
            }
            kl_rows[r] = acc;
            lse_t[r] = lt;
            lse_s[r] = ls;
        }
        free(st);
        free(ss);
    }
    double s = 0.0, c = 0.0;
    for (int r = 0; r < rows; ++r) {
        double x = kl_rows[r], t = s + x;
        if (fabs(s) >= fabs(x)) c += (s - t) + x;
        else c += (x - t) + s;
        s = t;
    }
    *kl_sum = s + c;
}

/*
 * Gradients of L = sum_r g_r KL_r with respect to the logits:
 *   dzs[r][v] = g_r * scale * (q[v] - p[v])
 *   dzt[r][v] = g_r * scale * p[v] (log p[v] - log q[v] - KL_r)   (if dzt != NULL)
 * (the derivations of row_dS and row_dS_teacher with s = scale * z).
 */
void oracle_vocab_bwd(const double *zt, const double *zs, int rows, int V, double scale,
                      const double *g_rows, double g_scalar, double *dzs, double *dzt)
{
#pragma omp parallel
    {
        double *st = (double *)malloc(sizeof(double) * (size_t)V);
        double *ss = (double *)malloc(sizeof(double) * (size_t)V);
#pragma omp for schedule(dynamic, 4)
        for (int r = 0; r < rows; ++r) {
            double g = g_rows ? g_rows[r] : g_scalar;
            for (int v = 0; v < V; ++v) {
                st[v] = scale * zt[(size_t)r * V + v];
                ss[v] = scale * zs[(size_t)r * V + v];
            }
            double lt = log_sum_exp(st, V), ls = log_sum_exp(ss, V), kl = 0.0;
            for (int v = 0; v < V; ++v) {
                double lp = st[v] - lt, lq = ss[v] - ls, p = exp(lp);
                if (p != 0.0)
                    kl += p * (lp - lq);
            }
            for (int v = 0; v < V; ++v) {
                double lp = st[v] - lt, lq = ss[v] - ls, p = exp(lp), q = exp(lq);
                dzs[(size_t)r * V + v] = g * scale * (q - p);
                if (dzt)
                    dzt[(size_t)r * V + v] = p != 0.0 ? g * scale * p * (lp - lq - kl) : 0.0;
            }
        }
        free(st);
        free(ss);
    }
}

/* Number of OpenMP threads the functions above run with (for reporting). */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
}
