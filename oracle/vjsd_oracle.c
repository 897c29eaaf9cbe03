/*
 * vjsd_oracle.c -- TEST INFRASTRUCTURE ONLY: the fp64 CPU oracle.
 *
 * A plain, slow, definition-level evaluation of what the GPU library computes:
 * per-token softmax statistics over a vocabulary split into ordered shards, the
 * generalized Jensen-Shannon divergence with its two KL endpoints, entropy and
 * log-probabilities, each with its gradient.  It shares no code, header or
 * constant with the GPU path.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the product never does.
 *
 * Page keys used in the citations below:
 *   [JSD-PR]  DeepSpeed PR #8958, "[VocabTP] Add vocabulary-parallel generalized
 *             JSD with Triton kernels".
 *   [OPS-PR]  DeepSpeed PR #8791, "Add vocabulary-parallel logprobs, entropy and
 *             KL ops", and its review thread.
 *
 * Conventions.
 *   Inputs are row-major matrices of fp32, fp16 or bf16 values, widened exactly to
 *   double, or of doubles (logits a caller has already transformed in fp64, such as
 *   logits divided by a distillation temperature).  Row r, column j of an input lives at element r*ld + j.  The vocabulary
 *   [0, V) is split into S consecutive shards of the given widths (a width may be
 *   0).  Only the rows listed in rows[0..nr) are evaluated; every output is packed
 *   by position in that list, so a caller can check single rows of a huge matrix.
 *   Gradient outputs have nr*V entries; a NULL output pointer skips that output.
 *   Rows are independent and are spread over OpenMP threads.
 *
 * Readings of the pages (where they leave a step open):
 *   - The JSD is the generalized JSD of GKD-style distillation [JSD-PR, Motivation]
 *     written as two KL-to-mixture expectations [JSD-PR, Changes]:
 *       M = beta*p_t + (1-beta)*p_s,
 *       loss = beta*KL(p_t||M) + (1-beta)*KL(p_s||M)   for 0 < beta < 1,
 *     natural logarithms.  beta = 0 is forward KL(p_t||p_s) and beta = 1 is reverse
 *     KL(p_s||p_t), as exact branches, not limits [JSD-PR, Changes].
 *   - A token whose log-probability is -inf contributes nothing; a row that is
 *     -inf everywhere (in either input of a two-input op) has no distribution: its
 *     value is NaN and every gradient in it is exactly 0 [OPS-PR, How; review].
 *   - KL is +inf when the target puts mass on a token the other side masked, decided
 *     on the logits, so it holds even when that mass underflows [OPS-PR, Tests].
 *   - An empty or fully masked shard joins the merge as (max, sum-exp) = (-inf, 0)
 *     [OPS-PR, review: empty shards].
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2, OR_F64 = 3 };

/* ---- exact widening of the stored input formats ------------------------------- */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double half_bits_to_double(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);               /* zero and subnormals */
    else if (e == 0x1f)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f | 0x400), e - 25);  /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
static double bf16_bits_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double elem(const void *x, int dt, int64_t i)
{
    if (dt == OR_F64)
        return ((const double *)x)[i];
    if (dt == OR_F32)
        return (double)((const float *)x)[i];
    if (dt == OR_F16)
        return half_bits_to_double(((const uint16_t *)x)[i]);
    return bf16_bits_to_double(((const uint16_t *)x)[i]);
}

/* ---- softmax statistics [OPS-PR, How] ------------------------------------------ */

/* One shard's statistics: m = max_j x_j and Z = sum_j exp(x_j - m) over the
 * shard's columns; an empty or fully -inf shard gives (-inf, 0). */
static void shard_stats(const void *x, int dt, int64_t row_off, int64_t c0, int64_t c1,
                        double *m_out, double *Z_out)
{
    double m = -INFINITY, Z = 0.0;
    for (int64_t j = c0; j < c1; ++j) {
        double v = elem(x, dt, row_off + j);
        if (v > m)
            m = v;
    }
    if (m > -INFINITY)
        for (int64_t j = c0; j < c1; ++j) {
            double v = elem(x, dt, row_off + j);
            if (v > -INFINITY)
                Z += exp(v - m);
        }
    *m_out = m;
    *Z_out = Z;
}

/* Row statistics as the cross-shard merge computes them: the global max is the max
 * of the shard maxima, and each shard's sum-exp is rescaled to it before summing;
 * shards with m_k = -inf add nothing.  The global max and the log-sum-exp are kept
 * apart (lnZ = ln Z, not m + ln Z), so a large common offset costs no precision. */
static void row_stats(const void *x, int dt, int64_t row_off, const int64_t *widths, int S,
                      double *m_out, double *lnZ_out)
{
    double mk[S > 0 ? S : 1], Zk[S > 0 ? S : 1];
    int64_t c = 0;
    double m = -INFINITY;
    for (int k = 0; k < S; ++k) {
        shard_stats(x, dt, row_off, c, c + widths[k], &mk[k], &Zk[k]);
        c += widths[k];
        if (mk[k] > m)
            m = mk[k];
    }
    double Z = 0.0;
    if (m > -INFINITY)
        for (int k = 0; k < S; ++k)
            if (mk[k] > -INFINITY)
                Z += Zk[k] * exp(mk[k] - m);
    *m_out = m;
    *lnZ_out = log(Z); /* -inf for an undefined row */
}

/* log-probability of value v under statistics (m, lnZ), in the order the pages
 * prescribe: shift by the max first, then subtract the log-sum-exp. */
static double logprob(double v, double m, double lnZ)
{
    return (v - m) - lnZ;
}

/* ln(exp(a) + exp(b)) without overflow; -inf only when both are -inf. */
static double logaddexp(double a, double b)
{
    if (a == -INFINITY && b == -INFINITY)
        return -INFINITY;
    double hi = a > b ? a : b, lo = a > b ? b : a;
    return hi + log1p(exp(lo - hi));
}

void or_stats(const void *x, int dt, int64_t ld, int64_t V, const int64_t *widths, int S,
              const int64_t *rows, int64_t nr, double *m, double *lnZ)
{
    (void)V;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < nr; ++q)
        row_stats(x, dt, rows[q] * ld, widths, S, &m[q], &lnZ[q]);
}

/* ---- generalized JSD and its KL endpoints [JSD-PR, Changes] --------------------- */

/*
 * Per row, with lp_x = log-probabilities and p_x = exp(lp_x):
 *   interior 0 < beta < 1:
 *     lM_j = logaddexp(ln beta + lp_t,j, ln(1-beta) + lp_s,j)
 *     KT = sum_{t_j > -inf} p_t,j (lp_t,j - lM_j)      = KL(p_t || M)
 *     KS = sum_{s_j > -inf} p_s,j (lp_s,j - lM_j)      = KL(p_s || M)
 *     loss = beta KT + (1 - beta) KS
 *     d/ds_j = g (1-beta) p_s,j (lp_s,j - lM_j - KS),  d/dt_j = g beta p_t,j (lp_t,j - lM_j - KT)
 *   beta = 0:  M = p_s, so KT = KL(p_t || p_s) is the loss and KS = 0;
 *     d/ds_j = g (p_s,j - p_t,j),  d/dt_j = g p_t,j (lp_t,j - lp_s,j - KT)
 *   beta = 1:  M = p_t, so KS = KL(p_s || p_t) is the loss and KT = 0;
 *     d/ds_j = g p_s,j (lp_s,j - lp_t,j - KS),  d/dt_j = g (p_t,j - p_s,j)
 * The gradients follow from dJ/dp_s,j = (1-beta)(lp_s,j - lM_j) and the softmax
 * Jacobian p_j (delta_ij - p_i); a term whose own logit is -inf is exactly 0.
 * The per-token value is reduced per shard and the shard partials are summed in
 * shard order, as the cross-shard SUM of the pages does [JSD-PR, Changes].
 */
static void jsd_row(const void *s, const void *t, int dt, int64_t off, int64_t V,
                    const int64_t *widths, int S, double beta, double g,
                    double *loss, double *kt_out, double *ks_out, double *gs, double *gt)
{
    double ms, lzs, mt, lzt;
    row_stats(s, dt, off, widths, S, &ms, &lzs);
    row_stats(t, dt, off, widths, S, &mt, &lzt);

    if (ms == -INFINITY || mt == -INFINITY) { /* undefined row */
        *loss = NAN;
        *kt_out = NAN;
        *ks_out = NAN;
        for (int64_t j = 0; j < V; ++j) {
            if (gs) gs[j] = 0.0;
            if (gt) gt[j] = 0.0;
        }
        return;
    }

    const int fwd_kl = (beta == 0.0), rev_kl = (beta == 1.0);
    const double lnb = log(beta), ln1mb = log1p(-beta);
    double KT = 0.0, KS = 0.0;
    int infinite = 0;
    int64_t c = 0;
    for (int k = 0; k < S; ++k) {
        double pKT = 0.0, pKS = 0.0; /* this shard's partials */
        for (int64_t j = c; j < c + widths[k]; ++j) {
            double sv = elem(s, dt, off + j), tv = elem(t, dt, off + j);
            double lps = logprob(sv, ms, lzs), lpt = logprob(tv, mt, lzt);
            if (fwd_kl) {
                if (tv > -INFINITY) {
                    if (sv == -INFINITY)
                        infinite = 1;
                    else
                        pKT += exp(lpt) * (lpt - lps);
                }
            } else if (rev_kl) {
                if (sv > -INFINITY) {
                    if (tv == -INFINITY)
                        infinite = 1;
                    else
                        pKS += exp(lps) * (lps - lpt);
                }
            } else {
                double lM = logaddexp(lnb + lpt, ln1mb + lps);
                if (tv > -INFINITY)
                    pKT += exp(lpt) * (lpt - lM);
                if (sv > -INFINITY)
                    pKS += exp(lps) * (lps - lM);
            }
        }
        KT += pKT;
        KS += pKS;
        c += widths[k];
    }
    if (fwd_kl) {
        if (infinite) KT = INFINITY;
        *loss = KT;
    } else if (rev_kl) {
        if (infinite) KS = INFINITY;
        *loss = KS;
    } else {
        *loss = beta * KT + (1.0 - beta) * KS;
    }
    *kt_out = KT;
    *ks_out = KS;

    if (!gs && !gt)
        return;
    for (int64_t j = 0; j < V; ++j) {
        double sv = elem(s, dt, off + j), tv = elem(t, dt, off + j);
        double lps = logprob(sv, ms, lzs), lpt = logprob(tv, mt, lzt);
        double ps = exp(lps), pt = exp(lpt);
        double dsj, dtj;
        if (fwd_kl) {
            dsj = g * (ps - pt);
            dtj = tv > -INFINITY ? g * pt * (lpt - lps - KT) : 0.0;
        } else if (rev_kl) {
            dsj = sv > -INFINITY ? g * ps * (lps - lpt - KS) : 0.0;
            dtj = g * (pt - ps);
        } else {
            double lM = logaddexp(lnb + lpt, ln1mb + lps);
            dsj = sv > -INFINITY ? g * (1.0 - beta) * ps * (lps - lM - KS) : 0.0;
            dtj = tv > -INFINITY ? g * beta * pt * (lpt - lM - KT) : 0.0;
        }
        if (gs) gs[j] = dsj;
        if (gt) gt[j] = dtj;
    }
}

void or_jsd(const void *s, const void *t, int dt, int64_t ld, int64_t V,
            const int64_t *widths, int S, double beta, const int64_t *rows, int64_t nr,
            const double *gout, double *loss, double *kt, double *ks, double *gs, double *gt)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < nr; ++q) {
        double l, a, b;
        jsd_row(s, t, dt, rows[q] * ld, V, widths, S, beta, gout ? gout[q] : 1.0, &l, &a, &b,
                gs ? gs + q * V : NULL, gt ? gt + q * V : NULL);
        loss[q] = l;
        if (kt) kt[q] = a;
        if (ks) ks[q] = b;
    }
}

/* ---- entropy [OPS-PR, What] ---------------------------------------------------- */

/* H = -sum_{x_j > -inf} p_j lp_j;  dH/dx_j = -p_j (lp_j + H). */
static void entropy_row(const void *x, int dt, int64_t off, int64_t V, const int64_t *widths,
                        int S, double g, double *H_out, double *gx)
{
    double m, lz;
    row_stats(x, dt, off, widths, S, &m, &lz);
    if (m == -INFINITY) {
        *H_out = NAN;
        if (gx)
            for (int64_t j = 0; j < V; ++j) gx[j] = 0.0;
        return;
    }
    double H = 0.0;
    int64_t c = 0;
    for (int k = 0; k < S; ++k) {
        double part = 0.0;
        for (int64_t j = c; j < c + widths[k]; ++j) {
            double v = elem(x, dt, off + j);
            if (v > -INFINITY) {
                double lp = logprob(v, m, lz);
                part -= exp(lp) * lp;
            }
        }
        H += part;
        c += widths[k];
    }
    *H_out = H;
    if (gx)
        for (int64_t j = 0; j < V; ++j) {
            double v = elem(x, dt, off + j);
            if (v > -INFINITY) {
                double lp = logprob(v, m, lz);
                gx[j] = -g * exp(lp) * (lp + H);
            } else {
                gx[j] = 0.0;
            }
        }
}

void or_entropy(const void *x, int dt, int64_t ld, int64_t V, const int64_t *widths, int S,
                const int64_t *rows, int64_t nr, const double *gout, double *H, double *gx)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < nr; ++q)
        entropy_row(x, dt, rows[q] * ld, V, widths, S, gout ? gout[q] : 1.0, &H[q],
                    gx ? gx + q * V : NULL);
}

/* ---- per-id and top-k log-probabilities [OPS-PR, What / How] -------------------- */

/*
 * out_k = lp_{id_k}, or exactly 0 where id_k == ignore_index.  An id outside
 * [0, V) that is not ignore_index is an argument error (*err is set; the outputs of
 * that row are then unspecified).  d/dx_j = sum_{valid k} g_k [j == id_k]
 *   - (sum_{valid k} g_k) p_j; repeated ids accumulate.  An undefined row gives NaN
 * for its valid ids, 0 for ignored ones, and a zero gradient.
 */
static void logprobs_row(const void *x, int dt, int64_t off, int64_t V, const int64_t *widths,
                         int S, const int64_t *ids, int K, int64_t ignore_index,
                         const double *g, double *out, double *gx, int *err)
{
    double m, lz;
    row_stats(x, dt, off, widths, S, &m, &lz);
    int defined = m > -INFINITY;
    double G = 0.0;
    for (int k = 0; k < K; ++k) {
        int64_t id = ids[k];
        if (id == ignore_index) {
            out[k] = 0.0;
            continue;
        }
        if (id < 0 || id >= V) {
#pragma omp atomic write
            *err = 1;
            out[k] = NAN;
            continue;
        }
        out[k] = defined ? logprob(elem(x, dt, off + id), m, lz) : NAN;
        if (g)
            G += g[k];
    }
    if (!gx)
        return;
    for (int64_t j = 0; j < V; ++j)
        gx[j] = defined ? -G * exp(logprob(elem(x, dt, off + j), m, lz)) : 0.0;
    if (!defined)
        return;
    for (int k = 0; k < K; ++k) {
        int64_t id = ids[k];
        if (id != ignore_index && id >= 0 && id < V)
            gx[id] += g[k];
    }
}

void or_logprobs(const void *x, int dt, int64_t ld, int64_t V, const int64_t *widths, int S,
                 const int64_t *rows, int64_t nr, const int64_t *ids, int K,
                 int64_t ignore_index, const double *gout, double *out, double *gx, int *err)
{
    *err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < nr; ++q)
        logprobs_row(x, dt, rows[q] * ld, V, widths, S, ids + q * K, K, ignore_index,
                     gout ? gout + q * K : NULL, out + q * K, gx ? gx + q * V : NULL, err);
}

int or_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
