/*
 * spec_oracle.c -- plain fp64 CPU oracle for the batched draft-verification
 * sampler.  TEST INFRASTRUCTURE ONLY: it exists to check the HIP library and
 * is called from tests/, the smoke check and the benchmark's CPU-baseline
 * leg, never from the product path.  It shares no code, header, table or
 * helper with the HIP library.
 *
 * Everything here is a direct, slow transcription of the definitions:
 *
 *   per logit row l[0..V):  M = max_t l_t,   g = min{t : l_t = M},
 *                           S = sum_t exp(l_t - M),
 *                           log p(t) = (l_t - M) - log S
 *   (softmax at temperature 1; the rows are the verify-pass logits of
 *   mini-sglang PR #134 "Modifications" / spec-decode README "How it works").
 *
 * Rules:
 *   greedy   -- accept the matching prefix of the K drafts against the
 *               target's argmax rows, then append the argmax of the first
 *               unmatched row (the bonus) (mini-sglang PR #134,
 *               "Modifications", verify_drafts).
 *   exact    -- accept draft j with probability min(1, p/q), in order; on the
 *               first rejection emit a sample of normalize(relu(p - q)) and
 *               stop; if all K are accepted emit a sample of the last target
 *               row (spec-decode README, "How it works" flowchart and the
 *               paragraph under it).
 *   relaxed  -- accept iff p >= tau or the draft is in the target's top-k;
 *               deterministic, so the behaviour probability of an accepted
 *               draft is 1 (nanospec README, acceptance-rule paragraph).
 *   tree     -- greedy verification of a draft tree: a node is accepted when
 *               its token is the argmax of its parent's row and its parent is
 *               accepted; emit the deepest accepted root path plus the argmax
 *               of its last node (nanospec README, intro and benchmark
 *               section: EAGLE trees, output identical to greedy decoding).
 *
 * Conventions where the pages are silent (each also listed with the design
 * notes): u_j drives test j and u_K drives the terminal sample; accept iff
 * u < r (strict); inverse CDF in ascending vocabulary order, y = smallest t
 * whose inclusive prefix exceeds u*Z; argmax ties go to the lowest index;
 * top-k membership is rank based (#{t : l_t > l_x} < k); behaviour log-prob
 * of an accepted exact draft is min(0, log p - log q), of a residual sample
 * log(1 - r) + log w(y) - log Z, of a bonus or relaxed sample log p(y).
 *
 * Near-tie flags: a decision whose outcome could flip under rounding that is
 * far below the tolerances (|u - r| < eps_accept, |p - tau| < eps_accept when
 * the rank test fails, or u within eps_sample of a CDF boundary) is reported
 * so that the comparison can exempt that position and everything after it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#include "spec_oracle.h"

/* ---------------------------------------------------------------- loads */
static double ld(const void *base, int dtype, size_t i)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[i];
    /* bf16: the 16 stored bits are the top half of an fp32 pattern */
    uint32_t w = (uint32_t)((const uint16_t *)base)[i] << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------ row stats */
typedef struct {
    double M;   /* row max */
    long g;     /* lowest index of the max */
    double S;   /* sum_t exp(l_t - M) */
    double lnS; /* log S */
} row_stats;

static void stats(const void *base, int dt, size_t row, int V, row_stats *st)
{
    size_t off = row * (size_t)V;
    double M = -INFINITY;
    long g = 0;
    for (int t = 0; t < V; ++t) {
        double v = ld(base, dt, off + t);
        if (v > M) {
            M = v;
            g = t;
        }
    }
    double S = 0.0;
    if (M > -INFINITY)
        for (int t = 0; t < V; ++t)
            S += exp(ld(base, dt, off + t) - M);
    st->M = M;
    st->g = g;
    st->S = S;
    st->lnS = log(S);
}

static double logp(const void *base, int dt, size_t row, int V, long t, const row_stats *st)
{
    return (ld(base, dt, row * (size_t)V + t) - st->M) - st->lnS;
}

/* ----------------------------------------------------------- inverse CDF
 * y = min{t : sum_{t' <= t} w(t') > target}; tokens with w = 0 are never
 * chosen.  If rounding leaves no such t, the last t with w > 0 is taken.
 * lo/hi receive the cumulative mass just before and through y.            */
static long inverse_cdf(const double *w, int V, double target, double *lo, double *hi)
{
    double c = 0.0, prev = 0.0;
    long last = -1;
    double last_lo = 0.0;
    for (int t = 0; t < V; ++t) {
        if (!(w[t] > 0.0))
            continue;
        prev = c;
        c += w[t];
        last = t;
        last_lo = prev;
        if (c > target) {
            *lo = prev;
            *hi = c;
            return t;
        }
    }
    *lo = last_lo;
    *hi = c;
    return last;
}

static int sample_flag(double target, double lo, double hi, double Z, double eps)
{
    double d1 = (target - lo) / Z, d2 = (hi - target) / Z;
    double d = d1 < d2 ? d1 : d2;
    return d < eps;
}

/* fill the padding of one request's outputs */
static void pad_row(int32_t *tok, double *tlp, double *blp, int L)
{
    for (int i = 0; i < L; ++i) {
        tok[i] = -1;
        tlp[i] = 0.0;
        blp[i] = 0.0;
    }
}

/* ------------------------------------------------------ terminal weights
 * The weights each rule's terminal draw inverts (spec-decode README, "How it
 * works": after the first rejection n the sampler draws from
 * normalize(relu(p_n - q_n)); with every draft accepted, from the last target
 * row).  Returns Z = sum_t w[t].                                          */

/* exact rule: relu(p_n - q_n) when n < K and it has mass, else p_n */
static double exact_terminal(const void *T, const void *D, int dt, int b, int K, int V, int n,
                             const row_stats *sp, double *w, int *residual)
{
    const int L = K + 1;
    double Z = 0.0;
    *residual = 0;
    if (n < K) {
        row_stats sq;
        stats(D, dt, (size_t)b * K + n, V, &sq);
        for (int t = 0; t < V; ++t) {
            double p = exp(logp(T, dt, (size_t)b * L + n, V, t, sp));
            double q = exp(logp(D, dt, (size_t)b * K + n, V, t, &sq));
            double d = p - q;
            w[t] = d > 0.0 ? d : 0.0;
            Z += w[t];
        }
        *residual = Z > 0.0;
    }
    if (!*residual) { /* bonus (n == K) or a residual with no mass */
        Z = 0.0;
        for (int t = 0; t < V; ++t) {
            w[t] = exp(logp(T, dt, (size_t)b * L + n, V, t, sp));
            Z += w[t];
        }
    }
    return Z;
}

/* p over one target row: the relaxed and power rules' terminal draw */
static double target_terminal(const void *T, int dt, size_t row, int V, const row_stats *sp,
                              double *w)
{
    double Z = 0.0;
    for (int t = 0; t < V; ++t) {
        w[t] = exp(logp(T, dt, row, V, t, sp));
        Z += w[t];
    }
    return Z;
}

/* exp(l - M) over one row (unnormalized q): the draft sampler's weights */
static double sampler_weights(const void *X, int dt, size_t r, int V, const row_stats *sq,
                              double *w)
{
    double Z = 0.0;
    for (int t = 0; t < V; ++t) {
        w[t] = exp(ld(X, dt, r * (size_t)V + t) - sq->M);
        Z += w[t];
    }
    return Z;
}

/* --------------------------------------------------------------- threads */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------- row stats */
void oracle_row_stats(const void *x, int dtype, long rows, int V, double *M, int64_t *g, double *S)
{
#pragma omp parallel for schedule(dynamic)
    for (long r = 0; r < rows; ++r) {
        row_stats st;
        stats(x, dtype, (size_t)r, V, &st);
        M[r] = st.M;
        g[r] = st.g;
        S[r] = st.S;
    }
}

/* ---------------------------------------------------------------- greedy */
void oracle_greedy(const void *T, int dt, const int32_t *x, int B, int K, int V,
                   int32_t *out_tok, int32_t *out_len, double *out_tlp, double *out_blp,
                   int32_t *out_status, int32_t *out_decisions)
{
#pragma omp parallel for schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        const int L = K + 1;
        int32_t *tok = out_tok + (size_t)b * L;
        double *tlp = out_tlp + (size_t)b * L, *blp = out_blp + (size_t)b * L;
        pad_row(tok, tlp, blp, L);
        int status = 0, n = K, dec = 0;
        for (int j = 0; j < K; ++j) {
            int32_t xj = x[(size_t)b * K + j];
            row_stats st;
            stats(T, dt, (size_t)b * L + j, V, &st);
            ++dec;
            if (xj < 0 || xj >= V) {
                status = 1;
                n = j;
                break;
            }
            if (xj != st.g) {
                n = j;
                break;
            }
            tok[j] = xj;
            tlp[j] = logp(T, dt, (size_t)b * L + j, V, xj, &st);
        }
        row_stats sn;
        stats(T, dt, (size_t)b * L + n, V, &sn);
        tok[n] = (int32_t)sn.g;
        tlp[n] = logp(T, dt, (size_t)b * L + n, V, sn.g, &sn);
        out_len[b] = n;
        out_status[b] = status;
        out_decisions[b] = dec;
    }
}

/* ----------------------------------------------------------------- exact */
void oracle_exact(const void *T, const void *D, int dt, const int32_t *x, const float *u,
                  int B, int K, int V, double eps_accept, double eps_sample,
                  int32_t *out_tok, int32_t *out_len, double *out_tlp, double *out_blp,
                  int32_t *out_status, int32_t *out_flag, int32_t *out_decisions)
{
#pragma omp parallel for schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        const int L = K + 1;
        int32_t *tok = out_tok + (size_t)b * L;
        double *tlp = out_tlp + (size_t)b * L, *blp = out_blp + (size_t)b * L;
        pad_row(tok, tlp, blp, L);
        int status = 0, n = K, flag = -1, dec = 0;
        double rn = 0.0;
        for (int j = 0; j < K; ++j) {
            int32_t xj = x[(size_t)b * K + j];
            ++dec;
            if (xj < 0 || xj >= V) { /* malformed draft: rejected, no test */
                status = 1;
                n = j;
                rn = 0.0;
                break;
            }
            row_stats sp, sq;
            stats(T, dt, (size_t)b * L + j, V, &sp);
            stats(D, dt, (size_t)b * K + j, V, &sq);
            double lp = logp(T, dt, (size_t)b * L + j, V, xj, &sp);
            double lq = logp(D, dt, (size_t)b * K + j, V, xj, &sq);
            double r;
            if (lp == -INFINITY)
                r = 0.0;
            else if (lq == -INFINITY)
                r = INFINITY;
            else
                r = exp(lp - lq);
            double uj = (double)u[(size_t)b * L + j];
            if (flag < 0 && fabs(uj - r) < eps_accept)
                flag = j;
            if (uj < r) {
                tok[j] = xj;
                tlp[j] = lp;
                blp[j] = (lp - lq) < 0.0 ? (lp - lq) : 0.0;
            } else {
                n = j;
                rn = r;
                break;
            }
        }
        /* terminal sample with u_K */
        double uK = (double)u[(size_t)b * L + K];
        double *w = (double *)malloc(sizeof(double) * (size_t)V);
        row_stats sp;
        stats(T, dt, (size_t)b * L + n, V, &sp);
        int residual;
        double Z = exact_terminal(T, D, dt, b, K, V, n, &sp, w, &residual);
        double lo, hi, target = uK * Z;
        long y = inverse_cdf(w, V, target, &lo, &hi);
        ++dec;
        if (flag < 0 && sample_flag(target, lo, hi, Z, eps_sample))
            flag = n;
        tok[n] = (int32_t)y;
        tlp[n] = logp(T, dt, (size_t)b * L + n, V, y, &sp);
        if (residual)
            blp[n] = log1p(-rn) + log(w[y]) - log(Z);
        else
            blp[n] = tlp[n];
        free(w);
        out_len[b] = n;
        out_status[b] = status;
        out_flag[b] = flag;
        out_decisions[b] = dec;
    }
}

/* --------------------------------------------------------------- relaxed */
void oracle_relaxed(const void *T, int dt, const int32_t *x, const float *u, int B, int K, int V,
                    double tau, int top_k, double eps_accept, double eps_sample,
                    int32_t *out_tok, int32_t *out_len, double *out_tlp, double *out_blp,
                    int32_t *out_status, int32_t *out_flag, int32_t *out_decisions)
{
#pragma omp parallel for schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        const int L = K + 1;
        int32_t *tok = out_tok + (size_t)b * L;
        double *tlp = out_tlp + (size_t)b * L, *blp = out_blp + (size_t)b * L;
        pad_row(tok, tlp, blp, L);
        int status = 0, n = K, flag = -1, dec = 0;
        for (int j = 0; j < K; ++j) {
            int32_t xj = x[(size_t)b * K + j];
            ++dec;
            if (xj < 0 || xj >= V) {
                status = 1;
                n = j;
                break;
            }
            size_t row = (size_t)b * L + j;
            row_stats sp;
            stats(T, dt, row, V, &sp);
            double lx = ld(T, dt, row * (size_t)V + xj);
            long c = 0; /* rank: number of tokens scored strictly above x */
            for (int t = 0; t < V; ++t)
                if (ld(T, dt, row * (size_t)V + t) > lx)
                    ++c;
            double lp = logp(T, dt, row, V, xj, &sp);
            double p = exp(lp);
            int in_topk = c < top_k;
            if (flag < 0 && !in_topk && fabs(p - tau) < eps_accept)
                flag = j;
            if (in_topk || p >= tau) {
                tok[j] = xj;
                tlp[j] = lp;
                blp[j] = 0.0;
            } else {
                n = j;
                break;
            }
        }
        size_t row = (size_t)b * L + n;
        row_stats sp;
        stats(T, dt, row, V, &sp);
        double *w = (double *)malloc(sizeof(double) * (size_t)V);
        double Z = target_terminal(T, dt, row, V, &sp, w);
        double uK = (double)u[(size_t)b * L + K];
        double lo, hi, target = uK * Z;
        long y = inverse_cdf(w, V, target, &lo, &hi);
        ++dec;
        if (flag < 0 && sample_flag(target, lo, hi, Z, eps_sample))
            flag = n;
        tok[n] = (int32_t)y;
        tlp[n] = logp(T, dt, row, V, y, &sp);
        blp[n] = tlp[n];
        free(w);
        out_len[b] = n;
        out_status[b] = status;
        out_flag[b] = flag;
        out_decisions[b] = dec;
    }
}

/* ------------------------------------------------------------------ tree */
void oracle_tree(const void *T, int dt, const int32_t *node_tok, const int32_t *parents,
                 const int32_t *num_nodes, int B, int N, int V,
                 int32_t *out_path, int32_t *out_tok, int32_t *out_len, double *out_tlp,
                 double *out_blp, int32_t *out_status)
{
#pragma omp parallel for schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        int nb = num_nodes ? num_nodes[b] : N;
        if (nb < 1)
            nb = 1;
        if (nb > N)
            nb = N;
        int32_t *path = out_path + (size_t)b * N, *tok = out_tok + (size_t)b * N;
        double *tlp = out_tlp + (size_t)b * N, *blp = out_blp + (size_t)b * N;
        pad_row(tok, tlp, blp, N);
        for (int i = 0; i < N; ++i)
            path[i] = -1;
        row_stats *st = (row_stats *)malloc(sizeof(row_stats) * (size_t)nb);
        int *acc = (int *)malloc(sizeof(int) * (size_t)nb);
        int *depth = (int *)malloc(sizeof(int) * (size_t)nb);
        int *par = (int *)malloc(sizeof(int) * (size_t)nb);
        for (int i = 0; i < nb; ++i)
            stats(T, dt, (size_t)b * N + i, V, &st[i]);
        int status = 0;
        acc[0] = 1;
        depth[0] = 0;
        par[0] = -1;
        for (int i = 1; i < nb; ++i) {
            int p = parents[(size_t)b * N + i];
            int32_t t = node_tok[(size_t)b * N + i];
            par[i] = p;
            depth[i] = 0;
            acc[i] = 0;
            if (p < 0 || p >= i || t < 0 || t >= V) {
                status = 1;
                par[i] = -1;
                continue;
            }
            depth[i] = depth[p] + 1;
            acc[i] = acc[p] && (t == st[p].g);
        }
        int e = 0;
        for (int i = 1; i < nb; ++i)
            if (acc[i] && depth[i] > depth[e])
                e = i;
        int d = depth[e];
        for (int v = e, k = d - 1; k >= 0; --k, v = par[v])
            path[k] = v;
        for (int k = 0; k < d; ++k) {
            int v = path[k];
            tok[k] = node_tok[(size_t)b * N + v];
            tlp[k] = logp(T, dt, (size_t)b * N + par[v], V, tok[k], &st[par[v]]);
        }
        tok[d] = (int32_t)st[e].g;
        tlp[d] = logp(T, dt, (size_t)b * N + e, V, st[e].g, &st[e]);
        out_len[b] = d;
        out_status[b] = status;
        free(st);
        free(acc);
        free(depth);
        free(par);
    }
}

/* ----------------------------------------------------------- draft sampler
 * Independent draws, one per logit row: y_r = inverse CDF of softmax(X_r) at
 * u_r (ascending token order, smallest t whose inclusive prefix exceeds
 * u_r * Z), and log q_r(y_r).  This is the draft model's proposal step that
 * feeds the verifier (spec-decode README, "How it works": the draft samples
 * its k tokens from q); the uniform per row and the inverse-CDF order are the
 * same conventions as the terminal sample above.                           */
void oracle_sample(const void *X, int dt, const float *u, long rows, int V, double eps_sample,
                   int32_t *out_tok, double *out_logq, int32_t *out_flag)
{
#pragma omp parallel for schedule(dynamic)
    for (long r = 0; r < rows; ++r) {
        row_stats sq;
        stats(X, dt, (size_t)r, V, &sq);
        double *w = (double *)malloc(sizeof(double) * (size_t)V);
        double Z = sampler_weights(X, dt, (size_t)r, V, &sq, w);
        double lo, hi, target = (double)u[r] * Z;
        long y = inverse_cdf(w, V, target, &lo, &hi);
        out_tok[r] = (int32_t)y;
        out_logq[r] = logp(X, dt, (size_t)r, V, y, &sq);
        out_flag[r] = sample_flag(target, lo, hi, Z, eps_sample);
        free(w);
    }
}

/* ----------------------------------------------------------------- power
 * Power acceptance (nanospec README, acceptance-rule paragraph: accept with
 * probability min(1, p/rest)^alpha; stochastic, full support, exact
 * weights).  Reading: "rest" is the draft probability q, so draft j is
 * accepted iff u_j < a_j = min(1, p_j(x_j)/q_j(x_j))^alpha; at the first
 * rejection n the sampler emits y ~ p_n (full support), and at n = K the
 * bonus y ~ p_K, both by inverse CDF at u_K.  Behaviour log-probs: log a_j
 * on accepted drafts, log(1 - a_n) + log p_n(y) after a rejection, and
 * log p_K(y) for the bonus.  alpha = 0 accepts every draft.                */
static double power_accept(double lp, double lq, double alpha)
{
    if (alpha == 0.0)
        return 1.0;
    if (lp == -INFINITY)
        return 0.0;
    if (lq == -INFINITY)
        return 1.0;
    double la = alpha * (lp - lq);
    return la >= 0.0 ? 1.0 : exp(la);
}

void oracle_power(const void *T, const void *D, int dt, const int32_t *x, const float *u,
                  int B, int K, int V, double alpha, double eps_accept, double eps_sample,
                  int32_t *out_tok, int32_t *out_len, double *out_tlp, double *out_blp,
                  int32_t *out_status, int32_t *out_flag, int32_t *out_decisions)
{
#pragma omp parallel for schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        const int L = K + 1;
        int32_t *tok = out_tok + (size_t)b * L;
        double *tlp = out_tlp + (size_t)b * L, *blp = out_blp + (size_t)b * L;
        pad_row(tok, tlp, blp, L);
        int status = 0, n = K, flag = -1, dec = 0;
        double an = 0.0;
        for (int j = 0; j < K; ++j) {
            int32_t xj = x[(size_t)b * K + j];
            ++dec;
            if (xj < 0 || xj >= V) {
                status = 1;
                n = j;
                an = 0.0;
                break;
            }
            size_t trow = (size_t)b * L + j, drow = (size_t)b * K + j;
            row_stats sp, sq;
            stats(T, dt, trow, V, &sp);
            stats(D, dt, drow, V, &sq);
            double lp = logp(T, dt, trow, V, xj, &sp);
            double lq = logp(D, dt, drow, V, xj, &sq);
            double a = power_accept(lp, lq, alpha);
            double uj = (double)u[(size_t)b * L + j];
            if (flag < 0 && fabs(uj - a) < eps_accept)
                flag = j;
            if (uj < a) {
                tok[j] = xj;
                tlp[j] = lp;
                blp[j] = log(a);
            } else {
                n = j;
                an = a;
                break;
            }
        }
        size_t row = (size_t)b * L + n;
        row_stats sp;
        stats(T, dt, row, V, &sp);
        double *w = (double *)malloc(sizeof(double) * (size_t)V);
        double Z = target_terminal(T, dt, row, V, &sp, w);
        double lo, hi, target = (double)u[(size_t)b * L + K] * Z;
        long y = inverse_cdf(w, V, target, &lo, &hi);
        ++dec;
        if (flag < 0 && sample_flag(target, lo, hi, Z, eps_sample))
            flag = n;
        tok[n] = (int32_t)y;
        tlp[n] = logp(T, dt, row, V, y, &sp);
        blp[n] = (n < K) ? log1p(-an) + tlp[n] : tlp[n];
        free(w);
        out_len[b] = n;
        out_status[b] = status;
        out_flag[b] = flag;
        out_decisions[b] = dec;
    }
}


/* ------------------------------------------------------ terminal weights
 * The weights a rule's terminal draw inverts, for a given first-rejection
 * position n[b], exactly as the rules above form them: rule 0 the exact rule
 * (relu(p_n - q_n), or p_n at n = K or when the residual has no mass), rule 1
 * target row n (relaxed and power rules), rule 2 the draft sampler (row b of
 * T, n and D unused).  Used by tests to place uniforms next to CDF
 * boundaries.                                                             */
void oracle_terminal_weights(int rule, const void *T, const void *D, int dt, const int32_t *n,
                             int B, int K, int V, double *out_w, double *out_Z,
                             int32_t *out_residual)
{
#pragma omp parallel for schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        double *w = out_w + (size_t)b * V;
        row_stats st;
        int residual = 0;
        if (rule == 2) {
            stats(T, dt, (size_t)b, V, &st);
            out_Z[b] = sampler_weights(T, dt, (size_t)b, V, &st, w);
        } else {
            size_t row = (size_t)b * (K + 1) + n[b];
            stats(T, dt, row, V, &st);
            if (rule == 0)
                out_Z[b] = exact_terminal(T, D, dt, b, K, V, n[b], &st, w, &residual);
            else
                out_Z[b] = target_terminal(T, dt, row, V, &st, w);
        }
        out_residual[b] = residual;
    }
}
