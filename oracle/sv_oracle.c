/*
 * sv_oracle.c -- plain fp64 CPU oracle for the speculative-decoding
 * verification step.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this file.  It shares no
 * code, header, table or helper with the HIP library; it is written from the
 * method's definition, index by index, in the plainest way:
 *
 *   - every sum runs over x = 0, 1, ..., V-1 in ascending order, in fp64, on
 *     exactly converted f32 inputs;
 *   - no blocking, no vectorisation, no fusion beyond what the definition
 *     states; the pthread split is over whole sequences only.
 *
 * Sources (the spec-verify kernel card, section "Method", and its
 * "Correctness" and "Requirements and limits" sections):
 *   greedy  - accept draft token t_i while it equals argmax of target row i;
 *             at the first miss emit that argmax and stop; if all K match,
 *             emit argmax of row K.
 *   sampled - accept t_i with probability min(1, p_i(t_i)/q_i(t_i)) on
 *             row-normalised masses (rows need not be normalised; their
 *             masses are summed); on the first rejection draw from
 *             norm(max(0, p_i - q_i)); if all K are accepted draw the bonus
 *             from p_K.  Randomness enters only through explicit uniforms.
 *
 * Readings where the card is silent (each one is a stated convention):
 *   R1  normalise each row by its own summed mass; test the acceptance
 *       scale-free as u * q(t) * P < p(t) * Q and build the residual as
 *       max(0, p(x) * Q - q(x) * P), which is P*Q*max(0, p/P - q/Q).
 *   R2  u_i (i < K) drives the test of t_i; u_K is the single final draw
 *       (residual when n < K, bonus when n == K).
 *   R3  accept iff u < ratio; the inverse CDF returns the smallest x whose
 *       running mass C(x) = sum_{y <= x} w(y) exceeds T = u_K * W.
 *   R4  the inverse CDF walks tokens in ascending index order.
 *   R6  argmax ties go to the lowest index (f32 values compared as given).
 *   R7  a draft token outside [0, V) is a miss: greedy never matches it, and
 *       in sampled mode p(t) = q(t) = 0, so it is rejected.
 *   R8  if a rejection leaves W = 0 (possible only through rounding), the
 *       final draw uses p_n itself.
 *   R9  K = 0 is allowed: greedy returns argmax(p_0); sampled draws from p_0
 *       with u_0.
 *   R10 inputs must be finite and non-negative, each P and Q positive, each
 *       uniform in [0, 1); otherwise the call fails (returns -1).
 *
 * The inverse CDF always finds its token (no rounding guard is needed).  The
 * running mass at the last token, C(V-1), is the same sequential fp64 sum as
 * the total W (same terms, same order), so C(V-1) == W bitwise.  W is a
 * normal fp64 number: for a draw from a row it is that row's mass, at least
 * 2^-149 (the smallest positive f32); for a residual, every term p*Q and q*P
 * is a product of an f32 (a multiple of 2^-149) and an fp64 mass of at least
 * 2^-149, so each rounded product is a multiple of 2^-350, and a positive
 * difference of two of them rounds to at least 2^-350.  With u <= 1 - 2^-24
 * (the largest f32 below 1) the product u*W is 0 or normal, and rounding to
 * nearest gives T = fl(u*W) <= (1 - 2^-24)(1 + 2^-53) W < W = C(V-1).  So
 * some x has C(x) > T.  The oracle checks this and returns -4 if it ever
 * failed, rather than picking a token by another rule.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off -pthread
 * (never -ffast-math).  oracle/build.py runs exactly that.
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

/* Per-row statistics, one per (b, i), i in [0, K].  Draft fields (sum_q,
 * sum_min, sum_pos, q_t) are 0 for i == K and in greedy mode; p_t is 0 for
 * i == K and for out-of-range tokens. */
typedef struct {
    int32_t argmax;
    float max_p;
    double sum_p, sum_q, sum_min, sum_pos;
    float p_t, q_t;
} svo_row_stats;

/* Per-sequence diagnostics of the sampled path. */
typedef struct {
    int32_t n_accepted;
    int32_t next_token;
    int32_t draw_row;      /* row whose distribution the final draw searched */
    int32_t draw_kind;     /* 1 residual, 2 bonus, 3 residual fell back to p_n (R8) */
    double accept_margin;  /* min over performed tests of |u q(t) P - p(t) Q| / (q(t) P);
                              +inf when no test was performed or q(t) P == 0 */
    double draw_margin;    /* min(T - C(x-1), C(x) - T) / W at the selected x */
    double W;              /* total mass of the searched distribution */
    double T;              /* u_K * W */
} svo_seq_diag;

/* ---------------------------------------------------------------- rows -- */

static int row_ok(const float* r, int64_t V)
{
    for (int64_t x = 0; x < V; ++x)
        if (!(isfinite(r[x]) && r[x] >= 0.0f)) return 0;
    return 1;
}

/* argmax with the lowest index winning ties (R6) */
static int32_t row_argmax(const float* r, int64_t V, float* maxval)
{
    int64_t best = 0;
    for (int64_t x = 1; x < V; ++x)
        if (r[x] > r[best]) best = x;
    *maxval = r[best];
    return (int32_t)best;
}

static double row_sum(const float* r, int64_t V)
{
    double s = 0.0;
    for (int64_t x = 0; x < V; ++x) s += (double)r[x];
    return s;
}

static float row_at(const float* r, int64_t V, int32_t t)
{
    return (t >= 0 && (int64_t)t < V) ? r[t] : 0.0f;
}

/* -------------------------------------------------------------- greedy -- */

static int greedy_one(const float* p, const int32_t* t, int32_t K, int64_t V,
                      int32_t* n_out, int32_t* next_out, svo_row_stats* st)
{
    int32_t amax[K + 1];
    for (int32_t i = 0; i <= K; ++i) {
        const float* pi = p + (int64_t)i * V;
        if (!row_ok(pi, V)) return -1;
        float mv;
        amax[i] = row_argmax(pi, V, &mv);
        if (st) {
            svo_row_stats z = {0};
            z.argmax = amax[i];
            z.max_p = mv;
            z.sum_p = row_sum(pi, V);
            z.p_t = (i < K) ? row_at(pi, V, t[i]) : 0.0f;
            st[i] = z;
        }
    }
    int32_t n = K;
    for (int32_t i = 0; i < K; ++i) {
        if (t[i] != amax[i]) { n = i; break; }   /* R7: out of range never matches */
    }
    *n_out = n;
    *next_out = amax[n];
    return 0;
}

/* ------------------------------------------------------------- sampled -- */

/* Residual mass of token x on the rejected row (R1, R5). */
static double residual_w(const float* p, const float* q, double P, double Q, int64_t x)
{
    double a = (double)p[x] * Q;
    double b = (double)q[x] * P;
    double w = a - b;
    return w > 0.0 ? w : 0.0;
}

static int sample_one(const float* p, const float* q, const int32_t* t, const float* u,
                      int32_t K, int64_t V, int32_t* n_out, int32_t* next_out,
                      svo_row_stats* st, svo_seq_diag* dg, double* alpha)
{
    double P[K + 1], Q[K + 1];
    for (int32_t i = 0; i <= K; ++i) {
        const float* pi = p + (int64_t)i * V;
        if (!row_ok(pi, V)) return -1;
        P[i] = row_sum(pi, V);
        if (!(P[i] > 0.0)) return -1;
        if (!(u[i] >= 0.0f && u[i] < 1.0f)) return -1;
        if (st) {
            svo_row_stats z = {0};
            float mv;
            z.argmax = row_argmax(pi, V, &mv);
            z.max_p = mv;
            z.sum_p = P[i];
            st[i] = z;
        }
    }
    /* per-row tests (steps of the sampled mode, R1, R3, R7) */
    int32_t n = K;
    double acc_margin = INFINITY;
    for (int32_t i = 0; i < K; ++i) {
        const float* pi = p + (int64_t)i * V;
        const float* qi = q + (int64_t)i * V;
        if (!row_ok(qi, V)) return -1;
        Q[i] = row_sum(qi, V);
        if (!(Q[i] > 0.0)) return -1;
        double pt = (double)row_at(pi, V, t[i]);
        double qt = (double)row_at(qi, V, t[i]);
        if (st || alpha) {
            double smin = 0.0, spos = 0.0, a = 0.0;
            for (int64_t x = 0; x < V; ++x) {
                double px = (double)pi[x], qx = (double)qi[x];
                smin += px < qx ? px : qx;
                double d = px - qx;
                spos += d > 0.0 ? d : 0.0;
                double pn = px / P[i], qn = qx / Q[i];
                a += pn < qn ? pn : qn;
            }
            if (st) {
                st[i].sum_q = Q[i];
                st[i].sum_min = smin;
                st[i].sum_pos = spos;
                st[i].p_t = (float)pt;
                st[i].q_t = (float)qt;
            }
            if (alpha) alpha[i] = a;
        }
        if (n == K) {
            double lhs = (double)u[i] * qt * P[i];
            double rhs = pt * Q[i];
            if (qt * P[i] > 0.0) {
                double m = fabs(lhs - rhs) / (qt * P[i]);
                if (m < acc_margin) acc_margin = m;
            }
            if (!(lhs < rhs)) n = i;    /* first rejection */
        }
    }

    /* final draw (R2, R3, R4, R8) */
    const float* pw = p + (int64_t)n * V;
    const float* qw = (n < K) ? q + (int64_t)n * V : NULL;
    int kind;
    double W = 0.0;
    if (n < K) {
        kind = 1;
        for (int64_t x = 0; x < V; ++x) W += residual_w(pw, qw, P[n], Q[n], x);
        if (W == 0.0) { kind = 3; qw = NULL; W = P[n]; }
    } else {
        kind = 2;
        W = P[K];
    }
    double T = (double)u[K] * W;
    double C = 0.0, Cprev = 0.0;
    int64_t pick = -1;
    for (int64_t x = 0; x < V; ++x) {
        double w = qw ? residual_w(pw, qw, P[n], Q[n], x) : (double)pw[x];
        Cprev = C;
        C += w;
        if (C > T) { pick = x; break; }
    }
    if (pick < 0) return -4;     /* unreachable (see the note at the top) */
    double lo = T - Cprev, hi = C - T;
    double dmargin = (lo < hi ? lo : hi) / W;
    *n_out = n;
    *next_out = (int32_t)pick;
    if (dg) {
        dg->n_accepted = n;
        dg->next_token = (int32_t)pick;
        dg->draw_row = n;
        dg->draw_kind = kind;
        dg->accept_margin = acc_margin;
        dg->draw_margin = dmargin;
        dg->W = W;
        dg->T = T;
    }
    return 0;
}

/* ------------------------------------------------------- batch drivers -- */

typedef struct {
    int sampled;
    const float *tp, *dp, *u;
    const int32_t* dt;
    int64_t b0, b1;
    int32_t K;
    int64_t V;
    int32_t *n, *next;
    svo_row_stats* stats;
    svo_seq_diag* diag;
    double* alpha;
    int status;
} job_t;

static void* run_job(void* arg)
{
    job_t* j = (job_t*)arg;
    const int64_t K = j->K, V = j->V;
    for (int64_t b = j->b0; b < j->b1; ++b) {
        const float* p = j->tp + b * (K + 1) * V;
        const int32_t* t = j->dt + b * K;
        svo_row_stats* st = j->stats ? j->stats + b * (K + 1) : NULL;
        int rc;
        if (!j->sampled) {
            rc = greedy_one(p, t, j->K, V, j->n + b, j->next + b, st);
        } else {
            rc = sample_one(p, j->dp + b * K * V, t, j->u + b * (K + 1), j->K, V,
                            j->n + b, j->next + b, st,
                            j->diag ? j->diag + b : NULL,
                            j->alpha ? j->alpha + b * K : NULL);
        }
        if (rc != 0) { j->status = rc; return NULL; }
    }
    return NULL;
}

static int run_batch(job_t proto, int64_t B, int32_t nthreads)
{
    if (B < 0 || proto.K < 0 || proto.V < 1) return -2;
    if (B == 0) return 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > B) nthreads = (int32_t)B;
    job_t* jobs = (job_t*)calloc((size_t)nthreads, sizeof(job_t));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); return -3; }
    for (int32_t k = 0; k < nthreads; ++k) {
        jobs[k] = proto;
        jobs[k].b0 = B * k / nthreads;
        jobs[k].b1 = B * (k + 1) / nthreads;
        jobs[k].status = 0;
    }
    for (int32_t k = 1; k < nthreads; ++k) pthread_create(&th[k], NULL, run_job, &jobs[k]);
    run_job(&jobs[0]);
    for (int32_t k = 1; k < nthreads; ++k) pthread_join(th[k], NULL);
    int rc = 0;
    for (int32_t k = 0; k < nthreads && rc == 0; ++k) rc = jobs[k].status;
    free(jobs);
    free(th);
    return rc;
}

/* Greedy verification of B sequences.  tp [B, K+1, V] f32, dt [B, K] int32.
 * Writes n_accepted [B], next_token [B] and, if non-NULL, stats [B, K+1].
 * Returns 0, or -1 on a violated precondition, -2 on bad sizes. */
int svo_verify_greedy(const float* tp, const int32_t* dt, int64_t B, int32_t K, int64_t V,
                      int32_t* n_accepted, int32_t* next_token, svo_row_stats* stats,
                      int32_t nthreads)
{
    job_t j = {0};
    j.sampled = 0;
    j.tp = tp; j.dt = dt; j.K = K; j.V = V;
    j.n = n_accepted; j.next = next_token; j.stats = stats;
    return run_batch(j, B, nthreads);
}

/* Sampled verification of B sequences.  tp [B, K+1, V], dp [B, K, V] f32,
 * dt [B, K] int32, u [B, K+1] f32.  Writes n_accepted, next_token and, if
 * non-NULL, stats [B, K+1], diag [B] and alpha [B, K] (the normalised
 * per-row acceptance sum_x min(p/P, q/Q)).  Returns 0, -1 on a violated
 * precondition, -2 on bad sizes, -4 if the inverse CDF found no token
 * (impossible for valid inputs; see the note at the top). */
int svo_verify_sample(const float* tp, const float* dp, const int32_t* dt, const float* u,
                      int64_t B, int32_t K, int64_t V,
                      int32_t* n_accepted, int32_t* next_token, svo_row_stats* stats,
                      svo_seq_diag* diag, double* alpha, int32_t nthreads)
{
    job_t j = {0};
    j.sampled = 1;
    j.tp = tp; j.dp = dp; j.dt = dt; j.u = u; j.K = K; j.V = V;
    j.n = n_accepted; j.next = next_token; j.stats = stats; j.diag = diag; j.alpha = alpha;
    return run_batch(j, B, nthreads);
}

/* sizeof checks for the Python side */
int32_t svo_sizeof_row_stats(void) { return (int32_t)sizeof(svo_row_stats); }
int32_t svo_sizeof_seq_diag(void) { return (int32_t)sizeof(svo_seq_diag); }
