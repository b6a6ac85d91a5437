/*
 * Plain fp64 CPU oracle for causal Taylor linear attention (BASED), its
 * JRT-RNN prefix variant and the single-token decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links or calls this
 * file: only the test-suite, the smoke check and the benchmark's CPU-baseline
 * leg use it.  It shares no code, header or constant with the HIP library.
 *
 * Sources (the reading-notes pages this follows):
 *   [BASED] "Simple linear attention language models balance the
 *           recall-throughput tradeoff" notes: §2.2 (recurrence s_i, z_i, y_i
 *           and its attention form), §2.3 (Taylor kernel, Eq. (4), feature map
 *           phi with the d'^(1/4) normalisation, D = 1 + d' + d'^2).
 *   [JRT]   "Just read twice: closing the recall gap for recurrent language
 *           models" notes: §2.5 (Eqs. (1)-(2)), §2.6 (prefix state s_E, z_E,
 *           Eq. (3) output, Eq. (4) merged state).
 *   [LG]    "Understanding and Improving Length Generalization in Recurrent
 *           Models" notes: §2.5 (Eq. (4): a non-zero initial state is carried
 *           by the same scan; with A_t = I it is simply added).
 *
 * Readings taken where the pages leave a step open:
 *   - the current token is included (sum over j <= i): state update first,
 *     then read ([BASED] §2.2);
 *   - vec(x x^T) is laid out a-major: feature index 1 + d + a*d + b;
 *   - numerator and denominator carry the initial state separately ([LG] §2.5
 *     applied to s and z each);
 *   - eps is added to the denominator ([BASED] §2.3 says only that an epsilon
 *     is added); parity runs use eps = 0;
 *   - JRT: the prefix sums run over all M prefix tokens (non-causal), the
 *     causal sums over every position 1..N ([JRT] §2.6, Eq. (3)); the cached
 *     state is initial + s_E + s_{D,N} ([JRT] Eq. (4)).
 *
 * Every array is contiguous row-major fp64:
 *   q, k [B][H][N][d]   v [B][H][N][dv]   ke [B][H][M][d]   ve [B][H][M][dv]
 *   S [B][H][D][dv]     z [B][H][D]       y [B][H][N][dv]
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

int oracle_feature_dim(int d) { return 1 + d + d * d; }

/* phi(x) = [1, x/d^(1/4), vec((x/d^(1/4))(x/d^(1/4))^T)/sqrt(2)]  ([BASED] §2.3) */
void oracle_feature_map(int d, const double *x, double *phi)
{
    double s = pow((double)d, -0.25);
    double r2 = 1.0 / sqrt(2.0);
    phi[0] = 1.0;
    for (int a = 0; a < d; ++a)
        phi[1 + a] = x[a] * s;
    for (int a = 0; a < d; ++a)
        for (int b = 0; b < d; ++b)
            phi[1 + d + a * d + b] = (x[a] * s) * (x[b] * s) * r2;
}

typedef struct {
    int B, H, N, M, d, dv;
    double eps;
    const double *q, *k, *v, *ke, *ve, *S0, *z0;
    double *y, *S_out, *z_out;
    long first, last; /* head range [first, last) of this worker */
} job_t;

/* s += phi(key) value^T ; z += phi(key)  ([BASED] §2.2, [JRT] Eq. (1)) */
static void absorb(int D, int dv, const double *phi, const double *val, double *S, double *z)
{
    for (int f = 0; f < D; ++f) {
        double p = phi[f];
        double *row = S + (long)f * dv;
        for (int c = 0; c < dv; ++c)
            row[c] += p * val[c];
        z[f] += p;
    }
}

/* y = s^T phi(query) / (z^T phi(query) + eps)  ([BASED] §2.2, [JRT] Eq. (3)) */
static void readout(int D, int dv, const double *phi, const double *S, const double *z, double eps,
                    double *out)
{
    double den = 0.0;
    for (int f = 0; f < D; ++f)
        den += phi[f] * z[f];
    den += eps;
    for (int c = 0; c < dv; ++c) {
        double num = 0.0;
        for (int f = 0; f < D; ++f)
            num += phi[f] * S[(long)f * dv + c];
        out[c] = num / den;
    }
}

static void run_head(const job_t *J, long bh, double *S, double *z, double *phi)
{
    const int d = J->d, dv = J->dv, D = oracle_feature_dim(d);
    const long N = J->N, M = J->M;

    /* initial state: given, or zero ([LG] §2.5) */
    if (J->S0)
        memcpy(S, J->S0 + bh * D * dv, sizeof(double) * D * dv);
    else
        memset(S, 0, sizeof(double) * D * dv);
    if (J->z0)
        memcpy(z, J->z0 + bh * D, sizeof(double) * D);
    else
        memset(z, 0, sizeof(double) * D);

    /* JRT encoder pass: s_E = sum_{j<=M} phi(k_e_j) v_e_j^T, z_E likewise ([JRT] §2.6) */
    for (long j = 0; j < M; ++j) {
        oracle_feature_map(d, J->ke + (bh * M + j) * d, phi);
        absorb(D, dv, phi, J->ve + (bh * M + j) * dv, S, z);
    }

    /* causal scan: update with token i, then read with query i */
    for (long i = 0; i < N; ++i) {
        oracle_feature_map(d, J->k + (bh * N + i) * d, phi);
        absorb(D, dv, phi, J->v + (bh * N + i) * dv, S, z);
        if (J->y) {
            oracle_feature_map(d, J->q + (bh * N + i) * d, phi);
            readout(D, dv, phi, S, z, J->eps, J->y + (bh * N + i) * dv);
        }
    }

    if (J->S_out)
        memcpy(J->S_out + bh * D * dv, S, sizeof(double) * D * dv);
    if (J->z_out)
        memcpy(J->z_out + bh * D, z, sizeof(double) * D);
}

static void *worker(void *arg)
{
    const job_t *J = (const job_t *)arg;
    const int D = oracle_feature_dim(J->d);
    double *S = (double *)malloc(sizeof(double) * D * J->dv);
    double *z = (double *)malloc(sizeof(double) * D);
    double *phi = (double *)malloc(sizeof(double) * D);
    for (long bh = J->first; bh < J->last; ++bh)
        run_head(J, bh, S, z, phi);
    free(S);
    free(z);
    free(phi);
    return NULL;
}

static void run_jobs(job_t base, int nthreads)
{
    long heads = (long)base.B * base.H;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > heads)
        nthreads = (int)(heads > 0 ? heads : 1);
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
    job_t *jobs = (job_t *)malloc(sizeof(job_t) * nthreads);
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = base;
        jobs[t].first = heads * t / nthreads;
        jobs[t].last = heads * (t + 1) / nthreads;
        pthread_create(&tid[t], NULL, worker, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t)
        pthread_join(tid[t], NULL);
    free(tid);
    free(jobs);
}

/* Causal prefill with optional initial state.  S0/z0 NULL -> zero state;
 * y, S_out, z_out may each be NULL (not produced). */
void oracle_prefill(int B, int H, int N, int d, int dv, const double *q, const double *k,
                    const double *v, const double *S0, const double *z0, double eps, double *y,
                    double *S_out, double *z_out, int nthreads)
{
    job_t J = {B, H, N, 0, d, dv, eps, q, k, v, NULL, NULL, S0, z0, y, S_out, z_out, 0, 0};
    run_jobs(J, nthreads);
}

/* JRT-RNN prefix linear attention: the prefix state from (ke, ve) over M
 * tokens is added to the initial state, then the causal scan runs over all
 * N positions; the final state is initial + s_E + s_{D,N}. */
void oracle_jrt(int B, int H, int N, int M, int d, int dv, const double *q, const double *k,
                const double *v, const double *ke, const double *ve, const double *S0,
                const double *z0, double eps, double *y, double *S_out, double *z_out,
                int nthreads)
{
    job_t J = {B, H, N, M, d, dv, eps, q, k, v, ke, ve, S0, z0, y, S_out, z_out, 0, 0};
    run_jobs(J, nthreads);
}

/* One recurrent step per head on a persistent state, updated in place:
 * S += phi(k) v^T, z += phi(k), then y = S^T phi(q) / (z^T phi(q) + eps).
 * Heads are independent; they are split over nthreads workers. */
typedef struct {
    int d, dv;
    double eps;
    const double *q, *k, *v;
    double *S, *z, *y;
    long first, last;
} step_job_t;

static void *step_worker(void *arg)
{
    const step_job_t *J = (const step_job_t *)arg;
    const int d = J->d, dv = J->dv, D = oracle_feature_dim(d);
    double *phi = (double *)malloc(sizeof(double) * D);
    for (long bh = J->first; bh < J->last; ++bh) {
        double *Sh = J->S + bh * D * dv, *zh = J->z + bh * D;
        oracle_feature_map(d, J->k + bh * d, phi);
        absorb(D, dv, phi, J->v + bh * dv, Sh, zh);
        oracle_feature_map(d, J->q + bh * d, phi);
        readout(D, dv, phi, Sh, zh, J->eps, J->y + bh * dv);
    }
    free(phi);
    return NULL;
}

void oracle_decode_step(int B, int H, int d, int dv, const double *q, const double *k,
                        const double *v, double *S, double *z, double eps, double *y, int nthreads)
{
    long heads = (long)B * H;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > heads)
        nthreads = (int)(heads > 0 ? heads : 1);
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
    step_job_t *jobs = (step_job_t *)malloc(sizeof(step_job_t) * nthreads);
    for (int t = 0; t < nthreads; ++t) {
        step_job_t J = {d, dv, eps, q, k, v, S, z, y, heads * t / nthreads, heads * (t + 1) / nthreads};
        jobs[t] = J;
        pthread_create(&tid[t], NULL, step_worker, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t)
        pthread_join(tid[t], NULL);
    free(tid);
    free(jobs);
}
