/*
 * gdr_oracle.c -- float64 CPU oracle of the gated delta-rule token mixer.
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the test suite, the
 * smoke check and the bench's CPU-baseline leg load this file's library.  It
 * shares no code, header, table or helper with the GPU library.
 *
 * What it computes.  "Super Apriel: One Checkpoint, Many Speeds"
 * (gist.science/paper/2604.19877), §2.A "The Supernet Architecture", lists
 * two recurrent token mixers with a fixed-size state and O(n) time: Gated
 * DeltaNet (GDN), a delta rule with a scalar gate, and Kimi Delta Attention
 * (KDA), delta attention with a channel-wise gate.  The pages print no update
 * rule.  This file takes the gated delta rule in its usual form, for each
 * batch b and head h independently, with state S in R^{dk x dv}:
 *
 *     S_t = (I - beta_t k_t k_t^T) D_t S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t
 *
 * where D_t = alpha_t I (GDN, alpha_t a scalar per token and head) or
 * D_t = diag(alpha_t) (KDA, alpha_t in R^dk acting on the key axis, i.e. the
 * rows of S).  The gate is applied before the delta correction, and the
 * output reads the post-update state.
 *
 * Layouts (all row-major, float64):
 *   q, k   [B, T, H, dk]      v, o   [B, T, H, dv]
 *   alpha  [B, T, H] (GDN) or [B, T, H, dk] (KDA)
 *   beta   [B, T, H]
 *   s0, sT [B, H, dk, dv]     (s0 may be NULL: zero initial state)
 * A single decode step is the T == 1 case: [B, 1, H, d] is [B, H, d].
 *
 * Two forms are provided:
 *   oracle_recurrent  the definition above, token by token (the main oracle);
 *   oracle_chunked    the exact chunked refactoring of the same recurrence
 *                     (WY/UT form), with decays taken as direct products of
 *                     the gates rather than exponentials of log sums, so a
 *                     zero gate is legal.  Used to pin that the chunked
 *                     algebra equals the definition.
 * Both thread across the independent (b, h) pairs with pthreads.
 */
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ENOMEM (-2)

typedef struct {
    int kda, B, T, H, dk, dv, chunk;
    double scale;
    const double *q, *k, *v, *alpha, *beta, *s0;
    double *o, *sT;
    int nthreads, tid, status;
} job_t;

/* Pointers to token t of (b, h) in a [B, T, H, d] tensor. */
static inline const double* tok(const double* base, const job_t* j, int b, int t, int h, int d) {
    return base + (((size_t)b * j->T + t) * j->H + h) * (size_t)d;
}
static inline double* tok_mut(double* base, const job_t* j, int b, int t, int h, int d) {
    return base + (((size_t)b * j->T + t) * j->H + h) * (size_t)d;
}
static inline double gate_at(const job_t* j, int b, int t, int h, int c) {
    if (j->kda) return tok(j->alpha, j, b, t, h, j->dk)[c];
    return j->alpha[((size_t)b * j->T + t) * j->H + h];
}
static inline double beta_at(const job_t* j, int b, int t, int h) {
    return j->beta[((size_t)b * j->T + t) * j->H + h];
}

static void load_state(const job_t* j, int b, int h, double* S) {
    size_t n = (size_t)j->dk * j->dv;
    if (j->s0) memcpy(S, j->s0 + ((size_t)b * j->H + h) * n, n * sizeof(double));
    else memset(S, 0, n * sizeof(double));
}
static void store_state(const job_t* j, int b, int h, const double* S) {
    size_t n = (size_t)j->dk * j->dv;
    if (j->sT) memcpy(j->sT + ((size_t)b * j->H + h) * n, S, n * sizeof(double));
}

/* ---------------------------------------------------------------- recurrent */

/* One (b, h) pair, token by token, exactly as the recurrence is written:
 *   S' = D_t S;  p = S'^T k;  S = S' + beta k (v - p)^T  (= (I - beta k k^T) S' + beta k v^T);
 *   o = scale * S^T q. */
static void recurrent_unit(const job_t* j, int b, int h, double* S, double* p) {
    const int dk = j->dk, dv = j->dv;
    load_state(j, b, h, S);
    for (int t = 0; t < j->T; ++t) {
        const double* q = tok(j->q, j, b, t, h, dk);
        const double* k = tok(j->k, j, b, t, h, dk);
        const double* v = tok(j->v, j, b, t, h, dv);
        const double beta = beta_at(j, b, t, h);
        for (int i = 0; i < dk; ++i) {
            const double a = gate_at(j, b, t, h, i);
            for (int c = 0; c < dv; ++c) S[(size_t)i * dv + c] *= a;
        }
        for (int c = 0; c < dv; ++c) p[c] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int c = 0; c < dv; ++c) p[c] += k[i] * S[(size_t)i * dv + c];
        for (int i = 0; i < dk; ++i) {
            const double bk = beta * k[i];
            for (int c = 0; c < dv; ++c) S[(size_t)i * dv + c] += bk * (v[c] - p[c]);
        }
        double* o = tok_mut(j->o, j, b, t, h, dv);
        for (int c = 0; c < dv; ++c) o[c] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int c = 0; c < dv; ++c) o[c] += q[i] * S[(size_t)i * dv + c];
        for (int c = 0; c < dv; ++c) o[c] *= j->scale;
    }
    store_state(j, b, h, S);
}

/* ------------------------------------------------------------------ chunked */

/* Scratch for one chunk of at most C tokens. */
typedef struct {
    double *S, *G, *Dl, *A, *P, *Tm, *W, *Ut, *U, *Kh, *Qh, *Kt, *O;
} chunk_scratch_t;

/*
 * One (b, h) pair by chunks.  For a chunk of tokens t0 .. t0+n-1 entering with
 * state S, write Gamma_t = prod_{s=t0..t} alpha_s (per channel) and
 * delta(j, t) = prod_{s=j+1..t} alpha_s for j <= t (empty product 1).  Unrolling
 * the recurrence inside the chunk gives S_t = Gamma_t S + sum_{j<=t} delta(j,t) k_j u_j^T
 * with u_t = beta_t (v_t - (D_t S_{t-1})^T k_t), which in matrix form (rows =
 * tokens of the chunk) is
 *   A_tj = beta_t sum_c k_tc k_jc delta(j,t)_c        (j < t, else 0)
 *   T    = (I + A)^{-1}                               (unit lower triangular)
 *   Khat = rows k_t (.) Gamma_t,  Qhat = rows q_t (.) Gamma_t
 *   W    = T diag(beta) Khat,     Ut = T diag(beta) V
 *   U    = Ut - W S
 *   P_tj = sum_c q_tc k_jc delta(j,t)_c               (j <= t, else 0)
 *   O    = scale (Qhat S + P U)
 *   Ktil = rows k_j (.) delta(j, t0+n-1)
 *   S   <- diag(Gamma_{t0+n-1}) S + Ktil^T U.
 */
static void chunked_unit(const job_t* j, int b, int h, chunk_scratch_t* w) {
    const int dk = j->dk, dv = j->dv, C = j->chunk;
    double* S = w->S;
    load_state(j, b, h, S);
    for (int t0 = 0; t0 < j->T; t0 += C) {
        const int n = (j->T - t0 < C) ? (j->T - t0) : C;
        /* Gamma_t per channel, by direct products from the chunk start. */
        for (int c = 0; c < dk; ++c) {
            double g = 1.0;
            for (int t = 0; t < n; ++t) {
                g *= gate_at(j, b, t0 + t, h, c);
                w->G[(size_t)t * dk + c] = g;
            }
        }
        /* delta(jj, t)_c for jj <= t, stored at Dl[(t * C + jj) * dk + c]. */
        for (int jj = 0; jj < n; ++jj) {
            for (int c = 0; c < dk; ++c) w->Dl[((size_t)jj * C + jj) * dk + c] = 1.0;
            for (int t = jj + 1; t < n; ++t)
                for (int c = 0; c < dk; ++c)
                    w->Dl[((size_t)t * C + jj) * dk + c] =
                        w->Dl[((size_t)(t - 1) * C + jj) * dk + c] * gate_at(j, b, t0 + t, h, c);
        }
        /* A and P. */
        for (int t = 0; t < n; ++t) {
            const double* kt = tok(j->k, j, b, t0 + t, h, dk);
            const double* qt = tok(j->q, j, b, t0 + t, h, dk);
            const double bt = beta_at(j, b, t0 + t, h);
            for (int jj = 0; jj < n; ++jj) {
                double a = 0.0, p = 0.0;
                if (jj <= t) {
                    const double* kj = tok(j->k, j, b, t0 + jj, h, dk);
                    const double* dl = w->Dl + ((size_t)t * C + jj) * dk;
                    for (int c = 0; c < dk; ++c) {
                        a += kt[c] * kj[c] * dl[c];
                        p += qt[c] * kj[c] * dl[c];
                    }
                }
                w->A[(size_t)t * C + jj] = (jj < t) ? bt * a : 0.0;
                w->P[(size_t)t * C + jj] = p;
            }
        }
        /* T = (I + A)^{-1} by forward substitution, row by row:
         * T[i][:] = e_i - sum_{jj < i} A[i][jj] T[jj][:]. */
        for (int i = 0; i < n; ++i) {
            for (int c = 0; c < n; ++c) w->Tm[(size_t)i * C + c] = (i == c) ? 1.0 : 0.0;
            for (int jj = 0; jj < i; ++jj) {
                const double a = w->A[(size_t)i * C + jj];
                for (int c = 0; c < n; ++c) w->Tm[(size_t)i * C + c] -= a * w->Tm[(size_t)jj * C + c];
            }
        }
        /* Gated rows. */
        for (int t = 0; t < n; ++t) {
            const double* kt = tok(j->k, j, b, t0 + t, h, dk);
            const double* qt = tok(j->q, j, b, t0 + t, h, dk);
            const double* dl = w->Dl + ((size_t)(n - 1) * C + t) * dk; /* delta(t, end) */
            for (int c = 0; c < dk; ++c) {
                const double g = w->G[(size_t)t * dk + c];
                w->Kh[(size_t)t * dk + c] = kt[c] * g;
                w->Qh[(size_t)t * dk + c] = qt[c] * g;
                w->Kt[(size_t)t * dk + c] = kt[c] * dl[c];
            }
        }
        /* W = T diag(beta) Khat (n x dk), Ut = T diag(beta) V (n x dv). */
        for (int t = 0; t < n; ++t) {
            for (int c = 0; c < dk; ++c) w->W[(size_t)t * dk + c] = 0.0;
            for (int c = 0; c < dv; ++c) w->Ut[(size_t)t * dv + c] = 0.0;
            for (int jj = 0; jj <= t; ++jj) {
                const double tb = w->Tm[(size_t)t * C + jj] * beta_at(j, b, t0 + jj, h);
                const double* vj = tok(j->v, j, b, t0 + jj, h, dv);
                for (int c = 0; c < dk; ++c) w->W[(size_t)t * dk + c] += tb * w->Kh[(size_t)jj * dk + c];
                for (int c = 0; c < dv; ++c) w->Ut[(size_t)t * dv + c] += tb * vj[c];
            }
        }
        /* U = Ut - W S. */
        for (int t = 0; t < n; ++t)
            for (int c = 0; c < dv; ++c) {
                double acc = w->Ut[(size_t)t * dv + c];
                for (int i = 0; i < dk; ++i) acc -= w->W[(size_t)t * dk + i] * S[(size_t)i * dv + c];
                w->U[(size_t)t * dv + c] = acc;
            }
        /* O = scale (Qhat S + P U). */
        for (int t = 0; t < n; ++t) {
            double* o = tok_mut(j->o, j, b, t0 + t, h, dv);
            for (int c = 0; c < dv; ++c) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i) acc += w->Qh[(size_t)t * dk + i] * S[(size_t)i * dv + c];
                for (int jj = 0; jj <= t; ++jj) acc += w->P[(size_t)t * C + jj] * w->U[(size_t)jj * dv + c];
                o[c] = j->scale * acc;
            }
        }
        /* S <- diag(Gamma_end) S + Ktil^T U. */
        for (int i = 0; i < dk; ++i) {
            const double ge = w->G[(size_t)(n - 1) * dk + i];
            for (int c = 0; c < dv; ++c) {
                double acc = ge * S[(size_t)i * dv + c];
                for (int t = 0; t < n; ++t) acc += w->Kt[(size_t)t * dk + i] * w->U[(size_t)t * dv + c];
                S[(size_t)i * dv + c] = acc;
            }
        }
    }
    store_state(j, b, h, S);
}

/* ------------------------------------------------------------------ driver */

static void* run_recurrent(void* arg) {
    job_t* j = (job_t*)arg;
    double* S = (double*)malloc(sizeof(double) * ((size_t)j->dk * j->dv + j->dv));
    if (!S) { j->status = ORACLE_ENOMEM; return NULL; }
    for (int u = j->tid; u < j->B * j->H; u += j->nthreads)
        recurrent_unit(j, u / j->H, u % j->H, S, S + (size_t)j->dk * j->dv);
    free(S);
    return NULL;
}

static void* run_chunked(void* arg) {
    job_t* j = (job_t*)arg;
    const size_t C = (size_t)j->chunk, dk = (size_t)j->dk, dv = (size_t)j->dv;
    chunk_scratch_t w;
    double** slots[] = {&w.S, &w.G, &w.Dl, &w.A, &w.P, &w.Tm, &w.W, &w.Ut, &w.U,
                        &w.Kh, &w.Qh, &w.Kt, &w.O};
    const size_t sizes[] = {dk * dv, C * dk, C * C * dk, C * C, C * C, C * C, C * dk,
                            C * dv, C * dv, C * dk, C * dk, C * dk, C * dv};
    int ok = 1;
    for (int s = 0; s < 13; ++s) {
        *slots[s] = (double*)malloc(sizeof(double) * sizes[s]);
        if (!*slots[s]) ok = 0;
    }
    if (ok) {
        for (int u = j->tid; u < j->B * j->H; u += j->nthreads)
            chunked_unit(j, u / j->H, u % j->H, &w);
    } else {
        j->status = ORACLE_ENOMEM;
    }
    for (int s = 0; s < 13; ++s) free(*slots[s]);
    return NULL;
}

static int launch(job_t* proto, void* (*fn)(void*)) {
    if (proto->B < 0 || proto->T < 0 || proto->H < 0 || proto->dk <= 0 || proto->dv <= 0)
        return ORACLE_EINVAL;
    if (!proto->q || !proto->k || !proto->v || !proto->alpha || !proto->beta || !proto->o)
        return (proto->B * proto->T * proto->H == 0) ? ORACLE_OK : ORACLE_EINVAL;
    int nt = proto->nthreads < 1 ? 1 : proto->nthreads;
    if (nt > proto->B * proto->H) nt = proto->B * proto->H > 0 ? proto->B * proto->H : 1;
    job_t* jobs = (job_t*)calloc((size_t)nt, sizeof(job_t));
    pthread_t* th = (pthread_t*)calloc((size_t)nt, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); return ORACLE_ENOMEM; }
    for (int i = 0; i < nt; ++i) {
        jobs[i] = *proto;
        jobs[i].nthreads = nt;
        jobs[i].tid = i;
        jobs[i].status = ORACLE_OK;
    }
    int status = ORACLE_OK;
    int started = 0;
    for (int i = 1; i < nt; ++i) {
        if (pthread_create(&th[i], NULL, fn, &jobs[i]) != 0) { status = ORACLE_ENOMEM; break; }
        started = i;
    }
    if (status == ORACLE_OK) fn(&jobs[0]);
    for (int i = 1; i <= started; ++i) pthread_join(th[i], NULL);
    for (int i = 0; i < nt && status == ORACLE_OK; ++i) status = jobs[i].status;
    free(jobs);
    free(th);
    return status;
}

int oracle_recurrent(int kda, int B, int T, int H, int dk, int dv, double scale,
                     const double* q, const double* k, const double* v,
                     const double* alpha, const double* beta, const double* s0,
                     double* o, double* sT, int nthreads) {
    job_t j = {kda, B, T, H, dk, dv, 1, scale, q, k, v, alpha, beta, s0, o, sT, nthreads, 0, 0};
    return launch(&j, run_recurrent);
}

int oracle_chunked(int kda, int B, int T, int H, int dk, int dv, int chunk, double scale,
                   const double* q, const double* k, const double* v,
                   const double* alpha, const double* beta, const double* s0,
                   double* o, double* sT, int nthreads) {
    if (chunk <= 0) return ORACLE_EINVAL;
    job_t j = {kda, B, T, H, dk, dv, chunk, scale, q, k, v, alpha, beta, s0, o, sT, nthreads, 0, 0};
    return launch(&j, run_chunked);
}

int oracle_abi_version(void) { return 1; }
