/*
 * C driver of the float64 oracle (oracle/gdr_oracle.c), built with
 * AddressSanitizer and UndefinedBehaviorSanitizer.  It runs both forms of
 * the recurrence (token by token, and chunked with several chunk sizes,
 * ragged tails and a zero gate) for both gate modes on small deterministic
 * inputs over several threads, and checks that the forms agree.  Exit
 * status 0 on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_recurrent(int kda, int B, int T, int H, int dk, int dv, double scale, const double* q,
                     const double* k, const double* v, const double* alpha, const double* beta,
                     const double* s0, double* o, double* sT, int nthreads);
int oracle_chunked(int kda, int B, int T, int H, int dk, int dv, int chunk, double scale,
                   const double* q, const double* k, const double* v, const double* alpha,
                   const double* beta, const double* s0, double* o, double* sT, int nthreads);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
/* uniform in [0, 1) from a 64-bit linear congruential generator */
static double uniform(void) {
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(rng_state >> 11) * (1.0 / 9007199254740992.0);
}

static double* fill(size_t n, double lo, double hi) {
    double* x = malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) x[i] = lo + (hi - lo) * uniform();
    return x;
}

static double max_abs_diff(const double* a, const double* b, size_t n) {
    double m = 0.0;
    for (size_t i = 0; i < n; ++i) m = fmax(m, fabs(a[i] - b[i]));
    return m;
}

int main(void) {
    const int B = 2, H = 3, dk = 8, dv = 5;
    const int lengths[] = {1, 37, 64, 130};
    const int chunks[] = {1, 4, 16, 64};
    int failures = 0;
    for (int kda = 0; kda <= 1; ++kda) {
        for (int li = 0; li < 4; ++li) {
            const int T = lengths[li];
            const size_t nq = (size_t)B * T * H * dk, nv = (size_t)B * T * H * dv;
            const size_t na = kda ? nq : (size_t)B * T * H, ns = (size_t)B * H * dk * dv;
            double *q = fill(nq, -0.4, 0.4), *k = fill(nq, -0.4, 0.4), *v = fill(nv, -1, 1);
            double *a = fill(na, 0.5, 1.0), *beta = fill((size_t)B * T * H, 0.0, 1.0);
            double* s0 = fill(ns, -0.1, 0.1);
            if (T > 20) a[(size_t)(T / 2) * H * (kda ? dk : 1)] = 0.0; /* a zero gate */
            double *o1 = malloc(nv * sizeof(double)), *o2 = malloc(nv * sizeof(double));
            double *s1 = malloc(ns * sizeof(double)), *s2 = malloc(ns * sizeof(double));
            if (oracle_recurrent(kda, B, T, H, dk, dv, 0.7, q, k, v, a, beta, s0, o1, s1, 3) != 0)
                ++failures;
            for (int ci = 0; ci < 4; ++ci) {
                if (oracle_chunked(kda, B, T, H, dk, dv, chunks[ci], 0.7, q, k, v, a, beta,
                                   s0, o2, s2, 2) != 0)
                    ++failures;
                const double eo = max_abs_diff(o1, o2, nv), es = max_abs_diff(s1, s2, ns);
                if (!(eo < 1e-12 && es < 1e-12)) {
                    fprintf(stderr, "kda=%d T=%d chunk=%d: |o| %.3e |S| %.3e\n", kda, T,
                            chunks[ci], eo, es);
                    ++failures;
                }
            }
            /* a zero initial state given as NULL */
            if (oracle_recurrent(kda, B, T, H, dk, dv, 1.0, q, k, v, a, beta, NULL, o1, s1, 4) != 0 ||
                oracle_chunked(kda, B, T, H, dk, dv, 16, 1.0, q, k, v, a, beta, NULL, o2, s2, 4) != 0)
                ++failures;
            if (!(max_abs_diff(o1, o2, nv) < 1e-12 && max_abs_diff(s1, s2, ns) < 1e-12)) ++failures;
            free(q); free(k); free(v); free(a); free(beta); free(s0);
            free(o1); free(o2); free(s1); free(s2);
        }
    }
    /* invalid arguments are rejected, not run */
    if (oracle_recurrent(0, -1, 4, 1, 4, 4, 1.0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1) == 0)
        ++failures;
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("all checks passed\n");
    return 0;
}
