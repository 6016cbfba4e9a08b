/* The C oracle under AddressSanitizer and UBSan (built with gcc by
 * tests/test_sanitizers.py): a forward with an initial state and a state
 * trace on a ragged shape with groups, then the same tokens one decode step
 * at a time, which must give the same outputs and final state. Exit status 0
 * when they agree to 1e-12 relative, 1 otherwise; the sanitizers abort on any
 * out-of-range access or undefined behaviour. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_ssd_fwd(const double *X, const double *dt, const double *A, const double *Bm, const double *Cm,
                   const double *D, const double *init_state, double *Y, double *final_state, double *trace,
                   int64_t trace_every, int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                   int64_t dstate, int64_t ngroups);
int oracle_ssd_step(double *state, const double *x, const double *dt, const double *A, const double *Bm,
                    const double *Cm, const double *D, double *y, int64_t batch, int64_t nheads, int64_t headdim,
                    int64_t dstate, int64_t ngroups);

static uint64_t rng = 88172645463325252ull;
static double uni(void) { /* xorshift64, uniform in (-1, 1) */
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return (double)(rng >> 11) / (double)(1ull << 52) - 1.0;
}
static double *alloc_fill(size_t n, double scale, double shift) {
    double *p = malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = shift + scale * uni();
    return p;
}

int main(void) {
    const int64_t Bz = 2, T = 37, H = 4, P = 8, N = 16, G = 2, TE = 5;
    double *X = alloc_fill(Bz * T * H * P, 1.0, 0.0), *dt = alloc_fill(Bz * T * H, 0.05, 0.06);
    double *A = alloc_fill(H, 0.9, -1.0), *Bm = alloc_fill(Bz * T * G * N, 0.3, 0.0);
    double *Cm = alloc_fill(Bz * T * G * N, 0.3, 0.0), *D = alloc_fill(H, 1.0, 0.0);
    double *h0 = alloc_fill(Bz * H * P * N, 1.0, 0.0);
    double *Y = malloc(Bz * T * H * P * sizeof(double)), *F = malloc(Bz * H * P * N * sizeof(double));
    double *trace = malloc(Bz * (T / TE) * H * P * N * sizeof(double));
    if (oracle_ssd_fwd(X, dt, A, Bm, Cm, D, h0, Y, F, trace, TE, Bz, T, H, P, N, G) != 0) return 1;
    if (oracle_ssd_fwd(X, dt, A, Bm, Cm, D, NULL, Y, NULL, NULL, 0, Bz, 0, H, P, N, G) != 0) return 1;
    if (oracle_ssd_fwd(X, dt, A, Bm, Cm, D, h0, Y, F, trace, TE, Bz, T, H, P, N, G) != 0) return 1;
    if (oracle_ssd_fwd(X, dt, A, Bm, Cm, D, h0, Y, F, trace, TE, Bz, T, 3, P, N, G) == 0) return 1; /* H % G */

    double *state = malloc(Bz * H * P * N * sizeof(double));
    memcpy(state, h0, Bz * H * P * N * sizeof(double));
    double *x = malloc(Bz * H * P * sizeof(double)), *d = malloc(Bz * H * sizeof(double));
    double *b = malloc(Bz * G * N * sizeof(double)), *c = malloc(Bz * G * N * sizeof(double));
    double *y = malloc(Bz * H * P * sizeof(double));
    double ymax = 0.0, err = 0.0;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t i = 0; i < Bz; ++i) {
            memcpy(x + i * H * P, X + (i * T + t) * H * P, H * P * sizeof(double));
            memcpy(d + i * H, dt + (i * T + t) * H, H * sizeof(double));
            memcpy(b + i * G * N, Bm + (i * T + t) * G * N, G * N * sizeof(double));
            memcpy(c + i * G * N, Cm + (i * T + t) * G * N, G * N * sizeof(double));
        }
        if (oracle_ssd_step(state, x, d, A, b, c, D, y, Bz, H, P, N, G) != 0) return 1;
        for (int64_t i = 0; i < Bz; ++i)
            for (int64_t k = 0; k < H * P; ++k) {
                const double ref = Y[(i * T + t) * H * P + k];
                ymax = fmax(ymax, fabs(ref));
                err = fmax(err, fabs(y[i * H * P + k] - ref));
            }
    }
    double fmax_ = 0.0, ferr = 0.0;
    for (int64_t k = 0; k < Bz * H * P * N; ++k) {
        fmax_ = fmax(fmax_, fabs(F[k]));
        ferr = fmax(ferr, fabs(state[k] - F[k]));
    }
    printf("step vs forward: Y %.3g, final state %.3g (relative)\n", err / ymax, ferr / fmax_);
    free(X); free(dt); free(A); free(Bm); free(Cm); free(D); free(h0); free(Y); free(F); free(trace);
    free(state); free(x); free(d); free(b); free(c); free(y);
    return (err / ymax < 1e-12 && ferr / fmax_ < 1e-12) ? 0 : 1;
}
