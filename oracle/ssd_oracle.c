/*
 * CPU oracle for the SSD core. TEST INFRASTRUCTURE ONLY: this file is built
 * and called by the test suite, the smoke check and the benchmark's CPU
 * baseline leg. The product (the HIP library) never links, loads or calls it,
 * and it shares no code, header or table with the HIP path.
 *
 * What it computes: the plain sequential recurrence of a selective SSM whose
 * state matrix is a scalar times the identity, one token at a time, in fp64.
 *
 *   a_t     = exp(dt[b,t,h] * A[h])                      decay (ZOH form)
 *   s_t     = a_t * s_{t-1} + dt[b,t,h] * x_t (outer) B_t  state, P x N per (b,h)
 *   y_t     = s_t . C_t + D[h] * x_t                       output with skip term
 *   s_{-1}  = init_state (zero when not given); final_state = s_{T-1}
 *
 * Sources (page title, section):
 *  - "Transformer vs Mamba/SSM: the next step of the architecture", core
 *    concepts: the discretised recurrence h_t = Abar h_{t-1} + Bbar x_t, y_t = C h_t.
 *  - "Mamba principles in depth", section 2.2: Mamba discretises with zero-order
 *    hold and folds the step size into the input matrix, Bbar = Delta * B.
 *  - "Mamba 2 state space duality deep theory", section 4.1 (ssd_scan): the
 *    decay is exp(dt * A) and the input term is dt * u.
 *  - "Transformers are SSMs" reading report (Mamba-2), sections 2.2 and 2.4:
 *    A is a scalar times the identity, one scalar a_t per head and step; the
 *    head dimension P > 1 turns the state into a P x N matrix per head.
 *  - "SSM and Mamba survey", section 2: the skip term, y = C h + D x.
 *  - Head h reads B/C group floor(h * G / H) (contiguous groups; the reading
 *    taken because the reading report's section 3.4 requires that a tensor-
 *    parallel shard of heads owns whole groups).
 *
 * Layouts (row-major, contiguous): X, Y (B,T,H,P); dt (B,T,H); A, D (H);
 * Bm, Cm (B,T,G,N); states (B,H,P,N). All arrays are double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL 1

static int shapes_ok(int64_t b, int64_t t, int64_t h, int64_t p, int64_t n, int64_t g) {
    if (b < 0 || t < 0 || h <= 0 || p <= 0 || n <= 0 || g <= 0) return 0;
    if (h % g != 0) return 0;
    return 1;
}

/* Number of threads OpenMP will use (for reporting in the CPU baseline). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Forward over a whole sequence. `trace_every` > 0 with a non-NULL `trace`
 * records the state after every trace_every-th token: trace has layout
 * (B, T / trace_every, H, P, N) and entry k is the state after token
 * (k + 1) * trace_every - 1.
 */
int oracle_ssd_fwd(const double *X, const double *dt, const double *A,
                   const double *Bm, const double *Cm, const double *D,
                   const double *init_state, double *Y, double *final_state,
                   double *trace, int64_t trace_every,
                   int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                   int64_t dstate, int64_t ngroups) {
    if (!shapes_ok(batch, seqlen, nheads, headdim, dstate, ngroups)) return ORACLE_EINVAL;
    if (!X || !dt || !A || !Bm || !Cm || !D || !Y) return ORACLE_EINVAL;
    const int64_t H = nheads, P = headdim, N = dstate, G = ngroups, T = seqlen;
    const int64_t ntrace = (trace && trace_every > 0) ? T / trace_every : 0;

    #pragma omp parallel for collapse(3) schedule(static)
    for (int64_t b = 0; b < batch; ++b)
    for (int64_t h = 0; h < H; ++h)
    for (int64_t p = 0; p < P; ++p) {
        const int64_t g = (h * G) / H;
        double *s = (double *)malloc((size_t)N * sizeof(double));
        for (int64_t n = 0; n < N; ++n)
            s[n] = init_state ? init_state[((b * H + h) * P + p) * N + n] : 0.0;
        for (int64_t t = 0; t < T; ++t) {
            const double d = dt[(b * T + t) * H + h];
            const double a = exp(d * A[h]);
            const double x = X[((b * T + t) * H + h) * P + p];
            const double *bt = Bm + ((b * T + t) * G + g) * N;
            const double *ct = Cm + ((b * T + t) * G + g) * N;
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                s[n] = a * s[n] + d * x * bt[n];
                acc += s[n] * ct[n];
            }
            Y[((b * T + t) * H + h) * P + p] = acc + D[h] * x;
            if (ntrace && (t + 1) % trace_every == 0) {
                const int64_t k = (t + 1) / trace_every - 1;
                double *dst = trace + (((b * ntrace + k) * H + h) * P + p) * N;
                memcpy(dst, s, (size_t)N * sizeof(double));
            }
        }
        if (final_state) memcpy(final_state + ((b * H + h) * P + p) * N, s, (size_t)N * sizeof(double));
        free(s);
    }
    return ORACLE_OK;
}

/*
 * One recurrent decode step on a given state (updated in place):
 * x, y (B,H,P); dt (B,H); Bm, Cm (B,G,N); state (B,H,P,N).
 * The constant-size state is the whole carried context of an SSM at
 * inference ("Transformer vs Mamba/SSM", why it matters: O(1) per step).
 */
int oracle_ssd_step(double *state, const double *x, const double *dt, const double *A,
                    const double *Bm, const double *Cm, const double *D, double *y,
                    int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate,
                    int64_t ngroups) {
    if (!shapes_ok(batch, 1, nheads, headdim, dstate, ngroups)) return ORACLE_EINVAL;
    if (!state || !x || !dt || !A || !Bm || !Cm || !D || !y) return ORACLE_EINVAL;
    const int64_t H = nheads, P = headdim, N = dstate, G = ngroups;

    #pragma omp parallel for collapse(3) schedule(static)
    for (int64_t b = 0; b < batch; ++b)
    for (int64_t h = 0; h < H; ++h)
    for (int64_t p = 0; p < P; ++p) {
        const int64_t g = (h * G) / H;
        const double d = dt[b * H + h];
        const double a = exp(d * A[h]);
        const double xv = x[(b * H + h) * P + p];
        const double *bt = Bm + (b * G + g) * N;
        const double *ct = Cm + (b * G + g) * N;
        double *s = state + ((b * H + h) * P + p) * N;
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            s[n] = a * s[n] + d * xv * bt[n];
            acc += s[n] * ct[n];
        }
        y[(b * H + h) * P + p] = acc + D[h] * xv;
    }
    return ORACLE_OK;
}
