/*
 * fp64 CPU oracle for the selective state-space recurrence that the chunked SSD forward
 * computes faster.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU
 * baseline leg of the benchmark may call it; the product path never does.
 *
 * What it computes (per batch b and head h, with group g = h / (H/G)):
 *
 *   h_0 = init_state[b,h]            (zeros when init_state is NULL)
 *   for t = 0 .. T-1:
 *     a_t        = exp(log_a[b,t,h])         scalar decay      (or exp(log_a[b,t,h,n]) per n)
 *     h_t[n,p]   = a_t * h_{t-1}[n,p] + B[b,t,g,n] * x[b,t,h,p]
 *     y[b,t,h,p] = sum_n C[b,t,g,n] * h_t[n,p] + D[h] * x[b,t,h,p]
 *   final_state[b,h] = h_T
 *
 * Sources (State Space Models and Mamba, llms.blog): the discrete recurrence h_t = A h_{t-1}
 * + B x_t, y_t = C h_t + D x_t in "Continuous-to-Discrete Discretization"; the scalar-times-
 * identity transition A_t = a_t I and the state-space view h_t = a_t h_{t-1} + K_t^T V_t,
 * y_t = Q_t h_t in "The SSD Theoretical Equivalence"; heads D = H*P with B, C shared by a
 * group of heads in "Multi-Head State Space Layers".  The diagonal transition (one decay per
 * state dimension) is the generalisation of "On Structured State-Space Duality" (ICML 2026
 * poster, abstract item (i)).
 *
 * Plain sequential loops, no blocking, no reordering: every output element is summed in
 * the order written above.  Decode (one token at a time) is this same loop run for T = 1
 * with init_state set to the running state.
 *
 * Layouts (row-major, last index fastest):
 *   x [B,T,H,P]  log_a [B,T,H] or [B,T,H,N]  Bm, Cm [B,T,G,N]  D [H]  init/final [B,H,N,P]
 *   y [B,T,H,P]
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int ssd_oracle_forward(int64_t nbatch, int64_t T, int64_t H, int64_t G, int64_t P, int64_t N,
                       int diag, const double* x, const double* log_a, const double* Bm,
                       const double* Cm, const double* D, const double* init_state, double* y,
                       double* final_state, int nthreads)
{
    if (nbatch < 0 || T < 0 || H <= 0 || G <= 0 || P <= 0 || N <= 0 || H % G != 0) return -1;
    if (nthreads <= 0) nthreads = 1;
    const int64_t heads_per_group = H / G;
    const int64_t units = nbatch * H;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t u = 0; u < units; ++u) {
        const int64_t b = u / H;
        const int64_t hd = u % H;
        const int64_t g = hd / heads_per_group;
        double* state = (double*)malloc((size_t)(N * P) * sizeof(double));
        double* decay = (double*)malloc((size_t)N * sizeof(double));
        if (!state || !decay) {
            free(state);
            free(decay);
#pragma omp atomic write
            failed = 1;
            continue;
        }
        for (int64_t n = 0; n < N; ++n)
            for (int64_t p = 0; p < P; ++p)
                state[n * P + p] = init_state ? init_state[((b * H + hd) * N + n) * P + p] : 0.0;

        for (int64_t t = 0; t < T; ++t) {
            const int64_t row = (b * T + t) * H + hd; /* index of (b,t,h) */
            const double* xt = x + row * P;
            const double* bt = Bm + ((b * T + t) * G + g) * N;
            const double* ct = Cm + ((b * T + t) * G + g) * N;
            for (int64_t n = 0; n < N; ++n)
                decay[n] = diag ? exp(log_a[row * N + n]) : exp(log_a[row]);
            /* state update: h_t = a_t h_{t-1} + B_t x_t^T */
            for (int64_t n = 0; n < N; ++n)
                for (int64_t p = 0; p < P; ++p)
                    state[n * P + p] = decay[n] * state[n * P + p] + bt[n] * xt[p];
            /* readout: y_t = C_t^T h_t + D x_t */
            double* yt = y + row * P;
            for (int64_t p = 0; p < P; ++p) {
                double acc = D ? D[hd] * xt[p] : 0.0;
                for (int64_t n = 0; n < N; ++n) acc += ct[n] * state[n * P + p];
                yt[p] = acc;
            }
        }
        if (final_state)
            for (int64_t n = 0; n < N; ++n)
                for (int64_t p = 0; p < P; ++p)
                    final_state[((b * H + hd) * N + n) * P + p] = state[n * P + p];
        free(state);
        free(decay);
    }
    return failed ? -2 : 0;
}

/* Number of OpenMP threads the oracle would use by default (for reporting). */
int ssd_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
