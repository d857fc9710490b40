/*
 * fp64 CPU oracle for the gradient of the SSD forward pass: the reverse-mode adjoint of the
 * recurrence that ssd_oracle.c runs forward.  TEST INFRASTRUCTURE ONLY: the tests, the smoke
 * check and the CPU baseline leg of the benchmark may call it; the product path never does.
 *
 * Forward (per batch b and head h, group g = h / (H/G)), as in ssd_oracle.c:
 *   h_{-1} = init_state[b,h] (zeros when NULL)
 *   h_t    = a_t h_{t-1} + B_t x_t^T,  a_t = exp(log_a[b,t,h])  (or exp(log_a[b,t,h,n]) per n)
 *   y_t    = C_t^T h_t + D_h x_t,      final = h_{T-1}
 *
 * Given dy = dL/dy and dfinal = dL/dfinal (zeros when NULL), the adjoint runs the chain rule
 * backwards through those steps, with G = dL/dh_t:
 *   G = dfinal
 *   for t = T-1 .. 0:
 *     G        += C_t dy_t^T                       (y_t reads h_t)
 *     dx_t      = G^T B_t + D_h dy_t               (h_t takes B_t x_t^T; y_t takes D x_t)
 *     dB_t     += G x_t        (summed over the heads of the group, which share B_t)
 *     dC_t     += h_t dy_t     (likewise for C_t)
 *     dlog_a_t  = sum_{n,p} a_t G[n,p] h_{t-1}[n,p]   (d a_t / d log a_t = a_t; per n for the
 *                                                      diagonal decay, summed over p only)
 *     G         = a_t G                            (h_{t-1} reaches h_t through a_t)
 *   dinit = G,   dD_h = sum_{b,t} dy_t . x_t
 *
 * Sources: the recurrence is the one of llms.blog "State Space Models and Mamba" sections
 * "Continuous-to-Discrete Discretization" and "The SSD Theoretical Equivalence"; the backward
 * pass is the chain rule through it, nothing the pages print.
 *
 * Plain loops: the forward states h_t of one head are kept whole (T * N * P doubles), then the
 * sweep above runs once.  Parallel over (batch, group) pairs; the heads of a group run in order
 * inside, so the sums over heads are taken in a fixed order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int ssd_oracle_backward(int64_t nbatch, int64_t T, int64_t H, int64_t G, int64_t P, int64_t N,
                        int diag, const double* x, const double* log_a, const double* Bm,
                        const double* Cm, const double* D, const double* init_state,
                        const double* dy, const double* dfinal, double* dx, double* dlog_a,
                        double* dB, double* dC, double* dD, double* dinit, int nthreads)
{
    if (nbatch < 0 || T < 0 || H <= 0 || G <= 0 || P <= 0 || N <= 0 || H % G != 0) return -1;
    if (nthreads <= 0) nthreads = 1;
    const int64_t hpg = H / G;
    const int64_t K = diag ? N : 1; /* decays per (b, t, h) */
    double* dD_part = (double*)calloc((size_t)(nbatch * H > 0 ? nbatch * H : 1), sizeof(double));
    if (!dD_part) return -2;
    memset(dB, 0, (size_t)(nbatch * T * G * N) * sizeof(double));
    memset(dC, 0, (size_t)(nbatch * T * G * N) * sizeof(double));
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t bg = 0; bg < nbatch * G; ++bg) {
        const int64_t b = bg / G, g = bg % G;
        double* hs = (double*)malloc((size_t)((T + 1) * N * P) * sizeof(double));
        double* Gs = (double*)malloc((size_t)(N * P) * sizeof(double));
        double* a = (double*)malloc((size_t)N * sizeof(double));
        if (!hs || !Gs || !a) {
            free(hs);
            free(Gs);
            free(a);
#pragma omp atomic write
            failed = 1;
            continue;
        }
        for (int64_t hd = g * hpg; hd < (g + 1) * hpg; ++hd) {
            /* forward: hs[t + 1] = h_t, hs[0] = h_{-1} */
            for (int64_t i = 0; i < N * P; ++i)
                hs[i] = init_state ? init_state[(b * H + hd) * N * P + i] : 0.0;
            for (int64_t t = 0; t < T; ++t) {
                const int64_t row = (b * T + t) * H + hd;
                const double* xt = x + row * P;
                const double* bt = Bm + ((b * T + t) * G + g) * N;
                const double* prev = hs + t * N * P;
                double* cur = hs + (t + 1) * N * P;
                for (int64_t n = 0; n < N; ++n) {
                    const double an = exp(log_a[row * K + (diag ? n : 0)]);
                    for (int64_t p = 0; p < P; ++p) cur[n * P + p] = an * prev[n * P + p] + bt[n] * xt[p];
                }
            }
            /* reverse sweep */
            for (int64_t i = 0; i < N * P; ++i) Gs[i] = dfinal ? dfinal[(b * H + hd) * N * P + i] : 0.0;
            double dDh = 0.0;
            for (int64_t t = T - 1; t >= 0; --t) {
                const int64_t row = (b * T + t) * H + hd;
                const double* xt = x + row * P;
                const double* dyt = dy + row * P;
                const double* bt = Bm + ((b * T + t) * G + g) * N;
                const double* ct = Cm + ((b * T + t) * G + g) * N;
                const double* ht = hs + (t + 1) * N * P;
                const double* hprev = hs + t * N * P;
                double* dbt = dB + ((b * T + t) * G + g) * N;
                double* dct = dC + ((b * T + t) * G + g) * N;
                for (int64_t n = 0; n < N; ++n)
                    for (int64_t p = 0; p < P; ++p) Gs[n * P + p] += ct[n] * dyt[p];
                for (int64_t p = 0; p < P; ++p) {
                    double acc = D ? D[hd] * dyt[p] : 0.0;
                    for (int64_t n = 0; n < N; ++n) acc += Gs[n * P + p] * bt[n];
                    dx[row * P + p] = acc;
                }
                for (int64_t n = 0; n < N; ++n) {
                    double gb = 0.0, gc = 0.0;
                    for (int64_t p = 0; p < P; ++p) {
                        gb += Gs[n * P + p] * xt[p];
                        gc += ht[n * P + p] * dyt[p];
                    }
                    dbt[n] += gb;
                    dct[n] += gc;
                }
                for (int64_t n = 0; n < N; ++n) a[n] = exp(log_a[row * K + (diag ? n : 0)]);
                if (diag) {
                    for (int64_t n = 0; n < N; ++n) {
                        double acc = 0.0;
                        for (int64_t p = 0; p < P; ++p) acc += Gs[n * P + p] * hprev[n * P + p];
                        dlog_a[row * N + n] = a[n] * acc;
                    }
                } else {
                    double acc = 0.0;
                    for (int64_t i = 0; i < N * P; ++i) acc += Gs[i] * hprev[i];
                    dlog_a[row] = a[0] * acc;
                }
                for (int64_t n = 0; n < N; ++n)
                    for (int64_t p = 0; p < P; ++p) Gs[n * P + p] *= a[n];
                for (int64_t p = 0; p < P; ++p) dDh += dyt[p] * xt[p];
            }
            if (dinit)
                for (int64_t i = 0; i < N * P; ++i) dinit[(b * H + hd) * N * P + i] = Gs[i];
            dD_part[b * H + hd] = dDh;
        }
        free(hs);
        free(Gs);
        free(a);
    }
    if (dD)
        for (int64_t hd = 0; hd < H; ++hd) {
            double acc = 0.0;
            for (int64_t b = 0; b < nbatch; ++b) acc += dD_part[b * H + hd];
            dD[hd] = acc;
        }
    free(dD_part);
    return failed ? -2 : 0;
}
