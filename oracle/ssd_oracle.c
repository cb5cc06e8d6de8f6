/*
 * Token-by-token SSD recurrence in double precision, plain C + OpenMP.
 * TEST INFRASTRUCTURE ONLY: called by the test suite, the smoke check and the benchmark's
 * CPU-baseline leg; nothing in the GPU library links or calls it, and it shares no code with it.
 *
 * Per (batch, head), with state S[P][N] (head-dim rows, state columns):
 *     a      = exp(dt[t,h] * A[h])                         one scalar decay per head and step
 *     S      = a * S + dt[t,h] * outer(x[t,h,:], B[t,g,:])
 *     y[t,h] = S @ C[t,g,:] + D[h] * x[t,h,:]
 * the selective state-space step of "Why SSM and linear-RNN FLOPs do not convert into GPU FLOPs"
 * (first paragraph) with the decay shared across the head, in its Mamba-2 SSD form.
 *
 * Inputs are float (bf16 workloads pass their values widened to float, which is exact) and are
 * widened to double; the initial state is double (so a carried state resumes exactly); outputs
 * are double. Layouts are row-major:
 *     x [Bt,L,H,P]  dt [Bt,L,H]  A [H]  B, C [Bt,L,G,N]  D [H]  h0, final [Bt,H,P,N]  y [Bt,L,H,P]
 * `units` / `nunits` optionally restrict the work to a list of (batch*H + head) indices, so a bounded
 * sample of a large workload can be timed; y and final are written only for those units.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int ssd_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

int ssd_oracle_forward(int64_t Bt, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                       const float* x, const float* dt, const float* A, const float* B,
                       const float* C, const float* D, const double* h0,
                       double* y, double* final_state,
                       const int64_t* units, int64_t nunits, int nthreads) {
    if (Bt <= 0 || L <= 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G) return 1;
    const int64_t per_group = H / G;
    const int64_t total = units ? nunits : Bt * H;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (int64_t k = 0; k < total; ++k) {
        const int64_t unit = units ? units[k] : k;
        const int64_t b = unit / H, h = unit % H, g = h / per_group;
        double* S = (double*)malloc((size_t)(P * N) * sizeof(double));
        double* u = (double*)malloc((size_t)P * sizeof(double));
        double* bn = (double*)malloc((size_t)N * sizeof(double));
        double* cn = (double*)malloc((size_t)N * sizeof(double));
        if (!S || !u || !bn || !cn) {
            failed |= 1;
        } else {
            for (int64_t i = 0; i < P * N; ++i)
                S[i] = h0 ? h0[(b * H + h) * P * N + i] : 0.0;
            const double a_h = (double)A[h], d_h = (double)D[h];
            for (int64_t t = 0; t < L; ++t) {
                const double dtv = (double)dt[(b * L + t) * H + h];
                const double a = exp(dtv * a_h);
                const float* xt = x + ((b * L + t) * H + h) * P;
                const float* bt = B + ((b * L + t) * G + g) * N;
                const float* ct = C + ((b * L + t) * G + g) * N;
                for (int64_t n = 0; n < N; ++n) { bn[n] = bt[n]; cn[n] = ct[n]; }
                for (int64_t p = 0; p < P; ++p) u[p] = dtv * (double)xt[p];
                double* yt = y + ((b * L + t) * H + h) * P;
                for (int64_t p = 0; p < P; ++p) {
                    double* Sp = S + p * N;
                    double acc = 0.0;
                    for (int64_t n = 0; n < N; ++n) {
                        Sp[n] = a * Sp[n] + u[p] * bn[n];
                        acc += Sp[n] * cn[n];
                    }
                    yt[p] = acc + d_h * (double)xt[p];
                }
            }
            if (final_state)
                memcpy(final_state + (b * H + h) * P * N, S, (size_t)(P * N) * sizeof(double));
        }
        free(S); free(u); free(bn); free(cn);
    }
    return failed ? 2 : 0;
}
