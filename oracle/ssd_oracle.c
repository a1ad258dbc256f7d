/*
 * CPU oracle for the Mamba-2 SSD selective scan and its cached decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no source, header or table with the HIP
 * library.
 *
 * What it computes.  State-space duality makes A a single scalar per head, so
 * the discretised transition of the selective recurrence is one scalar
 * exponential per token and head ("Compiler-First State Space Duality and
 * Portable O(1) Autoregressive Caching for Inference", paperlayer summary,
 * §3 Method, "State-space duality"; B, C and the step size are inputs that vary
 * per token).  With a = A[h], g the group of head h (heads split into ngroups
 * contiguous blocks), for each batch row b, head h and channel p:
 *
 *     s     <- init_state[b,h,p,:]            (zero when no init state)
 *     for t = 0 .. L-1:
 *         r      = exp(dt[b,t,h] * a)
 *         s[n]   = r * s[n] + dt[b,t,h] * x[b,t,h,p] * B[b,t,g,n]
 *         y[b,t,h,p] = sum_n C[b,t,g,n] * s[n] + D[h] * x[b,t,h,p]
 *     final_state[b,h,p,:] = s
 *
 * The output of token t therefore uses the state after token t's own update.
 * The decode step is the loop body once, with the state carried between calls
 * ("Compiler-First ...", §3 "Autoregressive cache": a fixed-size state makes
 * each next-token update independent of the prefix length).  The chunk size of
 * the chunked algorithm does not appear here: the recurrence is its definition.
 *
 * All arithmetic is IEEE double.  Rows (b, h, p) are independent and are the
 * only thing run in parallel (OpenMP); inside a row the order is the token
 * order above.  Build without fast-math and without FMA contraction.
 *
 * Layouts (row-major, contiguous):
 *   x [Bt,L,H,P]  dt [Bt,L,H]  A [H]  B,C [Bt,L,G,N]  D [H]
 *   init, final [Bt,H,P,N]  y [Bt,L,H,P]
 * Decode step:  state [Bt,H,P,N] (in/out)  x [Bt,H,P]  dt [Bt,H]
 *   B,C [Bt,G,N]  y [Bt,H,P]
 */
#include <math.h>
#include <stdlib.h>
#include <stddef.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One token of one (b,h,p) row: update the N-vector state in place and return
 * the output.  Shared by the scan and the step so that L steps reproduce the
 * scan exactly. */
static double row_update(double *s, int64_t N, double dt, double a, double xv,
                         const double *Bt_row, const double *Ct_row, double Dh)
{
    const double r = exp(dt * a);
    const double u = dt * xv;
    double acc = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        s[n] = r * s[n] + u * Bt_row[n];
        acc += Ct_row[n] * s[n];
    }
    return acc + Dh * xv;
}

static int bad_shape(int64_t Bt, int64_t H, int64_t P, int64_t N, int64_t G)
{
    return Bt < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0;
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* Returns the number of threads OpenMP will use for the next parallel region. */
int ssd_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Full-sequence scan.  D, init and final_state may be NULL (D, init -> 0;
 * final -> not written).  Returns 0, -1 for an invalid shape, or -2 when the
 * per-thread state rows cannot be allocated (nothing is written then). */
int ssd_oracle_scan(int64_t Bt, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                    const double *x, const double *dt, const double *A,
                    const double *Bm, const double *Cm, const double *D,
                    const double *init, double *y, double *final_state, int nthreads)
{
    if (bad_shape(Bt, H, P, N, G) || L < 0) return -1;
    set_threads(nthreads);
    const int64_t R = H / G;
    const int64_t rows = Bt * H * P;
    /* one state row per thread, allocated (and checked) before the threads start */
    const int nt = ssd_oracle_max_threads();
    double *srows = (double *)malloc((size_t)(nt > 0 ? nt : 1) * (size_t)N * sizeof(double));
    if (!srows) return -2;
#pragma omp parallel
    {
#ifdef _OPENMP
        double *s = srows + (size_t)omp_get_thread_num() * (size_t)N;
#else
        double *s = srows;
#endif
#pragma omp for schedule(static)
        for (int64_t row = 0; row < rows; ++row) {
            const int64_t p = row % P;
            const int64_t h = (row / P) % H;
            const int64_t b = row / (P * H);
            const int64_t g = h / R;
            const double a = A[h];
            const double Dh = D ? D[h] : 0.0;
            const int64_t sbase = ((b * H + h) * P + p) * N;
            for (int64_t n = 0; n < N; ++n) s[n] = init ? init[sbase + n] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                const int64_t bt = b * L + t;
                const double dtv = dt[bt * H + h];
                const double xv = x[(bt * H + h) * P + p];
                const double *Brow = Bm + (bt * G + g) * N;
                const double *Crow = Cm + (bt * G + g) * N;
                y[(bt * H + h) * P + p] = row_update(s, N, dtv, a, xv, Brow, Crow, Dh);
            }
            if (final_state)
                for (int64_t n = 0; n < N; ++n) final_state[sbase + n] = s[n];
        }
    }
    free(srows);
    return 0;
}

/* One cached decode step for every (b,h,p) row; the state is updated in place.
 * D may be NULL.  Returns 0, or -1 for an invalid shape. */
int ssd_oracle_step(int64_t Bt, int64_t H, int64_t P, int64_t N, int64_t G,
                    double *state, const double *x, const double *dt, const double *A,
                    const double *Bm, const double *Cm, const double *D, double *y,
                    int nthreads)
{
    if (bad_shape(Bt, H, P, N, G)) return -1;
    set_threads(nthreads);
    const int64_t R = H / G;
    const int64_t rows = Bt * H * P;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < rows; ++row) {
        const int64_t h = (row / P) % H;
        const int64_t b = row / (P * H);
        const int64_t g = h / R;
        y[row] = row_update(state + row * N, N, dt[b * H + h], A[h], x[row],
                            Bm + (b * G + g) * N, Cm + (b * G + g) * N, D ? D[h] : 0.0);
    }
    return 0;
}

/* Gradients of the scan (its vector-Jacobian product).  For the scalar
 *     J = sum(dy * y) + sum(dfinal * final_state)
 * the gradient with respect to every input, by the adjoint recurrence of the
 * loop above run backwards in time.  Per (b, h, p) row, with lam the
 * derivative of J with respect to the state s_t after token t:
 *
 *     lam   <- dfinal[b,h,p,:]                    (zero when dfinal is NULL)
 *     for t = L-1 .. 0:   (r_t = exp(dt_t a), s_t the forward state, s_{-1} = init)
 *         lam[n]  += dy[t,p] * C_t[n]              (y_t reads s_t)
 *         dx[t,p]  = dt_t * sum_n B_t[n] lam[n] + D * dy[t,p]
 *         dB_t[n] += dt_t * x[t,p] * lam[n]        (summed over heads of the group)
 *         dC_t[n] += dy[t,p] * s_t[n]
 *         ddt_t   += sum_n lam[n] * (x[t,p] B_t[n] + a r_t s_{t-1}[n])
 *         dA      += sum_n lam[n] * dt_t r_t s_{t-1}[n]
 *         dD      += dy[t,p] * x[t,p]
 *         lam[n]  *= r_t                           (s_t = r_t s_{t-1} + ...)
 *     dinit[b,h,p,:] = lam
 *
 * since s_t = r_t s_{t-1} + dt_t x_t B_t with r_t = exp(dt_t a) gives
 * ds_t/ddt_t = a r_t s_{t-1} + x_t B_t and ds_t/da = dt_t r_t s_{t-1}.  The
 * forward states of a row are recomputed and kept (L+1 vectors of N).
 * Parallel over batch rows only; heads, channels and the per-head sums over
 * batch rows run in a fixed order, so the result is deterministic.
 * dfinal, D and init may be NULL; every output is written (dD even when D is
 * NULL).  Returns 0, -1 for an invalid shape, -2 when out of memory. */
int ssd_oracle_scan_vjp(int64_t Bt, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                        const double *x, const double *dt, const double *A,
                        const double *Bm, const double *Cm, const double *D,
                        const double *init, const double *dy, const double *dfinal,
                        double *dx, double *ddt, double *dA, double *dB, double *dC,
                        double *dD, double *dinit, int nthreads)
{
    if (bad_shape(Bt, H, P, N, G) || L < 0) return -1;
    set_threads(nthreads);
    const int64_t R = H / G;
    /* per batch row partial sums of dA and dD, reduced in order afterwards */
    double *pA = (double *)calloc((size_t)(Bt > 0 ? Bt : 1) * H, sizeof(double));
    double *pD = (double *)calloc((size_t)(Bt > 0 ? Bt : 1) * H, sizeof(double));
    if (!pA || !pD) { free(pA); free(pD); return -2; }
    for (int64_t i = 0; i < Bt * L * G * N; ++i) { dB[i] = 0.0; dC[i] = 0.0; }
    for (int64_t i = 0; i < Bt * L * H; ++i) ddt[i] = 0.0;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(|:err)
    for (int64_t b = 0; b < Bt; ++b) {
        double *S = (double *)malloc((size_t)(L + 1) * N * sizeof(double));
        double *lam = (double *)malloc((size_t)N * sizeof(double));
        if (!S || !lam) { free(S); free(lam); err |= 1; continue; }
        for (int64_t h = 0; h < H; ++h) {
            const int64_t g = h / R;
            const double a = A[h];
            const double Dh = D ? D[h] : 0.0;
            for (int64_t p = 0; p < P; ++p) {
                const int64_t sbase = ((b * H + h) * P + p) * N;
                /* forward states: S[t+1] is s_t, S[0] is s_{-1} */
                for (int64_t n = 0; n < N; ++n) S[n] = init ? init[sbase + n] : 0.0;
                for (int64_t t = 0; t < L; ++t) {
                    const int64_t bt = b * L + t;
                    const double dtv = dt[bt * H + h];
                    const double r = exp(dtv * a);
                    const double u = dtv * x[(bt * H + h) * P + p];
                    const double *Brow = Bm + (bt * G + g) * N;
                    for (int64_t n = 0; n < N; ++n)
                        S[(t + 1) * N + n] = r * S[t * N + n] + u * Brow[n];
                }
                for (int64_t n = 0; n < N; ++n) lam[n] = dfinal ? dfinal[sbase + n] : 0.0;
                for (int64_t t = L - 1; t >= 0; --t) {
                    const int64_t bt = b * L + t;
                    const double dtv = dt[bt * H + h];
                    const double r = exp(dtv * a);
                    const double xv = x[(bt * H + h) * P + p];
                    const double dyv = dy[(bt * H + h) * P + p];
                    const double *Brow = Bm + (bt * G + g) * N;
                    const double *Crow = Cm + (bt * G + g) * N;
                    const double *s_t = S + (t + 1) * N, *s_prev = S + t * N;
                    double *dBrow = dB + (bt * G + g) * N, *dCrow = dC + (bt * G + g) * N;
                    double bl = 0.0, ddt_acc = 0.0, da_acc = 0.0;
                    for (int64_t n = 0; n < N; ++n) {
                        lam[n] += dyv * Crow[n];
                        bl += Brow[n] * lam[n];
                        dBrow[n] += dtv * xv * lam[n];
                        dCrow[n] += dyv * s_t[n];
                        ddt_acc += lam[n] * (xv * Brow[n] + a * r * s_prev[n]);
                        da_acc += lam[n] * dtv * r * s_prev[n];
                    }
                    dx[(bt * H + h) * P + p] = dtv * bl + Dh * dyv;
                    ddt[bt * H + h] += ddt_acc;
                    pA[b * H + h] += da_acc;
                    pD[b * H + h] += dyv * xv;
                    for (int64_t n = 0; n < N; ++n) lam[n] *= r;
                }
                if (dinit)
                    for (int64_t n = 0; n < N; ++n) dinit[sbase + n] = lam[n];
            }
        }
        free(S);
        free(lam);
    }
    for (int64_t h = 0; h < H; ++h) {
        double sa = 0.0, sd = 0.0;
        for (int64_t b = 0; b < Bt; ++b) { sa += pA[b * H + h]; sd += pD[b * H + h]; }
        dA[h] = sa;
        if (dD) dD[h] = sd;
    }
    free(pA);
    free(pD);
    return err ? -2 : 0;
}
