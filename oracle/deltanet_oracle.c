/*
 * Token-serial DeltaNet forward pass in fp64 -- the ORACLE.
 *
 * This file is test infrastructure. Only the tests, the smoke check and the
 * CPU-baseline leg of the benchmark load it. It shares no code, header or
 * constant with the HIP library and never runs on the product path.
 *
 * What it computes (column convention, the state S is dv x dk):
 *   "Linear Attention, Visualized" (Haoran Zhang), section "DeltaNet:
 *   correcting memory collisions" > "Recurrent form": for each token t
 *       vhat_t = S_{t-1} k_t                (the value the memory predicts for k_t)
 *       u_t    = beta_t (v_t - vhat_t)      (scaled correction)
 *       S_t    = S_{t-1} + u_t k_t^T        (rank-one write at k_t)
 *       o_t    = S_t q_t                    (read AFTER the write)
 *   The page writes the state as a dk x dv matrix acting on row vectors; the
 *   state kept here is its transpose, as in "Context Parallelism for DeltaNet"
 *   (yywangcs), section 2, chunk-state update equation. The rank-one form equals
 *   S_t = S_{t-1}(I - beta_t k_t k_t^T) + beta_t v_t k_t^T.
 *
 * Gated DeltaNet (same page, section "Gated DeltaNet (GDN)", token recurrence
 * in the first display): the previous state is first multiplied by the
 * token's scalar decay a_t, then corrected as above:
 *       S_t = a_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *   i.e. Sd = a_t S_{t-1}; vhat_t = Sd k_t; S_t = Sd + beta_t (v_t - vhat_t) k_t^T.
 *   The decay is passed as its natural logarithm g_t (a_t = exp(g_t), in
 *   fp64 here); a NULL gate array means a_t = 1 (plain DeltaNet).
 *
 * Layouts (all fp64, row-major, contiguous):
 *   q, k : [B, T, H, dk]     v, o : [B, T, H, dv]     beta, g : [B, T, H]
 *   S0, S_final : [B, H, dv, dk]   (S0 may be NULL: zero initial state)
 * Varlen: B = 1, T = cu_seqlens[N]; sequence n owns tokens
 *   [cu_seqlens[n], cu_seqlens[n+1]); S0/S_final are [N, H, dv, dk]; the state
 *   restarts at every sequence start.
 *
 * Units (b, h) -- or (n, h) -- are independent and run in an OpenMP loop.
 * Return value: 0 on success, -1 on invalid arguments, -2 on allocation failure.
 */
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One (sequence, head) unit. Row r of q/k lives at q + r*qk_stride, of v/o at
 * v + r*vo_stride, beta_r at beta[r*beta_stride] and g_r (log decay, or NULL)
 * at g[r*beta_stride]. S is dv x dk, updated in place. */
static void unit_forward(const double *q, const double *k, const double *v,
                         const double *beta, const double *g, double *o, ptrdiff_t qk_stride,
                         ptrdiff_t vo_stride, ptrdiff_t beta_stride, int64_t L,
                         int dk, int dv, double *S, double *vhat)
{
    for (int64_t t = 0; t < L; ++t) {
        const double *kt = k + t * qk_stride;
        const double *qt = q + t * qk_stride;
        const double *vt = v + t * vo_stride;
        const double bt = beta[t * beta_stride];
        /* decay of the previous state: S <- a_t S */
        if (g) {
            const double at = exp(g[t * beta_stride]);
            for (size_t e = 0; e < (size_t)dv * dk; ++e) S[e] *= at;
        }
        /* prediction: vhat = S k_t */
        for (int i = 0; i < dv; ++i) {
            const double *Si = S + (size_t)i * dk;
            double acc = 0.0;
            for (int j = 0; j < dk; ++j) acc += Si[j] * kt[j];
            vhat[i] = acc;
        }
        /* write: S += beta_t (v_t - vhat) k_t^T */
        for (int i = 0; i < dv; ++i) {
            double *Si = S + (size_t)i * dk;
            const double ui = bt * (vt[i] - vhat[i]);
            for (int j = 0; j < dk; ++j) Si[j] += ui * kt[j];
        }
        /* read-out after the write: o_t = S_t q_t */
        if (o) {
            double *ot = o + t * vo_stride;
            for (int i = 0; i < dv; ++i) {
                const double *Si = S + (size_t)i * dk;
                double acc = 0.0;
                for (int j = 0; j < dk; ++j) acc += Si[j] * qt[j];
                ot[i] = acc;
            }
        }
    }
}

static int run_units(const double *q, const double *k, const double *v,
                     const double *beta, const double *g, const double *S0, double *o,
                     double *S_final, int64_t n_units, int H, int dk, int dv,
                     const int64_t *starts, const int64_t *lens, int nthreads)
{
    const ptrdiff_t qk_stride = (ptrdiff_t)H * dk;
    const ptrdiff_t vo_stride = (ptrdiff_t)H * dv;
    const size_t sz = (size_t)dv * dk;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double *S = (double *)malloc(sizeof(double) * (sz + (size_t)dv));
        if (!S) {
#pragma omp atomic write
            failed = 1;
        } else {
            double *vhat = S + sz;
#pragma omp for schedule(dynamic, 1)
            for (int64_t u = 0; u < n_units; ++u) {
                const int64_t seq = u / H;
                const int h = (int)(u % H);
                const int64_t t0 = starts[seq];
                if (S0) memcpy(S, S0 + (size_t)u * sz, sizeof(double) * sz);
                else memset(S, 0, sizeof(double) * sz);
                unit_forward(q + t0 * qk_stride + (ptrdiff_t)h * dk,
                             k + t0 * qk_stride + (ptrdiff_t)h * dk,
                             v + t0 * vo_stride + (ptrdiff_t)h * dv,
                             beta + t0 * H + h,
                             g ? g + t0 * H + h : NULL,
                             o ? o + t0 * vo_stride + (ptrdiff_t)h * dv : NULL,
                             qk_stride, vo_stride, H, lens[seq], dk, dv, S, vhat);
                if (S_final) memcpy(S_final + (size_t)u * sz, S, sizeof(double) * sz);
            }
            free(S);
        }
    }
    return failed ? -2 : 0;
}

static int dense_fwd(const double *q, const double *k, const double *v,
                     const double *beta, const double *g, const double *S0, double *o,
                     double *S_final, int B, int H, int64_t T, int dk, int dv,
                     int nthreads)
{
    if (!q || !k || !v || !beta || B <= 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0)
        return -1;
    int64_t *starts = (int64_t *)malloc(sizeof(int64_t) * 2 * (size_t)B);
    if (!starts) return -2;
    int64_t *lens = starts + B;
    for (int b = 0; b < B; ++b) { starts[b] = (int64_t)b * T; lens[b] = T; }
    int rc = run_units(q, k, v, beta, g, S0, o, S_final, (int64_t)B * H, H, dk, dv,
                       starts, lens, nthreads);
    free(starts);
    return rc;
}

static int varlen_fwd(const double *q, const double *k, const double *v,
                      const double *beta, const double *g, const double *S0, double *o,
                      double *S_final, const int64_t *cu_seqlens, int N,
                      int H, int dk, int dv, int nthreads)
{
    if (!q || !k || !v || !beta || !cu_seqlens || N <= 0 || H <= 0 || dk <= 0 || dv <= 0)
        return -1;
    for (int n = 0; n < N; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    int64_t *starts = (int64_t *)malloc(sizeof(int64_t) * 2 * (size_t)N);
    if (!starts) return -2;
    int64_t *lens = starts + N;
    for (int n = 0; n < N; ++n) {
        starts[n] = cu_seqlens[n];
        lens[n] = cu_seqlens[n + 1] - cu_seqlens[n];
    }
    int rc = run_units(q, k, v, beta, g, S0, o, S_final, (int64_t)N * H, H, dk, dv,
                       starts, lens, nthreads);
    free(starts);
    return rc;
}

/* DeltaNet (no decay). */
int oracle_deltanet_fwd(const double *q, const double *k, const double *v,
                        const double *beta, const double *S0, double *o,
                        double *S_final, int B, int H, int64_t T, int dk, int dv,
                        int nthreads)
{
    return dense_fwd(q, k, v, beta, NULL, S0, o, S_final, B, H, T, dk, dv, nthreads);
}

int oracle_deltanet_fwd_varlen(const double *q, const double *k, const double *v,
                               const double *beta, const double *S0, double *o,
                               double *S_final, const int64_t *cu_seqlens, int N,
                               int H, int dk, int dv, int nthreads)
{
    return varlen_fwd(q, k, v, beta, NULL, S0, o, S_final, cu_seqlens, N, H, dk, dv, nthreads);
}

/* Gated DeltaNet: g holds log a_t, same layout as beta (required). */
int oracle_gated_deltanet_fwd(const double *q, const double *k, const double *v,
                              const double *beta, const double *g, const double *S0,
                              double *o, double *S_final, int B, int H, int64_t T, int dk,
                              int dv, int nthreads)
{
    if (!g) return -1;
    return dense_fwd(q, k, v, beta, g, S0, o, S_final, B, H, T, dk, dv, nthreads);
}

int oracle_gated_deltanet_fwd_varlen(const double *q, const double *k, const double *v,
                                     const double *beta, const double *g, const double *S0,
                                     double *o, double *S_final, const int64_t *cu_seqlens,
                                     int N, int H, int dk, int dv, int nthreads)
{
    if (!g) return -1;
    return varlen_fwd(q, k, v, beta, g, S0, o, S_final, cu_seqlens, N, H, dk, dv, nthreads);
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
