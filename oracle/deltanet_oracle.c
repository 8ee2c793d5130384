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

/*
 * Kimi Delta Attention (KDA), "Linear Attention, Visualized", section "Kimi
 * Delta Attention (KDA)": the previous state first decays channel by channel
 * (one decay a_{t,j} = exp(g_{t,j}) per key channel j), then the delta-rule
 * correction applies. In the column convention (S is dv x dk, key channels
 * are columns):
 *     Sd = S_{t-1} Diag(a_t);  vhat = Sd k_t;  S_t = Sd + beta_t (v_t - vhat) k_t^T;  o_t = S_t q_t.
 * g: [B, T, H, dk] (log decays per channel).
 */
static void unit_forward_kda(const double *q, const double *k, const double *v, const double *beta,
                             const double *g, double *o, ptrdiff_t qk_stride, ptrdiff_t vo_stride,
                             ptrdiff_t beta_stride, int64_t L, int dk, int dv, double *S, double *vhat)
{
    for (int64_t t = 0; t != L; ++t) {
        const double *kt = k + t * qk_stride, *qt = q + t * qk_stride, *vt = v + t * vo_stride;
        const double *gt = g + t * qk_stride;
        const double bt = beta[t * beta_stride];
        for (int i = 0; i < dv; ++i)
            for (int j = 0; j < dk; ++j) S[(size_t)i * dk + j] *= exp(gt[j]);
        for (int i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dk; ++j) acc += S[(size_t)i * dk + j] * kt[j];
            vhat[i] = acc;
        }
        for (int i = 0; i < dv; ++i) {
            const double corr = bt * (vt[i] - vhat[i]);
            for (int j = 0; j < dk; ++j) S[(size_t)i * dk + j] += corr * kt[j];
        }
        if (o) {
            double *ot = o + t * vo_stride;
            for (int i = 0; i < dv; ++i) {
                double acc = 0.0;
                for (int j = 0; j < dk; ++j) acc += S[(size_t)i * dk + j] * qt[j];
                ot[i] = acc;
            }
        }
    }
}

int oracle_kda_fwd(const double *q, const double *k, const double *v, const double *beta, const double *g,
                   const double *S0, double *o, double *S_final, int B, int H, int64_t T, int dk, int dv,
                   int nthreads)
{
    if (!q || !k || !v || !beta || !g || B <= 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0) return -1;
    const ptrdiff_t qk_stride = (ptrdiff_t)H * dk, vo_stride = (ptrdiff_t)H * dv;
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
#pragma omp for schedule(dynamic, 1)
            for (int64_t u = 0; u < (int64_t)B * H; ++u) {
                const int64_t b = u / H;
                const int h = (int)(u % H);
                const int64_t t0 = b * T;
                if (S0) memcpy(S, S0 + (size_t)u * sz, sizeof(double) * sz);
                else memset(S, 0, sizeof(double) * sz);
                unit_forward_kda(q + t0 * qk_stride + (ptrdiff_t)h * dk, k + t0 * qk_stride + (ptrdiff_t)h * dk,
                                 v + t0 * vo_stride + (ptrdiff_t)h * dv, beta + t0 * H + h,
                                 g + t0 * qk_stride + (ptrdiff_t)h * dk,
                                 o ? o + t0 * vo_stride + (ptrdiff_t)h * dv : NULL, qk_stride, vo_stride, H, T, dk,
                                 dv, S, S + sz);
                if (S_final) memcpy(S_final + (size_t)u * sz, S, sizeof(double) * sz);
            }
            free(S);
        }
    }
    return failed ? -2 : 0;
}

/*
 * Backward pass of the DeltaNet recurrence (reverse mode of the token-serial
 * definition above, in fp64). For a loss with upstream gradients dO_t of the
 * outputs and dS_T of the final state, reading the recurrence backwards:
 *   G  <- dS_T                                   (gradient of S_T)
 *   for t = T .. 1:
 *     G  += dO_t q_t^T ;      dq_t = S_t^T dO_t          (o_t = S_t q_t)
 *     r_t = v_t - S_{t-1} k_t                    (the residual of the write)
 *     du  = G k_t                                (S_t = S_{t-1} + beta_t r_t k_t^T)
 *     dk_t = beta_t G^T r_t - beta_t S_{t-1}^T du
 *     dv_t = beta_t du ;      dbeta_t = du . r_t
 *     G  <- G - beta_t du k_t^T                  (gradient of S_{t-1})
 *   dS_0 = G.
 * The pages derive no backward pass; this is the chain rule applied to the
 * recurrence of "Linear Attention, Visualized", DeltaNet > "Recurrent form".
 * States S_{t-1} are recomputed forward from checkpoints every kSeg tokens.
 */
enum { kSeg = 64 };

static void unit_backward(const double *q, const double *k, const double *v, const double *beta,
                          const double *dO, double *dq, double *dk, double *dv, double *dbeta,
                          ptrdiff_t qk_stride, ptrdiff_t vo_stride, ptrdiff_t beta_stride, int64_t L,
                          int dk_, int dv_, double *S, double *G, double *seg, double *tmp)
{
    /* S holds S0 on entry; G holds dS_T. seg: (kSeg + 1) states; tmp: dv + dk + dv */
    const size_t sz = (size_t)dv_ * dk_;
    const int64_t nseg = (L + kSeg - 1) / kSeg;
    double *ck = (double *)malloc(sizeof(double) * sz * (size_t)(nseg > 0 ? nseg : 1));
    if (!ck) return;
    /* forward: checkpoint the state at each segment start */
    for (int64_t sgi = 0; sgi < nseg; ++sgi) {
        memcpy(ck + (size_t)sgi * sz, S, sizeof(double) * sz);
        const int64_t t1 = (sgi + 1) * kSeg < L ? (sgi + 1) * kSeg : L;
        unit_forward(q + sgi * kSeg * qk_stride, k + sgi * kSeg * qk_stride, v + sgi * kSeg * vo_stride,
                     beta + sgi * kSeg * beta_stride, NULL, NULL, qk_stride, vo_stride, beta_stride,
                     t1 - sgi * kSeg, dk_, dv_, S, tmp);
    }
    double *r = tmp, *du = tmp + dv_, *vh = tmp + 2 * dv_;
    for (int64_t sgi = nseg - 1; sgi >= 0; --sgi) {
        const int64_t t0 = sgi * kSeg, t1 = (sgi + 1) * kSeg < L ? (sgi + 1) * kSeg : L;
        /* seg[j] = state before token t0 + j, j = 0 .. t1 - t0 */
        memcpy(seg, ck + (size_t)sgi * sz, sizeof(double) * sz);
        for (int64_t t = t0; t < t1; ++t) {
            double *Sn = seg + (size_t)(t - t0 + 1) * sz;
            memcpy(Sn, seg + (size_t)(t - t0) * sz, sizeof(double) * sz);
            unit_forward(q + t * qk_stride, k + t * qk_stride, v + t * vo_stride, beta + t * beta_stride,
                         NULL, NULL, qk_stride, vo_stride, beta_stride, 1, dk_, dv_, Sn, vh);
        }
        for (int64_t t = t1 - 1; t >= t0; --t) {
            const double *St = seg + (size_t)(t - t0 + 1) * sz, *Sp = seg + (size_t)(t - t0) * sz;
            const double *kt = k + t * qk_stride, *qt = q + t * qk_stride, *vt = v + t * vo_stride;
            const double *dot = dO + t * vo_stride;
            const double bt = beta[t * beta_stride];
            /* readout: G += dO q^T ; dq = S_t^T dO */
            for (int j = 0; j < dk_; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dv_; ++i) acc += St[(size_t)i * dk_ + j] * dot[i];
                dq[t * qk_stride + j] = acc;
            }
            for (int i = 0; i < dv_; ++i)
                for (int j = 0; j < dk_; ++j) G[(size_t)i * dk_ + j] += dot[i] * qt[j];
            /* residual r = v - S_{t-1} k ; du = G k */
            for (int i = 0; i < dv_; ++i) {
                double a = 0.0, b = 0.0;
                for (int j = 0; j < dk_; ++j) {
                    a += Sp[(size_t)i * dk_ + j] * kt[j];
                    b += G[(size_t)i * dk_ + j] * kt[j];
                }
                r[i] = vt[i] - a;
                du[i] = b;
            }
            double db = 0.0;
            for (int i = 0; i < dv_; ++i) db += du[i] * r[i];
            dbeta[t * beta_stride] = db;
            for (int i = 0; i < dv_; ++i) dv[t * vo_stride + i] = bt * du[i];
            for (int j = 0; j < dk_; ++j) {
                double a = 0.0, b = 0.0;
                for (int i = 0; i < dv_; ++i) {
                    a += G[(size_t)i * dk_ + j] * r[i];
                    b += Sp[(size_t)i * dk_ + j] * du[i];
                }
                dk[t * qk_stride + j] = bt * a - bt * b;
            }
            /* G <- G - beta du k^T */
            for (int i = 0; i < dv_; ++i)
                for (int j = 0; j < dk_; ++j) G[(size_t)i * dk_ + j] -= bt * du[i] * kt[j];
        }
    }
    free(ck);
}

/*
 * dq, dk [B,T,H,dk], dv [B,T,H,dv], dbeta [B,T,H], dS0 [B,H,dv,dk] (may be
 * NULL) for upstream gradients dO [B,T,H,dv] and dS_final [B,H,dv,dk] (NULL:
 * zero). S0 may be NULL (zero). Returns 0, -1 on bad arguments, -2 on
 * allocation failure.
 */
int oracle_deltanet_bwd(const double *q, const double *k, const double *v, const double *beta,
                        const double *S0, const double *dO, const double *dS_final, double *dq,
                        double *dk, double *dv, double *dbeta, double *dS0, int B, int H, int64_t T,
                        int dk_, int dv_, int nthreads)
{
    if (!q || !k || !v || !beta || !dO || !dq || !dk || !dv || !dbeta || B <= 0 || H <= 0 || T < 0 ||
        dk_ <= 0 || dv_ <= 0)
        return -1;
    const ptrdiff_t qk_stride = (ptrdiff_t)H * dk_, vo_stride = (ptrdiff_t)H * dv_;
    const size_t sz = (size_t)dv_ * dk_;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double *buf = (double *)malloc(sizeof(double) * (sz * (kSeg + 3) + 3 * (size_t)(dv_ + dk_)));
        if (!buf) {
#pragma omp atomic write
            failed = 1;
        } else {
            double *S = buf, *G = buf + sz, *seg = buf + 2 * sz, *tmp = seg + sz * (kSeg + 1);
#pragma omp for schedule(dynamic, 1)
            for (int64_t u = 0; u < (int64_t)B * H; ++u) {
                const int64_t b = u / H;
                const int h = (int)(u % H);
                const int64_t t0 = b * T;
                if (S0) memcpy(S, S0 + (size_t)u * sz, sizeof(double) * sz);
                else memset(S, 0, sizeof(double) * sz);
                if (dS_final) memcpy(G, dS_final + (size_t)u * sz, sizeof(double) * sz);
                else memset(G, 0, sizeof(double) * sz);
                unit_backward(q + t0 * qk_stride + (ptrdiff_t)h * dk_, k + t0 * qk_stride + (ptrdiff_t)h * dk_,
                              v + t0 * vo_stride + (ptrdiff_t)h * dv_, beta + t0 * H + h,
                              dO + t0 * vo_stride + (ptrdiff_t)h * dv_, dq + t0 * qk_stride + (ptrdiff_t)h * dk_,
                              dk + t0 * qk_stride + (ptrdiff_t)h * dk_, dv + t0 * vo_stride + (ptrdiff_t)h * dv_,
                              dbeta + t0 * H + h, qk_stride, vo_stride, H, T, dk_, dv_, S, G, seg, tmp);
                if (dS0) memcpy(dS0 + (size_t)u * sz, G, sizeof(double) * sz);
            }
            free(buf);
        }
    }
    return failed ? -2 : 0;
}

/*
 * Reverse mode of the Gated DeltaNet recurrence ("Linear Attention,
 * Visualized", "Gated DeltaNet (GDN)", transposed state), token by token:
 *     P_t = a_t S_{t-1}   (a_t = exp(g_t)),   S_t = P_t + beta_t (v_t - P_t k_t) k_t^T,
 *     o_t = S_t q_t.
 * With G the gradient of S_t (after adding dO_t q_t^T), the step from P_t is
 * the DeltaNet step, so its gradients follow with P_t in place of S_{t-1};
 * the gradient of P_t is H = G - beta_t (G k_t) k_t^T, and then
 *     dg_t = <H, P_t>  (= a_t <H, S_{t-1}>),   gradient of S_{t-1} = a_t H.
 * The pages derive no backward pass; this is the chain rule on that
 * recurrence. States are recomputed from checkpoints every kSeg tokens.
 */
static void unit_backward_decay(const double *q, const double *k, const double *v, const double *beta,
                                const double *g, const double *dO, double *dq, double *dk, double *dv,
                                double *dbeta, double *dg, ptrdiff_t qk_stride, ptrdiff_t vo_stride,
                                ptrdiff_t beta_stride, int64_t L, int dk_, int dv_, double *S, double *G,
                                double *seg, double *tmp)
{
    const size_t sz = (size_t)dv_ * dk_;
    const int64_t nseg = (L + kSeg - 1) / kSeg;
    double *ck = (double *)malloc(sizeof(double) * sz * (size_t)(nseg > 0 ? nseg : 1));
    double *Pt = (double *)malloc(sizeof(double) * sz);
    if (!ck || !Pt) {
        free(ck);
        free(Pt);
        return;
    }
    for (int64_t s0 = 0; s0 < nseg; ++s0) { /* checkpoints */
        memcpy(ck + (size_t)s0 * sz, S, sizeof(double) * sz);
        const int64_t e0 = (s0 + 1) * kSeg < L ? (s0 + 1) * kSeg : L;
        unit_forward(q + s0 * kSeg * qk_stride, k + s0 * kSeg * qk_stride, v + s0 * kSeg * vo_stride,
                     beta + s0 * kSeg * beta_stride, g + s0 * kSeg * beta_stride, NULL, qk_stride, vo_stride,
                     beta_stride, e0 - s0 * kSeg, dk_, dv_, S, tmp);
    }
    double *res = tmp, *gk = tmp + dv_, *scratch = tmp + 2 * dv_;
    for (int64_t s0 = nseg - 1; s0 >= 0; --s0) {
        const int64_t b0 = s0 * kSeg, e0 = (s0 + 1) * kSeg < L ? (s0 + 1) * kSeg : L;
        memcpy(seg, ck + (size_t)s0 * sz, sizeof(double) * sz); /* seg[j]: state before token b0 + j */
        for (int64_t t = b0; t < e0; ++t) {
            double *nxt = seg + (size_t)(t - b0 + 1) * sz;
            memcpy(nxt, seg + (size_t)(t - b0) * sz, sizeof(double) * sz);
            unit_forward(q + t * qk_stride, k + t * qk_stride, v + t * vo_stride, beta + t * beta_stride,
                         g + t * beta_stride, NULL, qk_stride, vo_stride, beta_stride, 1, dk_, dv_, nxt, scratch);
        }
        for (int64_t t = e0 - 1; t >= b0; --t) {
            const double *Snew = seg + (size_t)(t - b0 + 1) * sz, *Sold = seg + (size_t)(t - b0) * sz;
            const double *kv = k + t * qk_stride, *qv = q + t * qk_stride, *vv = v + t * vo_stride;
            const double *ov = dO + t * vo_stride;
            const double bb = beta[t * beta_stride], at = exp(g[t * beta_stride]);
            for (size_t e = 0; e < sz; ++e) Pt[e] = at * Sold[e];
            /* o_t = S_t q_t: dq_t = S_t^T dO_t and G += dO_t q_t^T */
            for (int c = 0; c < dk_; ++c) {
                double s = 0.0;
                for (int r = 0; r < dv_; ++r) s += Snew[(size_t)r * dk_ + c] * ov[r];
                dq[t * qk_stride + c] = s;
            }
            for (int r = 0; r < dv_; ++r)
                for (int c = 0; c < dk_; ++c) G[(size_t)r * dk_ + c] += ov[r] * qv[c];
            /* the write from P_t: res = v - P_t k, gk = G k */
            for (int r = 0; r < dv_; ++r) {
                double pk = 0.0, gkr = 0.0;
                for (int c = 0; c < dk_; ++c) {
                    pk += Pt[(size_t)r * dk_ + c] * kv[c];
                    gkr += G[(size_t)r * dk_ + c] * kv[c];
                }
                res[r] = vv[r] - pk;
                gk[r] = gkr;
            }
            double sb = 0.0;
            for (int r = 0; r < dv_; ++r) {
                sb += gk[r] * res[r];
                dv[t * vo_stride + r] = bb * gk[r];
            }
            dbeta[t * beta_stride] = sb;
            for (int c = 0; c < dk_; ++c) {
                double x = 0.0, y = 0.0;
                for (int r = 0; r < dv_; ++r) {
                    x += G[(size_t)r * dk_ + c] * res[r];
                    y += Pt[(size_t)r * dk_ + c] * gk[r];
                }
                dk[t * qk_stride + c] = bb * (x - y);
            }
            /* H = G - beta (G k) k^T is the gradient of P_t; dg_t = <H, P_t>; G <- a_t H */
            double sg = 0.0;
            for (int r = 0; r < dv_; ++r)
                for (int c = 0; c < dk_; ++c) {
                    const double hv = G[(size_t)r * dk_ + c] - bb * gk[r] * kv[c];
                    sg += hv * Pt[(size_t)r * dk_ + c];
                    G[(size_t)r * dk_ + c] = at * hv;
                }
            dg[t * beta_stride] = sg;
        }
    }
    free(Pt);
    free(ck);
}

/*
 * Gated DeltaNet backward: as oracle_deltanet_bwd, with the log decays g
 * [B,T,H] (layout of beta) as an input and their gradient dg [B,T,H] as an
 * output.
 */
int oracle_gated_deltanet_bwd(const double *q, const double *k, const double *v, const double *beta,
                              const double *g, const double *S0, const double *dO, const double *dS_final,
                              double *dq, double *dk, double *dv, double *dbeta, double *dg, double *dS0, int B,
                              int H, int64_t T, int dk_, int dv_, int nthreads)
{
    if (!q || !k || !v || !beta || !g || !dO || !dq || !dk || !dv || !dbeta || !dg || B <= 0 || H <= 0 ||
        T < 0 || dk_ <= 0 || dv_ <= 0)
        return -1;
    const ptrdiff_t qs = (ptrdiff_t)H * dk_, vs = (ptrdiff_t)H * dv_;
    const size_t sz = (size_t)dv_ * dk_;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (sz * (kSeg + 3) + 3 * (size_t)(dv_ + dk_)));
        if (!w) {
#pragma omp atomic write
            bad = 1;
        } else {
            double *S = w, *G = w + sz, *seg = w + 2 * sz, *tmp = seg + sz * (kSeg + 1);
#pragma omp for schedule(dynamic, 1)
            for (int64_t unit = 0; unit < (int64_t)B * H; ++unit) {
                const int64_t bi = unit / H, tok = bi * T;
                const int hi = (int)(unit % H);
                if (S0) memcpy(S, S0 + (size_t)unit * sz, sizeof(double) * sz);
                else memset(S, 0, sizeof(double) * sz);
                if (dS_final) memcpy(G, dS_final + (size_t)unit * sz, sizeof(double) * sz);
                else memset(G, 0, sizeof(double) * sz);
                unit_backward_decay(q + tok * qs + (ptrdiff_t)hi * dk_, k + tok * qs + (ptrdiff_t)hi * dk_,
                                    v + tok * vs + (ptrdiff_t)hi * dv_, beta + tok * H + hi, g + tok * H + hi,
                                    dO + tok * vs + (ptrdiff_t)hi * dv_, dq + tok * qs + (ptrdiff_t)hi * dk_,
                                    dk + tok * qs + (ptrdiff_t)hi * dk_, dv + tok * vs + (ptrdiff_t)hi * dv_,
                                    dbeta + tok * H + hi, dg + tok * H + hi, qs, vs, H, T, dk_, dv_, S, G, seg,
                                    tmp);
                if (dS0) memcpy(dS0 + (size_t)unit * sz, G, sizeof(double) * sz);
            }
            free(w);
        }
    }
    return bad ? -2 : 0;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
