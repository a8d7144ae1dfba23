/*
 * KDA oracle: the gated delta rule with per-channel decay, token by token, in float64.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path links, loads or calls this file;
 * only the test suite, the smoke check and the benchmark's CPU-baseline leg do. It shares
 * no code with the HIP kernels.
 *
 * Sources: the KV-cache page ("Starting from the KV-cache explosion: what KimiLinear's
 * linear attention solves") and the revolution page ("Linear attention revolution: Kimi
 * Linear ...").
 *
 * What it computes (Kimi Delta Attention). Each (sequence, head) keeps a d_k x d_v state
 * S whose rows are key channels; its size is fixed, whatever the sequence length (KV-cache
 * page, section 2). Per token t, with log-decay g_t <= 0 per key channel, write strength
 * beta_t, key k_t, value v_t and query q_t:
 *
 *   1. a   = exp(g_t)                 the forget gate, one value per channel (the per-channel
 *                                     gating that distinguishes KDA from Gated DeltaNet:
 *                                     revolution page, the KDA section)
 *   2. S  <- Diag(a) S                decay acts on the key channels (rows)
 *   3. p   = S^T k_t                  what the decayed state predicts for k_t
 *   4. S  <- S + beta_t k_t (v_t - p)^T
 *                                     delta-rule erase-and-write; steps 2-4 together are
 *                                     S_t = (I - beta k k^T) Diag(a) S_{t-1} + beta k v^T,
 *                                     with the erase term (I - beta k k^T) of the KV-cache
 *                                     page, section 5
 *   5. o_t = S^T (scale * q_t)        read-out with the updated state
 *
 * Plain float64 loops, no blocking or reordering beyond the definition; no compensated
 * summation (relative error ~ d_k * 2^-53). Sequences and heads are independent, so the
 * only parallelism is over (sequence, head) chains.
 *
 * Layouts (all dense, row-major, last dimension innermost):
 *   q, k, g : [T_total, H, K]     v, o : [T_total, H, V]     beta : [T_total, H]
 *   s0, s_out : [N, H, K, V]      cu_seqlens : [N + 1], cu[0] = 0, non-decreasing
 * s0 may be NULL (zero initial state); s_out may be NULL (not written) and may alias s0.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static void chain(int64_t t0, int64_t t1, int64_t h, int64_t H, int64_t K, int64_t V,
                  const double *q, const double *k, const double *v, const double *g,
                  const double *beta, double scale, const double *s0, double *o,
                  double *S, double *a, double *p)
{
    if (s0)
        memcpy(S, s0, (size_t)(K * V) * sizeof(double));
    else
        memset(S, 0, (size_t)(K * V) * sizeof(double));

    for (int64_t t = t0; t < t1; ++t) {
        const double *qt = q + (t * H + h) * K;
        const double *kt = k + (t * H + h) * K;
        const double *gt = g + (t * H + h) * K;
        const double *vt = v + (t * H + h) * V;
        const double bt = beta[t * H + h];
        double *ot = o + (t * H + h) * V;

        /* 1-2: decay every key channel (row) of the state */
        for (int64_t c = 0; c < K; ++c)
            a[c] = exp(gt[c]);
        for (int64_t c = 0; c < K; ++c)
            for (int64_t j = 0; j < V; ++j)
                S[c * V + j] *= a[c];

        /* 3: prediction p = S^T k */
        for (int64_t j = 0; j < V; ++j)
            p[j] = 0.0;
        for (int64_t c = 0; c < K; ++c)
            for (int64_t j = 0; j < V; ++j)
                p[j] += S[c * V + j] * kt[c];

        /* 4: erase-and-write with the correction u = beta (v - p) */
        for (int64_t j = 0; j < V; ++j)
            p[j] = bt * (vt[j] - p[j]);
        for (int64_t c = 0; c < K; ++c)
            for (int64_t j = 0; j < V; ++j)
                S[c * V + j] += kt[c] * p[j];

        /* 5: read-out with the updated state */
        for (int64_t j = 0; j < V; ++j)
            ot[j] = 0.0;
        for (int64_t c = 0; c < K; ++c) {
            const double qc = scale * qt[c];
            for (int64_t j = 0; j < V; ++j)
                ot[j] += S[c * V + j] * qc;
        }
    }
}

/* Returns 0 on success, 1 on invalid arguments, 2 on allocation failure. */
int kda_oracle_fwd(int64_t n_seqs, const int64_t *cu_seqlens, int64_t H, int64_t K, int64_t V,
                   const double *q, const double *k, const double *v, const double *g,
                   const double *beta, double scale, const double *s0, double *o,
                   double *s_out, int nthreads)
{
    if (n_seqs < 0 || H <= 0 || K <= 0 || V <= 0 || !cu_seqlens)
        return 1;
    if (cu_seqlens[0] != 0)
        return 1;
    for (int64_t n = 0; n < n_seqs; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n])
            return 1;
    if (cu_seqlens[n_seqs] > 0 && (!q || !k || !v || !g || !beta || !o))
        return 1;

    const int64_t items = n_seqs * H;
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel reduction(| : err)
#endif
    {
        double *S = (double *)malloc((size_t)(K * V + K + V) * sizeof(double));
        if (!S) {
            err |= 2;
        } else {
            double *a = S + K * V, *p = a + K;
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
            for (int64_t it = 0; it < items; ++it) {
                const int64_t n = it / H, h = it % H;
                const double *init = s0 ? s0 + (n * H + h) * K * V : NULL;
                chain(cu_seqlens[n], cu_seqlens[n + 1], h, H, K, V, q, k, v, g, beta, scale,
                      init, o, S, a, p);
                if (s_out)
                    memcpy(s_out + (n * H + h) * K * V, S, (size_t)(K * V) * sizeof(double));
            }
            free(S);
        }
    }
    return err ? 2 : 0;
}

int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Backward pass: the gradient of a scalar loss through the recurrence above, by reverse-mode
 * differentiation of its five steps, token by token in reverse order (the training side of
 * the layer: chunk mode is the one used for training, revolution page, the KDA section).
 *
 * Given the loss's gradients do_t = dL/do_t for every token and dS_T = dL/dS_final (NULL:
 * zero), it returns dL/dq, dL/dk, dL/dv, dL/dg, dL/dbeta per token and dL/dS_init per
 * (sequence, head). With dS the gradient with respect to the state after step t (from the
 * later tokens), each token t in reverse order takes
 *   5. o = S_t^T (scale q):  dq = scale S_t do,   dS += scale q do^T
 *   4. S_t = S' + k u^T:     dk = dS u,           du = dS^T k          (S' = Diag(a) S_{t-1})
 *      u = beta (v - p):     dv = beta du,        dbeta = du . (v - p),  dp = -beta du
 *   3. p = S'^T k:           dS' = dS + k dp^T,   dk += S' dp
 *   1-2. S' = Diag(e^g) S_{t-1}:
 *                            dg[c] = sum_j S'[c][j] dS'[c][j]   (d e^g / dg = e^g)
 *                            dS_{t-1} = Diag(a) dS'
 * and dS_init is dS after the first token. The states S_{t-1} of every token of the chain
 * are kept from a forward sweep (the same arithmetic as the forward above), so memory is
 * (tokens of the chain) x K x V doubles per thread.
 */
static int chain_bwd(int64_t t0, int64_t t1, int64_t h, int64_t H, int64_t K, int64_t V,
                     const double *q, const double *k, const double *v, const double *g,
                     const double *beta, double scale, const double *s0, const double *dout,
                     const double *dsT, double *dq, double *dk, double *dv, double *dg,
                     double *dbeta, double *ds0)
{
    const int64_t L = t1 - t0, KV = K * V;
    double *Sp = (double *)malloc((size_t)((L + 3) * KV + K + 4 * V + L * V) * sizeof(double));
    if (!Sp)
        return 2;
    double *S = Sp + L * KV;      /* running state */
    double *dS = S + KV;          /* gradient with respect to the state */
    double *Sd = dS + KV;         /* S' of the current token */
    double *a = Sd + KV;
    double *p = a + K, *du = p + V, *dp = du + V, *tv = dp + V;
    double *r = tv + V;           /* v_t - p_t of every token, [L][V] */

    /* forward sweep: keep S_{t-1} and v_t - p_t */
    if (s0)
        memcpy(S, s0, (size_t)KV * sizeof(double));
    else
        memset(S, 0, (size_t)KV * sizeof(double));
    for (int64_t t = t0; t < t1; ++t) {
        const int64_t i = t - t0;
        const double *kt = k + (t * H + h) * K, *gt = g + (t * H + h) * K;
        const double *vt = v + (t * H + h) * V;
        const double bt = beta[t * H + h];
        memcpy(Sp + i * KV, S, (size_t)KV * sizeof(double));
        for (int64_t c = 0; c < K; ++c)
            a[c] = exp(gt[c]);
        for (int64_t c = 0; c < K; ++c)
            for (int64_t j = 0; j < V; ++j)
                S[c * V + j] *= a[c];
        for (int64_t j = 0; j < V; ++j)
            p[j] = 0.0;
        for (int64_t c = 0; c < K; ++c)
            for (int64_t j = 0; j < V; ++j)
                p[j] += S[c * V + j] * kt[c];
        for (int64_t j = 0; j < V; ++j) {
            r[i * V + j] = vt[j] - p[j];
            p[j] = bt * r[i * V + j];
        }
        for (int64_t c = 0; c < K; ++c)
            for (int64_t j = 0; j < V; ++j)
                S[c * V + j] += kt[c] * p[j];
    }

    /* reverse sweep */
    if (dsT)
        memcpy(dS, dsT, (size_t)KV * sizeof(double));
    else
        memset(dS, 0, (size_t)KV * sizeof(double));
    for (int64_t t = t1 - 1; t >= t0; --t) {
        const int64_t i = t - t0;
        const double *qt = q + (t * H + h) * K, *kt = k + (t * H + h) * K;
        const double *gt = g + (t * H + h) * K, *dot = dout + (t * H + h) * V;
        const double bt = beta[t * H + h];
        const double *rt = r + i * V;
        double *dqt = dq + (t * H + h) * K, *dkt = dk + (t * H + h) * K;
        double *dgt = dg + (t * H + h) * K, *dvt = dv + (t * H + h) * V;

        /* recompute S' = Diag(a) S_{t-1}, u = beta (v - p) and S_t = S' + k u^T */
        for (int64_t c = 0; c < K; ++c)
            a[c] = exp(gt[c]);
        for (int64_t c = 0; c < K; ++c)
            for (int64_t j = 0; j < V; ++j)
                Sd[c * V + j] = Sp[i * KV + c * V + j] * a[c];
        for (int64_t j = 0; j < V; ++j)
            tv[j] = bt * rt[j];     /* u */

        /* 5: read-out */
        for (int64_t c = 0; c < K; ++c) {
            double acc = 0.0;
            for (int64_t j = 0; j < V; ++j)
                acc += (Sd[c * V + j] + kt[c] * tv[j]) * dot[j];
            dqt[c] = scale * acc;
        }
        for (int64_t c = 0; c < K; ++c)
            for (int64_t j = 0; j < V; ++j)
                dS[c * V + j] += scale * qt[c] * dot[j];

        /* 4: write with u = beta (v - p) */
        for (int64_t c = 0; c < K; ++c) {
            double acc = 0.0;
            for (int64_t j = 0; j < V; ++j)
                acc += dS[c * V + j] * tv[j];
            dkt[c] = acc;
        }
        for (int64_t j = 0; j < V; ++j) {
            double acc = 0.0;
            for (int64_t c = 0; c < K; ++c)
                acc += dS[c * V + j] * kt[c];
            du[j] = acc;
        }
        double db = 0.0;
        for (int64_t j = 0; j < V; ++j) {
            dvt[j] = bt * du[j];
            db += du[j] * rt[j];
            dp[j] = -bt * du[j];
        }
        dbeta[t * H + h] = db;

        /* 3: prediction p = S'^T k */
        for (int64_t c = 0; c < K; ++c)
            for (int64_t j = 0; j < V; ++j)
                dS[c * V + j] += kt[c] * dp[j];     /* dS now holds dS' */
        for (int64_t c = 0; c < K; ++c) {
            double acc = 0.0;
            for (int64_t j = 0; j < V; ++j)
                acc += Sd[c * V + j] * dp[j];
            dkt[c] += acc;
        }

        /* 1-2: decay */
        for (int64_t c = 0; c < K; ++c) {
            double acc = 0.0;
            for (int64_t j = 0; j < V; ++j)
                acc += Sd[c * V + j] * dS[c * V + j];
            dgt[c] = acc;
        }
        for (int64_t c = 0; c < K; ++c)
            for (int64_t j = 0; j < V; ++j)
                dS[c * V + j] *= a[c];
    }
    if (ds0)
        memcpy(ds0, dS, (size_t)KV * sizeof(double));
    free(Sp);
    return 0;
}

/* Layouts as kda_oracle_fwd; dout [T_total, H, V]; dsT, ds0 [N, H, K, V] (dsT may be NULL:
 * zero; ds0 may be NULL: not written). Returns 0, 1 (invalid arguments) or 2 (no memory). */
int kda_oracle_bwd(int64_t n_seqs, const int64_t *cu_seqlens, int64_t H, int64_t K, int64_t V,
                   const double *q, const double *k, const double *v, const double *g,
                   const double *beta, double scale, const double *s0, const double *dout,
                   const double *dsT, double *dq, double *dk, double *dv, double *dg,
                   double *dbeta, double *ds0, int nthreads)
{
    if (n_seqs < 0 || H <= 0 || K <= 0 || V <= 0 || !cu_seqlens)
        return 1;
    if (cu_seqlens[0] != 0)
        return 1;
    for (int64_t n = 0; n < n_seqs; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n])
            return 1;
    if (cu_seqlens[n_seqs] > 0 && (!q || !k || !v || !g || !beta || !dout || !dq || !dk || !dv ||
                                   !dg || !dbeta))
        return 1;

    const int64_t items = n_seqs * H;
    int err = 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
#endif
    for (int64_t it = 0; it < items; ++it) {
        const int64_t n = it / H, h = it % H;
        const int64_t off = (n * H + h) * K * V;
        err |= chain_bwd(cu_seqlens[n], cu_seqlens[n + 1], h, H, K, V, q, k, v, g, beta, scale,
                         s0 ? s0 + off : NULL, dout, dsT ? dsT + off : NULL, dq, dk, dv, dg,
                         dbeta, ds0 ? ds0 + off : NULL);
    }
    (void)nthreads;
    return err;
}
