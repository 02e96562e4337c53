/*
 * kda_oracle.c -- fp64 CPU oracle for Kimi Delta Attention (KDA).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness reference that the
 * HIP kernels are checked against.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it.  The product path never calls it,
 * and it shares no code, header or constant with the HIP library.
 *
 * What it computes (SemiAnalysis "Kimi K3" architecture primer, as summarised
 * on the bayesiansapien wiki page, section 1 "KDA is DeltaNet plus per-channel
 * decay"): per (batch, head), a dk x dv associative memory S is updated once
 * per token by
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = S_t^T q_t,              alpha_t = exp(g_t)  (per channel)
 *
 * i.e. decay each key channel of the old memory (the diagonal forget gate),
 * erase what the memory returns for k_t (the delta rule), write beta_t k_t v_t^T,
 * then read with q_t from the updated memory.  The chunked prefill and the
 * one-token decode described in section 2 ("FlashKDA's complexity") of the same
 * page are re-orderings of this arithmetic, so the oracle is the token-by-token
 * recurrence itself: no chunking, no inverse, no reordering.
 *
 * Readings taken where the pages are silent (stated once here):
 *   - g is a natural-log decay: alpha = exp(g) per key channel.
 *   - decay acts on S_{t-1} before the erase/write; the output uses S_t.
 *   - no 1/sqrt(dk) query scale; callers pre-scale q if they want one.
 *   - S0 == NULL means a zero initial state.
 *   - checkpoint j (1-based) is the state after token min(j*N, T); there are
 *     ceil(T/N) of them, the last one equal to S_T.
 *
 * Layouts (dense, row-major, fp64):
 *   q, k [B,T,H,dk]   v [B,T,H,dv]   g [B,T,H,dk]   beta [B,T,H]
 *   S0, S_T [B,H,dk,dv]   o [B,T,H,dv]   ckpt [ceil(T/N),B,H,dk,dv]
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#define KDA_MAX_THREADS() omp_get_max_threads()
#else
#define KDA_MAX_THREADS() 1
#endif

/* One token of the recurrence applied to S (dk x dv, row-major) in place.
 * `e` is caller scratch of length dv.  Writes o_t (length dv). */
static void kda_token_f64(double *S, const double *q, const double *k,
                          const double *v, const double *g, double beta,
                          double *o, double *e, int dk, int dv)
{
    int i, j;
    /* Diag(alpha_t) S_{t-1}: per-channel forget gate on the key axis. */
    for (i = 0; i < dk; ++i) {
        double alpha = exp(g[i]);
        for (j = 0; j < dv; ++j)
            S[i * dv + j] *= alpha;
    }
    /* e = k_t^T S' : what the decayed memory returns for the key k_t. */
    for (j = 0; j < dv; ++j)
        e[j] = 0.0;
    for (i = 0; i < dk; ++i)
        for (j = 0; j < dv; ++j)
            e[j] += k[i] * S[i * dv + j];
    /* (I - beta k k^T) S' + beta k v^T = S' - beta k e^T + beta k v^T. */
    for (i = 0; i < dk; ++i)
        for (j = 0; j < dv; ++j)
            S[i * dv + j] = S[i * dv + j] - beta * k[i] * e[j] + beta * k[i] * v[j];
    /* o_t = S_t^T q_t. */
    for (j = 0; j < dv; ++j)
        o[j] = 0.0;
    for (i = 0; i < dk; ++i)
        for (j = 0; j < dv; ++j)
            o[j] += S[i * dv + j] * q[i];
}

/* Full-sequence recurrence for every (b, h).  Returns 0 on success, -1 on bad
 * arguments, -2 if scratch memory could not be allocated.  `nthreads` <= 0
 * lets OpenMP choose; (b, h) pairs are independent and run in parallel. */
int kda_oracle_prefill_f64(const double *q, const double *k, const double *v,
                           const double *g, const double *beta, const double *S0,
                           double *o, double *S_T, double *ckpt, int ckpt_every,
                           int B, int T, int H, int dk, int dv, int nthreads)
{
    int n_bh, failed = 0;
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0 || ckpt_every < 0)
        return -1;
    if (!S_T || (T > 0 && (!q || !k || !v || !g || !beta || !o)))
        return -1;
    if (ckpt_every > 0 && !ckpt)
        return -1;
    n_bh = B * H;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : KDA_MAX_THREADS())
    for (int bh = 0; bh < n_bh; ++bh) {
        int b = bh / H, h = bh % H, t, n_ck = 0;
        int n_ck_total = ckpt_every > 0 ? (T + ckpt_every - 1) / ckpt_every : 0;
        size_t sd = (size_t)dk * dv;
        double *S = (double *)malloc(sd * sizeof(double));
        double *e = (double *)malloc((size_t)dv * sizeof(double));
        if (!S || !e) {
            free(S);
            free(e);
#pragma omp atomic write
            failed = 1;
            continue;
        }
        if (S0)
            memcpy(S, S0 + (size_t)bh * sd, sd * sizeof(double));
        else
            memset(S, 0, sd * sizeof(double));
        for (t = 0; t < T; ++t) {
            size_t row = ((size_t)b * T + t) * H + h; /* token (b, t, h) */
            kda_token_f64(S, q + row * dk, k + row * dk, v + row * dv,
                          g + row * dk, beta[row], o + row * dv, e, dk, dv);
            if (n_ck < n_ck_total && ((t + 1) % ckpt_every == 0 || t == T - 1)) {
                memcpy(ckpt + ((size_t)n_ck * n_bh + bh) * sd, S, sd * sizeof(double));
                ++n_ck;
            }
        }
        memcpy(S_T + (size_t)bh * sd, S, sd * sizeof(double));
        free(S);
        free(e);
    }
    return failed ? -2 : 0;
}

/* One decode step for N independent sequences: the same token update applied
 * to S [N,H,dk,dv] in place; q, k [N,H,dk], v [N,H,dv], g [N,H,dk],
 * beta [N,H]; writes o [N,H,dv]. */
int kda_oracle_decode_f64(const double *q, const double *k, const double *v,
                          const double *g, const double *beta, double *S,
                          double *o, int N, int H, int dk, int dv, int nthreads)
{
    int n_bh, failed = 0;
    if (N < 0 || H < 0 || dk <= 0 || dv <= 0)
        return -1;
    if (N * H > 0 && (!q || !k || !v || !g || !beta || !S || !o))
        return -1;
    n_bh = N * H;

#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : KDA_MAX_THREADS())
    for (int bh = 0; bh < n_bh; ++bh) {
        double *e = (double *)malloc((size_t)dv * sizeof(double));
        if (!e) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        kda_token_f64(S + (size_t)bh * dk * dv, q + (size_t)bh * dk, k + (size_t)bh * dk,
                      v + (size_t)bh * dv, g + (size_t)bh * dk, beta[bh],
                      o + (size_t)bh * dv, e, dk, dv);
        free(e);
    }
    return failed ? -2 : 0;
}
