/*
 * kda_oracle.c -- plain fp64 CPU reference for the Kimi Delta Attention (KDA) core.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file: only the test suite, the package's smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header or table with the HIP
 * library.
 *
 * Source: "Kimi K3 Technical Report: Open Frontier Intelligence", §2.1.1
 * (Kimi Delta Attention):
 *   - eq. (1): S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *              o_t = S_t^T q_t,  S in R^{d_k x d_v}.
 *   - eq. (5): g_t = g_min * Sigmoid(exp(A_h) * z_t),  alpha_t = exp(g_t).
 * The output is read after the token's own update (the text under eq. (4)
 * explains that Tril keeps the diagonal for exactly this reason).
 *
 * The recurrence is evaluated one token at a time, exactly as eq. (1) is
 * written, in double precision.  The only rewriting is the algebraic identity
 *   (I - b k k^T) D S + b k v^T  =  D S + b k (v - (D S)^T k)^T,
 * which avoids forming the d_k x d_k matrix; every step is a plain loop.
 *
 * Optional query scale: o_t = S_t^T (scale * q_t); eq. (1) itself has scale 1.
 *
 * Parity pins for this file live in tests/test_oracle_pins.py (closed forms,
 * invariants, a chunk-parallel evaluation, hand-worked examples); no function
 * here is unpinned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* eq. (5): lower-bounded log-decay from the decay logit z. */
static double kda_gate(double z, double A_h, double g_min)
{
    double x = exp(A_h) * z;
    double sig = 1.0 / (1.0 + exp(-x));
    return g_min * sig;
}

void kda_oracle_gate(int64_t n, const double *z, double A_h, double g_min, double *g)
{
    for (int64_t i = 0; i < n; ++i)
        g[i] = kda_gate(z[i], A_h, g_min);
}

/*
 * One sequence of one head, T tokens, in order.
 *   q, k, gz : row t at q + t*ldk (d_k values each)
 *   v        : row t at v + t*ldv (d_v values)
 *   beta     : beta[t*ldb]
 *   gz       : log-decay g_t (z_mode == 0) or decay logit z_t (z_mode != 0)
 *   S        : d_k x d_v row-major, entering state on input, final state on output
 *   o        : row t at o + t*ldo (d_v values)
 *   work     : scratch of d_k + d_v doubles
 */
void kda_oracle_sequence(int64_t T, int64_t Dk, int64_t Dv,
                         const double *q, const double *k, const double *v,
                         const double *gz, const double *beta,
                         int64_t ldk, int64_t ldv, int64_t ldb,
                         int z_mode, double A_h, double g_min, double scale,
                         double *S, double *o, int64_t ldo, double *work)
{
    double *alpha = work;      /* d_k */
    double *u = work + Dk;     /* d_v */
    for (int64_t t = 0; t < T; ++t) {
        const double *qt = q + t * ldk;
        const double *kt = k + t * ldk;
        const double *gt = gz + t * ldk;
        const double *vt = v + t * ldv;
        const double bt = beta[t * ldb];
        double *ot = o + t * ldo;

        /* alpha_t = exp(g_t), per key channel */
        for (int64_t j = 0; j < Dk; ++j)
            alpha[j] = exp(z_mode ? kda_gate(gt[j], A_h, g_min) : gt[j]);

        /* S <- Diag(alpha_t) S : row j of S is scaled by alpha_j */
        for (int64_t j = 0; j < Dk; ++j)
            for (int64_t c = 0; c < Dv; ++c)
                S[j * Dv + c] *= alpha[j];

        /* u = S^T k_t */
        for (int64_t c = 0; c < Dv; ++c)
            u[c] = 0.0;
        for (int64_t j = 0; j < Dk; ++j)
            for (int64_t c = 0; c < Dv; ++c)
                u[c] += S[j * Dv + c] * kt[j];

        /* S <- S + beta_t k_t (v_t - u)^T */
        for (int64_t j = 0; j < Dk; ++j)
            for (int64_t c = 0; c < Dv; ++c)
                S[j * Dv + c] += bt * kt[j] * (vt[c] - u[c]);

        /* o_t = S_t^T (scale q_t) */
        for (int64_t c = 0; c < Dv; ++c)
            ot[c] = 0.0;
        for (int64_t j = 0; j < Dk; ++j)
            for (int64_t c = 0; c < Dv; ++c)
                ot[c] += S[j * Dv + c] * (scale * qt[j]);
    }
}

/*
 * Many sequences and heads; (sequence, head) pairs are independent and run in
 * parallel with OpenMP.  Token-major layouts, as the library takes them:
 *   q, k, gz : [T_total][H][Dk]     v, o : [T_total][H][Dv]     beta : [T_total][H]
 *   cu_seqlens : [N+1], sequence s spans tokens [cu[s], cu[s+1])
 *   A_log : [H] (read only when z_mode != 0)
 *   h0 : [N][H][Dk][Dv] entering states, or NULL for zeros
 *   hT : [N][H][Dk][Dv] final states (may be NULL)
 * nthreads <= 0 uses the OpenMP default.  Returns the number of threads used,
 * or -1 when scratch memory cannot be allocated.
 */
int kda_oracle_forward(int64_t N, int64_t H, int64_t Dk, int64_t Dv,
                       const int64_t *cu_seqlens,
                       const double *q, const double *k, const double *v,
                       const double *gz, const double *beta,
                       int z_mode, const double *A_log, double g_min, double scale,
                       const double *h0, double *o, double *hT, int nthreads)
{
    int used = 1;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#endif
#pragma omp parallel
    {
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
        double *S = (double *)malloc(sizeof(double) * (size_t)(Dk * Dv));
        double *work = (double *)malloc(sizeof(double) * (size_t)(Dk + Dv));
        if (!S || !work) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t p = 0; p < N * H; ++p) {
            if (!S || !work)
                continue;
            int64_t s = p / H, h = p % H;
            int64_t t0 = cu_seqlens[s], len = cu_seqlens[s + 1] - cu_seqlens[s];
            if (h0)
                memcpy(S, h0 + (s * H + h) * Dk * Dv, sizeof(double) * (size_t)(Dk * Dv));
            else
                memset(S, 0, sizeof(double) * (size_t)(Dk * Dv));
            kda_oracle_sequence(len, Dk, Dv,
                                q + (t0 * H + h) * Dk, k + (t0 * H + h) * Dk,
                                v + (t0 * H + h) * Dv, gz + (t0 * H + h) * Dk,
                                beta + t0 * H + h,
                                H * Dk, H * Dv, H,
                                z_mode, z_mode ? A_log[h] : 0.0, g_min, scale,
                                S, o + (t0 * H + h) * Dv, H * Dv, work);
            if (hT)
                memcpy(hT + (s * H + h) * Dk * Dv, S, sizeof(double) * (size_t)(Dk * Dv));
        }
        free(S);
        free(work);
    }
    return failed ? -1 : used;
}
