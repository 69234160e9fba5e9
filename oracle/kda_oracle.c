/*
 * TEST INFRASTRUCTURE ONLY. This file is the CPU oracle for the KDA forward
 * prefill. Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load it; the library path never does.
 *
 * What it computes: the per-token Kimi Delta Attention (KDA) recurrence in
 * fp64. The chunked two-kernel prefill of
 *   "feat(kda/sm90): FlashKDA prefill port + intracard-CP prefill"
 *   (cuLA pull request #103; commit summary: K1 prepares decayed q/k, beta and
 *   the WY inverse, K2 runs the inter-chunk recurrence; CHUNK=16, D=128,
 *   forward only)
 * reaches it in exact arithmetic. That page names the method but prints no
 * equation; the rule below is the published KDA definition (a gated delta
 * rule with per-key-channel decay). For one sequence and one head, with the state
 * S (dk x dv, rows are key channels) and every token t in order:
 *
 *   S   <- Diag(exp(g_t)) S                      (per-key-channel decay)
 *   e   <- v_t - S^T k_t                         (delta-rule residual)
 *   S   <- S + beta_t k_t e^T                    (rank-one write)
 *   o_t <- scale * S^T q_t                       (read of the updated state)
 *
 * which is S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T
 * and o_t = S_t^T q_t (times scale). Sequences are packed token-major and
 * delimited by cu_seqlens (the FLA-compatible varlen convention named in the
 * same pull request's description). Plain loops, no blocking beyond splitting
 * the independent value columns across threads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/*
 * Layouts (all row-major, fp64):
 *   q, k, g : [Tt, H, dk]     v, o : [Tt, H, dv]     beta : [Tt, H]
 *   s0, sT  : [n_seqs, H, dk, dv]   (s0 may be NULL: zero state; sT may be NULL)
 *   cu      : [n_seqs + 1] int32, cu[0] = 0, non-decreasing, cu[n_seqs] = Tt
 * col_block: value columns per parallel work unit (columns of S evolve
 *   independently, so splitting them changes no arithmetic).
 * Returns 0 on success, -1 on invalid arguments, -2 on allocation failure.
 */
int kda_oracle_recurrent(int64_t Tt, int32_t H, int32_t dk, int32_t dv, int32_t n_seqs,
                         const int32_t *cu, const double *q, const double *k,
                         const double *v, const double *g, const double *beta,
                         double scale, const double *s0, double *o, double *sT,
                         int32_t col_block, int32_t n_threads)
{
    if (Tt < 0 || H < 1 || dk < 1 || dv < 1 || n_seqs < 0 || !cu) return -1;
    if (cu[0] != 0 || cu[n_seqs] != Tt) return -1;
    for (int32_t i = 0; i < n_seqs; ++i)
        if (cu[i + 1] < cu[i]) return -1;
    if (col_block < 1 || col_block > dv) col_block = dv;
    const int32_t n_cb = (dv + col_block - 1) / col_block;
    const int64_t n_units = (int64_t)n_seqs * H * n_cb;
    int failed = 0;

#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
#endif
    for (int64_t u = 0; u < n_units; ++u) {
        const int32_t cb = (int32_t)(u % n_cb);
        const int32_t h = (int32_t)((u / n_cb) % H);
        const int32_t i = (int32_t)(u / ((int64_t)n_cb * H));
        const int32_t c0 = cb * col_block;
        const int32_t nc = (c0 + col_block <= dv) ? col_block : dv - c0;

        double *S = (double *)malloc(sizeof(double) * (size_t)dk * nc);
        double *e = (double *)malloc(sizeof(double) * (size_t)nc);
        if (!S || !e) { free(S); free(e); failed = 1; continue; }

        const size_t st_off = ((size_t)i * H + h) * (size_t)dk * dv;
        for (int32_t a = 0; a < dk; ++a)
            for (int32_t c = 0; c < nc; ++c)
                S[(size_t)a * nc + c] = s0 ? s0[st_off + (size_t)a * dv + c0 + c] : 0.0;

        for (int64_t t = cu[i]; t < cu[i + 1]; ++t) {
            const size_t row_k = ((size_t)t * H + h) * dk;
            const size_t row_v = ((size_t)t * H + h) * dv;
            const double b = beta[(size_t)t * H + h];
            /* decay: S <- Diag(exp(g_t)) S */
            for (int32_t a = 0; a < dk; ++a) {
                const double gam = exp(g[row_k + a]);
                for (int32_t c = 0; c < nc; ++c) S[(size_t)a * nc + c] *= gam;
            }
            /* residual: e = v_t - S^T k_t */
            for (int32_t c = 0; c < nc; ++c) {
                double acc = 0.0;
                for (int32_t a = 0; a < dk; ++a) acc += k[row_k + a] * S[(size_t)a * nc + c];
                e[c] = v[row_v + c0 + c] - acc;
            }
            /* write: S <- S + beta_t k_t e^T */
            for (int32_t a = 0; a < dk; ++a) {
                const double bk = b * k[row_k + a];
                for (int32_t c = 0; c < nc; ++c) S[(size_t)a * nc + c] += bk * e[c];
            }
            /* read: o_t = scale * S^T q_t */
            for (int32_t c = 0; c < nc; ++c) {
                double acc = 0.0;
                for (int32_t a = 0; a < dk; ++a) acc += q[row_k + a] * S[(size_t)a * nc + c];
                o[row_v + c0 + c] = scale * acc;
            }
        }
        if (sT)
            for (int32_t a = 0; a < dk; ++a)
                for (int32_t c = 0; c < nc; ++c)
                    sT[st_off + (size_t)a * dv + c0 + c] = S[(size_t)a * nc + c];
        free(S);
        free(e);
    }
    return failed ? -2 : 0;
}

/* Threads the OpenMP runtime would use for the parallel loop above. */
int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
