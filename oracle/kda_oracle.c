/*
 * kda_oracle.c -- plain, slow, sequential fp64 reference for Kimi Delta
 * Attention (KDA).  TEST INFRASTRUCTURE ONLY: it exists to check the HIP
 * library and shares no code, header or constant with it.  Only the tests,
 * the smoke check and the benchmark's CPU-baseline leg may load it.
 *
 * What it computes.  "Kimi K3: Open Frontier Intelligence and Implementation
 * Framework" (gemslabs.io), section "Hybrid Attention Mechanism", describes
 * KDA as the delta-rule recurrence extended with a channel-wise forget gate.
 * The reading taken here (the delta rule with a per-key-channel decay applied
 * to the state before the delta correction, output read from the updated
 * state) is, per sequence and head, with S a K x V matrix whose rows are key
 * channels:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t,            alpha_t = exp(g_t)  (g = log alpha)
 *
 * The loop below is that definition with one association made explicit:
 * (k k^T) Y is evaluated as k (k^T Y), so each step costs O(K V) instead of
 * O(K^2 V).  There is no chunking, blocking or reordering over time.
 *
 * Layouts (row-major, contiguous), tokens packed along the first axis:
 *   q, k, g : [tokens, H, K]     v, o : [tokens, H, V]     beta : [tokens, H]
 *   s0, sT  : [N, H, K, V]       cu   : [N + 1] offsets, cu[0] = 0, nondecreasing
 * s0 may be NULL (zero initial state); sT may be NULL (not returned).
 * (sequence, head) units are independent and may run on separate threads;
 * time within a unit is strictly sequential.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

int kda_oracle_recurrence(const double *q, const double *k, const double *v,
                          const double *g, const double *beta, const double *s0,
                          double *o, double *sT, const int64_t *cu, int64_t N,
                          int64_t H, int64_t K, int64_t V, int nthreads)
{
    if (!q || !k || !v || !g || !beta || !o || !cu) return 1;
    if (N < 0 || H <= 0 || K <= 0 || V <= 0) return 2;
    if (cu[0] != 0) return 3;
    for (int64_t n = 0; n < N; ++n)
        if (cu[n + 1] < cu[n]) return 3;
    if (nthreads < 1) nthreads = 1;

    int failed = 0;
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 1) reduction(| : failed)
    for (int64_t unit = 0; unit < N * H; ++unit) {
        const int64_t n = unit / H, h = unit % H;
        double *S = (double *)malloc((size_t)(K * V) * sizeof(double));
        double *w = (double *)malloc((size_t)V * sizeof(double));
        if (!S || !w) {
            free(S);
            free(w);
            failed |= 1;
            continue;
        }
        if (s0)
            memcpy(S, s0 + unit * K * V, (size_t)(K * V) * sizeof(double));
        else
            memset(S, 0, (size_t)(K * V) * sizeof(double));

        for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
            const double *qt = q + (t * H + h) * K;
            const double *kt = k + (t * H + h) * K;
            const double *gt = g + (t * H + h) * K;
            const double *vt = v + (t * H + h) * V;
            const double bt = beta[t * H + h];
            double *ot = o + (t * H + h) * V;

            /* Y = Diag(alpha_t) S_{t-1}: row c (key channel c) scaled by exp(g_t[c]). */
            for (int64_t c = 0; c < K; ++c) {
                const double a = exp(gt[c]);
                for (int64_t j = 0; j < V; ++j) S[c * V + j] *= a;
            }
            /* w = k_t^T Y (a length-V row). */
            for (int64_t j = 0; j < V; ++j) w[j] = 0.0;
            for (int64_t c = 0; c < K; ++c)
                for (int64_t j = 0; j < V; ++j) w[j] += kt[c] * S[c * V + j];
            /* S_t = Y - beta k (k^T Y) + beta k v^T = Y + beta k (v - w)^T. */
            for (int64_t c = 0; c < K; ++c) {
                const double bk = bt * kt[c];
                for (int64_t j = 0; j < V; ++j) S[c * V + j] += bk * (vt[j] - w[j]);
            }
            /* o_t = S_t^T q_t. */
            for (int64_t j = 0; j < V; ++j) ot[j] = 0.0;
            for (int64_t c = 0; c < K; ++c)
                for (int64_t j = 0; j < V; ++j) ot[j] += qt[c] * S[c * V + j];
        }
        if (sT) memcpy(sT + unit * K * V, S, (size_t)(K * V) * sizeof(double));
        free(S);
        free(w);
    }
    return failed ? 4 : 0;
}
