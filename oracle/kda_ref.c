/*
 * kda_ref.c -- CPU oracle for the Kimi Delta Attention (KDA) forward pass.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
 * baseline may load this file's library. The product path never calls it.
 *
 * What it computes: the plain token-by-token recurrence of KDA, in fp64.
 * KDA is described as a refinement of Gated DeltaNet with fine-grained,
 * channel-wise gating (toolarium.ru, "FlashKDA: Moonshot открыла ядра Kimi
 * Delta Attention для H20", §"Почему это новость про инфраструктуру";
 * donniechu.com, "FlashKDA … Kimi Delta Attention", §"Số liệu kỹ thuật").
 * Per (sequence, head), with state S in R^{K x V} (K = V = 128):
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t
 *
 * Evaluated in this equivalent order, one token at a time:
 *     S   <- Diag(exp(g_t)) S            (per-channel decay of the K rows)
 *     e   <- v_t - S^T k_t               (delta-rule prediction error)
 *     S   <- S + beta_t k_t e^T
 *     o_t <- S^T q_t                     (the updated state; no 1/sqrt(K) scale)
 *
 * Sequences: B fixed-length rows of T tokens, or, when cu_seqlens is given
 * (B must then be 1), N sequences packed along T at [cu[n], cu[n+1]).
 * The state starts at h0[n, h] (or zero) and its final value goes to hT[n, h].
 * The pages name batch, varlen cu_seqlens and initial/final recurrent states as
 * the kernel's interface (donniechu.com page, §"Số liệu kỹ thuật").
 *
 * Layouts (row-major, innermost last): q, k, v, g [B, T, H, K]; beta [B, T, H];
 * h0, hT [N, H, K, V]; o [B, T, H, V]. q, k, v, g, beta are float32 values
 * (exactly what the device receives); h0 is fp64 so that a final state can be
 * handed back in without rounding; all arithmetic and the outputs are fp64.
 *
 * The only parallelism is over independent (sequence, head) pairs.
 *
 * gdn_ref_fwd is the same recurrence with one scalar gate per (token, head),
 * g [B, T, H]: Gated DeltaNet, the method KDA refines by making the gate
 * channel-wise (toolarium.ru page, section "Почему это новость про
 * инфраструктуру"; the pages' second baseline, "gdn", in the H20 benchmark
 * table of the same page). Every channel then decays by the same exp(g_t).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* gate_ch: number of gate values per (token, head): K (channel-wise) or 1. */
static int ref_fwd(const float* q, const float* k, const float* v, const float* g, int64_t gate_ch,
                   const float* beta, const int64_t* cu_seqlens, int64_t num_seqs,
                   int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                   const double* h0, double* o, double* hT) {
    if (K <= 0 || V <= 0 || H <= 0 || B <= 0 || T < 0) return -2;
    if (cu_seqlens && B != 1) return -2;
    const int64_t N = cu_seqlens ? num_seqs : B;
    const int64_t units = N * H;

    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < units; ++u) {
        const int64_t n = u / H, h = u % H;
        const int64_t row = cu_seqlens ? 0 : n;
        const int64_t t0 = cu_seqlens ? cu_seqlens[n] : 0;
        const int64_t t1 = cu_seqlens ? cu_seqlens[n + 1] : T;

        double* S = (double*)malloc(sizeof(double) * (size_t)(K * V));
        double* e = (double*)malloc(sizeof(double) * (size_t)V);
        if (!S || !e) {
            free(S); free(e);
#pragma omp atomic write
            failed = 1;
            continue;
        }
        for (int64_t i = 0; i < K * V; ++i)
            S[i] = h0 ? h0[(n * H + h) * K * V + i] : 0.0;

        for (int64_t t = t0; t < t1; ++t) {
            const int64_t tok = (row * T + t) * H + h;   /* (b, t, h) index */
            const float* kt = k + tok * K;
            const float* qt = q + tok * K;
            const float* vt = v + tok * V;
            const float* gt = g + tok * gate_ch;
            const double bt = (double)beta[tok];

            /* decay: row c of S scales by alpha_c = exp(g_c) (g_0 for all rows if scalar) */
            for (int64_t c = 0; c < K; ++c) {
                const double a = exp((double)gt[gate_ch == 1 ? 0 : c]);
                for (int64_t j = 0; j < V; ++j) S[c * V + j] *= a;
            }
            /* prediction error e = v - S^T k */
            for (int64_t j = 0; j < V; ++j) e[j] = (double)vt[j];
            for (int64_t c = 0; c < K; ++c) {
                const double kc = (double)kt[c];
                for (int64_t j = 0; j < V; ++j) e[j] -= S[c * V + j] * kc;
            }
            /* rank-1 correction S += beta k e^T */
            for (int64_t c = 0; c < K; ++c) {
                const double w = bt * (double)kt[c];
                for (int64_t j = 0; j < V; ++j) S[c * V + j] += w * e[j];
            }
            /* output o = S^T q */
            double* ot = o + tok * V;
            for (int64_t j = 0; j < V; ++j) ot[j] = 0.0;
            for (int64_t c = 0; c < K; ++c) {
                const double qc = (double)qt[c];
                for (int64_t j = 0; j < V; ++j) ot[j] += S[c * V + j] * qc;
            }
        }
        if (hT) memcpy(hT + (n * H + h) * K * V, S, sizeof(double) * (size_t)(K * V));
        free(S);
        free(e);
    }
    return failed ? -1 : 0;
}

int kda_ref_fwd(const float* q, const float* k, const float* v, const float* g,
                const float* beta, const int64_t* cu_seqlens, int64_t num_seqs,
                int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                const double* h0, double* o, double* hT) {
    return ref_fwd(q, k, v, g, K, beta, cu_seqlens, num_seqs, B, T, H, K, V, h0, o, hT);
}

/* g: [B, T, H], one gate per (token, head). */
int gdn_ref_fwd(const float* q, const float* k, const float* v, const float* g,
                const float* beta, const int64_t* cu_seqlens, int64_t num_seqs,
                int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                const double* h0, double* o, double* hT) {
    return ref_fwd(q, k, v, g, 1, beta, cu_seqlens, num_seqs, B, T, H, K, V, h0, o, hT);
}

int kda_ref_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
