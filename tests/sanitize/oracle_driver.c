/* Drives the fp64 oracle (oracle/kda_ref.c) on small inputs under
 * -fsanitize=address,undefined: fixed-length and varlen batches (with empty
 * sequences), with and without h0 and hT, and the one-token closed form
 * o = beta (q . k) v from a zero state. Exits non-zero on a failed check. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int kda_ref_fwd(const float* q, const float* k, const float* v, const float* g, const float* beta,
                const int64_t* cu, int64_t N, int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                const double* h0, double* o, double* hT);
int gdn_ref_fwd(const float* q, const float* k, const float* v, const float* g, const float* beta,
                const int64_t* cu, int64_t N, int64_t B, int64_t T, int64_t H, int64_t K, int64_t V,
                const double* h0, double* o, double* hT);

static float urand(unsigned* s) {
    *s = *s * 1664525u + 1013904223u;
    return (float)((*s >> 8) & 0xffff) / 65536.0f - 0.5f;
}

int main(void) {
    enum { T = 70, H = 2, D = 128 };
    const size_t n = (size_t)T * H * D;
    float *q = malloc(n * 4), *k = malloc(n * 4), *v = malloc(n * 4), *g = malloc(n * 4);
    float* beta = malloc((size_t)T * H * 4);
    float* gs = malloc((size_t)T * H * 4);
    unsigned s = 1;
    for (size_t i = 0; i < n; ++i) {
        q[i] = urand(&s); k[i] = urand(&s); v[i] = urand(&s); g[i] = -fabsf(urand(&s));
    }
    for (int i = 0; i < T * H; ++i) { beta[i] = 0.5f + urand(&s); gs[i] = -fabsf(urand(&s)); }
    const int64_t cu[5] = {0, 1, 1, 33, 70};   /* lengths 1, 0, 32, 37 */
    const int64_t N = 4;
    double* h0 = calloc((size_t)N * H * D * D, 8);
    for (size_t i = 0; i < (size_t)N * H * D * D; ++i) h0[i] = 0.1 * urand(&s);
    double* o = malloc(n * 8);
    double* hT = malloc((size_t)N * H * D * D * 8);
    int bad = 0;
    bad |= kda_ref_fwd(q, k, v, g, beta, NULL, 1, 1, T, H, D, D, NULL, o, NULL) != 0;
    bad |= kda_ref_fwd(q, k, v, g, beta, cu, N, 1, T, H, D, D, h0, o, hT) != 0;
    bad |= gdn_ref_fwd(q, k, v, gs, beta, cu, N, 1, T, H, D, D, h0, o, hT) != 0;
    /* the empty sequence keeps its initial state */
    for (size_t i = 0; i < (size_t)H * D * D; ++i)
        if (hT[(size_t)1 * H * D * D + i] != h0[(size_t)1 * H * D * D + i]) { bad = 1; break; }
    /* one token from zero: o = beta (q . k) v */
    bad |= kda_ref_fwd(q, k, v, g, beta, NULL, 1, 1, 1, H, D, D, NULL, o, hT) != 0;
    for (int h = 0; h < H; ++h) {
        double qk = 0.0;
        for (int c = 0; c < D; ++c) qk += (double)q[h * D + c] * k[h * D + c];
        for (int c = 0; c < D; ++c) {
            const double want = beta[h] * qk * v[h * D + c];
            if (fabs(o[h * D + c] - want) > 1e-12 * (1.0 + fabs(want))) { bad = 1; break; }
        }
    }
    free(q); free(k); free(v); free(g); free(beta); free(gs); free(h0); free(o); free(hT);
    if (bad) { fprintf(stderr, "oracle driver: a check failed\n"); return 1; }
    printf("oracle driver: all checks passed\n");
    return 0;
}
