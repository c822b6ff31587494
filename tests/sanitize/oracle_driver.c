/* Drives oracle/oracle.c on small inputs for its AddressSanitizer /
 * UndefinedBehaviorSanitizer build (tests/test_sanitizers.py): every mode
 * and input type, empty and length-1 chunks, a row range, the unmasked
 * flag, top-k with ties and signed zeros, and the budget. Checks the impact
 * mass (rows x H over all keys) so a run that reads garbage also fails. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_attn(int dtype, int mode, int causal, const void *Q, const void *const *K, const void *const *V,
                const int32_t *lens, int m, int q_len, int H, int H_kv, int d, int row_lo, int row_hi,
                double *out, double *impact, double *lse, int n_threads);
long oracle_budget(long n_doc, double r);
int oracle_topk(const float *value, int n, int k, int32_t *idx);

static unsigned g_s = 12345u;
static float rnd(void)
{
    g_s = g_s * 1664525u + 1013904223u;
    return ((g_s >> 8) & 0xFFFF) / 32768.0f - 1.0f;
}

static void *fill(int dtype, size_t n)
{
    size_t esz = dtype == 0 ? 4 : dtype == 1 ? 2 : 8;
    unsigned char *p = malloc(n * esz + 1);
    for (size_t i = 0; i < n; ++i) {
        float f = rnd();
        if (dtype == 0)
            memcpy(p + 4 * i, &f, 4);
        else if (dtype == 2) {
            double x = f;
            memcpy(p + 8 * i, &x, 8);
        } else {
            uint32_t u;
            memcpy(&u, &f, 4);
            uint16_t b = (uint16_t)(u >> 16);
            memcpy(p + 2 * i, &b, 2);
        }
    }
    return p;
}

static int run(int dtype, int mode, int causal, const int *doc, int m, int q_len, int H, int H_kv, int d,
               int row_lo, int row_hi)
{
    int32_t lens[16];
    const void *K[16], *V[16];
    int N = 0;
    for (int c = 0; c <= m; ++c) {
        lens[c] = c < m ? doc[c] : q_len;
        K[c] = fill(dtype, (size_t)H_kv * lens[c] * d);
        V[c] = fill(dtype, (size_t)H_kv * lens[c] * d);
        N += lens[c];
    }
    const int rows = mode == 0 ? q_len : N;
    void *Q = fill(dtype, (size_t)H * rows * d);
    double *out = calloc((size_t)H * rows * d, sizeof(double));
    double *imp = calloc(N ? N : 1, sizeof(double));
    double *lse = calloc((size_t)H * rows, sizeof(double));
    int rc = oracle_attn(dtype, mode, causal, Q, K, V, lens, m, q_len, H, H_kv, d, row_lo, row_hi, out, imp,
                         lse, 3);
    int bad = rc != 0;
    if (!bad && row_lo == 0 && row_hi == 0) {
        double s = 0;
        for (int i = 0; i < N; ++i)
            s += imp[i];
        /* query and all-rows modes: every row's weights sum to 1 */
        if (mode != 1 && fabs(s - (double)rows * H) > 1e-9 * rows * H) {
            fprintf(stderr, "impact mass %.17g != %d\n", s, rows * H);
            bad = 1;
        }
    }
    for (int c = 0; c <= m; ++c) {
        free((void *)K[c]);
        free((void *)V[c]);
    }
    free(Q);
    free(out);
    free(imp);
    free(lse);
    return bad;
}

int main(void)
{
    int fails = 0;
    const int docs_a[4] = {65, 0, 1, 130};
    const int docs_b[2] = {33, 91};
    for (int dtype = 0; dtype <= 2; ++dtype)
        for (int mode = 0; mode <= 2; ++mode) {
            fails += run(dtype, mode, 1, docs_a, 4, 17, 4, 2, 64, 0, 0);
            fails += run(dtype, mode, 1, docs_b, 2, 5, 6, 3, 128, 0, 0);
        }
    fails += run(1, 0, 0, docs_b, 2, 9, 2, 2, 64, 0, 0);   /* the listing's unmasked softmax */
    fails += run(1, 1, 1, docs_a, 4, 12, 4, 4, 64, 70, 150); /* a row range */
    fails += run(0, 0, 1, NULL, 0, 21, 2, 1, 64, 0, 0);    /* no documents */
    fails += run(1, 0, 1, docs_b, 2, 1, 8, 8, 128, 0, 0);  /* one query row */

    float v[64];
    int32_t idx[64];
    for (int i = 0; i < 64; ++i)
        v[i] = (float)(i % 5) * 0.25f;
    v[3] = -0.0f;
    v[9] = 0.0f;
    for (int k = 1; k <= 64; k += 9)
        fails += oracle_topk(v, 64, k, idx) != 0;
    fails += oracle_topk(v, 64, 65, idx) == 0; /* k > n is refused */
    fails += oracle_budget(10000, 0.15) != 1500 || oracle_budget(3, 0.1) != 1 || oracle_budget(8192, 0.05) != 409;
    if (fails) {
        fprintf(stderr, "%d oracle checks failed\n", fails);
        return 1;
    }
    printf("ORACLE_SANITIZE_OK\n");
    return 0;
}
