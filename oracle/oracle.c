/*
 * Reference oracle for attention over precomputed per-chunk K/V caches,
 * CacheBlend impact and top-k selection.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check of the package
 * entry point and the CPU-baseline leg of the benchmark may load this code.
 * It shares nothing with the HIP library (no headers, helpers or tables), and
 * the library never calls it.
 *
 * Everything is computed in float64 with plain loops, in the order the pages
 * state the method. Inputs (fp32 or bf16 bit patterns) are widened exactly to
 * float64 before any arithmetic; float64 inputs (values of a dequantised
 * cache, which need not fit float32) are taken as they are.
 *
 * Sources (the pages are blog summaries of the papers):
 *  - TurboRAG summary, "Precomputing the KV cache": the combined K (and V) is
 *    the concatenation K^(1), ..., K^(m), K^(Q) along the sequence axis; the
 *    query block's own K/V comes last.
 *  - TurboRAG summary, "Causal vs non-causal attention" equation:
 *    Attention(Q,K,V) = softmax(Q K^T / sqrt(d_k) + M_causal) V, where M_causal
 *    lets each token see only itself and earlier tokens.
 *  - CacheBlend summary, "Mathematical formulation": full prefill over
 *    X = [D_1; ...; D_m; q]; the Impact equation sums the attention weight
 *    alpha_{j,i} that token j puts on token i over tokens j of other documents.
 *  - CacheBlend summary, selective-recompute listing: softmax over all keys
 *    (documents and query), column sum over the query rows, slice to document
 *    tokens, k = max(1, int(N_doc * r)), top-k.
 *
 * Readings taken where the pages are silent or garbled:
 *  - The mask is causal over the whole concatenated sequence. For query rows
 *    this is "causal only inside the query block". A flag turns it off to give
 *    the listing's unmasked softmax.
 *  - The Impact equation's index set prints as "j != doc(i)"; it is read as
 *    "rows j whose segment differs from the segment of key i". The query block
 *    is its own segment (index m). Same-segment rows are left out of the
 *    impact sum only, never out of the softmax.
 *  - Impact is summed over all H query heads. Query head h reads KV head
 *    h / (H / H_kv) (contiguous head groups).
 *  - Top-k orders by the float32 value's bits mapped to an order-preserving
 *    unsigned key, then by lower index; output sorted (value desc, index asc).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1, OR_F64 = 2 };
enum { OR_QUERY_ROWS = 0, OR_CROSS_DOC = 1, OR_ALL_ROWS = 2 };

/* Exact widening of one stored element to float64. */
static double widen(const void *base, int dtype, size_t i)
{
    if (dtype == OR_BF16) {
        uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    if (dtype == OR_F64)
        return ((const double *)base)[i];
    return (double)((const float *)base)[i];
}

/*
 * Attention of every row over the concatenated segments, plus impact.
 *
 * Q      [H][rows][d]; rows = q_len (query-row mode) or N = sum of lens.
 * K, V   m + 1 pointers; segment c is [H_kv][lens[c]][d]; lens[m] >= q_len.
 *        Segment m holds the query block's own keys: in query-row mode the
 *        q_len rows are the last q_len positions of the concatenation (in a
 *        decode step segment m also holds the earlier generated tokens, and
 *        the one row is the newest token, which sees every key: TurboRAG
 *        summary, the generation loop that appends each token's K/V).
 * causal 1: key i is visible to the row at position p iff pos(i) <= p.
 *        0: every key is visible (the listing's unmasked softmax).
 * row_lo, row_hi  only rows in [row_lo, row_hi) are computed (row_hi <= 0:
 *        all rows). Impact then sums those rows only; in the causal
 *        all-position modes this is exact for every key at position >= the
 *        position of row_lo.
 * out    [H][rows][d] float64 (rows outside the range are left untouched).
 * impact [N] float64, overwritten; NULL to skip.
 * lse    [H][rows] float64 natural-log sum-exp of the row; NULL to skip.
 * Returns 0, or -1 on invalid arguments, -2 on allocation failure.
 */
int oracle_attn(int dtype, int mode, int causal, const void *Q, const void *const *K,
                const void *const *V, const int32_t *lens, int m, int q_len, int H, int H_kv,
                int d, int row_lo, int row_hi, double *out, double *impact, double *lse,
                int n_threads)
{
    if (!Q || !K || !V || !lens || m < 0 || q_len < 1 || H < 1 || H_kv < 1 || d < 1 ||
        H % H_kv != 0 || lens[m] < q_len)
        return -1;
    long n_doc = 0;
    for (int c = 0; c < m; ++c) {
        if (lens[c] < 0)
            return -1;
        n_doc += lens[c];
    }
    const long N = n_doc + lens[m];
    const long rows = (mode == OR_QUERY_ROWS) ? q_len : N;
    if (row_hi <= 0 || row_hi > rows)
        row_hi = (int)rows;
    if (row_lo < 0)
        row_lo = 0;
    const int G = H / H_kv;
    const double inv_sqrt_d = 1.0 / sqrt((double)d);

    /* Global key index -> (segment, offset inside the segment). */
    int *seg_of = malloc(sizeof(int) * (size_t)N);
    long *off_of = malloc(sizeof(long) * (size_t)N);
    if (!seg_of || !off_of) {
        free(seg_of);
        free(off_of);
        return -2;
    }
    {
        long i = 0;
        for (int c = 0; c <= m; ++c)
            for (long t = 0; t < lens[c]; ++t, ++i) {
                seg_of[i] = c;
                off_of[i] = t;
            }
    }

    int nt = 1;
#ifdef _OPENMP
    nt = n_threads > 0 ? n_threads : omp_get_max_threads();
#endif
    double *partial = calloc((size_t)nt * (size_t)N, sizeof(double));
    if (!partial) {
        free(seg_of);
        free(off_of);
        return -2;
    }
    const long n_rows_run = row_hi - row_lo;
    const long n_tasks = (long)H * n_rows_run;
    int failed = 0;

#pragma omp parallel num_threads(nt)
    {
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
        double *imp = partial + (size_t)tid * (size_t)N;
        double *s = malloc(sizeof(double) * (size_t)N);
        double *acc = malloc(sizeof(double) * (size_t)d);
        if (!s || !acc) {
#pragma omp atomic write
            failed = 1;
        }
        /* A fixed cyclic schedule keeps the summation order reproducible. */
#pragma omp for schedule(static, 1)
        for (long task = 0; task < n_tasks; ++task) {
            if (!s || !acc)
                continue;
            const int h = (int)(task / n_rows_run);
            const long j = row_lo + task % n_rows_run;
            const int hk = h / G;
            const long pos = (mode == OR_QUERY_ROWS) ? N - q_len + j : j;
            const int seg_row = seg_of[pos];
            const long n_vis = causal ? pos + 1 : N;
            const size_t qbase = ((size_t)h * (size_t)rows + (size_t)j) * (size_t)d;

            /* Scores s_i = q . k_i / sqrt(d) over the visible keys. */
            double mx = -INFINITY;
            for (long i = 0; i < n_vis; ++i) {
                const int c = seg_of[i];
                const size_t kbase = ((size_t)hk * (size_t)lens[c] + (size_t)off_of[i]) * (size_t)d;
                double dot = 0.0;
                for (int t = 0; t < d; ++t)
                    dot += widen(Q, dtype, qbase + t) * widen(K[c], dtype, kbase + t);
                s[i] = dot * inv_sqrt_d;
                if (s[i] > mx)
                    mx = s[i];
            }
            /* Softmax normaliser: lse = mx + log(sum exp(s - mx)). */
            double l = 0.0;
            for (long i = 0; i < n_vis; ++i)
                l += exp(s[i] - mx);
            const double row_lse = mx + log(l);
            if (lse)
                lse[(size_t)h * (size_t)rows + (size_t)j] = row_lse;

            /* Weights, output and impact. */
            for (int t = 0; t < d; ++t)
                acc[t] = 0.0;
            for (long i = 0; i < n_vis; ++i) {
                const double p = exp(s[i] - row_lse);
                const int c = seg_of[i];
                const size_t vbase = ((size_t)hk * (size_t)lens[c] + (size_t)off_of[i]) * (size_t)d;
                for (int t = 0; t < d; ++t)
                    acc[t] += p * widen(V[c], dtype, vbase + t);
                const int counted = (mode != OR_CROSS_DOC) || (seg_row != c);
                if (counted)
                    imp[i] += p;
            }
            if (out)
                for (int t = 0; t < d; ++t)
                    out[qbase + t] = acc[t];
        }
        free(s);
        free(acc);
    }

    if (impact) {
        for (long i = 0; i < N; ++i) {
            double sum = 0.0;
            for (int t = 0; t < nt; ++t)
                sum += partial[(size_t)t * (size_t)N + (size_t)i];
            impact[i] = sum;
        }
    }
    free(partial);
    free(seg_of);
    free(off_of);
    return failed ? -2 : 0;
}

/* k = max(1, floor(r * n_doc)) in float64 (CacheBlend listing's max(1, int(.))). */
long oracle_budget(long n_doc, double r)
{
    double x = floor(r * (double)n_doc);
    long k = (long)x;
    return k < 1 ? 1 : k;
}

/* Order-preserving map of float32 bits to an unsigned key (-0 < +0). */
static uint32_t order_key(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (u >> 31) ? ~u : (u | 0x80000000u);
}

typedef struct {
    uint32_t key;
    int32_t idx;
} keyed;

static int by_key_desc_idx_asc(const void *a, const void *b)
{
    const keyed *x = a, *y = b;
    if (x->key != y->key)
        return x->key > y->key ? -1 : 1;
    return (x->idx > y->idx) - (x->idx < y->idx);
}

/*
 * The k largest of value[0..n) by the float32 order, ties to the lower
 * index, written sorted (value desc, index asc) to idx[0..k).
 * Returns 0, -1 on invalid arguments, -2 on allocation failure.
 */
int oracle_topk(const float *value, int n, int k, int32_t *idx)
{
    if (!value || !idx || n < 1 || k < 1 || k > n)
        return -1;
    keyed *all = malloc(sizeof(keyed) * (size_t)n);
    if (!all)
        return -2;
    for (int i = 0; i < n; ++i) {
        all[i].key = order_key(value[i]);
        all[i].idx = i;
    }
    qsort(all, (size_t)n, sizeof(keyed), by_key_desc_idx_asc);
    for (int i = 0; i < k; ++i)
        idx[i] = all[i].idx;
    free(all);
    return 0;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
