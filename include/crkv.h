/*
 * crkv: attention of a query block over precomputed per-chunk K/V caches,
 * CacheBlend impact, and top-k selection, for AMD Instinct MI355X (gfx950).
 *
 * The operation (TurboRAG summary, "Precomputing the KV cache" and the causal
 * attention equation; CacheBlend summary, "Mathematical formulation", the
 * Impact equation and the selective-recompute listing):
 *
 *   K = Concat(K^(1), ..., K^(m), K^(Q)),  V likewise (query block last),
 *   out = softmax(Q K^T / sqrt(d) + M) V,
 *   impact[i] = sum over heads h and counted rows j of softmax weight p_{h,j,i},
 *   idx = the k = max(1, floor(r * N_doc)) largest impact[0..N_doc).
 *
 * M is causal over the concatenated sequence: the key at position i is
 * visible to the row at position p iff i <= p. For query rows (positions
 * N_doc + j) this is "causal only inside the query block".
 *
 * Conventions shared by every entry point:
 *  - Device pointers are owned by the caller; the library never frees or
 *    retains them. Host arrays (the chunk pointer tables, lengths, problem
 *    lists) are read during the call only and may be freed when it returns.
 *  - Work is enqueued asynchronously on opts->stream (a hipStream_t; NULL
 *    means the null stream). No call synchronises the stream. A kernel fault
 *    surfaces at the caller's next synchronisation.
 *  - Every argument is validated before anything is enqueued. Failures return
 *    a negative crkv_status and never abort; crkv_last_error() gives the
 *    reason (per thread).
 *  - Segment c of a problem stores K and V as [H_kv][chunk_len[c]][d],
 *    contiguous, in the element type opts->dtype. Entries 0..m-1 are document
 *    chunks (length 0 allowed: the chunk is skipped); N_doc is their total
 *    length. Entry m holds the query block's own K/V, chunk_len[m] >= q_len:
 *    the q_len query rows are the last q_len positions of the concatenation,
 *    and any earlier keys of entry m are tokens generated before them (a
 *    decode step has q_len = 1 and a growing entry m). N = N_doc +
 *    chunk_len[m] is the number of keys. Chunks are never copied or
 *    concatenated in memory: the library reads them through the pointer table.
 *  - Q and out are [H][rows][d] in opts->dtype. rows = q_len in
 *    CRKV_IMPACT_QUERY_ROWS mode, and N (every position of the concatenated
 *    sequence) in the two all-position modes.
 *  - Query head h reads KV head h / (H / H_kv).
 *  - impact is float32 [N] (document keys first, then entry m's keys),
 *    overwritten, summed over all H query heads.
 *  - Supported: d in {64, 128}; H % H_kv == 0; N < 2^30.
 */
#ifndef CRKV_H
#define CRKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CRKV_VERSION 1

typedef enum {
    CRKV_OK = 0,
    CRKV_E_INVAL = -1,       /* an argument is out of its documented range */
    CRKV_E_UNSUPPORTED = -2, /* valid, but outside what the kernels handle  */
    CRKV_E_HIP = -3,         /* a HIP runtime call or launch failed          */
    CRKV_E_NOMEM = -4        /* device or pinned host allocation failed      */
} crkv_status;

/* CRKV_KV_Q8: K/V segments in the 8-bit format of crkv_quantize_q8 (every
 * segment, documents and the query block's own), Q and out bf16; accepted by
 * the attention entry points (crkv_attn_chunks[_batched][_static], the plan
 * and size functions) and by crkv_decode_chunks_batched; the gather/scatter,
 * rotation and quantise entry points refuse it. */
typedef enum { CRKV_F32 = 0, CRKV_BF16 = 1, CRKV_KV_Q8 = 2 } crkv_dtype;

/*
 * Which rows are attended and which rows count towards impact.
 *  QUERY_ROWS: the q_len query rows; impact sums all of them (CacheBlend
 *              listing: softmax over all keys, column sum over query rows).
 *  CROSS_DOC:  every position is a row (full causal prefill of
 *              [D_1; ...; D_m; q]); impact of key i sums only rows j whose
 *              segment differs from key i's segment (CacheBlend Impact
 *              equation, index set read as doc(j) != doc(i); the query block
 *              is segment m). Same-segment rows still take part in softmax.
 *  ALL_ROWS:   every position is a row; impact sums every row (a check mode:
 *              the impact vector then sums to N * H).
 */
typedef enum {
    CRKV_IMPACT_QUERY_ROWS = 0,
    CRKV_IMPACT_CROSS_DOC = 1,
    CRKV_IMPACT_ALL_ROWS = 2
} crkv_mode;

typedef struct crkv_opts {
    int dtype;              /* crkv_dtype of Q, K, V and out                   */
    int mode;               /* crkv_mode                                        */
    void *stream;           /* hipStream_t, NULL = null stream                  */
    void *workspace;        /* device scratch, or NULL: the library uses a
                               buffer it keeps per device (grown on demand,
                               held until exit); calls on different streams
                               that share it run one after another on the
                               device, so pass a workspace per stream for
                               concurrent calls                                 */
    size_t workspace_bytes; /* size of `workspace`; see crkv_workspace_size     */
    void *timing_events[2]; /* optional hipEvent_t pair recorded on `stream`
                               immediately before and after the attention
                               kernel (for measuring that kernel alone)         */
    int deterministic;      /* 1 (the default) or 0; results are bit-identical
                               from call to call either way: every reduction
                               (impact partials, split ranges, top-k) runs in
                               a fixed order without atomics, so there is no
                               faster nondeterministic mode to select. Other
                               values are CRKV_E_INVAL                          */
} crkv_opts;

/* Defaults: fp32, query-row mode, null stream, library-managed scratch,
 * deterministic = 1. */
void crkv_opts_init(crkv_opts *opts);

/*
 * Attention of one problem over m document chunks plus the query block.
 *  Q          device, [H][rows][d]
 *  chunk_K/V  host arrays of m + 1 device pointers (see conventions)
 *  chunk_len  host array of m + 1 lengths; chunk_len[m] >= q_len
 *  out        device, [H][rows][d], written
 *  impact     device, float32 [N], written
 *  opts       NULL for the defaults
 */
int crkv_attn_chunks(const void *Q, const void *const *chunk_K, const void *const *chunk_V,
                     const int32_t *chunk_len, int m, int q_len, int H, int H_kv, int d,
                     void *out, float *impact, const crkv_opts *opts);

/*
 * Top-k selection (CacheBlend listing's topk over the document slice of the
 * impact vector): the k largest of impact[0..n) by float32 order (-0 < +0),
 * ties broken by the lower index, written to idx[0..k) sorted by (value
 * descending, index ascending). Requires 1 <= k <= n and k <= 8192; NaN
 * inputs are outside the contract.
 *  impact  device float32 [n]; idx device int32 [k], written.
 */
int crkv_topk(const float *impact, int n, int k, int32_t *idx, const crkv_opts *opts);

/* One problem of a batch (a layer, or a request). Pointer fields as in
 * crkv_attn_chunks; chunk_K/chunk_V/chunk_len are host arrays. */
typedef struct crkv_problem {
    const void *Q;
    const void *const *chunk_K;
    const void *const *chunk_V;
    const int32_t *chunk_len;
    int m;
    int q_len;
    void *out;
    float *impact;
} crkv_problem;

/* All problems of a batch (shared H, H_kv, d, dtype and mode; each with its
 * own chunks, lengths and q_len) in one attention launch.
 * With opts->dtype == CRKV_KV_Q8 every chunk_K[c] / chunk_V[c] is a buffer in
 * the 8-bit format of crkv_quantize_q8 (kinds CRKV_Q8_K and CRKV_Q8_V,
 * 16-byte aligned) for chunk_len[c] keys, and Q and out are bf16. The call is
 * the attention over the dequantised cache (code * scale): key tiles are
 * widened to bf16 while they are staged, K as a hi/lo pair of bf16 values
 * (Q . K carried to about 17 significant bits, for the impact) and V with its
 * token scale applied and rounded once to bf16. */
int crkv_attn_chunks_batched(const crkv_problem *problems, int n_problems, int H, int H_kv,
                             int d, const crkv_opts *opts);

/*
 * For callers that cannot allocate device memory (code under stream capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same batched
 * attention as crkv_attn_chunks_batched (same kernels, same results bit for
 * bit), with its plan tables and impact partials in a static device array
 * the library holds on each device it runs on (crkv_static_scratch_bytes()
 * bytes, 64 MiB, held until the process ends) instead of a workspace or a
 * library-grown buffer. The call allocates no device or pinned host memory;
 * it copies the plan tables from pageable host memory into the array with
 * hipMemcpyAsync on opts->stream (the call returns once the host copy has
 * been read). The first call on a device looks up the array's device
 * address. opts->workspace must be NULL (else CRKV_E_INVAL). A call whose
 * tables plus partials exceed the array returns CRKV_E_UNSUPPORTED before
 * enqueuing anything (the 32-layer Llama-3-8B-shaped batch needs about
 * 11 MB). Every call on a device shares the one array and leaves its
 * contents behind (nothing in it has to start at zero): calls that overlap
 * on one device, from different streams or threads, race; calls on one
 * stream are ordered.
 */
int crkv_attn_chunks_batched_static(const crkv_problem *problems, int n_problems, int H, int H_kv,
                                    int d, const crkv_opts *opts);

/* Size in bytes of the static device array crkv_attn_chunks_batched_static uses. */
size_t crkv_static_scratch_bytes(void);

/* Top-k for n_problems vectors in one launch. impact and idx are host arrays
 * of device pointers; n and k are host arrays. Same contract as crkv_topk. */
int crkv_topk_batched(const float *const *impact, const int32_t *n, const int32_t *k,
                      int32_t *const *idx, int n_problems, const crkv_opts *opts);

/* Recompute budget k = max(1, floor(r * n_doc)) (CacheBlend: r times the
 * summed document lengths; the listing's max(1, int(N_doc * r))). Computed
 * in double. Returns -1 if n_doc < 0 or r is not in [0, 1]. */
int64_t crkv_budget(int64_t n_doc, double r);

/*
 * A batched attention call planned once, for launch-bound shapes and for
 * capture into a hipGraph (the per-call path uploads its tables through a
 * ring of reused buffers, which a replayed graph must not depend on).
 * crkv_plan_create validates like crkv_attn_chunks_batched, builds the plan,
 * allocates its device tables and impact partials (or uses opts->workspace,
 * which must then outlive the plan) and copies the tables synchronously; the
 * problems' device buffers (Q, segments, out, impact) are fixed into the
 * plan. k (host, n_problems entries, 0 = no selection for that problem) and
 * idx (host array of device int32 [k[i]] pointers) add the top-k of each
 * problem's document impact, as crkv_topk_batched; pass k = NULL for none.
 * crkv_plan_launch enqueues the attention kernel, the impact combine and the
 * top-k on `stream` and nothing else (no allocation, copy or host wait), on
 * the device the plan was made on (else CRKV_E_INVAL); timing_events (NULL
 * or a hipEvent_t pair) bracket the attention kernel. Launches of one plan
 * share its partials: concurrent launches of the same plan race.
 * crkv_plan_destroy waits for the device, then frees the plan (NULL: no-op).
 */
typedef struct crkv_plan crkv_plan;

int crkv_plan_create(const crkv_problem *problems, int n_problems, int H, int H_kv, int d, const int32_t *k,
                     int32_t *const *idx, const crkv_opts *opts, crkv_plan **plan);
int crkv_plan_launch(const crkv_plan *plan, void *stream, void *const *timing_events);
int crkv_plan_destroy(crkv_plan *plan);

/* Bytes of device scratch a crkv_attn_chunks_batched call with these
 * arguments needs when the caller passes opts->workspace (256-byte aligned
 * pointer). Returns 0 if the arguments are invalid. */
size_t crkv_workspace_size(const crkv_problem *problems, int n_problems, int H, int H_kv, int d,
                           const crkv_opts *opts);

/*
 * One decode step over the segment table, for a batch of problems (TurboRAG
 * summary: the generation loop appends each generated token's K/V to the
 * cache and the newest token attends to every cached key). Each problem has
 * q_len == 1; chunk_len[m] >= 1 counts the tokens generated so far including
 * the current one, whose query row (the last position) sees every key.
 * Computes out only: the problems' impact pointers are ignored (may be NULL).
 *  Q    device, [H][1][d]; out device, [H][1][d], written
 *  opts->dtype == CRKV_BF16: segments bf16 [H_kv][len][d]. opts->dtype ==
 *  CRKV_KV_Q8: chunk_K[c] and chunk_V[c] are buffers in the 8-bit format of
 *  crkv_quantize_q8 (kinds CRKV_Q8_K and CRKV_Q8_V, 16-byte aligned) for
 *  chunk_len[c] keys; the step is the decode over the dequantised cache
 *  (code * scale), with the scales applied outside the matrix products (Q
 *  times the segment's K channel scales, rounded to bf16 once per segment;
 *  softmax weight times the key's V scale before P.V); Q and out bf16.
 *  Requires opts->dtype CRKV_BF16 or CRKV_KV_Q8 (else CRKV_E_UNSUPPORTED) and
 *  H / H_kv <= 16. opts->mode is ignored. The keys of each (problem, KV head)
 *  are split into ranges processed in parallel and merged in range order, so
 *  results are deterministic. Scratch: opts->workspace of at least
 *  crkv_decode_workspace_size bytes, or library-managed (stream-ordered).
 *  opts->timing_events bracket the two decode kernels.
 */
int crkv_decode_chunks_batched(const crkv_problem *problems, int n_problems, int H, int H_kv, int d,
                               const crkv_opts *opts);

/* Bytes of device scratch crkv_decode_chunks_batched needs for these
 * arguments (256-byte aligned workspace). Returns 0 if they are invalid. */
size_t crkv_decode_workspace_size(const crkv_problem *problems, int n_problems, int H, int H_kv, int d,
                                  const crkv_opts *opts);

/*
 * The 8-bit K/V segment format (CacheGen summary: loading a precomputed
 * cache dominates, and caches can be stored in a much smaller form; the page
 * gives no codec, so this format is this library's own). bf16 values become
 * int8 codes with float32 scales, one scale per group, with float32 IEEE
 * divisions and round-half-to-even:
 *   scale = max over the group of |x| / 127,   code = clamp(rint(x / scale), -127, 127)
 * (an all-zero group: scale 0, codes 0). Value = code * scale. K groups are
 * (KV head, channel) over the segment's tokens, because cached keys carry a
 * few large-magnitude channels; V groups are (KV head, token). A segment of
 * len keys is one buffer of crkv_q8_bytes(H_kv, len, d, kind) bytes: the
 * codes [H_kv][len][d] (int8), then at byte offset H_kv * len * d the scales,
 * float32 [H_kv][d] (K) or [H_kv][len] (V). At d = 128 and 2,500 keys a K/V
 * pair is 0.51x the bf16 bytes, and the decode step (CRKV_KV_Q8) reads that.
 * K scales cover the tokens present when the segment was quantised: a
 * segment that grows (the generated tokens' segment) is quantised again.
 */
typedef enum { CRKV_Q8_K = 0, CRKV_Q8_V = 1 } crkv_q8_kind;

typedef struct crkv_q8_seg {
    const void *x;   /* device bf16 [H_kv][len][d], read; 16-byte aligned       */
    void *q8;        /* device, crkv_q8_bytes(H_kv, len, d, kind) bytes, written;
                        16-byte aligned; must not overlap x                     */
    int len;         /* >= 0 (0: nothing is written)                            */
    int kind;        /* crkv_q8_kind: the segment holds keys or values          */
} crkv_q8_seg;

/* Bytes of one segment in the 8-bit format (0 for len = 0); 0 if an argument
 * is negative, d is not 64 or 128, or kind is not a crkv_q8_kind. */
size_t crkv_q8_bytes(int H_kv, int len, int d, int kind);

/* Quantises n segments (K and V kinds mixed) in one call: one launch per
 * kind present. Requires opts->dtype == CRKV_BF16 (the input type), H_kv >= 1,
 * d in {64, 128}, H_kv * len < 2^31. opts->mode is ignored;
 * opts->timing_events bracket the launches. */
int crkv_quantize_q8(const crkv_q8_seg *segs, int n, int H_kv, int d, const crkv_opts *opts);

/* The launch configuration crkv_attn_chunks_batched would use for these
 * arguments: *kernel = 0 for the fp32 kernel, 1 for the bf16 kernel with one
 * wave per SIMD, 2 for the bf16 kernel with producer/consumer wave pairs;
 * *row_tiles = 16-row tiles per wave (or wave pair), *workgroups = grid size.
 * Host-only (no device work); for inspection and tuning. Returns CRKV_OK, or
 * CRKV_E_INVAL for invalid arguments or NULL outputs. */
int crkv_plan_info(const crkv_problem *problems, int n_problems, int H, int H_kv, int d,
                   const crkv_opts *opts, int *kernel, int *row_tiles, int *workgroups);

/* The plan crkv_attn_chunks_batched would make for these arguments, in more
 * detail than crkv_plan_info (host-only, for inspection and tuning):
 * kernel, row_tiles, workgroups as there; pass1_separate = 1 when the row
 * log-sum-exp runs as a kernel of its own before pass 2; split_blocks = row
 * blocks whose keys are cut into ranges (max_ranges at most per block; their
 * fp32 output partials are summed by combine_workgroups workgroups);
 * model_cycles = the planner's modelled duration of pass 2 in shader cycles
 * (items dealt to XCDs, one workgroup per CU) and work_cycles = the modelled
 * work summed over items, so model_cycles * 256 / work_cycles - 1 is the
 * modelled load imbalance; scratch_bytes = crkv_workspace_size. Returns
 * CRKV_OK, or CRKV_E_INVAL for invalid arguments or a NULL st. */
typedef struct crkv_plan_stat {
    int kernel;
    int row_tiles;
    int workgroups;
    int pass1_separate;
    int split_blocks;
    int max_ranges;
    int combine_workgroups;
    int pad;
    double model_cycles;
    double work_cycles;
    size_t scratch_bytes;
} crkv_plan_stat;

int crkv_plan_stats(const crkv_problem *problems, int n_problems, int H, int H_kv, int d,
                    const crkv_opts *opts, crkv_plan_stat *st);

/*
 * Moving the K/V rows of selected keys (CacheBlend summary, the three-phase
 * flowchart: the K/V values of exactly the selected high-impact tokens are
 * recomputed, and generation then runs on the fused cache). The recompute
 * needs model weights and is the caller's; these calls move the rows:
 *   crkv_gather_kv:  K_sel[h][j] = K_cat[h][idx[j]], V_sel likewise;
 *   crkv_scatter_kv: K_cat[h][idx[j]] = K_sel[h][j], V_cat likewise;
 * K_cat is the concatenation of the m + 1 segments (never formed). Rows are
 * copied bit for bit in opts->dtype (opts->mode is ignored). idx holds
 * positions in the concatenation: crkv_topk's output over the document keys
 * can be passed as it is. A position outside [0, N) gathers a zero row and
 * scatters nothing. Scatter indices must be distinct (with duplicates, which
 * row lands is unspecified). Every selection of the array is done in one
 * launch; opts->timing_events bracket it.
 */
typedef struct crkv_kv_select {
    void *const *chunk_K;      /* host array of m + 1 device pointers, [H_kv][chunk_len[c]][d];
                                  written by crkv_scatter_kv, only read by crkv_gather_kv */
    void *const *chunk_V;
    const int32_t *chunk_len;  /* host array of m + 1 lengths (>= 0) */
    int m;
    const int32_t *idx;        /* device int32 [k] */
    int k;                     /* >= 0; 0 moves nothing */
    void *K_sel;               /* device [H_kv][k][d], written by gather, read by scatter */
    void *V_sel;
} crkv_kv_select;

/* All pointers 16-byte aligned; H_kv >= 1; d in {64, 128}; N < 2^30. */
int crkv_gather_kv(const crkv_kv_select *sel, int n, int H_kv, int d, const crkv_opts *opts);
int crkv_scatter_kv(const crkv_kv_select *sel, int n, int H_kv, int d, const crkv_opts *opts);

/*
 * Moving cached keys to new positions under rotary position embedding
 * (TurboRAG summary, implementation notes: with rotary embedding the
 * position IDs a chunk's cache was built with must agree with those it is
 * used at, e.g. a chunk precomputed at positions 0 .. len-1 and placed at
 * offset o of the concatenation). The pages give no formula; this is the
 * standard rotary embedding in the rotate-half arrangement. For each key row
 * x of a segment and i < d/2, with a_i = delta * base^(-2i/d):
 *   y_i       = x_i cos(a_i) - x_{i+d/2} sin(a_i)
 *   y_{i+d/2} = x_{i+d/2} cos(a_i) + x_i sin(a_i)
 * in place, in opts->dtype (float32 arithmetic, cos and sin evaluated in
 * double on the host, one rounding to the stored type). Rotations compose:
 * delta moves keys by delta positions, -delta moves them back. Segments with
 * len == 0 or delta == 0 are left untouched (no memory traffic). V has no
 * positional rotation and is not an argument. opts->mode is ignored;
 * opts->timing_events bracket the launch.
 */
typedef struct crkv_rope_seg {
    void *K;     /* device [H_kv][len][d], rotated in place; 16-byte aligned */
    int len;     /* >= 0 */
    int delta;   /* new position minus old position */
} crkv_rope_seg;

/* All segments in one launch. H_kv >= 1, d in {64, 128}, base finite > 1
 * (10000 in the common models), H_kv * len < 2^31. */
int crkv_rope_shift(const crkv_rope_seg *segs, int n, int H_kv, int d, double base, const crkv_opts *opts);

const char *crkv_status_string(int status);
const char *crkv_last_error(void);
int crkv_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CRKV_H */
