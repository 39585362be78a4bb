/*
 * pivot.h - C ABI of the PIVOT group-shared sparse-attention indexer for
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed (PIVOT paper summary page, picx.dev):
 *   eq. (1)  I_{t,s} = sum_{j<H} w_{t,j} ReLU(q_{t,j} . k_s),   T_t = TopK(I_{t,:}, k)
 *   eq. (2)  prefill groups: g consecutive query rows
 *   eq. (3)  decode groups: the current token and its d drafts, g = d + 1
 *   eq. (4)  proxy: per-head mean of the group's q and w
 *   eq. (5)  proxy scan: Ibar_s = sum_j wbar_j ReLU(qbar_j . k_s), s <= t
 *   eq. (6)  PIVOT-Reuse: the proxy's top-k is every member's T_t
 *   eq. (7)  PIVOT-Refine candidates: C = TopK(Ibar, c), c = 2k by default
 *   eqs. (8)-(9)  each member re-scores only C with its own q, w; TopK(., k)
 *
 * Conventions fixed by this library (the pages leave them open):
 *   - a query row r of a sequence sits at position t = lk - lq + r; it scores
 *     keys s <= t (inclusive);
 *   - a group's proxy scans s <= t_last (its last member's position) once;
 *     Reuse gives that one row to every member (so an earlier member may get
 *     positions in (t, t_last]); a Refine member at t drops candidates s > t;
 *   - the proxy is an fp32 sum over members in order, one division by the
 *     member count (a short last group uses its own count), rounded to the
 *     q storage type (RNE); wbar stays fp32;
 *   - selection order: higher score first, equal scores by lower position;
 *   - every output row lists the selected positions in ASCENDING order,
 *     followed by -1 (scores: the matching values, then -INFINITY), unless
 *     the config asks for rank order (pivot_config.order);
 *   - a row holds min(k, #eligible keys) valid entries; |C| = min(c, t_last+1).
 *
 * Layouts (dense, row-major, device memory unless stated):
 *   q        [batch, lq, heads, dim]   dtype (bf16 or f32)
 *   w        [batch, lq, heads]        f32
 *   k        [batch, lk, dim]          dtype; one key per token, shared by all heads
 *   indices  [batch, lq, topk]         int32 (required output)
 *   scores   [batch, lq, topk]         f32 (optional output, may be NULL)
 *   candidates        [batch, G, c]    int32 (optional Refine output, ascending, -1 pad)
 *   candidate_counts  [batch, G]       int32 (optional Refine output, |C|)
 *   where G = ceil(lq / g).
 *
 * Alignment: q, w and k start on 16-byte boundaries (any torch allocation
 * does); the workspace on 256-byte boundaries.
 *
 * Ownership and execution: the caller owns every buffer (the library never
 * allocates or frees device memory). All work is enqueued on `stream` (a
 * hipStream_t passed as void*; NULL = default stream) and the call returns
 * without synchronising. Arguments are validated before anything is enqueued;
 * on error nothing is written and a status is returned; pivot_last_error()
 * then describes it (thread-local). Calls are re-entrant; calls that share a
 * workspace must not overlap on different streams.
 *
 * Kernels: bf16 with heads == 64 or 32 and dim == 128 runs on bf16 MFMA with
 * fp32 accumulation, at any size. Every other shape, and f32 inputs, runs the exact-order kernels:
 * one lane per key, fp32 in the definition's order (heads ascending, dims
 * ascending, one rounding per product and per sum), so their results equal
 * a plain CPU evaluation bit for bit. They are meant for small problems: a
 * call whose scan and refine need more than 2^36 multiply-adds, estimated
 * as (batch * G * lk + batch * lq * min(c, lk)) * heads * dim, returns
 * PIVOT_ERR_UNSUPPORTED instead of running slowly.
 *
 * Row order: by default rows list positions in ascending order, not by
 * descending score. T_t is a set in the pages' definitions; the kernels'
 * selections are stable compactions in position order, and sparse attention
 * over T_t does not need a ranking. pivot_config.order = PIVOT_ORDER_SCORE
 * (pivot_index, pivot_index_kv, pivot_index_static) adds one pass that puts
 * every row in rank order (score descending, equal scores by lower position).
 */
#ifndef PIVOT_H
#define PIVOT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PIVOT_ABI_VERSION 7

typedef enum {
    PIVOT_OK = 0,
    PIVOT_ERR_INVALID_ARG = 1, /* null pointer, bad size, bad relation between sizes */
    PIVOT_ERR_UNSUPPORTED = 2, /* a shape or mode this build has no kernel for */
    PIVOT_ERR_WORKSPACE = 3,   /* workspace missing or smaller than pivot_workspace_size() */
    PIVOT_ERR_HIP = 4          /* a HIP launch or runtime call failed */
} pivot_status;

typedef enum { PIVOT_F32 = 0, PIVOT_BF16 = 1 } pivot_dtype;

/* PIVOT_AUTO (pivot_index only): the short-context guardrail of the pages'
 * efficiency results (PIVOT falls back to dense DSA at short context): dense
 * when lk < dense_below, else the configured auto_variant. */
typedef enum { PIVOT_DENSE = 0, PIVOT_REUSE = 1, PIVOT_REFINE = 2, PIVOT_AUTO = 3 } pivot_variant;

/* How a group becomes its proxy (the pages' aggregation hyperparameter,
 * section "Ablation Studies"): the per-head mean of eq. (4), or the first or
 * the last member's own q and w taken unchanged. */
typedef enum { PIVOT_AGG_MEAN = 0, PIVOT_AGG_FIRST = 1, PIVOT_AGG_LAST = 2 } pivot_aggregation;

/* Which proxy-scan kernel family runs on the MFMA shapes (bf16, 64 or 32 heads,
 * 128 dims); the results are the same either way:
 *   PIVOT_PATH_FUSED  one wave per group streams the group's key prefix
 *                     through LDS tiles shared by 8 groups and keeps only the
 *                     entries above a running threshold (no score row is
 *                     written); fills the GPU from 256 groups up;
 *   PIVOT_PATH_SPLIT  each group's key range is split over many workgroups,
 *                     which write the group's full score row [lk] to the
 *                     workspace for a block-wide select (decode: few groups,
 *                     long prefixes); the workspace grows with groups * lk;
 *   PIVOT_PATH_AUTO   SPLIT below 256 groups (batch * ceil(lq / g)), else
 *                     FUSED. */
typedef enum { PIVOT_PATH_AUTO = 0, PIVOT_PATH_FUSED = 1, PIVOT_PATH_SPLIT = 2 } pivot_scan_path;

/* Order of the entries inside an output row (indices and scores alike; the
 * pages define T_t = TopK(I_{t,:}, k) as a set, eq. (1), and fix no order):
 *   PIVOT_ORDER_POSITION  ascending position, then -1 (the default; what the
 *                         kernels emit, and what pivot_index_stats reads);
 *   PIVOT_ORDER_SCORE     rank order: score descending, equal scores by
 *                         lower position (the selection rule itself), then
 *                         -1. A pass over the finished rows permutes each
 *                         row in place (one read and one write of indices
 *                         and scores); it needs the scores output (its sort
 *                         key) and 1 <= topk <= 8192. The Refine candidate
 *                         set C stays in ascending position. */
typedef enum { PIVOT_ORDER_POSITION = 0, PIVOT_ORDER_SCORE = 1 } pivot_order;

/* Default guardrail of PIVOT_AUTO: the key count below which dense (g = 1) is
 * faster than PIVOT-Refine (g = 8, k = 2048, c = 4096) on MI355X, measured on
 * one GPU over L = 4K..64K (dense 0.18 / 0.85 / 1.62 ms against Refine
 * 0.38 / 0.80 / 1.32 ms at L = 4096 / 8192 / 12288). */
#define PIVOT_DENSE_BELOW_DEFAULT 8192

/* Problem shape. Prefill: batch = 1 (or more independent sequences), lq = lk.
 * Decode (eq. 3): lq = g rows at the last g positions of each sequence. */
typedef struct {
    int64_t batch; /* >= 1 */
    int64_t lq;    /* query rows per sequence, 1 <= lq <= lk */
    int64_t lk;    /* key rows per sequence, lk < 2^31 */
    int32_t heads; /* H_I >= 1 */
    int32_t dim;   /* d >= 1 (multiple of 8 for bf16, of 4 for f32) */
    int32_t dtype; /* pivot_dtype of q and k */
} pivot_problem;

/* Bytes of device workspace a call needs (variant: pivot_variant; g, c are
 * ignored where the variant has no such parameter). */
pivot_status pivot_workspace_size(const pivot_problem *p, int32_t variant, int32_t g, int32_t topk, int32_t c,
                                  size_t *bytes);

/* eq. (1) with T_t = TopK(I_{t,:}, topk): the dense DSA indexer (PIVOT with
 * g = 1). indices/scores as above. */
pivot_status pivot_index_dense(const pivot_problem *p, const void *q, const float *w, const void *k, int32_t topk,
                               int32_t *indices, float *scores, void *workspace, size_t workspace_bytes,
                               void *stream);

/* eqs. (4)-(6): PIVOT-Reuse with groups of g rows (g >= 1). */
pivot_status pivot_index_reuse(const pivot_problem *p, const void *q, const float *w, const void *k, int32_t g,
                               int32_t topk, int32_t *indices, float *scores, void *workspace,
                               size_t workspace_bytes, void *stream);

/* eqs. (4)-(5), (7)-(9): PIVOT-Refine with groups of g rows and c >= topk
 * candidates per group. candidates / candidate_counts may be NULL. */
pivot_status pivot_index_refine(const pivot_problem *p, const void *q, const float *w, const void *k, int32_t g,
                                int32_t topk, int32_t c, int32_t *indices, float *scores, int32_t *candidates,
                                int32_t *candidate_counts, void *workspace, size_t workspace_bytes, void *stream);

/* One call with every knob (eqs. (1)-(9), the aggregation ablation and the
 * guardrail). Zero-initialise the struct or start from pivot_config_init. */
typedef struct {
    int32_t variant;       /* pivot_variant */
    int32_t g;             /* group size, >= 1 (Reuse, Refine) */
    int32_t topk;          /* k, >= 1 */
    int32_t c;             /* candidates per group, >= topk (Refine) */
    int32_t aggregation;   /* pivot_aggregation of the proxy (Reuse, Refine) */
    int32_t member_causal; /* 1: a Reuse member at t keeps the proxy's top-k over s <= t (eq. (6) read
                              per member) instead of the group's one row over s <= t_last; needs
                              topk + g - 1 <= 4096. Valid with PIVOT_REUSE, and with PIVOT_AUTO,
                              where it applies when the call resolves to Reuse; an error with an
                              explicit dense or Refine variant (Refine members already drop s > t) */
    int32_t auto_variant;  /* PIVOT_AUTO: PIVOT_REUSE or PIVOT_REFINE above the guardrail */
    int32_t scan_path;     /* pivot_scan_path; 0 = PIVOT_PATH_AUTO */
    int64_t dense_below;   /* PIVOT_AUTO: dense when lk < dense_below; 0 = PIVOT_DENSE_BELOW_DEFAULT */
    int32_t order;         /* pivot_order of the output rows; 0 = PIVOT_ORDER_POSITION */
    int32_t reserved;      /* must be 0 */
} pivot_config;

/* Defaults: Refine, g = 8, topk = 2048, c = 4096, mean proxy, group rows,
 * auto_variant = Refine, automatic scan path, default guardrail, rows in
 * ascending position. */
pivot_status pivot_config_init(pivot_config *cfg);

/* The variant a pivot_index call with this config runs (resolves PIVOT_AUTO). */
pivot_status pivot_resolve_variant(const pivot_problem *p, const pivot_config *cfg, int32_t *variant);

/* Bytes of workspace pivot_index needs for this config. */
pivot_status pivot_index_workspace_size(const pivot_problem *p, const pivot_config *cfg, size_t *bytes);

/* The indexer under cfg; outputs as for the three calls above. candidates /
 * candidate_counts (may be NULL) are written only when the resolved variant is
 * Refine. With member_causal, row t holds min(k, t + 1) entries, all s <= t. */
pivot_status pivot_index(const pivot_problem *p, const pivot_config *cfg, const void *q, const float *w,
                         const void *k, int32_t *indices, float *scores, int32_t *candidates,
                         int32_t *candidate_counts, void *workspace, size_t workspace_bytes, void *stream);

/* pivot_index without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The call allocates nothing: its scratch
 * is a static device array of PIVOT_STATIC_SCRATCH_BYTES in the library, one
 * per GPU (the calling thread's current device, which `stream` must belong
 * to), held until the process ends. Every call on a GPU shares that GPU's
 * array, so calls that overlap on one GPU (other threads, other streams, or
 * a stream not yet drained of an earlier call) race and must be serialised
 * by the caller. Nothing in the scratch needs to start at any value: each
 * call writes every scratch word it reads. A call whose scratch need
 * (pivot_index_workspace_size) exceeds the array returns PIVOT_ERR_WORKSPACE
 * before anything is enqueued. Contiguous keys only; timing hooks are not
 * recorded. Outputs and errors as for pivot_index. */
#define PIVOT_STATIC_SCRATCH_BYTES (64u << 20)
pivot_status pivot_index_static(const pivot_problem *p, const pivot_config *cfg, const void *q, const float *w,
                                const void *k, int32_t *indices, float *scores, int32_t *candidates,
                                int32_t *candidate_counts, void *stream);

/* Keys of a ragged and/or paged batch (batched decode with per-sequence
 * prefixes, in the page layout of a serving KV cache). The pages print no
 * batch format; this one is the library's own.
 *   k           contiguous: [batch, lk, dim] (row stride lk per sequence);
 *               paged: a pool [num_pages, page_size, dim]; q's dtype, device.
 *   seq_lens    [batch] int32 (device) or NULL: sequence b holds seq_lens[b]
 *               keys (its key positions 0 .. seq_lens[b] - 1), and its lq
 *               query rows sit at its last lq positions; NULL: lk each.
 *               Values are expected in [lq, lk]; values outside [0, lk] are
 *               clamped (no key outside the storage is read), and a row whose
 *               position falls below 0 selects nothing (all -1).
 *   page_table  [batch, max_pages] int32 (device) or NULL (contiguous): the
 *               pool page holding keys [j * page_size, (j + 1) * page_size)
 *               of sequence b is page_table[b * max_pages + j]; entries
 *               outside [0, num_pages) are clamped into the pool. Only the
 *               pages covering each sequence's keys are read.
 *   page_size   keys per page (>= 1); max_pages >= ceil(lk / page_size).
 * Positions in the outputs are logical (0 .. seq_lens[b] - 1). */
typedef struct {
    const void *k;
    const int32_t *seq_lens;
    const int32_t *page_table;
    int64_t num_pages;
    int32_t page_size;
    int32_t max_pages;
} pivot_keys;

/* pivot_index over a ragged / paged batch (p->lk is the key capacity per
 * sequence). Every kernel reads keys through the page table, so paged keys
 * take the same scan path as contiguous ones. */
pivot_status pivot_index_kv(const pivot_problem *p, const pivot_config *cfg, const void *q, const float *w,
                            const pivot_keys *keys, int32_t *indices, float *scores, int32_t *candidates,
                            int32_t *candidate_counts, void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace pivot_index_kv needs. */
pivot_status pivot_index_kv_workspace_size(const pivot_problem *p, const pivot_config *cfg, const pivot_keys *keys,
                                           size_t *bytes);

/* eq. (4) alone: qbar [batch, G, heads, dim] in the q dtype, wbar [batch, G,
 * heads] f32. Needs no workspace. */
pivot_status pivot_pool(const pivot_problem *p, int32_t g, const void *q, const float *w, void *qbar, float *wbar,
                        void *stream);

/* pivot_pool with a pivot_aggregation (PIVOT_AGG_FIRST / LAST copy that
 * member's q and w). */
pivot_status pivot_pool_ex(const pivot_problem *p, int32_t g, int32_t aggregation, const void *q, const float *w,
                           void *qbar, float *wbar, void *stream);

/* eq. (5) alone, for inspection: out [batch, G, lk] f32 receives the proxy
 * score of every key s <= t_last of each group and -INFINITY after it.
 * qbar/wbar as produced by pivot_pool (pass q, w with g = 1 for eq. 1). */
pivot_status pivot_proxy_scores(const pivot_problem *p, int32_t g, const void *qbar, const float *wbar,
                                const void *k, float *out, void *stream);

/* O1-O3 diagnostics of index rows (the key observations of the pages'
 * summary, Figure 2) on device buffers, for any rows the calls above return:
 * indices [batch, lq, k] int32, each row its selected positions ascending,
 * then -1. Outputs (each may be NULL; at least one must be given):
 *   overlap     [batch, lq] int32: |T_t ∩ T_{t+d}| for rows t and t + d of
 *               one sequence (d = 1: adjacent queries; d = g - 1: across a
 *               group), -1 where t + d >= lq;
 *   group_union / group_inter [batch, ceil(lq / g)] int32: the size of the
 *               union and of the intersection of each group of g consecutive
 *               rows (the last group may be short);
 *   mass        [batch, lq, 3] f32: for f = 1/4, 1/2, 3/4, the sum of the
 *               floor(f k) largest scores of the row over the sum of all its
 *               scores (the whole row when it is shorter), NaN when that sum
 *               is not positive; needs scores [batch, lq, k] f32 aligned with
 *               indices.
 * Limits: 1 <= k <= 4096; d >= 1; for the group outputs 1 <= g <= 64 and
 * P * K <= 16384, P the next power of two >= g and K = k rounded up to a
 * multiple of 32 (g = 8, k = 2048 fits). Sums are fp32. Enqueued on
 * `stream`; nothing allocated. */
pivot_status pivot_index_stats(int64_t batch, int64_t lq, int32_t k, const int32_t *indices, const float *scores,
                               int32_t d, int32_t g, int32_t *overlap, int32_t *group_union, int32_t *group_inter,
                               float *mass, void *stream);

/* Optional per-kernel timing (instrumentation for benchmarks). While enabled
 * on the calling thread, every kernel a pivot_* call enqueues is bracketed by
 * a pair of hipEvents on the same stream. pivot_timing_read waits for the
 * recorded events, adds the elapsed milliseconds of each stage into ms[s] and
 * the number of launches into launches[s] (arrays of PIVOT_STAGES entries;
 * either may be NULL), then forgets the records. Disabling also forgets them. */
#define PIVOT_STAGES 6
/* POOL: eq. (4) as its own launch (shapes without an MFMA scan; the MFMA
 * scans pool inside and record none); SCAN: eq. (5) with its streaming
 * filter; SCAN_SELECT: the
 * group's final top-k / top-c of eqs. (6)-(7) when the scan leaves survivors
 * for a separate kernel; SELECT: per-row selects (eq. (9), few-groups rows);
 * REFINE: eq. (8); ORDER: the rank-order pass of PIVOT_ORDER_SCORE. */
typedef enum {
    PIVOT_STAGE_POOL = 0,
    PIVOT_STAGE_SCAN = 1,
    PIVOT_STAGE_SELECT = 2,
    PIVOT_STAGE_REFINE = 3,
    PIVOT_STAGE_SCAN_SELECT = 4,
    PIVOT_STAGE_ORDER = 5
} pivot_stage;
pivot_status pivot_timing_enable(int32_t on);
pivot_status pivot_timing_read(double *ms, int64_t *launches);

const char *pivot_status_str(pivot_status s);
const char *pivot_last_error(void);
int32_t pivot_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PIVOT_H */
