/*
 * Plain CPU oracle of the PIVOT group-shared sparse-attention indexer.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library. It shares no code,
 * header or table with the HIP library; both sides are fed from the seeded
 * input generators alone.
 *
 * Sources (web pages on PIVOT):
 *   "PIVOT paper summary" (picx.dev), section "Introduction and Theoretical
 *   Foundation", eq. (1): the DSA indexer score
 *        I_{t,s} = sum_j w_{t,j} ReLU(q_{t,j} . k_s),  T_t = TopK(I_{t,:}, k);
 *   section "Methodology": eq. (2)/(3) grouping, eq. (4) per-head mean-pool
 *   proxy, eq. (5) proxy scan over s <= t, eq. (6) PIVOT-Reuse, eq. (7)
 *   candidate set C = TopK(proxy scores, c), eqs. (8)-(9) PIVOT-Refine.
 *
 * Conventions (the pages leave these open; each is a stated reading):
 *   - arithmetic: float32, products and sums rounded one at a time in the
 *     order written below (build with -ffp-contract=off, no fast-math);
 *     bf16 inputs are widened to float32 exactly;
 *   - causal bound: a query at position t scores keys s <= t (inclusive);
 *   - the proxy of a group scans s <= t_last, the position of the group's
 *     last member, once per group; a Refine member at t drops candidates
 *     s > t; Reuse hands the one proxy row to every member;
 *   - the proxy: fp32 sum over members in ascending order, one IEEE division
 *     by the member count g_m (a short last group divides by its own size),
 *     then round-to-nearest-even to the q storage type; w-bar stays fp32;
 *   - selection order: higher score first, equal scores by lower position;
 *   - output rows list the selected set in ascending position, then -1
 *     (scores: the matching values, then -inf);
 *   - |C| = min(c, t_last + 1), and a Refine row keeps min(k, |C with s<=t|).
 *
 * Variant knobs (section "Ablation Studies", proxy aggregation, and the
 * per-member reading of eq. (6)):
 *   - aggregation: the proxy is the per-head mean of eq. (4) (default), or
 *     the first or the last member's own q and w, unchanged;
 *   - member-causal Reuse: every member at t keeps the proxy's top-k over
 *     s <= t (eq. (6) with the member's own bound) instead of the group's
 *     one row over s <= t_last.
 *
 * Positions: query row r of a sequence sits at position Lk - Lq + r.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
    int64_t B, Lq, Lk;
    int32_t H, d;
    int32_t dtype; /* 0: float32, 1: bf16 stored as uint16 bit patterns */
} oracle_problem;

enum { OR_OK = 0, OR_BAD_ARG = 1, OR_NO_MEM = 2 };
enum { VAR_DENSE = 0, VAR_REUSE = 1, VAR_REFINE = 2 };
enum { AGG_MEAN = 0, AGG_FIRST = 1, AGG_LAST = 2 };

/* ---------------------------------------------------------------- storage */
static float widen(const void *base, int dtype, int64_t i)
{
    if (dtype == 0) return ((const float *)base)[i];
    uint32_t u = (uint32_t)((const uint16_t *)base)[i] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* float32 -> nearest bf16 (ties to even), returned widened back to float32 */
static float round_to_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static int check_problem(const oracle_problem *p)
{
    if (!p || p->B < 1 || p->Lq < 1 || p->Lk < 1 || p->Lq > p->Lk) return 0;
    if (p->H < 1 || p->d < 1 || (p->dtype != 0 && p->dtype != 1)) return 0;
    if (p->Lk >= ((int64_t)1 << 31)) return 0;
    return 1;
}

static int64_t n_groups(const oracle_problem *p, int g) { return (p->Lq + g - 1) / g; }

/* --------------------------------------------------------------- eq. (1) */
/* I = sum_j w_j * ReLU(q_j . k): heads ascending, dims ascending, fp32. */
static float index_score(int H, int d, const float *qv, const float *wv, const float *ks)
{
    float acc = 0.0f;
    for (int j = 0; j < H; ++j) {
        float dot = 0.0f;
        for (int i = 0; i < d; ++i) {
            float prod = qv[(int64_t)j * d + i] * ks[i];
            dot = dot + prod;
        }
        float relu = dot > 0.0f ? dot : 0.0f;
        float term = wv[j] * relu;
        acc = acc + term;
    }
    if (acc == 0.0f) acc = 0.0f; /* one zero: +0 */
    return acc;
}

/* --------------------------------------------------------------- top-k */
typedef struct {
    float s;
    int32_t i;
} scored_t;

/* higher score first, then lower position */
static int cmp_rank(const void *a, const void *b)
{
    const scored_t *x = a, *y = b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->i > y->i) - (x->i < y->i);
}

static int cmp_pos(const void *a, const void *b)
{
    const scored_t *x = a, *y = b;
    return (x->i > y->i) - (x->i < y->i);
}

/* Keep the best `keep` of v[0..n) and leave them in v[0..keep) in
 * ascending position. Returns keep = min(k, n). */
static int64_t top_k_by_rank(scored_t *v, int64_t n, int64_t k)
{
    qsort(v, (size_t)n, sizeof *v, cmp_rank);
    int64_t keep = n < k ? n : k;
    qsort(v, (size_t)keep, sizeof *v, cmp_pos);
    return keep;
}

static void write_row(int32_t *idx_row, float *score_row, int64_t topk, const scored_t *v, int64_t n)
{
    for (int64_t j = 0; j < topk; ++j) {
        if (j < n) {
            idx_row[j] = v[j].i;
            if (score_row) score_row[j] = v[j].s;
        } else {
            idx_row[j] = -1;
            if (score_row) score_row[j] = -INFINITY;
        }
    }
}

/* ------------------------------------------------------------- helpers */
static float *widen_keys(const oracle_problem *p, const void *k, int64_t b)
{
    int64_t n = p->Lk * p->d;
    float *kf = malloc(sizeof(float) * (size_t)n);
    if (!kf) return NULL;
    for (int64_t i = 0; i < n; ++i) kf[i] = widen(k, p->dtype, b * n + i);
    return kf;
}

static void widen_query_row(const oracle_problem *p, const void *q, const float *w, int64_t b, int64_t r,
                            float *qv, float *wv)
{
    int64_t hd = (int64_t)p->H * p->d;
    int64_t base = (b * p->Lq + r) * hd;
    for (int64_t i = 0; i < hd; ++i) qv[i] = widen(q, p->dtype, base + i);
    for (int j = 0; j < p->H; ++j) wv[j] = w[(b * p->Lq + r) * p->H + j];
}

/* --------------------------------------------------------------- eq. (4) */
/* Proxy of group m of sequence b: per-head mean of the members' q and w. */
static void pool_group(const oracle_problem *p, int g, const void *q, const float *w, int64_t b, int64_t m,
                       float *qbar, float *wbar)
{
    int64_t r0 = m * g, r1 = r0 + g < p->Lq ? r0 + g : p->Lq;
    float gm = (float)(r1 - r0);
    int64_t hd = (int64_t)p->H * p->d;
    for (int64_t i = 0; i < hd; ++i) {
        float sum = 0.0f;
        for (int64_t r = r0; r < r1; ++r) sum = sum + widen(q, p->dtype, (b * p->Lq + r) * hd + i);
        float mean = sum / gm;
        qbar[i] = p->dtype == 1 ? round_to_bf16(mean) : mean;
    }
    for (int j = 0; j < p->H; ++j) {
        float sum = 0.0f;
        for (int64_t r = r0; r < r1; ++r) sum = sum + w[(b * p->Lq + r) * p->H + j];
        wbar[j] = sum / gm;
    }
}

/* The proxy of group m under an aggregation: the mean of eq. (4), or one
 * member's (first or last) q and w taken as they are. */
static void proxy_of_group(const oracle_problem *p, int g, int agg, const void *q, const float *w, int64_t b,
                           int64_t m, float *qbar, float *wbar)
{
    int64_t r0 = m * g, r1 = r0 + g < p->Lq ? r0 + g : p->Lq;
    if (agg == AGG_FIRST)
        widen_query_row(p, q, w, b, r0, qbar, wbar);
    else if (agg == AGG_LAST)
        widen_query_row(p, q, w, b, r1 - 1, qbar, wbar);
    else
        pool_group(p, g, q, w, b, m, qbar, wbar);
}

int oracle_pool2(const oracle_problem *p, int32_t g, int32_t agg, const void *q, const float *w,
                 float *qbar_out, float *wbar_out)
{
    if (!check_problem(p) || g < 1 || !q || !w || !qbar_out || !wbar_out) return OR_BAD_ARG;
    if (agg < AGG_MEAN || agg > AGG_LAST) return OR_BAD_ARG;
    int64_t G = n_groups(p, g), hd = (int64_t)p->H * p->d;
    for (int64_t b = 0; b < p->B; ++b)
        for (int64_t m = 0; m < G; ++m)
            proxy_of_group(p, g, agg, q, w, b, m, qbar_out + (b * G + m) * hd, wbar_out + (b * G + m) * p->H);
    return OR_OK;
}

int oracle_pool(const oracle_problem *p, int32_t g, const void *q, const float *w, float *qbar_out,
                float *wbar_out)
{
    return oracle_pool2(p, g, AGG_MEAN, q, w, qbar_out, wbar_out);
}

/* ------------------------------------------------------------ eq. (5) */
/* Proxy score row of one group: out[s] for s in [0, t_last]. */
int oracle_proxy_row2(const oracle_problem *p, int32_t g, int32_t agg, const void *q, const float *w,
                      const void *k, int64_t b, int64_t m, float *out)
{
    if (!check_problem(p) || g < 1 || b < 0 || b >= p->B || m < 0 || m >= n_groups(p, g)) return OR_BAD_ARG;
    if (agg < AGG_MEAN || agg > AGG_LAST) return OR_BAD_ARG;
    int64_t hd = (int64_t)p->H * p->d;
    int64_t last = (m + 1) * g - 1 < p->Lq - 1 ? (m + 1) * g - 1 : p->Lq - 1;
    int64_t t_last = p->Lk - p->Lq + last;
    float *kf = widen_keys(p, k, b);
    float *qbar = malloc(sizeof(float) * (size_t)hd), *wbar = malloc(sizeof(float) * (size_t)p->H);
    int rc = OR_OK;
    if (!kf || !qbar || !wbar) {
        rc = OR_NO_MEM;
    } else {
        proxy_of_group(p, g, agg, q, w, b, m, qbar, wbar);
        for (int64_t s = 0; s <= t_last; ++s) out[s] = index_score(p->H, p->d, qbar, wbar, kf + s * p->d);
    }
    free(kf);
    free(qbar);
    free(wbar);
    return rc;
}

int oracle_proxy_row(const oracle_problem *p, int32_t g, const void *q, const float *w, const void *k,
                     int64_t b, int64_t m, float *out)
{
    return oracle_proxy_row2(p, g, AGG_MEAN, q, w, k, b, m, out);
}

/* ------------------------------------------------------------ variants */
/*
 * oracle_run: the indexer for one variant.
 *
 *   variant   0 dense (eq. 1), 1 Reuse (eqs. 4-6), 2 Refine (eqs. 4-5, 7-9)
 *   g         group size (ignored by dense)
 *   topk, c   k of eq. (1)/(6)/(9) and c of eq. (7) (Refine only; c >= topk)
 *   units     optional list of the work units to compute: flat row ids
 *             b*Lq + r for dense, flat group ids b*G + m otherwise; NULL = all
 *   indices   [B, Lq, topk] int32; rows of the listed units are written
 *   scores    [B, Lq, topk] float or NULL
 *   cand      [B, G, c] int32 or NULL (Refine: C in ascending position, -1 pad)
 *   cand_n    [B, G] int32 or NULL (Refine: |C|)
 *   cand_in / cand_in_n: optional candidate sets to use in place of eq. (7)
 *             (Refine only; same layout as cand / cand_n)
 *   counters  double[3] or NULL: proxy dot products (H per scored key of a
 *             proxy), member re-score dot products, dense dot products
 *
 * oracle_run2 adds the variant knobs: agg (0 mean, 1 first member, 2 last
 * member) for the proxy of Reuse and Refine, and member_causal (Reuse only:
 * each member keeps the proxy's top-k over s <= its own t).
 */
int oracle_run2(const oracle_problem *p, int32_t variant, int32_t g, int32_t topk, int32_t c, int32_t agg,
                int32_t member_causal, const void *q, const float *w, const void *k, const int64_t *units,
                int64_t n_units, int32_t *indices, float *scores, int32_t *cand, int32_t *cand_n,
                const int32_t *cand_in, const int32_t *cand_in_n, double *counters)
{
    if (!check_problem(p) || !q || !w || !k || !indices || topk < 1) return OR_BAD_ARG;
    if (variant < VAR_DENSE || variant > VAR_REFINE) return OR_BAD_ARG;
    if (agg < AGG_MEAN || agg > AGG_LAST) return OR_BAD_ARG;
    if (member_causal && variant != VAR_REUSE) return OR_BAD_ARG;
    if (variant == VAR_DENSE) g = 1;
    if (g < 1) return OR_BAD_ARG;
    if (variant == VAR_REFINE && c < topk) return OR_BAD_ARG;
    if (variant != VAR_REFINE && (cand_in || cand_in_n)) return OR_BAD_ARG;
    if ((cand_in == NULL) != (cand_in_n == NULL)) return OR_BAD_ARG;

    const int64_t G = n_groups(p, g);
    const int64_t total_units = variant == VAR_DENSE ? p->B * p->Lq : p->B * G;
    if (!units) n_units = total_units;
    for (int64_t u = 0; units && u < n_units; ++u)
        if (units[u] < 0 || units[u] >= total_units) return OR_BAD_ARG;

    const int64_t hd = (int64_t)p->H * p->d;
    double c_proxy = 0.0, c_refine = 0.0, c_dense = 0.0;
    int rc = OR_OK;

    /* widened keys, one sequence at a time */
    for (int64_t b = 0; b < p->B && rc == OR_OK; ++b) {
        float *kf = widen_keys(p, k, b);
        if (!kf) return OR_NO_MEM;

#pragma omp parallel reduction(+ : c_proxy, c_refine, c_dense)
        {
            float *qv = malloc(sizeof(float) * (size_t)hd);
            float *wv = malloc(sizeof(float) * (size_t)p->H);
            scored_t *row = malloc(sizeof(scored_t) * (size_t)p->Lk);
            scored_t *cset = malloc(sizeof(scored_t) * (size_t)p->Lk);
            int local_ok = qv && wv && row && cset;
            if (!local_ok) {
#pragma omp atomic write
                rc = OR_NO_MEM;
            }

#pragma omp for schedule(dynamic, 1)
            for (int64_t u = 0; u < n_units; ++u) {
                int64_t unit = units ? units[u] : u;
                int64_t per_seq = variant == VAR_DENSE ? p->Lq : G;
                if (!local_ok || unit / per_seq != b) continue;
                int64_t local = unit % per_seq;

                if (variant == VAR_DENSE) {
                    /* eq. (1): the query scores every key s <= t */
                    int64_t r = local, t = p->Lk - p->Lq + r;
                    widen_query_row(p, q, w, b, r, qv, wv);
                    for (int64_t s = 0; s <= t; ++s) {
                        row[s].s = index_score(p->H, p->d, qv, wv, kf + s * p->d);
                        row[s].i = (int32_t)s;
                    }
                    c_dense += (double)p->H * (double)(t + 1);
                    int64_t n = top_k_by_rank(row, t + 1, topk);
                    int64_t o = (b * p->Lq + r) * topk;
                    write_row(indices + o, scores ? scores + o : NULL, topk, row, n);
                    continue;
                }

                /* eqs. (2)-(4): the group and its proxy */
                int64_t m = local, r0 = m * g, r1 = r0 + g < p->Lq ? r0 + g : p->Lq;
                int64_t t_last = p->Lk - p->Lq + (r1 - 1);
                int64_t nc = 0; /* |C| */

                if (!(variant == VAR_REFINE && cand_in)) {
                    proxy_of_group(p, g, agg, q, w, b, m, qv, wv);
                    /* eq. (5): one scan of the prefix s <= t_last */
                    for (int64_t s = 0; s <= t_last; ++s) {
                        row[s].s = index_score(p->H, p->d, qv, wv, kf + s * p->d);
                        row[s].i = (int32_t)s;
                    }
                    c_proxy += (double)p->H * (double)(t_last + 1);
                }

                if (variant == VAR_REUSE && member_causal) {
                    /* eq. (6) per member: the proxy's top-k over s <= t */
                    for (int64_t r = r0; r < r1; ++r) {
                        int64_t t = p->Lk - p->Lq + r;
                        memcpy(cset, row, sizeof(scored_t) * (size_t)(t + 1));
                        int64_t n = top_k_by_rank(cset, t + 1, topk);
                        int64_t o = (b * p->Lq + r) * topk;
                        write_row(indices + o, scores ? scores + o : NULL, topk, cset, n);
                    }
                    continue;
                }
                if (variant == VAR_REUSE) {
                    /* eq. (6): the proxy's top-k is every member's row */
                    int64_t n = top_k_by_rank(row, t_last + 1, topk);
                    for (int64_t r = r0; r < r1; ++r) {
                        int64_t o = (b * p->Lq + r) * topk;
                        write_row(indices + o, scores ? scores + o : NULL, topk, row, n);
                    }
                    continue;
                }

                /* eq. (7): candidate set C (ascending position) */
                if (cand_in) {
                    nc = cand_in_n[b * G + m];
                    if (nc < 0 || nc > c || nc > t_last + 1) {
#pragma omp atomic write
                        rc = OR_BAD_ARG;
                        continue;
                    }
                    for (int64_t j = 0; j < nc; ++j) {
                        cset[j].i = cand_in[(b * G + m) * c + j];
                        cset[j].s = 0.0f;
                    }
                } else {
                    nc = top_k_by_rank(row, t_last + 1, c);
                    memcpy(cset, row, sizeof(scored_t) * (size_t)nc);
                }
                if (cand) {
                    for (int64_t j = 0; j < c; ++j) cand[(b * G + m) * c + j] = j < nc ? cset[j].i : -1;
                }
                if (cand_n) cand_n[b * G + m] = (int32_t)nc;

                /* eqs. (8)-(9): each member re-scores C with its own q, w and
                 * keeps its top-k among the candidates s <= t */
                for (int64_t r = r0; r < r1; ++r) {
                    int64_t t = p->Lk - p->Lq + r, nv = 0;
                    widen_query_row(p, q, w, b, r, qv, wv);
                    for (int64_t j = 0; j < nc; ++j) {
                        int32_t s = cset[j].i;
                        float sc = index_score(p->H, p->d, qv, wv, kf + (int64_t)s * p->d);
                        if (s <= t) {
                            row[nv].s = sc;
                            row[nv].i = s;
                            ++nv;
                        }
                    }
                    c_refine += (double)p->H * (double)nc;
                    int64_t n = top_k_by_rank(row, nv, topk);
                    int64_t o = (b * p->Lq + r) * topk;
                    write_row(indices + o, scores ? scores + o : NULL, topk, row, n);
                }
            }
            free(qv);
            free(wv);
            free(row);
            free(cset);
        }
        free(kf);
    }
    if (counters) {
        counters[0] = c_proxy;
        counters[1] = c_refine;
        counters[2] = c_dense;
    }
    return rc;
}

int oracle_run(const oracle_problem *p, int32_t variant, int32_t g, int32_t topk, int32_t c, const void *q,
               const float *w, const void *k, const int64_t *units, int64_t n_units, int32_t *indices,
               float *scores, int32_t *cand, int32_t *cand_n, const int32_t *cand_in, const int32_t *cand_in_n,
               double *counters)
{
    return oracle_run2(p, variant, g, topk, c, AGG_MEAN, 0, q, w, k, units, n_units, indices, scores, cand, cand_n,
                       cand_in, cand_in_n, counters);
}

/* ------------------------------------------ scores at chosen positions */
/*
 * oracle_scores_at: eq. (1) scores of chosen query rows (proxy = 0; unit =
 * flat row b*Lq + r, scored with its own q and w) or eq. (5) scores of
 * chosen group proxies (proxy = 1; unit = flat group b*G + m, its proxy from
 * g and agg as in oracle_run2), at chosen key positions:
 *   out[i * npos + j] = score of units[i] at key pos[i * npos + j],
 * NaN where that position is negative or not below Lk. No causal bound is
 * applied: this is the score function itself, for checking the scores (and
 * the near-boundary positions) another implementation selected.
 */
int oracle_scores_at(const oracle_problem *p, int32_t proxy, int32_t g, int32_t agg, const void *q, const float *w,
                     const void *k, const int64_t *units, int64_t n_units, const int32_t *pos, int64_t npos,
                     float *out)
{
    if (!check_problem(p) || !q || !w || !k || !units || !pos || !out || n_units < 0 || npos < 0) return OR_BAD_ARG;
    if (proxy != 0 && proxy != 1) return OR_BAD_ARG;
    if (proxy && (g < 1 || agg < AGG_MEAN || agg > AGG_LAST)) return OR_BAD_ARG;
    const int64_t per_seq = proxy ? n_groups(p, g) : p->Lq;
    for (int64_t u = 0; u < n_units; ++u)
        if (units[u] < 0 || units[u] >= p->B * per_seq) return OR_BAD_ARG;
    const int64_t hd = (int64_t)p->H * p->d;
    int rc = OR_OK;
#pragma omp parallel
    {
        float *qv = malloc(sizeof(float) * (size_t)hd);
        float *wv = malloc(sizeof(float) * (size_t)p->H);
        float *ks = malloc(sizeof(float) * (size_t)p->d);
        int local_ok = qv && wv && ks;
        if (!local_ok) {
#pragma omp atomic write
            rc = OR_NO_MEM;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t u = 0; u < n_units; ++u) {
            if (!local_ok) continue;
            const int64_t b = units[u] / per_seq, local = units[u] % per_seq;
            if (proxy)
                proxy_of_group(p, g, agg, q, w, b, local, qv, wv);
            else
                widen_query_row(p, q, w, b, local, qv, wv);
            for (int64_t j = 0; j < npos; ++j) {
                const int64_t s = pos[u * npos + j];
                if (s < 0 || s >= p->Lk) {
                    out[u * npos + j] = NAN;
                    continue;
                }
                for (int i = 0; i < p->d; ++i) ks[i] = widen(k, p->dtype, (b * p->Lk + s) * p->d + i);
                out[u * npos + j] = index_score(p->H, p->d, qv, wv, ks);
            }
        }
        free(qv);
        free(wv);
        free(ks);
    }
    return rc;
}

/* Threads of the OpenMP loops above (n >= 1); results never depend on it. */
int oracle_set_threads(int32_t n)
{
    if (n < 1) return OR_BAD_ARG;
#ifdef _OPENMP
    omp_set_num_threads(n);
#endif
    return OR_OK;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
