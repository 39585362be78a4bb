// C ABI of the PIVOT indexer: argument checks, workspace layout and the
// launch sequence (pool -> scan/select -> refine) on the caller's stream.
// Declarations and conventions: include/pivot.h.

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "pivot.h"
#include "pivot_kernels.h"

#include <atomic>
#include <mutex>
#include <vector>

namespace {

thread_local char g_last_error[512] = "";

// ---------------------------------------------------------------- timing
struct TimedLaunch {
    int stage;
    hipEvent_t start, stop;
};
thread_local bool g_timing = false;
thread_local bool g_timing_off = false;  // set while pivot_index_static runs (it creates no events)
thread_local std::vector<TimedLaunch> g_timed;

void forget_timing()
{
    for (auto &t : g_timed) {
        (void)hipEventDestroy(t.start);
        (void)hipEventDestroy(t.stop);
    }
    g_timed.clear();
}

// Brackets one kernel launch with events when timing is enabled.
struct StageTimer {
    TimedLaunch rec{};
    bool armed = false;
    hipStream_t stream;
    StageTimer(int stage, hipStream_t s) : stream(s)
    {
        if (!g_timing || g_timing_off) return;
        rec.stage = stage;
        if (hipEventCreate(&rec.start) != hipSuccess) return;
        if (hipEventCreate(&rec.stop) != hipSuccess) {
            (void)hipEventDestroy(rec.start);
            return;
        }
        armed = hipEventRecord(rec.start, stream) == hipSuccess;
    }
    ~StageTimer()
    {
        if (!armed) return;
        if (hipEventRecord(rec.stop, stream) == hipSuccess) {
            g_timed.push_back(rec);
        } else {
            (void)hipEventDestroy(rec.start);
            (void)hipEventDestroy(rec.stop);
        }
    }
};

pivot_status fail(pivot_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return s;
}

constexpr size_t kAlign = 256;
// bound on topk and c: keeps a group's survivor buffer (2 cap words, cap <=
// 2 K) addressable by one 32-bit buffer resource and its indices in int32
constexpr int64_t kMaxSel = int64_t(1) << 27;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

pivot_status check_problem(const pivot_problem *p)
{
    if (!p) return fail(PIVOT_ERR_INVALID_ARG, "problem is NULL");
    if (p->batch < 1 || p->lq < 1 || p->lk < 1) return fail(PIVOT_ERR_INVALID_ARG, "batch, lq and lk must be >= 1");
    if (p->lq > p->lk) return fail(PIVOT_ERR_INVALID_ARG, "lq (%lld) must not exceed lk (%lld)", (long long)p->lq,
                                   (long long)p->lk);
    if (p->lk >= (int64_t(1) << 31)) return fail(PIVOT_ERR_INVALID_ARG, "lk must be < 2^31");
    if (p->heads < 1 || p->dim < 1) return fail(PIVOT_ERR_INVALID_ARG, "heads and dim must be >= 1");
    if (p->dtype != PIVOT_F32 && p->dtype != PIVOT_BF16) return fail(PIVOT_ERR_INVALID_ARG, "unknown dtype %d", p->dtype);
    const int vec = p->dtype == PIVOT_BF16 ? 8 : 4;
    if (p->dim % vec != 0)
        return fail(PIVOT_ERR_UNSUPPORTED, "dim must be a multiple of %d for this dtype (got %d)", vec, p->dim);
    if (p->heads > 4096 || p->dim > 4096) return fail(PIVOT_ERR_UNSUPPORTED, "heads and dim are limited to 4096");
    return PIVOT_OK;
}

pivot::LaunchShape shape_of(const pivot_problem *p)
{
    return pivot::LaunchShape{p->batch, p->lq, p->lk, p->heads, p->dim, p->dtype == PIVOT_BF16};
}

// A call after PIVOT_AUTO has been resolved: variant is DENSE, REUSE or
// REFINE, g = 1 for DENSE.
struct Cfg {
    int variant;
    int32_t g, topk, c;
    int agg;      // pivot_aggregation
    bool causal;  // member-causal Reuse
    int path;     // pivot_scan_path
    bool rank;    // rows in rank order (PIVOT_ORDER_SCORE)
};

struct Layout {
    int64_t G;
    int g, K, cap;
    bool pool;
    bool few;               // few groups: split scan into score rows + block selects
    int scan_splits, refine_splits;
    size_t qbar, wbar, buf, buf_n, smp, rows, hist, cand, cand_n, cand_sc, scratch, nvalid, total;
};

// Below this many groups the per-group fused scan cannot fill 256 CUs; the
// key axis is split over workgroups instead (decode shapes). A config's
// scan_path can name either path explicitly.
constexpr int64_t kFewGroups = 256;
#ifndef PIVOT_SPLIT_SCAN_WGS
#define PIVOT_SPLIT_SCAN_WGS 512
#endif
// Workgroups of the split scan over all groups: two per CU, the waves of
// which stay resident for the whole launch (its key streams are one quarter
// deep per wave, so long-lived waves keep HBM busy).
constexpr int64_t kSplitScanWorkgroups = PIVOT_SPLIT_SCAN_WGS;

// Shapes without an MFMA kernel (f32, or bf16 with heads other than 32 or
// 64, or dim != 128) run the exact-order kernels: one lane per key, fp32 in the
// definition's order. They are meant for small problems (and for bit-exact
// checks); a call whose scan and refine need more multiply-adds than this is
// refused rather than run slowly.
constexpr double kExactMaxMacs = 68719476736.0;  // 2^36

pivot_status check_exact_work(const pivot_problem *p, int64_t G, int64_t c)
{
    if (pivot::mfma_shape(shape_of(p))) return PIVOT_OK;
    const double pairs = double(p->batch) * double(G) * double(p->lk) +
                         double(p->batch) * double(p->lq) * double(c < p->lk ? c : p->lk);
    const double macs = pairs * double(p->heads) * double(p->dim);
    if (macs > kExactMaxMacs)
        return fail(PIVOT_ERR_UNSUPPORTED,
                    "no MFMA kernel for %s with %d heads and dim %d (MFMA: bf16, 64 or 32 heads, dim 128); the exact-order "
                    "kernels take at most 2^36 multiply-adds per call, this one needs about %.3g",
                    p->dtype == PIVOT_BF16 ? "bf16" : "f32", p->heads, p->dim, macs);
    return PIVOT_OK;
}

// The short-context guardrail of PIVOT_AUTO: dense below this many keys.
int64_t dense_below(const pivot_config *cfg)
{
    return cfg->dense_below > 0 ? cfg->dense_below : PIVOT_DENSE_BELOW_DEFAULT;
}

pivot_status resolve(const pivot_problem *p, const pivot_config *cfg, Cfg *out)
{
    if (!cfg) return fail(PIVOT_ERR_INVALID_ARG, "config is NULL");
    pivot_status st = check_problem(p);
    if (st != PIVOT_OK) return st;
    Cfg c{};
    c.variant = cfg->variant;
    if (c.variant == PIVOT_AUTO) {
        if (cfg->auto_variant != PIVOT_REUSE && cfg->auto_variant != PIVOT_REFINE)
            return fail(PIVOT_ERR_INVALID_ARG, "auto_variant must be PIVOT_REUSE or PIVOT_REFINE (got %d)",
                        cfg->auto_variant);
        c.variant = p->lk < dense_below(cfg) ? PIVOT_DENSE : cfg->auto_variant;
    }
    if (c.variant < PIVOT_DENSE || c.variant > PIVOT_REFINE)
        return fail(PIVOT_ERR_INVALID_ARG, "unknown variant %d", cfg->variant);
    if (cfg->aggregation < PIVOT_AGG_MEAN || cfg->aggregation > PIVOT_AGG_LAST)
        return fail(PIVOT_ERR_INVALID_ARG, "unknown aggregation %d", cfg->aggregation);
    if (cfg->member_causal != 0 && cfg->member_causal != 1)
        return fail(PIVOT_ERR_INVALID_ARG, "member_causal must be 0 or 1");
    if (cfg->member_causal && cfg->variant != PIVOT_REUSE && !(cfg->variant == PIVOT_AUTO))
        return fail(PIVOT_ERR_INVALID_ARG, "member_causal applies to PIVOT_REUSE only");
    c.g = c.variant == PIVOT_DENSE ? 1 : cfg->g;
    c.topk = cfg->topk;
    c.c = c.variant == PIVOT_REFINE ? cfg->c : 0;
    c.agg = c.variant == PIVOT_DENSE ? PIVOT_AGG_MEAN : cfg->aggregation;
    c.causal = c.variant == PIVOT_REUSE && cfg->member_causal != 0;
    if (cfg->scan_path < PIVOT_PATH_AUTO || cfg->scan_path > PIVOT_PATH_SPLIT)
        return fail(PIVOT_ERR_INVALID_ARG, "unknown scan_path %d", cfg->scan_path);
    c.path = cfg->scan_path;
    if (cfg->reserved != 0) return fail(PIVOT_ERR_INVALID_ARG, "pivot_config.reserved must be 0");
    if (cfg->order != PIVOT_ORDER_POSITION && cfg->order != PIVOT_ORDER_SCORE)
        return fail(PIVOT_ERR_INVALID_ARG, "unknown order %d", cfg->order);
    c.rank = cfg->order == PIVOT_ORDER_SCORE;
    if (c.rank && (c.topk < 1 || c.topk > pivot::rank_rows_max()))
        return fail(PIVOT_ERR_UNSUPPORTED, "PIVOT_ORDER_SCORE needs 1 <= topk <= %d (got %d)",
                    pivot::rank_rows_max(), c.topk);
    *out = c;
    return PIVOT_OK;
}

// paged: keys in pages (every kernel translates the key rows it reads;
// the layout does not depend on it).
pivot_status plan(const pivot_problem *p, const Cfg &cfg, bool paged, Layout *L)
{
    pivot_status st = check_problem(p);
    if (st != PIVOT_OK) return st;
    const int variant = cfg.variant;
    const int32_t g = cfg.g, topk = cfg.topk, c = cfg.c;
    if (g < 1) return fail(PIVOT_ERR_INVALID_ARG, "group size g must be >= 1 (got %d)", g);
    if (topk < 1 || topk > kMaxSel) return fail(PIVOT_ERR_INVALID_ARG, "topk must be in [1, 2^27] (got %d)", topk);
    if (variant == PIVOT_REFINE) {
        if (c < topk) return fail(PIVOT_ERR_INVALID_ARG, "refine needs c >= topk (c=%d, topk=%d)", c, topk);
        if (c > kMaxSel) return fail(PIVOT_ERR_INVALID_ARG, "c must be <= 2^27");
    }
    const pivot::LaunchShape sh = shape_of(p);
    if (variant == PIVOT_REFINE && pivot::mfma_shape(sh) && g > 1024)
        return fail(PIVOT_ERR_UNSUPPORTED, "refine supports g <= 1024");
    Layout l{};
    l.g = g;
    l.G = (p->lq + g - 1) / g;
    st = check_exact_work(p, l.G, variant == PIVOT_REFINE ? c : 0);
    if (st != PIVOT_OK) return st;
    // scan selection size: c (Refine), k (Reuse, dense) or k + g - 1
    // (member-causal Reuse: every member's top-k over s <= t lies in the
    // group's top-(k + g - 1) over s <= t_last, since at most g - 1
    // positions in (t, t_last] are dropped)
    int64_t K = variant == PIVOT_REFINE ? c : topk;
    if (cfg.causal) {
        K = int64_t(topk) + g - 1;
        if (pivot::member_select_slabs(static_cast<int>(K > kMaxSel ? kMaxSel : K)) == 0)
            return fail(PIVOT_ERR_UNSUPPORTED, "member-causal Reuse needs topk + g - 1 <= 4096 (got %lld)",
                        (long long)K);
    }
    l.K = static_cast<int>(K);
    int64_t cap = 2 * int64_t(l.K);
    if (cap < l.K + 64) cap = l.K + 64;
    cap = (cap + 63) / 64 * 64;
    l.cap = static_cast<int>(cap);
    l.pool = g > 1;
    const size_t elt = p->dtype == PIVOT_BF16 ? 2 : 4;
    const size_t groups = static_cast<size_t>(p->batch) * static_cast<size_t>(l.G);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + bytes);
        return at;
    };
    l.few = pivot::mfma_shape(sh) &&
            (cfg.path == PIVOT_PATH_SPLIT || (cfg.path == PIVOT_PATH_AUTO && static_cast<int64_t>(groups) < kFewGroups));
    // the proxies go through HBM only where the pool kernel forms them (the
    // MFMA scans, fused and split, form them from the member rows themselves)
    const bool pool_kernel = l.pool && !pivot::mfma_shape(sh);
    l.qbar = pool_kernel ? take(groups * p->heads * p->dim * elt) : 0;
    l.wbar = pool_kernel ? take(groups * p->heads * sizeof(float)) : 0;
    if (l.few) {
        // split scan: about kSplitScanWorkgroups workgroups of four waves
        // over all groups, each wave streaming at least one 64-key quarter
        const int64_t quarters = (p->lk + 63) / 64;
        const int64_t most = (quarters + 3) / 4;
        int64_t ss = (kSplitScanWorkgroups + static_cast<int64_t>(groups) - 1) / static_cast<int64_t>(groups);
        l.scan_splits = static_cast<int>(ss < most ? ss : most);
        const int64_t rt = pivot::refine_tile();
        const int64_t ctiles = (int64_t(variant == PIVOT_REFINE ? c : 1) + rt - 1) / rt;  // refine tiles
        // refine: as many slices of C per group as fill the 256 CUs once
        // (each workgroup then scores several tiles, so its start-up
        // latency is paid once)
        int64_t rs = (256 + static_cast<int64_t>(groups) - 1) / static_cast<int64_t>(groups);
        l.refine_splits = static_cast<int>(rs < ctiles ? rs : ctiles);
        l.rows = take(groups * static_cast<size_t>(p->lk) * sizeof(float));
        l.hist = take(groups * static_cast<size_t>(l.scan_splits) * pivot::row_hist_bins() * sizeof(uint32_t));
    } else {
        l.scan_splits = l.refine_splits = 1;
        l.buf = take(groups * 2 * cap * sizeof(float));
        l.buf_n = take(groups * sizeof(int32_t));
        if (pivot::mfma_shape(sh)) l.smp = take(groups * static_cast<size_t>(pivot::scan_sample_slots()) * sizeof(float));
    }
    if (variant == PIVOT_REFINE || cfg.causal) {
        l.cand = take(groups * static_cast<size_t>(l.K) * sizeof(int32_t));
        l.cand_n = take(groups * sizeof(int32_t));
    }
    if (cfg.causal) l.cand_sc = take(groups * static_cast<size_t>(l.K) * sizeof(float));
    if (variant == PIVOT_REFINE) {
        l.scratch = take(groups * static_cast<size_t>(g) * static_cast<size_t>(c) * sizeof(float));
        l.nvalid = take(static_cast<size_t>(p->batch) * static_cast<size_t>(p->lq) * sizeof(int32_t));
    }
    l.total = off;
    *L = l;
    return PIVOT_OK;
}

pivot_status hip_status(hipError_t e, const char *what)
{
    if (e == hipSuccess) return PIVOT_OK;
    return fail(PIVOT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// The keys of a call: contiguous [batch, lk, dim] (lens, pages.table null)
// or ragged / paged (pivot_keys).
struct KeysIn {
    const void *k;
    const int32_t *lens;
    pivot::KeyPages pages;
};

KeysIn contiguous(const void *k) { return KeysIn{k, nullptr, pivot::KeyPages{nullptr, 0, 0, 0, 0, 0}}; }

pivot_status check_keys(const pivot_problem *p, const pivot_keys *keys, KeysIn *out)
{
    if (!keys) return fail(PIVOT_ERR_INVALID_ARG, "keys is NULL");
    KeysIn kin = contiguous(keys->k);
    kin.lens = keys->seq_lens;
    if (keys->page_table) {
        if (keys->page_size < 1) return fail(PIVOT_ERR_INVALID_ARG, "page_size must be >= 1 (got %d)", keys->page_size);
        if (keys->num_pages < 1) return fail(PIVOT_ERR_INVALID_ARG, "num_pages must be >= 1");
        const int64_t need = (p->lk + keys->page_size - 1) / keys->page_size;
        if (keys->max_pages < need)
            return fail(PIVOT_ERR_INVALID_ARG, "max_pages (%d) must cover lk keys (%lld pages)", keys->max_pages,
                        (long long)need);
        if (keys->num_pages * int64_t(keys->page_size) >= (int64_t(1) << 40))
            return fail(PIVOT_ERR_UNSUPPORTED, "key pool too large");
        kin.pages = pivot::make_key_pages(keys->page_table, keys->num_pages, keys->page_size, keys->max_pages);
    }
    *out = kin;
    return PIVOT_OK;
}

// The indexer's kernels up to the finished rows (each row's set in ascending
// position).
pivot_status run_rows(const pivot_problem *p, const Cfg &cfg, const void *q, const float *w, const KeysIn &kin,
                      int32_t *indices, float *scores, int32_t *candidates, int32_t *cand_counts, void *ws,
                      size_t ws_bytes, void *stream)
{
    Layout L;
    const void *k = kin.k;
    pivot_status st = plan(p, cfg, kin.pages.table != nullptr, &L);
    if (st != PIVOT_OK) return st;
    const int variant = cfg.variant;
    const int32_t topk = cfg.topk, c = cfg.c;
    if (!q || !w || !k || !indices) return fail(PIVOT_ERR_INVALID_ARG, "q, w, k and indices must be non-NULL");
    if (!ws || ws_bytes < L.total)
        return fail(PIVOT_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", L.total, ws ? ws_bytes : size_t(0));
    if (reinterpret_cast<uintptr_t>(ws) % kAlign != 0)
        return fail(PIVOT_ERR_WORKSPACE, "workspace must be %zu-byte aligned", kAlign);
    if (reinterpret_cast<uintptr_t>(q) % 16 != 0 || reinterpret_cast<uintptr_t>(k) % 16 != 0 ||
        reinterpret_cast<uintptr_t>(w) % 16 != 0)
        return fail(PIVOT_ERR_INVALID_ARG, "q, w and k must be 16-byte aligned");

    pivot::LaunchShape sh = shape_of(p);
    sh.lens = kin.lens;
    sh.pages = kin.pages;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *base = static_cast<char *>(ws);

    const void *qsrc = q;
    const float *wsrc = w;
    // the MFMA scans (fused and split) form each group's proxy from the
    // member rows themselves (the same arithmetic as k_pool): no pool launch
    // and no proxy round trip through HBM
    const bool pool_inline = L.pool && pivot::mfma_shape(sh);
    if (L.pool && !pool_inline) {
        void *qbar = base + L.qbar;
        float *wbar = reinterpret_cast<float *>(base + L.wbar);
        {
            StageTimer tm(PIVOT_STAGE_POOL, s);
            st = hip_status(pivot::launch_pool(sh, L.g, L.G, q, w, qbar, wbar, cfg.agg, s), "pool launch");
        }
        if (st != PIVOT_OK) return st;
        qsrc = qbar;
        wsrc = wbar;
    }

    const bool to_cand = variant == PIVOT_REFINE || cfg.causal;
    int32_t *cand = (variant == PIVOT_REFINE && candidates) ? candidates : reinterpret_cast<int32_t *>(base + L.cand);
    int32_t *cand_n =
        (variant == PIVOT_REFINE && cand_counts) ? cand_counts : reinterpret_cast<int32_t *>(base + L.cand_n);
    float *cand_sc = cfg.causal ? reinterpret_cast<float *>(base + L.cand_sc) : nullptr;

    pivot::ScanLaunch sl{};
    sl.qsrc = qsrc;
    sl.wsrc = wsrc;
    sl.pool_inline = pool_inline ? 1 : 0;
    sl.agg = cfg.agg;
    sl.k = k;
    sl.G = L.G;
    sl.g = L.g;
    sl.K = L.K;
    sl.cap = L.cap;
    sl.buf = L.few ? nullptr : reinterpret_cast<float *>(base + L.buf);
    sl.buf_n = L.few ? nullptr : reinterpret_cast<int32_t *>(base + L.buf_n);
    sl.smp = (L.few || !pivot::mfma_shape(sh)) ? nullptr : reinterpret_cast<float *>(base + L.smp);
    if (to_cand) {
        sl.out_idx = cand;
        sl.out_sc = cand_sc;
        sl.out_count = cand_n;
        sl.out_stride = L.K;
        sl.to_candidates = 1;
    } else {
        sl.out_idx = indices;
        sl.out_sc = scores;
        sl.out_count = nullptr;
        sl.out_stride = topk;
        sl.to_candidates = 0;
    }
    sl.rows = nullptr;
    if (L.few) {
        sl.rows = reinterpret_cast<float *>(base + L.rows);
        sl.hist = reinterpret_cast<uint32_t *>(base + L.hist);
        {
            StageTimer tm(PIVOT_STAGE_SCAN, s);
            st = hip_status(pivot::launch_scan_split(sh, sl, L.scan_splits, s), "split scan launch");
        }
        if (st != PIVOT_OK) return st;
        pivot::RowSelectLaunch rs{};
        rs.G = L.G;
        rs.g = L.g;
        rs.kind = 0;
        rs.rows = sl.rows;
        rs.K = L.K;
        rs.to_candidates = sl.to_candidates;
        rs.out_idx = sl.out_idx;
        rs.out_sc = sl.out_sc;
        rs.out_count = sl.out_count;
        rs.out_stride = sl.out_stride;
        rs.hist = sl.hist;
        rs.hist_splits = L.scan_splits;
        StageTimer tm(PIVOT_STAGE_SELECT, s);
        st = hip_status(pivot::launch_select_rows(sh, rs, s), "select launch");
    } else {
        {
            StageTimer tm(PIVOT_STAGE_SCAN, s);
            st = hip_status(pivot::launch_scan(sh, sl, s), "scan launch");
        }
        if (st == PIVOT_OK && pivot::mfma_shape(sh)) {
            StageTimer tm(PIVOT_STAGE_SCAN_SELECT, s);
            st = hip_status(pivot::launch_select_groups(sh, sl, s), "group select launch");
        }
    }
    if (st != PIVOT_OK) return st;

    if (cfg.causal) {
        // eq. (6) per member: each member's top-k of the shared proxy
        // scores over the candidates s <= t
        pivot::MemberSelectLaunch ml{};
        ml.G = L.G;
        ml.g = L.g;
        ml.topk = topk;
        ml.c = L.K;
        ml.cand = cand;
        ml.cand_n = cand_n;
        ml.row_nvalid = nullptr;
        ml.scores = cand_sc;
        ml.shared = 1;
        ml.out_idx = indices;
        ml.out_sc = scores;
        StageTimer tm(PIVOT_STAGE_SELECT, s);
        return hip_status(pivot::launch_select_members(sh, ml, s), "member select launch");
    }
    if (variant != PIVOT_REFINE) return st;

    pivot::RefineLaunch rl{};
    rl.q = q;
    rl.w = w;
    rl.k = k;
    rl.G = L.G;
    rl.g = L.g;
    rl.topk = topk;
    rl.c = c;
    rl.cand = cand;
    rl.cand_n = cand_n;
    rl.scratch = reinterpret_cast<float *>(base + L.scratch);
    rl.out_idx = indices;
    rl.out_sc = scores;
    rl.splits = L.refine_splits;
    // MFMA refine over many groups with c <= 4096: the member selection
    // runs as its own kernel (one wave per row), so the refine kernel's
    // matrix work is never idle behind it. With few groups (few rows) the
    // block-wide row select is faster: it spreads each row over 1024 lanes.
    const bool member_kernel = pivot::mfma_shape(sh) && !L.few && pivot::member_select_slabs(c) > 0;
    rl.finish = !member_kernel;
    rl.row_nvalid = member_kernel ? reinterpret_cast<int32_t *>(base + L.nvalid) : nullptr;
    {
        StageTimer tm(PIVOT_STAGE_REFINE, s);
        st = hip_status(pivot::launch_refine(sh, rl, s), "refine launch");
    }
    if (st != PIVOT_OK) return st;
    if (member_kernel) {
        pivot::MemberSelectLaunch ml{};
        ml.G = L.G;
        ml.g = L.g;
        ml.topk = topk;
        ml.c = c;
        ml.cand = cand;
        ml.cand_n = cand_n;
        ml.row_nvalid = rl.row_nvalid;
        ml.scores = rl.scratch;
        ml.shared = 0;
        ml.out_idx = indices;
        ml.out_sc = scores;
        StageTimer tm(PIVOT_STAGE_SELECT, s);
        return hip_status(pivot::launch_select_members(sh, ml, s), "member select launch");
    }
    if (rl.splits <= 1) return st;
    pivot::RowSelectLaunch ms{};
    ms.G = L.G;
    ms.g = L.g;
    ms.kind = 1;
    ms.rows = rl.scratch;
    ms.K = topk;
    ms.out_idx = indices;
    ms.out_sc = scores;
    ms.out_stride = topk;
    ms.cand = cand;
    ms.cand_n = cand_n;
    ms.c = c;
    StageTimer tm(PIVOT_STAGE_SELECT, s);
    return hip_status(pivot::launch_select_rows(sh, ms, s), "member select launch");
}

// run_rows, then (PIVOT_ORDER_SCORE) the rank-order pass over every row.
pivot_status run(const pivot_problem *p, const Cfg &cfg, const void *q, const float *w, const KeysIn &kin,
                 int32_t *indices, float *scores, int32_t *candidates, int32_t *cand_counts, void *ws,
                 size_t ws_bytes, void *stream)
{
    if (cfg.rank && !scores)
        return fail(PIVOT_ERR_INVALID_ARG, "PIVOT_ORDER_SCORE needs the scores output (its sort key)");
    if (cfg.rank && p->batch * p->lq > 0x7FFFFFFF)
        return fail(PIVOT_ERR_UNSUPPORTED, "PIVOT_ORDER_SCORE sorts at most 2^31 - 1 rows per call");
    pivot_status st = run_rows(p, cfg, q, w, kin, indices, scores, candidates, cand_counts, ws, ws_bytes, stream);
    if (st != PIVOT_OK || !cfg.rank) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    StageTimer tm(PIVOT_STAGE_ORDER, s);
    return hip_status(pivot::launch_rank_rows(indices, scores, p->batch * p->lq, cfg.topk, s), "rank order launch");
}

Cfg basic(int variant, int32_t g, int32_t topk, int32_t c)
{
    Cfg cfg{};
    cfg.variant = variant;
    cfg.g = variant == PIVOT_DENSE ? 1 : g;
    cfg.topk = topk;
    cfg.c = variant == PIVOT_REFINE ? c : 0;
    cfg.agg = PIVOT_AGG_MEAN;
    cfg.causal = false;
    cfg.path = PIVOT_PATH_AUTO;
    return cfg;
}

}  // namespace

extern "C" {

pivot_status pivot_workspace_size(const pivot_problem *p, int32_t variant, int32_t g, int32_t topk, int32_t c,
                                  size_t *bytes)
{
    if (!bytes) return fail(PIVOT_ERR_INVALID_ARG, "bytes is NULL");
    if (variant < PIVOT_DENSE || variant > PIVOT_REFINE) return fail(PIVOT_ERR_INVALID_ARG, "unknown variant %d", variant);
    Layout L;
    pivot_status st = plan(p, basic(variant, g, topk, c), false, &L);
    if (st != PIVOT_OK) return st;
    *bytes = L.total;
    return PIVOT_OK;
}

pivot_status pivot_index_dense(const pivot_problem *p, const void *q, const float *w, const void *k, int32_t topk,
                               int32_t *indices, float *scores, void *workspace, size_t workspace_bytes, void *stream)
{
    return run(p, basic(PIVOT_DENSE, 1, topk, 0), q, w, contiguous(k), indices, scores, nullptr, nullptr,
               workspace, workspace_bytes, stream);
}

pivot_status pivot_index_reuse(const pivot_problem *p, const void *q, const float *w, const void *k, int32_t g,
                               int32_t topk, int32_t *indices, float *scores, void *workspace, size_t workspace_bytes,
                               void *stream)
{
    return run(p, basic(PIVOT_REUSE, g, topk, 0), q, w, contiguous(k), indices, scores, nullptr, nullptr,
               workspace, workspace_bytes, stream);
}

pivot_status pivot_index_refine(const pivot_problem *p, const void *q, const float *w, const void *k, int32_t g,
                                int32_t topk, int32_t c, int32_t *indices, float *scores, int32_t *candidates,
                                int32_t *candidate_counts, void *workspace, size_t workspace_bytes, void *stream)
{
    return run(p, basic(PIVOT_REFINE, g, topk, c), q, w, contiguous(k), indices, scores, candidates,
               candidate_counts, workspace, workspace_bytes, stream);
}

pivot_status pivot_config_init(pivot_config *cfg)
{
    if (!cfg) return fail(PIVOT_ERR_INVALID_ARG, "config is NULL");
    std::memset(cfg, 0, sizeof *cfg);
    cfg->variant = PIVOT_REFINE;
    cfg->g = 8;
    cfg->topk = 2048;
    cfg->c = 4096;
    cfg->aggregation = PIVOT_AGG_MEAN;
    cfg->member_causal = 0;
    cfg->auto_variant = PIVOT_REFINE;
    cfg->scan_path = PIVOT_PATH_AUTO;
    cfg->dense_below = 0;
    cfg->order = PIVOT_ORDER_POSITION;
    return PIVOT_OK;
}

pivot_status pivot_resolve_variant(const pivot_problem *p, const pivot_config *cfg, int32_t *variant)
{
    if (!variant) return fail(PIVOT_ERR_INVALID_ARG, "variant is NULL");
    Cfg c;
    pivot_status st = resolve(p, cfg, &c);
    if (st != PIVOT_OK) return st;
    *variant = c.variant;
    return PIVOT_OK;
}

pivot_status pivot_index_workspace_size(const pivot_problem *p, const pivot_config *cfg, size_t *bytes)
{
    if (!bytes) return fail(PIVOT_ERR_INVALID_ARG, "bytes is NULL");
    Cfg c;
    pivot_status st = resolve(p, cfg, &c);
    if (st != PIVOT_OK) return st;
    Layout L;
    st = plan(p, c, false, &L);
    if (st != PIVOT_OK) return st;
    *bytes = L.total;
    return PIVOT_OK;
}

pivot_status pivot_index_kv_workspace_size(const pivot_problem *p, const pivot_config *cfg, const pivot_keys *keys,
                                           size_t *bytes)
{
    if (!bytes) return fail(PIVOT_ERR_INVALID_ARG, "bytes is NULL");
    Cfg c;
    pivot_status st = resolve(p, cfg, &c);
    if (st != PIVOT_OK) return st;
    KeysIn kin;
    st = check_keys(p, keys, &kin);
    if (st != PIVOT_OK) return st;
    Layout L;
    st = plan(p, c, kin.pages.table != nullptr, &L);
    if (st != PIVOT_OK) return st;
    *bytes = L.total;
    return PIVOT_OK;
}

pivot_status pivot_index(const pivot_problem *p, const pivot_config *cfg, const void *q, const float *w,
                         const void *k, int32_t *indices, float *scores, int32_t *candidates,
                         int32_t *candidate_counts, void *workspace, size_t workspace_bytes, void *stream)
{
    Cfg c;
    pivot_status st = resolve(p, cfg, &c);
    if (st != PIVOT_OK) return st;
    return run(p, c, q, w, contiguous(k), indices, scores, candidates, candidate_counts, workspace, workspace_bytes,
               stream);
}

pivot_status pivot_index_kv(const pivot_problem *p, const pivot_config *cfg, const void *q, const float *w,
                            const pivot_keys *keys, int32_t *indices, float *scores, int32_t *candidates,
                            int32_t *candidate_counts, void *workspace, size_t workspace_bytes, void *stream)
{
    Cfg c;
    pivot_status st = resolve(p, cfg, &c);
    if (st != PIVOT_OK) return st;
    KeysIn kin;
    st = check_keys(p, keys, &kin);
    if (st != PIVOT_OK) return st;
    return run(p, c, q, w, kin, indices, scores, candidates, candidate_counts, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ------------------------------------------------ allocation-free entry
// The scratch of pivot_index_static: one array per GPU, held until the
// process ends. In host code `scratch` names a host-side stand-in, not the
// device array; its device address comes from hipGetSymbolAddress, looked up
// once per device (with that device current) and kept in g_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[PIVOT_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

pivot_status static_scratch(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(PIVOT_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    void *ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!ptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
        if (!ptr) {
            e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
            if (!ptr) return fail(PIVOT_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
            g_scratch_ptr[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = ptr;
    return PIVOT_OK;
}

}  // namespace

extern "C" {

pivot_status pivot_index_static(const pivot_problem *p, const pivot_config *cfg, const void *q, const float *w,
                                const void *k, int32_t *indices, float *scores, int32_t *candidates,
                                int32_t *candidate_counts, void *stream)
{
    Cfg c;
    pivot_status st = resolve(p, cfg, &c);
    if (st != PIVOT_OK) return st;
    Layout L;
    st = plan(p, c, false, &L);
    if (st != PIVOT_OK) return st;
    if (L.total > PIVOT_STATIC_SCRATCH_BYTES)
        return fail(PIVOT_ERR_WORKSPACE,
                    "this call needs %zu bytes of scratch; pivot_index_static holds %zu (use pivot_index with a "
                    "workspace)",
                    L.total, static_cast<size_t>(PIVOT_STATIC_SCRATCH_BYTES));
    void *ws = nullptr;
    st = static_scratch(&ws);
    if (st != PIVOT_OK) return st;
    g_timing_off = true;
    st = run(p, c, q, w, contiguous(k), indices, scores, candidates, candidate_counts, ws,
             PIVOT_STATIC_SCRATCH_BYTES, stream);
    g_timing_off = false;
    return st;
}

pivot_status pivot_index_stats(int64_t batch, int64_t lq, int32_t k, const int32_t *indices, const float *scores,
                               int32_t d, int32_t g, int32_t *overlap, int32_t *group_union, int32_t *group_inter,
                               float *mass, void *stream)
{
    if (batch < 1 || lq < 1) return fail(PIVOT_ERR_INVALID_ARG, "batch and lq must be >= 1");
    if (k < 1 || k > pivot::stats_row_max())
        return fail(PIVOT_ERR_UNSUPPORTED, "row width k must be in [1, %d] (got %d)", pivot::stats_row_max(), k);
    if (!indices) return fail(PIVOT_ERR_INVALID_ARG, "indices is NULL");
    if (!overlap && !group_union && !group_inter && !mass) return fail(PIVOT_ERR_INVALID_ARG, "no output requested");
    if (overlap && d < 1) return fail(PIVOT_ERR_INVALID_ARG, "overlap distance d must be >= 1 (got %d)", d);
    const bool groups = group_union || group_inter;
    if (groups && (g < 1 || g > 64)) return fail(PIVOT_ERR_INVALID_ARG, "group size g must be in [1, 64] (got %d)", g);
    if (groups && !pivot::stats_group_fits(g, k))
        return fail(PIVOT_ERR_UNSUPPORTED,
                    "group sets need pow2ceil(g) * roundup(k, 32) <= 16384 (got g = %d, k = %d)", g, k);
    if (mass && !scores) return fail(PIVOT_ERR_INVALID_ARG, "mass needs scores");
    pivot::StatsArgs a{};
    a.idx = indices;
    a.scores = scores;
    a.B = batch;
    a.Lq = lq;
    a.k = k;
    a.d = overlap ? d : 1;
    a.g = groups ? g : 1;
    a.G = (lq + a.g - 1) / a.g;
    a.overlap = overlap;
    a.group_union = group_union;
    a.group_inter = group_inter;
    a.mass = mass;
    return hip_status(pivot::launch_stats(a, static_cast<hipStream_t>(stream)), "stats launch");
}

pivot_status pivot_pool(const pivot_problem *p, int32_t g, const void *q, const float *w, void *qbar, float *wbar,
                        void *stream)
{
    return pivot_pool_ex(p, g, PIVOT_AGG_MEAN, q, w, qbar, wbar, stream);
}

pivot_status pivot_pool_ex(const pivot_problem *p, int32_t g, int32_t aggregation, const void *q, const float *w,
                           void *qbar, float *wbar, void *stream)
{
    pivot_status st = check_problem(p);
    if (st != PIVOT_OK) return st;
    if (g < 1) return fail(PIVOT_ERR_INVALID_ARG, "group size g must be >= 1 (got %d)", g);
    if (aggregation < PIVOT_AGG_MEAN || aggregation > PIVOT_AGG_LAST)
        return fail(PIVOT_ERR_INVALID_ARG, "unknown aggregation %d", aggregation);
    if (!q || !w || !qbar || !wbar) return fail(PIVOT_ERR_INVALID_ARG, "q, w, qbar and wbar must be non-NULL");
    if (reinterpret_cast<uintptr_t>(q) % 16 != 0 || reinterpret_cast<uintptr_t>(qbar) % 16 != 0)
        return fail(PIVOT_ERR_INVALID_ARG, "q and qbar must be 16-byte aligned");
    const int64_t G = (p->lq + g - 1) / g;
    return hip_status(
        pivot::launch_pool(shape_of(p), g, G, q, w, qbar, wbar, aggregation, static_cast<hipStream_t>(stream)),
        "pool launch");
}

pivot_status pivot_proxy_scores(const pivot_problem *p, int32_t g, const void *qbar, const float *wbar, const void *k,
                                float *out, void *stream)
{
    pivot_status st = check_problem(p);
    if (st != PIVOT_OK) return st;
    if (g < 1) return fail(PIVOT_ERR_INVALID_ARG, "group size g must be >= 1 (got %d)", g);
    if (!qbar || !wbar || !k || !out) return fail(PIVOT_ERR_INVALID_ARG, "qbar, wbar, k and out must be non-NULL");
    if (reinterpret_cast<uintptr_t>(qbar) % 16 != 0 || reinterpret_cast<uintptr_t>(k) % 16 != 0)
        return fail(PIVOT_ERR_INVALID_ARG, "qbar and k must be 16-byte aligned");
    st = check_exact_work(p, (p->lq + g - 1) / g, 0);
    if (st != PIVOT_OK) return st;
    pivot::ScanLaunch sl{};
    sl.qsrc = qbar;
    sl.wsrc = wbar;
    sl.k = k;
    sl.G = (p->lq + g - 1) / g;
    sl.g = g;
    sl.rows = out;
    return hip_status(pivot::launch_scan(shape_of(p), sl, static_cast<hipStream_t>(stream)), "scan launch");
}

pivot_status pivot_timing_enable(int32_t on)
{
    g_timing = on != 0;
    if (!g_timing) forget_timing();
    return PIVOT_OK;
}

pivot_status pivot_timing_read(double *ms, int64_t *launches)
{
    pivot_status st = PIVOT_OK;
    for (auto &t : g_timed) {
        float e = 0.0f;
        hipError_t err = hipEventSynchronize(t.stop);
        if (err == hipSuccess) err = hipEventElapsedTime(&e, t.start, t.stop);
        if (err != hipSuccess) {
            st = hip_status(err, "timing event");
            continue;
        }
        if (ms) ms[t.stage] += e;
        if (launches) launches[t.stage] += 1;
    }
    forget_timing();
    return st;
}

const char *pivot_status_str(pivot_status s)
{
    switch (s) {
    case PIVOT_OK: return "ok";
    case PIVOT_ERR_INVALID_ARG: return "invalid argument";
    case PIVOT_ERR_UNSUPPORTED: return "unsupported";
    case PIVOT_ERR_WORKSPACE: return "workspace too small";
    case PIVOT_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

const char *pivot_last_error(void) { return g_last_error; }

int32_t pivot_abi_version(void) { return PIVOT_ABI_VERSION; }

}  // extern "C"
