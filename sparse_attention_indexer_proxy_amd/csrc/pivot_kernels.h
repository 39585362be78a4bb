// Internal interface between the C ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pivot {

// Key storage: contiguous [B, Lk, D], or pages [num_pages, page, D] named by
// a per-sequence table [B, max_pages] of physical page ids (device memory).
struct KeyPages {
    const int32_t *table;  // null: contiguous
    int64_t num_pages;
    int page, max_pages;
    // s / page == (s * page_magic) >> page_shift for every s < 2^31:
    // page_shift = 31 + ceil(log2 page), page_magic = 2^page_shift / page + 1
    // (then page_magic * page - 2^page_shift lies in (0, page] and at most
    // 2^(page_shift - 31), which keeps the rounding error below 1 / page)
    uint32_t page_magic;
    int page_shift;
};

inline KeyPages make_key_pages(const int32_t *table, int64_t num_pages, int page, int max_pages)
{
    int l = 0;
    while ((int64_t(1) << l) < page) ++l;
    const uint64_t magic = (uint64_t(1) << (31 + l)) / static_cast<uint64_t>(page) + 1;
    return KeyPages{table, num_pages, page, max_pages, static_cast<uint32_t>(magic), 31 + l};
}

struct LaunchShape {
    int64_t B, Lq, Lk;              // Lk: key capacity per sequence
    int H, D;
    bool bf16;
    const int32_t *lens = nullptr;  // [B] keys of each sequence (device), null: Lk each
    KeyPages pages{};               // table == null: contiguous keys
};

// One scan launch: eq. (5) for every group, then either the streaming
// selection of the best K (rows != nullptr selects the score-row output).
struct ScanLaunch {
    const void *qsrc;   // [B, G, H, D], or with pool_inline the queries [B, Lq, H, D]
    const float *wsrc;  // [B, G, H], or with pool_inline the weights [B, Lq, H]
    int pool_inline;    // MFMA scans (fused, split): form each group's proxy (eq. 4) in the kernel
    int agg;            // pool_inline: 0 mean, 1 first member, 2 last member
    const void *k;      // [B, Lk, D]
    int64_t G;
    int g;
    int K, cap;         // selection size and per-group buffer capacity
    float *buf;         // [B*G, 2*cap]: cap scores then cap int32 positions per group
    int32_t *buf_n;     // [B*G] buffered entries (MFMA shape, selection mode)
    float *smp;         // [B*G, scan_sample_slots()] sampled scores (MFMA shape, selection mode)
    int32_t *out_idx;   // rows [B, Lq, stride] or candidates [B, G, stride]
    float *out_sc;      // rows only, nullable
    int32_t *out_count; // candidates only, nullable
    int out_stride;
    int to_candidates;
    float *rows;        // [B, G, Lk] score rows, or nullptr for selection
    uint32_t *hist;     // split scan: [B*G, splits, row_hist_bins()] score counts
};

struct RefineLaunch {
    const void *q;
    const float *w;
    const void *k;
    int64_t G;
    int g;
    int topk, c;
    const int32_t *cand;
    const int32_t *cand_n;
    float *scratch;     // [B*G, g, c]
    int32_t *out_idx;
    float *out_sc;
    int splits;         // > 1: split C over workgroups
    int finish;         // splits == 1: select each member's top-k inside the refine kernel;
                        // otherwise launch_select_members / launch_select_rows does it
    int32_t *row_nvalid;  // [B, Lq], nullable, splits == 1: #{j : C[j] <= t} per row
};

// Per-member top-k over candidate score rows (c <= 4096): the members'
// re-scores of C (Refine), or the group's proxy scores of C shared by every
// member, each member keeping only C[j] <= its own position (member-causal
// Reuse).
struct MemberSelectLaunch {
    int64_t G;
    int g;
    int topk, c;
    const int32_t *cand;
    const int32_t *cand_n;      // read when row_nvalid is null
    const int32_t *row_nvalid;  // [B, Lq] from the refine launch, or null
    const float *scores;        // [B*G, g, c], or [B*G, c] when shared
    int shared;
    int32_t *out_idx;
    float *out_sc;
};

// Block-wide selection of rows held in memory (few-groups path).
struct RowSelectLaunch {
    int64_t G;
    int g;
    int kind;           // 0: group score rows [B*G, Lk]; 1: member rows of the split refine
    const float *rows;
    int K;
    int to_candidates;
    int32_t *out_idx;
    float *out_sc;
    int32_t *out_count;
    int out_stride;
    const int32_t *cand;
    const int32_t *cand_n;
    int c;
    const uint32_t *hist;  // kind 0: the split scan's score counts, or null
    int hist_splits;
};

// O1-O3 diagnostics of index rows (pivot_diag.hip).
struct StatsArgs {
    const int32_t *idx;     // [B, Lq, k] ascending valid prefix, then -1
    const float *scores;    // [B, Lq, k] aligned with idx (mass only)
    int64_t B, Lq;
    int k, d, g;
    int64_t G;              // ceil(Lq / g)
    int32_t *overlap;       // [B, Lq] |T_t ∩ T_{t+d}|, -1 past the sequence; nullable
    int32_t *group_union;   // [B, G]; nullable
    int32_t *group_inter;   // [B, G]; nullable
    float *mass;            // [B, Lq, 3]; nullable
};
hipError_t launch_stats(const StatsArgs &a, hipStream_t st);
int stats_row_max();    // largest row width k
// Whether groups of g rows of width k fit the group-set kernel: the next
// power of two >= g, times k rounded up to 32, at most 16384.
int stats_group_fits(int g, int k);

bool mfma_shape(const LaunchShape &sh);
// Sampled scores the fused scan keeps per group (its workspace share).
int scan_sample_slots();
// Score-count words per split-scan workgroup (its workspace share).
int row_hist_bins();
// Candidates per refine tile.
int refine_tile();
// agg: 0 mean of the members (eq. 4), 1 first member, 2 last member.
hipError_t launch_pool(const LaunchShape &sh, int g, int64_t G, const void *q, const float *w, void *qbar,
                       float *wbar, int agg, hipStream_t st);
// eqs. (5)-(7). On the MFMA shape in selection mode the scan leaves each
// group's survivors in L.buf / L.buf_n and launch_select_groups must follow
// on the same stream; the exact-order kernels select in-kernel.
hipError_t launch_scan(const LaunchShape &sh, const ScanLaunch &L, hipStream_t st);
// The final top-K of every group's survivor buffer into L's outputs.
hipError_t launch_select_groups(const LaunchShape &sh, const ScanLaunch &L, hipStream_t st);
hipError_t launch_refine(const LaunchShape &sh, const RefineLaunch &L, hipStream_t st);
// Proxy score rows with the key axis split over `splits` workgroups per group.
hipError_t launch_scan_split(const LaunchShape &sh, const ScanLaunch &L, int splits, hipStream_t st);
hipError_t launch_select_rows(const LaunchShape &sh, const RowSelectLaunch &L, hipStream_t st);
// Register-resident member selection needs c <= 4096; returns its slab count or 0.
int member_select_slabs(int c);
hipError_t launch_select_members(const LaunchShape &sh, const MemberSelectLaunch &L, hipStream_t st);
// Rank order (pivot_order.hip): rows [rows, k] of positions and scores
// reordered in place by score descending, equal scores by lower position,
// -1 padding last; k <= rank_rows_max().
int rank_rows_max();
hipError_t launch_rank_rows(int32_t *idx, float *sc, int64_t rows, int k, hipStream_t st);

}  // namespace pivot
