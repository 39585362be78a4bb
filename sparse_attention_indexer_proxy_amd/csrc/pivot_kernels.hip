// PIVOT group-shared sparse-attention indexer: HIP kernels for gfx950.
//
// Method (PIVOT paper summary page, picx.dev, sections "Introduction and
// Theoretical Foundation" and "Methodology"):
//   eq. (1)  I_{t,s} = sum_j w_{t,j} ReLU(q_{t,j} . k_s)      (dense indexer)
//   eq. (4)  proxy qbar_j, wbar_j = per-head mean over the group
//   eq. (5)  Ibar_s = sum_j wbar_j ReLU(qbar_j . k_s), s <= t_last
//   eq. (6)  Reuse: TopK(Ibar, k) for every member
//   eq. (7)  Refine candidates C = TopK(Ibar, c)
//   eqs. (8)-(9)  member re-score over C and per-member TopK(., k)
//
// Kernels:
//   k_pool                  eq. (4), HBM-bound streaming mean
//   k_scan_mfma<Mode>       eq. (5) on bf16 MFMA (heads on the M axis, keys on
//                           N, d as the contraction), ReLU + weighted head
//                           reduction in registers, then either the streaming
//                           top-K filter (Mode = kFilter, eqs. 6-7) or a plain
//                           score row (Mode = kRows)
//   k_scan_exact<T, Mode>   the same for any shape/dtype, in the exact fp32
//                           order of the definition (heads, then dims ascending)
//   k_select_groups<NV>     the final top-K of each group's survivors (eqs. 6-7)
//   k_scan_split            eq. (5) with the key axis split over many waves
//                           (few groups: decode), keys streamed from HBM
//                           straight into MFMA operands, score rows to HBM
//   k_select_rows           block-wide selects of those rows (eqs. 6-7, 9)
//   k_refine_mfma           eq. (8) over gathered candidate tiles
//   k_select_members<NV>    eq. (9): each member's top-k of its re-scored C
//   k_refine_exact<T>       eqs. (8)-(9) in exact order
//
// Selection: a wave keeps its group's survivors (score > tau) in a private
// buffer in HBM, appended in ascending position. When the buffer is full the
// wave radix-selects the K-th best (score desc, position asc), compacts the
// buffer in place (stable) to exactly K entries and raises tau. At the end
// k_select_groups (or, in the exact-order scan, the same wave select) picks
// the best K and writes them in ascending position. The full L/g x L score
// matrix never exists in memory.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "pivot_kernels.h"
#include "pivot_launch.h"

namespace pivot {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Loads and stores through a typed address space (1: global, 3: LDS), so
// the compiler emits global_load / ds_read rather than flat accesses, whose
// completion shares the LDS wait counter (each LDS wait would also wait for
// every global load in flight).
constexpr int kGlobal = 1, kLds = 3;

template <int AS, class T>
__device__ __forceinline__ T load_as(const T *p, int64_t j)
{
    return ((const __attribute__((address_space(AS))) T *)p)[j];
}

template <int AS, class T>
__device__ __forceinline__ void store_as(T *p, int64_t j, T v)
{
    ((__attribute__((address_space(AS))) T *)p)[j] = v;
}

// ------------------------------------------------------------ lane helpers
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ int mbcnt(uint64_t m)
{
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

__device__ __forceinline__ int popc(uint64_t m) { return __popcll(m); }

// Value of v in lane `src` (wave-uniform), without a trip through LDS.
__device__ __forceinline__ uint32_t lane_value(uint32_t v, int src)
{
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), src));
}

// DPP lane moves within the wave (gfx9 encodings): row_shr:n shifts each
// 16-lane row right by n, row_bcast:15 / row_bcast:31 pass lane 15 of a row
// (31 of the half) on to the next row(s); lanes without a source (or outside
// row_mask) take `fill`.
template <int Ctrl, int RowMask = 0xF>
__device__ __forceinline__ uint32_t dpp_move(uint32_t v, uint32_t fill)
{
    return static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(static_cast<int>(fill), static_cast<int>(v), Ctrl, RowMask, 0xF, false));
}

// Inclusive prefix sum over the lanes of a wave (Hillis-Steele on DPP).
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v)
{
    v += dpp_move<0x111>(v, 0u);
    v += dpp_move<0x112>(v, 0u);
    v += dpp_move<0x114>(v, 0u);
    v += dpp_move<0x118>(v, 0u);
    v += dpp_move<0x142, 0xA>(v, 0u);
    v += dpp_move<0x143, 0xC>(v, 0u);
    return v;
}

// Inclusive suffix sum over lanes: lane l gets the sum over lanes >= l.
__device__ __forceinline__ uint32_t wave_suffix_sum(uint32_t v)
{
    const uint32_t inc = wave_incl_sum(v);
    return lane_value(inc, kWave - 1) - inc + v;
}

// Sum over the wave (wave-uniform).
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) { return lane_value(wave_incl_sum(v), kWave - 1); }

// Sum over lanes 0..15 (wave-uniform).
__device__ __forceinline__ uint32_t row0_sum(uint32_t v)
{
    v += dpp_move<0x111>(v, 0u);
    v += dpp_move<0x112>(v, 0u);
    v += dpp_move<0x114>(v, 0u);
    v += dpp_move<0x118>(v, 0u);
    return lane_value(v, 15);
}

// Sum over the wave of a per-lane count in [0, 127].
__device__ __forceinline__ int wave_total(uint32_t c)
{
    int t = 0;
#pragma unroll
    for (int bit = 0; bit < 7; ++bit) t += popc(ballot((c >> bit) & 1u)) << bit;
    return t;
}

// Order-preserving map of a float to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t ord_key(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_float(uint32_t k)
{
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }

__device__ __forceinline__ uint16_t float_to_bf16_rne(float x)
{
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

template <typename T> __device__ __forceinline__ float widen(T x);
template <> __device__ __forceinline__ float widen<float>(float x) { return x; }
template <> __device__ __forceinline__ float widen<uint16_t>(uint16_t x) { return bf16_bits_to_float(x); }

// Workgroup-scope fence: orders this wave's global and LDS accesses so that
// other lanes of the wave observe them (buffers are wave-private).
__device__ __forceinline__ void wave_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup"); }

// ------------------------------------------------------ group geometry
// Sequence b holds lk(b) keys (lens[b], or the capacity Lk); its query row r
// sits at position lk(b) - Lq + r (a ragged batch: each sequence's queries
// are the last Lq positions of its own prefix).
struct Geo {
    int64_t B, G, Lq, Lk;
    int g;
    const int32_t *lens;  // [B] or null
    __device__ __forceinline__ int64_t first_row(int64_t m) const { return m * g; }
    __device__ __forceinline__ int64_t end_row(int64_t m) const { return (m + 1) * g < Lq ? (m + 1) * g : Lq; }
    // lens outside [0, Lk] are clamped, so no key outside the storage is read
    __device__ __forceinline__ int64_t lk(int64_t b) const
    {
        if (!lens) return Lk;
        const int64_t v = lens[b];
        return v < 0 ? 0 : (v > Lk ? Lk : v);
    }
    __device__ __forceinline__ int64_t pos(int64_t b, int64_t r) const { return lk(b) - Lq + r; }
    __device__ __forceinline__ int64_t t_last(int64_t b, int64_t m) const { return lk(b) - Lq + end_row(m) - 1; }
};

// Row index of key s of sequence b in the key storage: contiguous rows
// b * Lk + s, or page table[b][s / page] (clamped into the pool, so a
// malformed table cannot address outside it), row s % page.
struct Keys {
    const void *base;
    KeyPages pg;
    int64_t Lk;
    __device__ __forceinline__ int64_t flat(int64_t b, int64_t s) const { return b * Lk + s; }
    // A paged lookup in two halves, so that a kernel can read the table
    // entries a tile ahead of the rows they yield. Positions are below 2^31,
    // so s / page is one 32x32->64-bit multiply and a shift (the host's
    // round-up reciprocal), with no branch between the table loads.
    __device__ __forceinline__ uint32_t page_index(uint32_t s) const
    {
        return static_cast<uint32_t>((static_cast<uint64_t>(s) * pg.page_magic) >> pg.page_shift);
    }
    __device__ __forceinline__ int32_t entry(int64_t b, uint32_t s) const
    {
        return pg.table[b * pg.max_pages + page_index(s)];
    }
    __device__ __forceinline__ uint32_t page_offset(uint32_t s) const
    {
        return s - page_index(s) * static_cast<uint32_t>(pg.page);
    }
    // row `off` of page table entry `e`
    __device__ __forceinline__ int64_t paged_row(int32_t e, uint32_t off) const
    {
        const int64_t ph = e < 0 ? 0 : (e >= pg.num_pages ? pg.num_pages - 1 : e);
        return ph * pg.page + off;
    }
    __device__ __forceinline__ int64_t row(int64_t b, int64_t s) const
    {
        if (!pg.table) return flat(b, s);
        const uint32_t su = static_cast<uint32_t>(s);
        return paged_row(entry(b, su), page_offset(su));
    }
};

// ------------------------------------------------------------ wave select
// Result of selecting the best K of n entries by (score desc, position asc),
// with entries stored in ascending position: every entry whose key is above
// `kth`, plus the first `quota` entries whose key equals `kth`.
struct Sel {
    uint32_t kth;
    int quota;
    bool all;
};

constexpr int kVec = 4;                // entries per lane per step
constexpr int kStep = kWave * kVec;    // 256 entries per step; lane l owns j0 + 4l .. j0 + 4l + 3

// Exclusive prefix over lanes of a per-lane count c in [0, 7]; *total = sum.
__device__ __forceinline__ int lane_prefix(int c, int *total)
{
    const uint64_t b0 = ballot(c & 1), b1 = ballot(c & 2), b2 = ballot(c & 4);
    *total = popc(b0) + 2 * popc(b1) + 4 * popc(b2);
    return mbcnt(b0) + 2 * mbcnt(b1) + 4 * mbcnt(b2);
}

// Count one entry per lane into the 256-bin histogram of digit `shift` of
// its key, if its key matches the selected prefix. When every matching lane
// has the same digit (the common case for the leading digits), one lane adds
// the whole count.
__device__ __forceinline__ void hist_add(bool in, uint32_t key, uint32_t prefix, uint32_t pmask, int shift,
                                         uint32_t *hist, int l)
{
    const bool match = in && (key & pmask) == prefix;
    const uint32_t digit = (key >> shift) & 0xFFu;
    const uint64_t mm = ballot(match);
    if (mm == 0) return;
    const int first = __ffsll(static_cast<long long>(mm)) - 1;
    const uint32_t d0 = lane_value(digit, first);
    const uint64_t same = ballot(match && digit == d0);
    if (same == mm) {
        if (l == first) atomicAdd(&hist[d0], static_cast<uint32_t>(popc(mm)));
    } else if (match) {
        atomicAdd(&hist[digit], 1u);
    }
}

// hist_add for wave-private histograms: the lanes sharing the first matching
// lane's digit (most of them in the leading digits) add with one atomic, the
// others one each, so no address takes many atomics at once.
__device__ __forceinline__ void hist_add_peel(bool in, uint32_t key, uint32_t prefix, uint32_t pmask, int shift,
                                              uint32_t *hist, int l)
{
    const bool match = in && (key & pmask) == prefix;
    const uint32_t digit = (key >> shift) & 0xFFu;
    const uint64_t mm = ballot(match);
    if (mm == 0) return;
    const int first = __ffsll(static_cast<long long>(mm)) - 1;
    const uint32_t d0 = lane_value(digit, first);
    const bool other = match && digit != d0;
    const uint64_t same = mm & ~ballot(other);
    if (l == first) atomicAdd(&hist[d0], static_cast<uint32_t>(popc(same)));
    if (other) atomicAdd(&hist[digit], 1u);
}

// One count per lane with `in` into bins[bin] (LDS); the lanes sharing the
// first counted lane's bin add with one atomic, the others one each.
__device__ __forceinline__ void bin_add(bool in, uint32_t bin, uint32_t *bins, int l)
{
    const uint64_t mm = ballot(in);
    if (mm == 0) return;
    const int first = __ffsll(static_cast<long long>(mm)) - 1;
    const uint32_t b0 = lane_value(bin, first);
    const bool other = in && bin != b0;
    const uint64_t same = mm & ~ballot(other);
    if (l == first) atomicAdd(&bins[b0], static_cast<uint32_t>(popc(same)));
    if (other) atomicAdd(&bins[bin], 1u);
}

// Radix select over 8-bit digits of ord_key(score), most significant first,
// with a per-wave 256-bin histogram in LDS. sc may point to global memory;
// each lane keeps 8 loads in flight.
__device__ Sel wave_select(const float *sc, int n, int K, uint32_t *hist)
{
    Sel r;
    if (n <= K) {
        r.all = true;
        r.kth = 0;
        r.quota = 0;
        return r;
    }
    r.all = false;
    const int l = lane_id();
    uint32_t prefix = 0, pmask = 0;
    uint32_t remaining = static_cast<uint32_t>(K);
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = l; i < 256; i += kWave) hist[i] = 0u;
        wave_fence();
        for (int j0 = 0; j0 < n; j0 += 2 * kStep) {
            float v[2 * kVec];
            bool in[2 * kVec];
#pragma unroll
            for (int e = 0; e < 2 * kVec; ++e) {
                const int j = j0 + (e / kVec) * kStep + kVec * l + (e % kVec);
                in[e] = j < n;
                v[e] = in[e] ? sc[j] : 0.0f;
            }
#pragma unroll
            for (int e = 0; e < 2 * kVec; ++e) hist_add(in[e], ord_key(v[e]), prefix, pmask, shift, hist, l);
        }
        wave_fence();
        const uint32_t c0 = hist[4 * l], c1 = hist[4 * l + 1], c2 = hist[4 * l + 2], c3 = hist[4 * l + 3];
        const uint32_t tot = c0 + c1 + c2 + c3;
        // inclusive suffix sum over lanes (higher lanes hold higher bins);
        // shuffles rather than DPP here: inlined into the fused scan, the
        // DPP form shifts that kernel's register allocation and costs ~2%
        uint32_t suf = tot;
        for (int o = 1; o < kWave; o <<= 1) {
            const uint32_t t = __shfl_down(suf, o);
            if (l + o < kWave) suf += t;
        }
        const uint32_t above = suf - tot;
        const bool here = above < remaining && remaining <= suf;
        const uint64_t hm = ballot(here);
        const int src = __ffsll(static_cast<long long>(hm)) - 1;
        uint32_t dig = 0, abv = 0;
        if (here) {
            uint32_t cum = above;
            if (cum + c3 >= remaining) {
                dig = 4 * l + 3;
            } else {
                cum += c3;
                if (cum + c2 >= remaining) {
                    dig = 4 * l + 2;
                } else {
                    cum += c2;
                    if (cum + c1 >= remaining) {
                        dig = 4 * l + 1;
                    } else {
                        cum += c1;
                        dig = 4 * l;
                    }
                }
            }
            abv = cum;
        }
        dig = __shfl(dig, src);
        abv = __shfl(abv, src);
        remaining -= abv;
        prefix |= dig << shift;
        pmask |= 0xFFu << shift;
        wave_fence();
    }
    r.kth = prefix;
    r.quota = static_cast<int>(remaining);
    return r;
}

// Walk sc[0..n) in order and call emit(slot, position, score) for every
// selected entry, where position is pos[j] (or j when pos is null); slots are
// dense and ascending. Every entry of a step is loaded before any emit, so
// emit may write back into sc/pos (in-place compaction: slot <= j).
template <class F> __device__ int wave_emit(const float *sc, const int32_t *pos, int n, Sel s, F &&emit)
{
    const int l = lane_id();
    int eq_seen = 0, out = 0;
    for (int j0 = 0; j0 < n; j0 += kStep) {
        float v[kVec];
        int32_t p[kVec];
        bool take[kVec];
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            const int j = j0 + kVec * l + e;
            take[e] = j < n;
            v[e] = take[e] ? sc[j] : 0.0f;
            p[e] = take[e] ? (pos ? pos[j] : j) : 0;
        }
        if (!s.all) {
            bool eq[kVec];
            int neq = 0;
#pragma unroll
            for (int e = 0; e < kVec; ++e) {
                const uint32_t key = ord_key(v[e]);
                eq[e] = take[e] && key == s.kth;
                take[e] = take[e] && key > s.kth;
                neq += eq[e];
            }
            int eq_tot;
            int rank = eq_seen + lane_prefix(neq, &eq_tot);
            eq_seen += eq_tot;
#pragma unroll
            for (int e = 0; e < kVec; ++e) {
                if (eq[e]) {
                    take[e] = rank < s.quota;
                    ++rank;
                }
            }
        }
        int nt = 0;
#pragma unroll
        for (int e = 0; e < kVec; ++e) nt += take[e];
        int t_tot;
        int slot = out + lane_prefix(nt, &t_tot);
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            if (take[e]) emit(slot++, p[e], v[e]);
        }
        out += t_tot;
    }
    return out;
}

// ------------------------------------------------- per-group filter state
struct Filter {
    float *bs;    // buffered scores (wave-private, ascending position)
    int32_t *bi;  // buffered positions (bs + cap)
    __amdgpu_buffer_rsrc_t rs;  // bs as one raw buffer of 2 cap words (appends: one offset per lane)
    int cap;      // buffer capacity (>= K + 64)
    int K;        // entries to keep
    int cnt;      // buffered entries (wave-uniform)
    float tau;    // admission threshold (wave-uniform): keep score > tau
    uint32_t *hist;

    // One 64-key step: lane holds (score, position) or !valid. The branch
    // conditions are wave-uniform (ballots, readfirstlane'd counters).
    __device__ __forceinline__ void push(bool valid, float score, int32_t pos)
    {
        bool pass = valid && score > tau;
        uint64_t pm = ballot(pass);
        if (pm == 0) return;
        int n = popc(pm);
        if (cnt + n > cap) {
            compact();
            pass = valid && score > tau;
            pm = ballot(pass);
            n = popc(pm);
        }
        if (pass) {
            // score at byte 4 slot, position at byte 4 (cap + slot)
            const int slot = cnt + mbcnt(pm);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(score), rs, slot * 4, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32(static_cast<uint32_t>(pos), rs, slot * 4, cap * 4, 0);
        }
        cnt = __builtin_amdgcn_readfirstlane(cnt + n);
    }

    __device__ __forceinline__ void set_buffer(float *base, int capacity)
    {
        bs = base;
        bi = reinterpret_cast<int32_t *>(base + capacity);
        cap = capacity;
        rs = __builtin_amdgcn_make_buffer_rsrc(base, 0, static_cast<uint32_t>(capacity) * 8u, 0x00020000);
    }

    // Keep exactly the best K buffered entries, in order; tau := K-th score.
    __device__ void compact()
    {
        wave_fence();
        const Sel s = wave_select(bs, cnt, K, hist);
        float *bsl = bs;
        int32_t *bil = bi;
        const int kept = wave_emit(bs, bi, cnt, s, [&](int slot, int32_t p, float v) {
            bsl[slot] = v;
            bil[slot] = p;
        });
        wave_fence();
        cnt = __builtin_amdgcn_readfirstlane(kept);
        tau = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(s.all ? tau : key_float(s.kth))));
    }
};

// Final selection of a group's buffer into its outputs.
struct SelectionOut {
    int32_t *idx;    // rows [B, Lq, stride] or candidates [B, G, stride]
    float *sc;       // rows only (may be null)
    int32_t *count;  // candidates only (may be null)
    int stride;      // topk (rows) or c (candidates)
    int to_candidates;
};

__device__ void finish_group(const Geo &geo, const SelectionOut &o, int64_t b, int64_t m, Filter &f)
{
    wave_fence();
    const Sel s = wave_select(f.bs, f.cnt, f.K, f.hist);
    const int l = lane_id();
    if (o.to_candidates) {
        int32_t *ci = o.idx + (b * geo.G + m) * o.stride;
        float *cs = o.sc ? o.sc + (b * geo.G + m) * o.stride : nullptr;
        const int n = wave_emit(f.bs, f.bi, f.cnt, s, [&](int slot, int32_t p, float v) {
            ci[slot] = p;
            if (cs) cs[slot] = v;
        });
        for (int t = n + l; t < o.stride; t += kWave) {
            ci[t] = -1;
            if (cs) cs[t] = -INFINITY;
        }
        if (o.count && l == 0) o.count[b * geo.G + m] = n;
        return;
    }
    const int64_t r0 = geo.first_row(m), r1 = geo.end_row(m);
    const int64_t stride = o.stride;
    int32_t *idx = o.idx;
    float *scr = o.sc;
    const int n = wave_emit(f.bs, f.bi, f.cnt, s, [&](int slot, int32_t p, float v) {
        for (int64_t r = r0; r < r1; ++r) {
            const int64_t off = (b * geo.Lq + r) * stride + slot;
            idx[off] = p;
            if (scr) scr[off] = v;
        }
    });
    for (int64_t r = r0; r < r1; ++r) {
        for (int t = n + l; t < o.stride; t += kWave) {
            const int64_t off = (b * geo.Lq + r) * stride + t;
            idx[off] = -1;
            if (scr) scr[off] = -INFINITY;
        }
    }
}

// ---------------------------------------------------------------- pool
// eq. (4): thread per (b, m, head, VEC-element chunk). fp32 sum over members
// in order, one IEEE division by the member count, RNE to the q dtype.
// agg = 1 / 2 (the first / last-query proxies of the aggregation ablation):
// the proxy is that member's q and w, copied unchanged.
template <typename T>
__global__ __launch_bounds__(256) void k_pool(const T *__restrict__ q, const float *__restrict__ w,
                                              T *__restrict__ qbar, float *__restrict__ wbar, Geo geo, int H,
                                              int D, int agg)
{
    constexpr int VEC = 16 / sizeof(T);
    const int chunks = D / VEC;
    const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t total = geo.B * geo.G * H * chunks;
    if (tid >= total) return;
    const int ch = static_cast<int>(tid % chunks);
    const int64_t t2 = tid / chunks;
    const int h = static_cast<int>(t2 % H);
    const int64_t bm = t2 / H;
    const int64_t b = bm / geo.G, m = bm % geo.G;
    const int64_t r0 = geo.first_row(m), r1 = geo.end_row(m);
    const float gm = static_cast<float>(r1 - r0);
    if (agg != 0) {
        const int64_t r = agg == 1 ? r0 : r1 - 1;
        *reinterpret_cast<uint4 *>(qbar + (bm * H + h) * D + ch * VEC) =
            *reinterpret_cast<const uint4 *>(q + ((b * geo.Lq + r) * H + h) * D + ch * VEC);
        if (ch == 0) wbar[bm * H + h] = w[(b * geo.Lq + r) * H + h];
        return;
    }

    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.0f;
    // eight member rows are requested before the first is added (a short
    // batch repeats its last row and skips the repeats); the sum still runs
    // in member order
    constexpr int kRows = 8;
    for (int64_t r = r0; r < r1; r += kRows) {
        uint4 v[kRows];
#pragma unroll
        for (int j = 0; j < kRows; ++j) {
            const int64_t rr = r + j < r1 ? r + j : r1 - 1;
            v[j] = *reinterpret_cast<const uint4 *>(q + ((b * geo.Lq + rr) * H + h) * D + ch * VEC);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < kRows; ++j) {
            if (r + j < r1) {
                union {
                    uint4 v;
                    T e[VEC];
                } u;
                u.v = v[j];
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[e] = acc[e] + widen<T>(u.e[e]);
            }
        }
    }
    union {
        uint4 v;
        T e[VEC];
    } o;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        const float mean = acc[e] / gm;  // IEEE division (HIP default)
        if constexpr (sizeof(T) == 2) {
            o.e[e] = float_to_bf16_rne(mean);
        } else {
            o.e[e] = mean;
        }
    }
    *reinterpret_cast<uint4 *>(qbar + (bm * H + h) * D + ch * VEC) = o.v;
    if (ch == 0) {
        float s = 0.0f;
        for (int64_t r = r0; r < r1; ++r) s = s + w[(b * geo.Lq + r) * H + h];
        wbar[bm * H + h] = s / gm;
    }
}

// -------------------------------------------------------- MFMA scan (bf16)
// One workgroup = kScanWaves waves = as many consecutive groups of one
// sequence. The WG streams tiles of k into LDS (double-buffered; LDS DMA puts
// each 16-byte chunk straight into LDS at an XOR-swizzled slot, so the MFMA
// operand reads are bank-conflict free) and every wave multiplies its proxy
// (H x D, held in registers as MFMA A fragments) by the tile:
//   v_mfma_f32_16x16x32_bf16: A = 16 heads x 32 dims, B = 32 dims x 16 keys.
// Output lane l holds key (l % 16) and heads 4*(l/16) + v, v = 0..3, so the
// ReLU and w-weighted sum over the lane's heads stays in registers; two
// permlane swaps across the 16-lane quarters then leave lane l with the full
// score of key l of the tile.
enum ScanMode { kFilter = 0, kRows = 1 };

struct ScanArgs {
    const void *qsrc;   // [B, G, H, D] proxies (the queries themselves when g == 1), or, with
    const float *wsrc;  // [B, G, H]    pool_inline, the member rows q [B, Lq, H, D], w [B, Lq, H]
    int pool_inline;    // MFMA scans: 1 = form each group's proxy (eq. 4) from its members' rows
    int agg;            // pool_inline: 0 mean, 1 first member, 2 last member
    Keys keys;          // [B, Lk, D] contiguous, or paged
    Geo geo;
    int H, D;
    // kFilter
    int K, cap;
    float *buf_s;     // [B*G][2*cap]: cap scores, then cap positions (int32)
    int32_t *buf_n;   // [B*G] entries buffered (MFMA scan; k_select_groups selects them)
    float *smp;       // [B*G][kSampleSlots] sampled scores (MFMA scan)
    SelectionOut out; // exact-order scan: selected in-kernel
    // kRows
    float *rows;  // [B, G, Lk]
    uint32_t *hist;  // split scan: [B*G, splits, kRowHistWords] counts of the scores' leading key bits
};

// The split scan counts every score of its key range by the leading
// kRowHistBits bits of its order-preserving key (sign, exponent, 3 mantissa
// bits: bins an eighth of an octave wide); the row select finds the bin that
// holds the K-th largest score from these counts. Each workgroup writes the
// kRowHistBins fine counts, then kRowCoarseBins coarse ones (sixteen fine
// bins each, two octaves), so the select finds the coarse bin first and then
// reads only its sixteen fine counts.
constexpr int kRowHistBits = 12;
constexpr int kRowHistBins = 1 << kRowHistBits;
constexpr int kRowCoarseBins = kRowHistBins / 16;
constexpr int kRowHistWords = kRowHistBins + kRowCoarseBins;

typedef __attribute__((address_space(1))) const void *global_cptr;
typedef __attribute__((address_space(3))) void *lds_ptr;

// Lane l of the wave's 1 KiB slice `slice` (0..15) of a 64 x 128 bf16 tile:
// the tile row it fills and the element offset of its 16-byte chunk within
// the key row, so that LDS slot (row, l % 16) holds logical chunk
// (l % 16) ^ (row % 16).
__device__ __forceinline__ int slice_row(int slice, int l) { return slice * 4 + (l >> 4); }
__device__ __forceinline__ int slice_col(int slice, int l) { return (((l & 15) ^ (slice_row(slice, l) & 15)) * 8); }

// B fragment for key block cb (16 keys), dim block kb (32 dims): lane l reads
// key 16*cb + l%16, dims 32*kb + 8*(l/16) .. +8, from the swizzled tile.
__device__ __forceinline__ bf16x8 b_frag(const uint16_t *tile, int cb, int kb, int l)
{
    const int row = 16 * cb + (l & 15);
    const int chunk = (4 * kb + (l >> 4)) ^ (l & 15);
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(tile + row * 128 + chunk * 8));
}

template <int RB>
__device__ __forceinline__ void mfma_block(const bf16x8 (&afr)[RB][4], const uint16_t *tile, int cb, int l,
                                           f32x4 (&acc)[RB])
{
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        const bf16x8 bfr = b_frag(tile, cb, kb, l);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[rb][kb], bfr, acc[rb], 0, 0, 0);
    }
}

template <int RB>
__device__ __forceinline__ float relu_weighted(const f32x4 (&acc)[RB], const float (&wr)[RB][4])
{
    float s = 0.0f;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            // ReLU on the bit pattern: negative floats (and -0) are negative
            // int32, so max(bits, 0) gives +0 for them and keeps the rest.
            const float relu = __int_as_float(max(__float_as_int(acc[rb][v]), 0));
            s = fmaf(wr[rb][v], relu, s);
        }
    }
    return s;
}

// Sum p[cb] over the four 16-lane quarters so lane l ends with key l's total.
__device__ __forceinline__ float quarter_transpose_sum(const float (&p)[4])
{
    // halves: lanes 0-31 collect key blocks 0 and 1, lanes 32-63 blocks 2 and 3
    const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[0]), __float_as_uint(p[2]), false, false);
    const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[1]), __float_as_uint(p[3]), false, false);
    const float x0 = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);
    const float x1 = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);
    // rows: quarter 0 keeps block 0, 1 block 1, 2 block 2, 3 block 3
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x0), __float_as_uint(x1), false, false);
    return (__uint_as_float(r[0]) + __uint_as_float(r[1])) + 0.0f;  // + 0: one zero, +0
}

// B fragments of one 16-key block (all four 32-dim slices).
__device__ __forceinline__ void load_b(const uint16_t *tile, int cb, int l, bf16x8 (&bfr)[4])
{
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) bfr[kb] = b_frag(tile, cb, kb, l);
}

// Fence for the instruction scheduler: nothing moves across it, so the
// source order below is the issue order.
#define PIVOT_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// One tile of NBLK 16-key blocks, software-pipelined in issue order: the 16
// MFMAs of block cb alternate one-for-one with the ReLU-weighted reduction
// of block cb - 1 (one max and one FMA each), so the matrix core never waits
// on the reduction and the reduction reads accumulators finished 16 MFMAs
// earlier; the B fragments of block cb + 2 are read from LDS while block cb
// runs. The pipeline also runs across tiles: the last block of a tile is
// handed over in `carry` (its MFMAs may still be in flight through the
// barrier) and reduced beside the next tile's first block, with `pc` holding
// the reduced blocks NBLK - 4 .. NBLK - 2 of that last 64-key quarter.
// emit(q, score) receives each finished quarter: q = -1 for the previous
// tile's last quarter (only when have_prev), q = 0 .. NBLK / 4 - 2 for this
// tile's; lane l's score is that of key 64 q + l.
template <int RB, int NBLK, class Emit>
__device__ __forceinline__ void tile_step(const bf16x8 (&afr)[RB][4], const float (&wr)[RB][4], const uint16_t *tile,
                                          int l, f32x4 (&carry)[RB], float (&pc)[3], bool have_prev, Emit &&emit)
{
    // a block is 4 RB MFMAs and leaves 4 RB accumulator elements per lane:
    // one element of block cb - 1 is reduced beside each MFMA of block cb
    static_assert(RB >= 1 && RB <= 4, "16 to 64 heads");
    static_assert(NBLK % 4 == 0 && NBLK >= 4, "whole 64-key quarters");
    f32x4 acc[2][RB];
    bf16x8 bq[2][4];
    float p[NBLK];
    load_b(tile, 0, l, bq[0]);
    load_b(tile, 1, l, bq[1]);
    PIVOT_SCHED_FENCE();
#pragma unroll
    for (int cb = 0; cb < NBLK; ++cb) {
        f32x4 (&ac)[RB] = acc[cb & 1];
        const f32x4 (&pv)[RB] = cb == 0 ? carry : acc[(cb + 1) & 1];  // block cb - 1
        float sum = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                ac[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[rb][kb], bq[cb & 1][kb],
                                                                kb == 0 ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : ac[rb], 0, 0, 0);
                // element kb RB + rb of block cb - 1: accumulator (kb RB + rb) / 4,
                // lane slot (kb RB + rb) % 4 (for RB = 4: accumulator kb, slot rb)
                const int el = kb * RB + rb;
                const float relu = __int_as_float(max(__float_as_int(pv[el >> 2][el & 3]), 0));
                sum = fmaf(wr[el >> 2][el & 3], relu, sum);
                asm volatile("" : "+v"(sum));  // keep the partial sum here, beside this MFMA
                PIVOT_SCHED_FENCE();
            }
            if (cb + 2 < NBLK) {
                bq[cb & 1][kb] = b_frag(tile, cb + 2, kb, l);
                PIVOT_SCHED_FENCE();
            }
        }
        if (cb == 0) {
            if (have_prev) {
                const float q4[4] = {pc[0], pc[1], pc[2], sum};
                emit(-1, quarter_transpose_sum(q4));
            }
        } else {
            p[cb - 1] = sum;
            if (cb % 4 == 0) {
                const float q4[4] = {p[cb - 4], p[cb - 3], p[cb - 2], p[cb - 1]};
                emit(cb / 4 - 1, quarter_transpose_sum(q4));
            }
        }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) carry[rb] = acc[(NBLK - 1) & 1][rb];
    pc[0] = p[NBLK - 4];
    pc[1] = p[NBLK - 3];
    pc[2] = p[NBLK - 2];
}

template <int H>
__device__ __forceinline__ void load_a(const uint16_t *src, int l, bf16x8 (&afr)[H / 16][4])
{
#pragma unroll
    for (int rb = 0; rb < H / 16; ++rb) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
            afr[rb][kb] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const uint4 *>(src + (16 * rb + (l & 15)) * 128 + 32 * kb + 8 * (l >> 4)));
    }
}

template <int H>
__device__ __forceinline__ void load_w(const float *src, int l, float (&wr)[H / 16][4])
{
#pragma unroll
    for (int rb = 0; rb < H / 16; ++rb) {
#pragma unroll
        for (int v = 0; v < 4; ++v) wr[rb][v] = src[16 * rb + 4 * (l >> 4) + v];
    }
}

// eq. (4) inside the scan: row block rb (heads 16 rb .. 16 rb + 15) of the
// proxy of rows [r0, r1) of q (row stride H D) straight into this lane's A
// fragments and w slots, with the arithmetic of k_pool (fp32 sum in member
// order, one IEEE division by the member count, RNE to bf16; the first /
// last member copied unchanged for agg 1 / 2). The q and w rows of ROWS
// members are requested together, so ROWS members cost one memory latency.
template <int H, int ROWS = 8>
__device__ __forceinline__ void pool_rb(const uint16_t *q, const float *w, int64_t r0, int64_t r1, int agg, int l,
                                        int rb, bf16x8 (&afr)[4], float (&wr)[4])
{
    constexpr int D = 128;
    if (agg != 0) {
        const int64_t r = agg == 1 ? r0 : r1 - 1;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
            afr[kb] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const uint4 *>(q + (r * H + 16 * rb + (l & 15)) * D + 32 * kb + 8 * (l >> 4)));
        const float4 v = *reinterpret_cast<const float4 *>(w + r * H + 16 * rb + 4 * (l >> 4));
        wr[0] = v.x;
        wr[1] = v.y;
        wr[2] = v.z;
        wr[3] = v.w;
        return;
    }
    const float gm = static_cast<float>(r1 - r0);
    float acc[4][8];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[kb][e] = 0.0f;
    // w: the lane's four heads of the block are contiguous (one float4 per member)
    float sum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t r = r0; r < r1; r += ROWS) {
        uint4 v[ROWS][4];
        float4 vw[ROWS];
#pragma unroll
        for (int i = 0; i < ROWS; ++i) {
            const int64_t rr = r + i < r1 ? r + i : r1 - 1;  // a short batch repeats its last row
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                v[i][kb] =
                    *reinterpret_cast<const uint4 *>(q + (rr * H + 16 * rb + (l & 15)) * D + 32 * kb + 8 * (l >> 4));
            vw[i] = *reinterpret_cast<const float4 *>(w + rr * H + 16 * rb + 4 * (l >> 4));
        }
#pragma unroll
        for (int i = 0; i < ROWS; ++i) {
            if (r + i < r1) {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const uint32_t u[4] = {v[i][kb].x, v[i][kb].y, v[i][kb].z, v[i][kb].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        acc[kb][e] = acc[kb][e] + bf16_bits_to_float(static_cast<uint16_t>(u[e / 2] >> (16 * (e % 2))));
                }
                sum[0] = sum[0] + vw[i].x;
                sum[1] = sum[1] + vw[i].y;
                sum[2] = sum[2] + vw[i].z;
                sum[3] = sum[3] + vw[i].w;
            }
        }
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        uint32_t u[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            u[e] = static_cast<uint32_t>(float_to_bf16_rne(acc[kb][2 * e] / gm)) |
                   static_cast<uint32_t>(float_to_bf16_rne(acc[kb][2 * e + 1] / gm)) << 16;
        afr[kb] = __builtin_bit_cast(bf16x8, uint4{u[0], u[1], u[2], u[3]});
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) wr[v] = sum[v] / gm;
}

// The whole proxy (every row block) in this lane's A fragments and w slots.
template <int H>
__device__ __forceinline__ void pool_a(const uint16_t *q, const float *w, int64_t r0, int64_t r1, int agg, int l,
                                       bf16x8 (&afr)[H / 16][4], float (&wr)[H / 16][4])
{
#pragma unroll
    for (int rb = 0; rb < H / 16; ++rb) pool_rb<H, 4>(q, w, r0, r1, agg, l, rb, afr[rb], wr[rb]);
}

// Sampled admission threshold (filter mode). Before the full pass the WG
// scores every `stride`-th tile; each wave sets tau a few standard deviations
// below its sample's estimate of the K-th best score, so the full pass admits
// about 1.5 K survivors instead of c (1 + ln(n / c)). If a group still ends
// with fewer than K survivors the WG repeats the pass for it with tau = -inf,
// so the selection is exact whatever the sample shows.
constexpr int kSampleStride = 32;     // tiles between sampled tiles (>= this)
constexpr float kSampleSigmas = 6.0f;
constexpr int kSampleSlots = 4096;    // sampled scores kept per group (16 tiles of 256 keys)

// Fused-scan workgroup shape: kScanWaves groups (one per wave) share each
// 256-key tile (64 KiB); kScanBufs tiles are in LDS or in flight at once.
// The kernel needs about 220 VGPRs, so a CU holds eight of its waves: one
// workgroup of eight waves with two buffers measured faster than two
// workgroups of four (each key tile is fetched once per eight groups instead
// of four) and than a third buffer (L=128K, g=8: 16.4 ms vs 20.8 and 16.8);
// 256-key tiles (half the barriers) beat 128-key ones by 1.5% (13.6 vs 13.8 ms).
#ifndef PIVOT_SCAN_WAVES
#define PIVOT_SCAN_WAVES 8
#endif
#ifndef PIVOT_SCAN_TILE
#define PIVOT_SCAN_TILE 256
#endif
#ifndef PIVOT_SCAN_BUFS
#define PIVOT_SCAN_BUFS 2
#endif
constexpr int kScanWaves = PIVOT_SCAN_WAVES;
constexpr int kScanBufs = PIVOT_SCAN_BUFS;
constexpr int kScanTileKeys = PIVOT_SCAN_TILE;  // keys per LDS tile (one barrier each)
static_assert(kScanTileKeys % 64 == 0, "whole 64-key quarters");
static_assert(kScanBufs == 2 || kScanBufs == 3, "two or three tile buffers");

// One wave's share of a key tile: rows [base, base + NT) of kseq become one
// buffer resource of the bytes that exist, so rows past lk read as zero
// (their scores are masked) and each 1 KiB slice is one LDS DMA instruction
// on the lane's fixed byte offset voff[j]; slice j lands at dst + 512 j.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t key_tile_rsrc(const uint16_t *kseq, int64_t base, int64_t lk)
{
    constexpr int NT = kScanTileKeys, D = 128;
    const int64_t rows_left = lk - base;
    const uint32_t nbytes = static_cast<uint32_t>(rows_left < NT ? rows_left : NT) * (D * 2);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(kseq + base * D), 0, nbytes, 0x00020000);
}

__device__ __forceinline__ void dma_key_slice(__amdgpu_buffer_rsrc_t rs, uint16_t *dst, uint32_t voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)dst, 16, voff, 0, 0, 0);
}

// Workgroup barrier without a memory fence. LDS tiles are written only by
// global_load_lds, whose completion each wave establishes with an explicit
// vmcnt wait before the barrier, and every wave has consumed its own LDS
// reads of a tile before it arrives; the signal fences keep the compiler
// from moving memory operations across the barrier.
__device__ __forceinline__ void tile_barrier()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int H, int D, int Mode, bool PAGED>
__global__ __launch_bounds__(kScanWaves * 64) void k_scan_mfma(ScanArgs a)
{
    static_assert(H % 16 == 0 && D == 128, "tile layout assumes 128-dim keys (16 chunks of 8 bf16 per row)");
    static_assert(!PAGED || kScanBufs == 2, "paged keys: two tile buffers");
    constexpr int RB = H / 16;
    constexpr int NT = kScanTileKeys;                     // keys per tile
    constexpr int NQ = NT / kWave;                        // 64-key quarters per tile
    constexpr int SLICES = NT * D * 2 / 1024;             // 1 KiB slices per tile
    constexpr int SLICES_PER_WAVE = SLICES / kScanWaves;  // DMA instructions per lane per tile
    static_assert(SLICES % kScanWaves == 0, "each wave issues the same number of slices");
    constexpr int NB = kScanBufs;
    constexpr int AHEAD = (NB - 2) * SLICES_PER_WAVE;     // vmcnt that leaves the newer tiles in flight

    // NB tile buffers, each its own LDS object so the compiler can tell that
    // the tile being read is not one the in-flight DMAs are filling. Tile i
    // of a pass lives in buffer i % NB; the DMA for tile i + NB - 1 is issued
    // while tile i is scored.
    __shared__ __attribute__((aligned(1024))) uint16_t tile0[NT * D];
    __shared__ __attribute__((aligned(1024))) uint16_t tile1[NT * D];
    __shared__ __attribute__((aligned(1024))) uint16_t tile2[NB == 3 ? NT * D : 8];
    __shared__ uint32_t hist[kScanWaves][256];

    const Geo &geo = a.geo;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: per-wave values live in SGPRs
    const int l = threadIdx.x & 63;
    const int64_t nblk = (geo.G + kScanWaves - 1) / kScanWaves;
    const int64_t b = blockIdx.x % geo.B;
    const int64_t blk = nblk - 1 - blockIdx.x / geo.B;  // longest prefixes first
    const int64_t m = blk * kScanWaves + wv;
    const bool active = m < geo.G;
    const int64_t m_hi = (blk * kScanWaves + kScanWaves - 1 < geo.G - 1) ? blk * kScanWaves + kScanWaves - 1 : geo.G - 1;
    const int64_t wg_tlast = geo.t_last(b, m_hi);
    const int64_t my_tlast = active ? geo.t_last(b, m) : -1;
    const int ntiles = static_cast<int>(wg_tlast / NT) + 1;
    // contiguous keys: rows up to the capacity exist, those past the
    // sequence are masked
    const uint16_t *kseq = static_cast<const uint16_t *>(a.keys.base) + b * geo.Lk * D;
    const int64_t gid = b * geo.G + (active ? m : blk * kScanWaves);

    bf16x8 afr[RB][4];
    float wr[RB][4];
    if (a.pool_inline) {
        const int64_t mm = active ? m : blk * kScanWaves;
        pool_a<H>(static_cast<const uint16_t *>(a.qsrc) + b * geo.Lq * H * D, a.wsrc + b * geo.Lq * H,
                  geo.first_row(mm), geo.end_row(mm), a.agg, l, afr, wr);
    } else {
        load_a<H>(static_cast<const uint16_t *>(a.qsrc) + gid * H * D, l, afr);
        load_w<H>(a.wsrc + gid * H, l, wr);
    }

    Filter f;
    f.K = a.K;
    f.cap = a.cap;
    f.cnt = 0;
    f.tau = -INFINITY;
    f.hist = hist[wv];
    if (Mode == kFilter) f.set_buffer(a.buf_s + gid * 2 * static_cast<int64_t>(a.cap), a.cap);  // [cap scores | cap positions]
    float *row = (Mode == kRows) ? a.rows + gid * geo.Lk : nullptr;

    // This lane's byte offset within a tile for each of its DMA slices
    // (slices wv * SLICES_PER_WAVE + j).
    uint32_t slice_voff[SLICES_PER_WAVE];
#pragma unroll
    for (int j = 0; j < SLICES_PER_WAVE; ++j) {
        const int slice = wv * SLICES_PER_WAVE + j;
        slice_voff[j] = static_cast<uint32_t>((slice_row(slice, l) * D + slice_col(slice, l)) * 2);
    }
    // Paged keys: lane l's row of slice j of the tile at `base` is key
    // base + slice_row(slice, l) (clamped to the sequence's last key; those
    // past t_last are masked), whose page table entry is read one tile
    // ahead of its DMA, so the DMA issue never waits for a table load.
    const int64_t lkb = geo.lk(b);
    int32_t ent[PAGED ? SLICES_PER_WAVE : 1];
    auto key_of = [&](int64_t base, int j) {
        const int64_t s = base + slice_row(wv * SLICES_PER_WAVE + j, l);
        return static_cast<uint32_t>(s < lkb ? s : (lkb > 0 ? lkb - 1 : 0));
    };
    auto load_entries = [&](int64_t base) {
        if constexpr (PAGED) {
#pragma unroll
            for (int j = 0; j < SLICES_PER_WAVE; ++j) {
                const uint32_t s = key_of(base, j);
                ent[j] = load_as<kGlobal>(a.keys.pg.table, b * a.keys.pg.max_pages + a.keys.page_index(s));
            }
        }
    };
    // slice j (of this wave's SLICES_PER_WAVE) of the tile at `base` into
    // tile buffer `buf`
    auto issue_tile = [&](int buf, int64_t base) {
        uint16_t *dst = buf == 0 ? tile0 : (buf == 1 ? tile1 : tile2);
        const __amdgpu_buffer_rsrc_t rs = key_tile_rsrc(kseq, base, geo.Lk);
#pragma unroll
        for (int j = 0; j < SLICES_PER_WAVE; ++j) {
            const int slice = wv * SLICES_PER_WAVE + j;
            if constexpr (PAGED) {
                const uint16_t *kbase = static_cast<const uint16_t *>(a.keys.base);
                const uint32_t s = key_of(base, j);
                const int64_t r = a.keys.paged_row(ent[j], a.keys.page_offset(s));
                __builtin_amdgcn_global_load_lds((global_cptr)(kbase + r * D + slice_col(slice, l)),
                                                 (lds_ptr)(dst + slice * 512), 16, 0, 0);
            } else {
                dma_key_slice(rs, dst + slice * 512, slice_voff[j]);
            }
        }
    };

    // Phases of a pass over the tiles; the per-score work is chosen at run
    // time so the tile pipeline below is compiled once.
    enum { kPhaseRows = 0, kPhaseSample = 1, kPhaseFilter = 2, kPhaseRedo = 3 };
    int stride = 1;
    int nsv = 0;          // valid sampled keys (phase Sample)
    bool redo = false;    // phase Redo: this wave repeats its selection
    // the group's sampled scores (phase Sample), kept for the filter pass
    float *smp = Mode == kFilter ? a.smp + gid * static_cast<int64_t>(kSampleSlots) : nullptr;
    auto on_score = [&](int phase, int it, int quarter, int64_t base, float score) {
        const int64_t s = base + l;
        // lanes at or below lim hold keys s <= t_last (wave-uniform; positions
        // are below 2^31, so the difference fits 32 bits)
        const int lim = static_cast<int>(my_tlast) - static_cast<int>(base);
        const bool valid = l <= lim;
        if (phase == kPhaseRows) {
            if (active && s < geo.Lk) row[s] = valid ? score : -INFINITY;
        } else if (phase == kPhaseSample) {
            if (active) smp[(it / stride) * NT + quarter * kWave + l] = valid ? score : -INFINITY;
            nsv += popc(ballot(valid));
        } else if (phase == kPhaseFilter) {
            if (active) f.push(valid, score, static_cast<int32_t>(s));
        } else {
            if (redo) f.push(valid, score, static_cast<int32_t>(s));
        }
    };
    // A pass computes tiles tile_of(i), i < nt, in ascending order: every
    // step-th tile (step > 1: the sample), or, with skip > 0 (the filter
    // pass after a sample of every skip-th tile), every tile except the
    // sampled ones, whose scores were stored by the sample pass and are
    // handed to on_score in their place (so the per-score work still sees
    // every tile in position order). Sampled tiles are isolated (skip >= 2).
    auto pass = [&](int phase, int step, int skip) {
        auto tile_of = [&](int i) { return skip ? i + i / (skip - 1) + 1 : i * step; };
        const int nt = skip ? ntiles - ((ntiles - 1) / skip + 1) : (ntiles - 1) / step + 1;
        float gapv[NQ];  // a sampled tile's stored scores, loaded one tile before their turn
        auto load_gap = [&](int t) {
#pragma unroll
            for (int q = 0; q < NQ; ++q) gapv[q] = load_as<kGlobal>(smp, (t / skip) * NT + q * kWave + l);
        };
        auto push_gap = [&](int t) {
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                on_score(phase, t, q, static_cast<int64_t>(t) * NT + q * kWave, gapv[q]);
        };
        if (skip) {  // tile 0 is sampled
            load_gap(0);
            push_gap(0);
        }
        if (nt == 0) return;  // wave-uniform over the workgroup (ntiles is)
        const int64_t first = static_cast<int64_t>(tile_of(0)) * NT;
        load_entries(first);
        issue_tile(0, first);
        if (PAGED && nt > 1) load_entries(static_cast<int64_t>(tile_of(1)) * NT);
        if (NB == 3 && nt > 1) {
            issue_tile(1, static_cast<int64_t>(tile_of(1)) * NT);
            __builtin_amdgcn_s_waitcnt(0x0F70 | SLICES_PER_WAVE);  // tile 0 has landed, tile 1 may not
        } else {
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        }
        tile_barrier();
        int buf = 0;
        f32x4 carry[RB];  // the previous tile's last block, not yet reduced
        float pc[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) carry[rb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        int prev_it = 0;
        // the carried last quarter of tile prev_it
        auto flush = [&]() {
            const float q4[4] = {pc[0], pc[1], pc[2], relu_weighted<RB>(carry, wr)};
            on_score(phase, prev_it, NQ - 1, static_cast<int64_t>(prev_it) * NT + (NQ - 1) * kWave,
                     quarter_transpose_sum(q4));
        };
        for (int i = 0; i < nt; ++i) {
            const int it = tile_of(i);
            const int64_t base = static_cast<int64_t>(it) * NT;
            // a stored tile between the previous computed tile and this one:
            // finish the previous tile, then hand over the stored scores
            // (without skip the previous tile's last quarter is carried into
            // this tile's first block, whatever the step)
            const bool contiguous = i > 0 && (!skip || prev_it == it - 1);
            if (skip && i > 0 && !contiguous) {
                flush();
                push_gap(it - 1);
            }
            if (skip && it + 1 < ntiles && (it + 1) % skip == 0) load_gap(it + 1);
            // the buffer of tile i + NB - 1 held tile i - 1, which every wave
            // finished reading before the last barrier (paged keys: the
            // entries of the tile after it are then read)
            const bool ahead = i + NB - 1 < nt;
            if (ahead) {
                issue_tile(buf == 0 ? NB - 1 : buf - 1, static_cast<int64_t>(tile_of(i + NB - 1)) * NT);
                if (PAGED && i + 2 < nt) load_entries(static_cast<int64_t>(tile_of(i + 2)) * NT);
            }
            auto emit = [&](int qt, float score) {
                if (qt < 0)
                    on_score(phase, prev_it, NQ - 1, static_cast<int64_t>(prev_it) * NT + (NQ - 1) * kWave, score);
                else
                    on_score(phase, it, qt, base + qt * kWave, score);
            };
            if (buf == 0)
                tile_step<RB, NT / 16>(afr, wr, tile0, l, carry, pc, contiguous, emit);
            else if (NB == 2 || buf == 1)
                tile_step<RB, NT / 16>(afr, wr, tile1, l, carry, pc, contiguous, emit);
            else
                tile_step<RB, NT / 16>(afr, wr, tile2, l, carry, pc, contiguous, emit);
            prev_it = it;
            // tile i + 1 must be in LDS; with three buffers tile i + 2's DMAs
            // may stay in flight (vector memory counts complete in issue
            // order, so stores issued after them only make this wait longer)
            if (NB == 3 && ahead)
                __builtin_amdgcn_s_waitcnt(0x0F70 | AHEAD);
            else
                __builtin_amdgcn_s_waitcnt(0x0F70);
            tile_barrier();
            buf = buf == NB - 1 ? 0 : buf + 1;
        }
        flush();  // the last computed tile's last quarter
        if (skip && prev_it + 1 < ntiles) push_gap(prev_it + 1);  // a stored tile after it
    };

    if (Mode == kRows) {
        pass(kPhaseRows, 1, 0);
        if (!active) return;
        for (int64_t s = static_cast<int64_t>(ntiles) * NT + l; s < geo.Lk; s += kWave) row[s] = -INFINITY;
        return;
    }

    // ---- phase A: sampled threshold, the sampled scores kept in smp
    const int64_t n_valid = my_tlast + 1;
    const int sample_cap_tiles = kSampleSlots / NT;
    stride = kSampleStride;
    if ((ntiles + stride - 1) / stride > sample_cap_tiles) stride = (ntiles + sample_cap_tiles - 1) / sample_cap_tiles;
    const bool sample = ntiles * NT > 4 * a.K && sample_cap_tiles > 0;  // short prefixes: plain streaming
    if (sample) {
        pass(kPhaseSample, stride, 0);
        if (active) {
            const int nslots = ((ntiles - 1) / stride + 1) * NT;
            const float expect = static_cast<float>(a.K) * static_cast<float>(nsv) / static_cast<float>(n_valid);
            const int r = static_cast<int>(ceilf(expect + kSampleSigmas * sqrtf(expect) + 8.0f));
            if (n_valid > 2 * static_cast<int64_t>(a.K) && r < nsv) {
                wave_fence();
                const Sel sel = wave_select(smp, nslots, r, f.hist);
                f.tau = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(key_float(sel.kth))));
            }
        }
    }

    // ---- phase B: the full pass with the streaming filter (the sampled
    // tiles' scores come from smp)
    pass(kPhaseFilter, 1, sample ? stride : 0);

    // exactness guard: a group with fewer than min(K, n_valid) survivors had
    // its sampled tau set too high; the WG repeats the pass for it from -inf
    const int64_t need = n_valid < a.K ? n_valid : a.K;
    const bool failed = active && f.cnt < need;
    if (__syncthreads_or(failed)) {
        redo = failed;
        if (redo) {
            f.cnt = 0;
            f.tau = -INFINITY;
        }
        pass(kPhaseRedo, 1, 0);
    }

    // the group's survivors (ascending position, at least min(K, n_valid)
    // of them) are selected by k_select_groups, at full occupancy
    if (active && l == 0) a.buf_n[gid] = f.cnt;
}

// ---------------------------------------------- split scan (few groups)
// When there are too few groups to fill the GPU (decode: one group per
// sequence), the key axis of each group is split over many waves and the
// proxy scores go to a row buffer [B*G, Lk] for k_select_rows. Each key meets
// only the group's H proxy rows, so the scan is HBM-bound and its keys skip
// LDS: every wave streams 64-key quarters of its group (quarters u, u + U,
// u + 2U, ... with U waves per group, so the waves of a group sweep the
// prefix together) straight from HBM into MFMA B fragments. The next
// quarter's 16-key blocks are requested one by one as the current quarter's
// blocks are consumed, so a quarter (16 KiB) per wave is always in flight,
// with no LDS and no barrier. Paged keys: each lane reads the table entries
// of its keys two quarters ahead of their rows.
template <int RB>
__device__ __forceinline__ void mfma_block_regs(const bf16x8 (&afr)[RB][4], const bf16x8 (&bfr)[4], f32x4 (&acc)[RB])
{
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[rb][kb], bfr[kb], acc[rb], 0, 0, 0);
    }
}

constexpr int kSplitWaves = 4;  // waves per split-scan workgroup

template <int H, int D, bool PAGED>
__global__ __launch_bounds__(kSplitWaves * 64, 2) void k_scan_split(ScanArgs a, int splits)
{
    static_assert(H % 16 == 0 && D == 128, "B fragments assume 128-dim keys");
    constexpr int RB = H / 16;
    __shared__ __attribute__((aligned(16))) uint32_t hist[kRowHistBins];  // this workgroup's score counts
    __shared__ uint4 pool_f[RB][4][kWave];   // pool_inline: the proxy's A fragments, per lane
    __shared__ float4 pool_w[RB][kWave];     // and its w slots
    const Geo &geo = a.geo;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = threadIdx.x & 63;
    const int64_t gid = blockIdx.x / splits;
    const int split = blockIdx.x % splits;
    const int64_t b = gid / geo.G, m = gid % geo.G;
    const int64_t tl = geo.t_last(b, m);
    for (int i = threadIdx.x; i < kRowHistBins; i += kSplitWaves * 64) hist[i] = 0u;
    // the workgroup's counts go out whatever it scored (zeros when nothing)
    auto flush_hist = [&]() {
        __syncthreads();
        uint32_t *out = a.hist + (gid * splits + split) * kRowHistWords;
        for (int i = threadIdx.x; i < kRowHistBins; i += kSplitWaves * 64) out[i] = hist[i];
        static_assert(kRowCoarseBins == kSplitWaves * 64, "one coarse bin per thread");
        const uint4 *h4 = reinterpret_cast<const uint4 *>(hist + 16 * threadIdx.x);
        uint32_t c = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 v = h4[i];
            c += v.x + v.y + v.z + v.w;
        }
        out[kRowHistBins + threadIdx.x] = c;
    };
    const int nq = tl < 0 ? 0 : static_cast<int>(tl / kWave) + 1;  // quarters holding keys 0 .. tl
    const int U = kSplitWaves * splits;
    const int u = kSplitWaves * split + wv;
    const bool has = u < nq;  // wave-uniform: this wave has quarters
    const int n = has ? (nq - 1 - u) / U + 1 : 0;  // this wave's quarters: qidx(i), i < n

    const uint16_t *kbase = static_cast<const uint16_t *>(a.keys.base);
    const int64_t lkb = geo.lk(b);
    float *row = a.rows + gid * geo.Lk;

    // the wave's i-th quarter: the groups start their sweeps at staggered
    // offsets (group gid of N at nq gid / N), so that the groups do not
    // read the same offsets of their key ranges at the same time (4.5%
    // faster on 32 sequences of 64K keys)
    const int rot = static_cast<int>((static_cast<int64_t>(nq) * gid) / (geo.B * geo.G));
    auto qidx = [&](int i) {
        const int j = u + U * i + rot;
        return j < nq ? j : j - nq;
    };
    // lane l's key in block cb of quarter i (past the sequence: its last
    // key, whose score is never stored)
    auto key_pos = [&](int i, int cb) {
        const int64_t s = static_cast<int64_t>(qidx(i)) * kWave + 16 * cb + (l & 15);
        return static_cast<uint32_t>(s < lkb ? s : (lkb > 0 ? lkb - 1 : 0));
    };
    auto load_entries = [&](int i, int32_t (&e)[4]) {
        if constexpr (PAGED) {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) e[cb] = a.keys.entry(b, key_pos(i, cb));
        }
    };
    // B fragments of block cb of quarter i: lane l takes key 16 cb + l % 16,
    // dims 32 kb + 8 (l / 16) .. + 8 for kb = 0..3 (64 contiguous bytes of
    // each key row per load instruction)
    auto load_block = [&](int i, int cb, const int32_t (&e)[4], bf16x8 (&bfr)[4]) {
        const uint32_t s = key_pos(i, cb);
        const int64_t r = PAGED ? a.keys.paged_row(e[cb], a.keys.page_offset(s)) : a.keys.flat(b, s);
        const bf16x8 *src = reinterpret_cast<const bf16x8 *>(kbase + r * D + 8 * (l >> 4));
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) bfr[kb] = load_as<kGlobal>(src, 4 * kb);
    };

    // Every load and store below is unconditional (past the wave's last
    // quarter the loads repeat it; each quarter's store goes through a
    // buffer resource of its keys up to tl, which drops the lanes past tl),
    // so the compiler can count the loads in flight exactly and waits for
    // each block only, not for the whole next quarter.
    const int last = n - 1;
    // DEPTH quarters of keys per wave in registers: the one being scored
    // and the next DEPTH - 1, each block replaced by the block DEPTH
    // quarters later as soon as it is consumed (contiguous keys: two, i.e.
    // 32 KiB in flight per wave; paged keys need registers for the table
    // entries and keep one; deeper rings measured no faster)
    constexpr int DEPTH = PAGED ? 1 : 2;
    bf16x8 bq[DEPTH][4][4];
    int32_t e[2][4] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
    // the first quarter's keys are requested before the proxy is formed, so
    // their latency and the proxy's overlap
    if (has) {
        load_entries(0, e[1]);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) load_block(0, cb, e[1], bq[0][cb]);
    }
    if (a.pool_inline) {
        // eq. (4) once per workgroup: wave wv pools row blocks wv, wv + 4,
        // ... of the group's proxy from the member rows and leaves them in
        // LDS for every wave (no pool launch, no proxy round trip through
        // HBM); four members per memory round trip
        for (int rb = wv; rb < RB; rb += kSplitWaves) {
            bf16x8 f[4];
            float wq[4];
            pool_rb<H, 4>(static_cast<const uint16_t *>(a.qsrc) + b * geo.Lq * H * D, a.wsrc + b * geo.Lq * H,
                          geo.first_row(m), geo.end_row(m), a.agg, l, rb, f, wq);
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) pool_f[rb][kb][l] = __builtin_bit_cast(uint4, f[kb]);
            pool_w[rb][l] = float4{wq[0], wq[1], wq[2], wq[3]};
        }
    }
    __syncthreads();
    if (!has) {  // a wave without a quarter (or a group without keys)
        flush_hist();
        return;
    }

    bf16x8 afr[RB][4];
    float wr[RB][4];
    if (a.pool_inline) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) afr[rb][kb] = __builtin_bit_cast(bf16x8, pool_f[rb][kb][l]);
            const float4 v = pool_w[rb][l];
            wr[rb][0] = v.x;
            wr[rb][1] = v.y;
            wr[rb][2] = v.z;
            wr[rb][3] = v.w;
        }
    } else {
        load_a<H>(static_cast<const uint16_t *>(a.qsrc) + gid * H * D, l, afr);
        load_w<H>(a.wsrc + gid * H, l, wr);
    }
#pragma unroll
    for (int d = 1; d < DEPTH; ++d) {
        load_entries(d < last ? d : last, e[1]);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) load_block(d < last ? d : last, cb, e[1], bq[d][cb]);
    }
    load_entries(DEPTH < last ? DEPTH : last, e[0]);

    // quarter i (in slot i % DEPTH): score it while its slot fills with
    // quarter i + DEPTH (rows from e[i % 2], that quarter's table entries
    // when paged) and e[(i + 1) % 2] receives the entries of quarter
    // i + DEPTH + 1
    auto quarter = [&](int i, int slot, const int32_t (&use)[4], int32_t (&fill)[4]) {
        const int in = i + DEPTH < last ? i + DEPTH : last, ie = i + DEPTH + 1 < last ? i + DEPTH + 1 : last;
        load_entries(ie, fill);
        float p[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            f32x4 acc[RB];
            mfma_block_regs<RB>(afr, bq[slot][cb], acc);
            // the block's replacement is requested right here, DEPTH
            // quarters before its use (the scheduler would otherwise sink
            // the loads toward their use)
            __builtin_amdgcn_sched_barrier(0);
            load_block(in, cb, use, bq[slot][cb]);
            __builtin_amdgcn_sched_barrier(0);
            p[cb] = relu_weighted<RB>(acc, wr);
        }
        const float score = quarter_transpose_sum(p);
        const int64_t q0 = static_cast<int64_t>(qidx(i)) * kWave;  // <= tl
        const int64_t left = tl + 1 - q0;
        const __amdgpu_buffer_rsrc_t out = __builtin_amdgcn_make_buffer_rsrc(
            row + q0, 0, static_cast<uint32_t>((left < kWave ? left : kWave) * sizeof(float)), 0x00020000);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(score), out, l * 4, 0, 0);
        // count the lanes' scores (keys <= tl) by their leading key bits;
        // the lanes sharing the first lane's bin add with one atomic
        bin_add(l < left, ord_key(score) >> (32 - kRowHistBits), hist, l);
    };
    // UNROLL quarters per trip (a multiple of 2 and of DEPTH), so the key
    // slots and the entry arrays trade roles without copies (a copy of a
    // loaded register would wait for its load)
    constexpr int UNROLL = DEPTH % 2 == 0 ? DEPTH : 2 * DEPTH;
    int i = 0;
    for (; i + UNROLL - 1 <= last; i += UNROLL) {
#pragma unroll
        for (int k = 0; k < UNROLL; ++k) quarter(i + k, k % DEPTH, e[k % 2], e[(k + 1) % 2]);
    }
#pragma unroll
    for (int k = 0; k < UNROLL - 1; ++k)
        if (i + k <= last) quarter(i + k, k % DEPTH, e[k % 2], e[(k + 1) % 2]);
    flush_hist();
}

// Raw buffer descriptor over n 32-bit entries at p (gfx9 family: fourth
// word 0x00020000 = 32-bit data format, no swizzle); loads past the end
// return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_buffer(const void *p, int n)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, n * 4, 0x00020000);
}

// Number of keys in kv[] that are >= x (a wave-uniform count).
template <int N>
__device__ __forceinline__ int count_ge(const uint32_t (&kv)[N], uint32_t x)
{
    int n = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) n += popc(ballot(kv[i] >= x));
    return n;
}

constexpr int kMsMid = 1024;    // LDS keys per wave for the final bits (a bin bisected in registers)

// The K-th largest key when it lies in a bin [lo, hi] whose n keys are in
// mid (LDS) and `above` keys exceed the bin: the largest x in [lo, hi] with
// above + #{bin keys >= x} >= K, plus the keys above it and equal to it
// (counted over the bin alone), with the bin held R keys per lane.
struct BinKth {
    uint32_t kth;
    int n_gt, n_eq;
};

template <int R>
__device__ __forceinline__ BinKth bisect_bin(const uint32_t *mid, int n, uint32_t lo, uint32_t hi, int above, int K)
{
    const int l = lane_id();
    uint32_t mv[R];
#pragma unroll
    for (int q = 0; q < R; ++q) {
        const int j = kWave * q + l;
        mv[q] = j < n ? mid[j] : 0u;
    }
    while (lo < hi) {
        const uint32_t x = lo + (hi - lo) / 2u + 1u;
        if (above + count_ge(mv, x) >= K)
            lo = x;
        else
            hi = x - 1u;
    }
    BinKth r;
    r.kth = lo;
    r.n_gt = above + (lo == 0xFFFFFFFFu ? 0 : count_ge(mv, lo + 1u));
    r.n_eq = above + count_ge(mv, lo) - r.n_gt;
    return r;
}

__device__ __forceinline__ BinKth bisect_bin_any(const uint32_t *mid, int n, uint32_t lo, uint32_t hi, int above,
                                                 int K)
{
    if (n <= kWave) return bisect_bin<1>(mid, n, lo, hi, above, K);
    if (n <= 4 * kWave) return bisect_bin<4>(mid, n, lo, hi, above, K);
    return bisect_bin<kMsMid / kWave>(mid, n, lo, hi, above, K);
}

// --------------------------------------------------- block-wide select
// Selection of one row by a whole workgroup (1024 threads), for rows too
// long for one wave: the proxy rows of the split scan and the member rows of
// the split refine. Same radix select and stable emission as the wave
// versions, with the lane prefix extended across waves through LDS.
struct RowSelectArgs {
    Geo geo;
    int kind;              // 0: group rows (decode scan); 1: member rows (split refine)
    const float *rows;     // kind 0: [B*G, Lk]; kind 1: scratch [B*G, g, c]
    const uint32_t *hist;  // kind 0: the split scan's score counts [B*G, splits, kRowHistWords]
    int splits;
    int K;                 // kind 0: c (to candidates) or topk (to member rows); kind 1: topk
    int to_candidates;     // kind 0 only
    int32_t *out_idx;      // rows [B, Lq, topk] or candidates [B, G, c]
    float *out_sc;         // rows only, nullable
    int32_t *out_count;    // candidates only, nullable
    int out_stride;
    const int32_t *cand;   // kind 1: [B*G, c]
    const int32_t *cand_n; // kind 1: [B*G]
    int c;                 // kind 1
};

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;

struct BlockShared {
    alignas(16) uint32_t hist[kSelWaves][256];  // one histogram per wave (no inter-wave atomic contention)
    int wave_sum[2][kSelWaves];
    uint32_t bcast[4];
    uint32_t key_and[kSelWaves], key_or[kSelWaves];  // block_select_keys
    uint32_t small[4 * kWave];                        // block_select_keys: the last bin's keys
    uint32_t digit_hist[256];                         // block_select_bin: one histogram for the block
};

// Exclusive prefix over the block's threads of per-thread counts c0, c1 in
// [0, 7]; returns them and the block totals.
__device__ __forceinline__ void block_prefix2(int c0, int c1, int *p0, int *p1, int *t0, int *t1, BlockShared &sh)
{
    const int wv = threadIdx.x >> 6, l = threadIdx.x & 63;
    int w0, w1;
    const int e0 = lane_prefix(c0, &w0);
    const int e1 = lane_prefix(c1, &w1);
    if (l == 0) {
        sh.wave_sum[0][wv] = w0;
        sh.wave_sum[1][wv] = w1;
    }
    __syncthreads();
    // lane i < kSelWaves reads wave i's sums; sums over lanes 0..15 give
    // the waves below this one and all waves
    static_assert(kSelWaves == 16, "one DPP row of wave sums");
    const int i = l & (kSelWaves - 1);
    const uint32_t x0 = sh.wave_sum[0][i], x1 = sh.wave_sum[1][i];
    const int b0 = static_cast<int>(row0_sum(i < wv ? x0 : 0u)), b1 = static_cast<int>(row0_sum(i < wv ? x1 : 0u));
    const int s0 = static_cast<int>(row0_sum(x0)), s1 = static_cast<int>(row0_sum(x1));
    __syncthreads();
    *p0 = b0 + e0;
    *p1 = b1 + e1;
    *t0 = s0;
    *t1 = s1;
}

__device__ Sel block_select(const float *sc, int n, int K, BlockShared &sh)
{
    Sel r;
    if (n <= K) {
        r.all = true;
        r.kth = 0;
        r.quota = 0;
        return r;
    }
    r.all = false;
    const int tid = threadIdx.x, l = tid & 63;
    uint32_t prefix = 0, pmask = 0;
    uint32_t remaining = static_cast<uint32_t>(K);
    const int wv = tid >> 6;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < kSelWaves * 256; i += kSelThreads) (&sh.hist[0][0])[i] = 0u;
        __syncthreads();
        float vn[kVec];
        auto fetch = [&](int j0) {
#pragma unroll
            for (int e = 0; e < kVec; ++e) {
                const int j = j0 + kVec * tid + e;
                vn[e] = j < n ? sc[j] : 0.0f;
            }
        };
        fetch(0);
        for (int j0 = 0; j0 < n; j0 += kVec * kSelThreads) {
            float v[kVec];
#pragma unroll
            for (int e = 0; e < kVec; ++e) v[e] = vn[e];
            if (j0 + kVec * kSelThreads < n) fetch(j0 + kVec * kSelThreads);
#pragma unroll
            for (int e = 0; e < kVec; ++e)
                hist_add(j0 + kVec * tid + e < n, ord_key(v[e]), prefix, pmask, shift, sh.hist[wv], l);
        }
        __syncthreads();
        if (tid < 256) {  // fold the wave histograms into wave 0's
            uint32_t t = 0;
            for (int i = 0; i < kSelWaves; ++i) t += sh.hist[i][tid];
            sh.hist[0][tid] = t;
        }
        __syncthreads();
        if (tid < kWave) {
            const uint32_t c0 = sh.hist[0][4 * l], c1 = sh.hist[0][4 * l + 1], c2 = sh.hist[0][4 * l + 2],
                           c3 = sh.hist[0][4 * l + 3];
            const uint32_t tot = c0 + c1 + c2 + c3;
            const uint32_t suf = wave_suffix_sum(tot);
            const uint32_t above = suf - tot;
            if (above < remaining && remaining <= suf) {
                uint32_t cum = above, dig;
                if (cum + c3 >= remaining) {
                    dig = 4 * l + 3;
                } else {
                    cum += c3;
                    if (cum + c2 >= remaining) {
                        dig = 4 * l + 2;
                    } else {
                        cum += c2;
                        if (cum + c1 >= remaining) {
                            dig = 4 * l + 1;
                        } else {
                            cum += c1;
                            dig = 4 * l;
                        }
                    }
                }
                sh.bcast[0] = dig;
                sh.bcast[1] = cum;
            }
        }
        __syncthreads();
        const uint32_t dig = sh.bcast[0], abv = sh.bcast[1];
        remaining -= abv;
        prefix |= dig << shift;
        pmask |= 0xFFu << shift;
        __syncthreads();
    }
    r.kth = prefix;
    r.quota = static_cast<int>(remaining);
    return r;
}

// Block radix select over keys held in registers: thread tid holds the keys
// of entries j = e * kSelThreads + tid (e < kSelRegs), valid for j < n. The
// leading bits that every valid key shares (block AND / OR) are skipped, so
// the first digit already splits the keys; per 8-bit digit each wave counts
// its keys into its own 256-bin histogram (clearing it itself, so no atomics
// meet across waves) and wave 0 sums the 16 histograms and finds the digit:
// two barriers per digit. Digits are taken from the highest differing bit
// down; the last one may overlap the prefix (those bits agree already).
constexpr int kSelRegs = 16;  // keys per thread: rows of up to 16384 entries

__device__ __forceinline__ uint32_t wave_and(uint32_t v)
{
    v &= dpp_move<0x111>(v, ~0u);
    v &= dpp_move<0x112>(v, ~0u);
    v &= dpp_move<0x114>(v, ~0u);
    v &= dpp_move<0x118>(v, ~0u);
    v &= dpp_move<0x142, 0xA>(v, ~0u);
    v &= dpp_move<0x143, 0xC>(v, ~0u);
    return lane_value(v, kWave - 1);
}

__device__ __forceinline__ uint32_t wave_or(uint32_t v)
{
    v |= dpp_move<0x111>(v, 0u);
    v |= dpp_move<0x112>(v, 0u);
    v |= dpp_move<0x114>(v, 0u);
    v |= dpp_move<0x118>(v, 0u);
    v |= dpp_move<0x142, 0xA>(v, 0u);
    v |= dpp_move<0x143, 0xC>(v, 0u);
    return lane_value(v, kWave - 1);
}

// Generic form: N keys per thread, valid(e) this lane's key e is an entry,
// any(e) a wave-uniform "slot e may hold entries" (false skips the slot); n
// is the number of entries. Once the chosen digit's bin holds at most
// kSmall keys, they are compacted into LDS and wave 0 resolves the remaining
// bits by bisection over them (two barriers instead of further digits).
constexpr int kSmall = 4 * kWave;

template <int N, class Valid, class Any>
__device__ __forceinline__ Sel block_select_keys(const uint32_t (&key)[N], Valid &&valid, Any &&any, int n, int K, BlockShared &sh)
{
    Sel r;
    if (n <= K) {
        r.all = true;
        r.kth = 0;
        r.quota = 0;
        return r;
    }
    r.all = false;
    const int tid = threadIdx.x, l = tid & 63, wv = tid >> 6;
    // bits shared by every valid key
    uint32_t kand = ~0u, kor = 0u;
#pragma unroll
    for (int e = 0; e < N; ++e) {
        if (any(e)) {
            const bool in = valid(e);
            kand &= in ? key[e] : ~0u;
            kor |= in ? key[e] : 0u;
        }
    }
    kand = wave_and(kand);
    kor = wave_or(kor);
    if (l == 0) {
        sh.key_and[wv] = kand;
        sh.key_or[wv] = kor;
    }
    __syncthreads();
    {
        const int i = l & (kSelWaves - 1);
        kand = wave_and(sh.key_and[i]);
        kor = wave_or(sh.key_or[i]);
    }
    const uint32_t diff = kand ^ kor;
    if (diff == 0u) {  // every key equal: the first K of them
        __syncthreads();  // key_and / key_or read before a next call rewrites them
        r.kth = kand;
        r.quota = K;
        return r;
    }
    const int top = 31 - __builtin_clz(diff);  // highest differing bit
    uint32_t pmask = top == 31 ? 0u : ~((2u << top) - 1u);
    uint32_t prefix = kand & pmask;
    uint32_t remaining = static_cast<uint32_t>(K);
    uint32_t *own = sh.hist[wv];
    for (int sft = top - 7;; sft -= 8) {
        const int shift = sft > 0 ? sft : 0;
        for (int i = l; i < 256; i += kWave) own[i] = 0u;
        wave_fence();
#pragma unroll
        for (int e = 0; e < N; ++e)
            if (any(e)) hist_add_peel(valid(e), key[e], prefix, pmask, shift, own, l);
        __syncthreads();
        if (tid < kWave) {
            uint32_t c0 = 0, c1 = 0, c2 = 0, c3 = 0;
#pragma unroll
            for (int w = 0; w < kSelWaves; ++w) {
                const uint4 h = *reinterpret_cast<const uint4 *>(&sh.hist[w][4 * l]);
                c0 += h.x;
                c1 += h.y;
                c2 += h.z;
                c3 += h.w;
            }
            const uint32_t tot = c0 + c1 + c2 + c3;
            const uint32_t suf = wave_suffix_sum(tot);
            const uint32_t above = suf - tot;
            if (above < remaining && remaining <= suf) {
                uint32_t cum = above, dig, cnt;
                if (cum + c3 >= remaining) {
                    dig = 4 * l + 3, cnt = c3;
                } else {
                    cum += c3;
                    if (cum + c2 >= remaining) {
                        dig = 4 * l + 2, cnt = c2;
                    } else {
                        cum += c2;
                        if (cum + c1 >= remaining) {
                            dig = 4 * l + 1, cnt = c1;
                        } else {
                            cum += c1;
                            dig = 4 * l, cnt = c0;
                        }
                    }
                }
                sh.bcast[0] = dig;
                sh.bcast[1] = cum;
                sh.bcast[2] = cnt;
                sh.bcast[3] = 0u;  // compaction counter of the small path
            }
        }
        __syncthreads();
        remaining -= sh.bcast[1];
        prefix |= sh.bcast[0] << shift;
        pmask |= 0xFFu << shift;
        if (shift == 0) break;
        if (sh.bcast[2] <= static_cast<uint32_t>(kSmall)) {
            // few keys left in the bin: compact them, wave 0 bisects the
            // bits below this digit
#pragma unroll
            for (int e = 0; e < N; ++e) {
                if (any(e)) {
                    const bool m = valid(e) && (key[e] & pmask) == prefix;
                    const uint64_t mm = ballot(m);
                    if (mm != 0) {
                        const int first = __ffsll(static_cast<long long>(mm)) - 1;
                        uint32_t base = 0;
                        if (l == first) base = atomicAdd(&sh.bcast[3], static_cast<uint32_t>(popc(mm)));
                        base = lane_value(base, first);
                        if (m) sh.small[base + mbcnt(mm)] = key[e];
                    }
                }
            }
            __syncthreads();
            if (tid < kWave) {
                const int ns = static_cast<int>(sh.bcast[2]);
                uint32_t v[kSmall / kWave];
#pragma unroll
                for (int q = 0; q < kSmall / kWave; ++q) v[q] = kWave * q + l < ns ? sh.small[kWave * q + l] : 0u;
                auto count_ge_small = [&](uint32_t x) {
                    int c = 0;
#pragma unroll
                    for (int q = 0; q < kSmall / kWave; ++q) c += popc(ballot(v[q] >= x));
                    return c;
                };
                // the largest x with #{v >= x} >= remaining (bits below shift)
                uint32_t x = prefix;
                for (int bit = shift - 1; bit >= 0; --bit) {
                    const uint32_t t = x | (1u << bit);
                    if (count_ge_small(t) >= static_cast<int>(remaining)) x = t;
                }
                const int gt = x == 0xFFFFFFFFu ? 0 : count_ge_small(x + 1u);
                if (l == 0) {
                    sh.bcast[0] = x;
                    sh.bcast[1] = remaining - static_cast<uint32_t>(gt);
                }
            }
            __syncthreads();
            r.kth = sh.bcast[0];
            r.quota = static_cast<int>(sh.bcast[1]);
            __syncthreads();  // bcast read before a next call rewrites it
            return r;
        }
    }
    r.kth = prefix;
    r.quota = static_cast<int>(remaining);
    return r;
}

__device__ __forceinline__ Sel block_select_regs(const uint32_t (&key)[kSelRegs], int n, int K, BlockShared &sh)
{
    const int tid = threadIdx.x;
    return block_select_keys(
        key, [&](int e) { return e * kSelThreads + tid < n; }, [&](int e) { return e * kSelThreads < n; }, n, K, sh);
}

// Keys of entries j = e * kSelThreads + tid of sc[0, n) (n <= kSelRegs *
// kSelThreads); every load instruction reads 256 contiguous bytes per wave,
// and all of them are issued before the first key is formed.
template <int AS>
__device__ __forceinline__ void block_load_keys(const float *sc, int n, uint32_t (&key)[kSelRegs])
{
    const int tid = threadIdx.x;
    float x[kSelRegs];
#pragma unroll
    for (int e = 0; e < kSelRegs; ++e) {
        const int j = e * kSelThreads + tid;
        x[e] = e * kSelThreads < n ? load_as<AS>(sc, j < n ? j : n - 1) : 0.0f;
    }
#pragma unroll
    for (int e = 0; e < kSelRegs; ++e) key[e] = e * kSelThreads + tid < n ? ord_key(x[e]) : 0u;
}

// Walk sc[0..n) in order (AS: the address space of sc and pos) and call
// emit(slot, position, score) for every entry selected by s, where position
// is pos[j] (or j when pos is null); slots are dense and ascending. One
// block prefix per chunk counts both the entries above kth and those equal
// to it: an entry's slot is (entries above before it) + min(equal entries
// before it, quota).
template <int AS, class F>
__device__ __forceinline__ int block_emit(const float *sc, const int32_t *pos, int n, Sel s, BlockShared &sh, F &&emit)
{
    constexpr int CH = kVec * kSelThreads;
    const int tid = threadIdx.x;
    int ab_seen = 0, eq_seen = 0;
    // the next chunk's loads are issued before the current chunk is processed
    float vn[kVec];
    int32_t pn[kVec];
    auto fetch = [&](int j0) {
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            const int j = j0 + kVec * tid + e;
            const int jc = j < n ? j : n - 1;
            vn[e] = load_as<AS>(sc, jc);
            pn[e] = pos ? load_as<AS>(pos, jc) : j;
        }
    };
    if (n > 0) fetch(0);
    for (int j0 = 0; j0 < n; j0 += CH) {
        float v[kVec];
        int32_t p[kVec];
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            v[e] = vn[e];
            p[e] = pn[e];
        }
        if (j0 + CH < n) fetch(j0 + CH);
        bool ab[kVec], eq[kVec];
        int nab = 0, neq = 0;
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            const bool in = j0 + kVec * tid + e < n;
            const uint32_t key = ord_key(v[e]);
            ab[e] = in && (s.all || key > s.kth);
            eq[e] = in && !s.all && key == s.kth;
            nab += ab[e];
            neq += eq[e];
        }
        int pab, peq, tab, teq;
        block_prefix2(nab, neq, &pab, &peq, &tab, &teq, sh);
        int a_ = ab_seen + pab, q_ = eq_seen + peq;
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            if (ab[e]) {
                emit(a_ + (q_ < s.quota ? q_ : s.quota), p[e], v[e]);
                ++a_;
            } else if (eq[e]) {
                if (q_ < s.quota) emit(a_ + q_, p[e], v[e]);
                ++q_;
            }
        }
        ab_seen += tab;
        eq_seen += teq;
    }
    return ab_seen + (eq_seen < s.quota ? eq_seen : s.quota);
}

constexpr int kSurvivors = 12288;  // LDS capacity of the prefilter (entries)

// The fine bin holding the K-th largest of a row's scores, from the split
// scan's counts at h ([splits][kRowHistWords]: kRowHistBins fine counts,
// then kRowCoarseBins coarse ones): the coarse counts are summed over the
// splits (one 16-byte load per thread per 16 splits), wave 0 finds the
// coarse bin, then only its sixteen fine counts are read from every split.
// above: entries in higher bins; inbin: entries in the bin.
struct RowBin {
    bool found;
    uint32_t bin, above, inbin;
};

__device__ __forceinline__ RowBin row_bin(const uint32_t *h, int splits, int K, BlockShared &sh)
{
    static_assert(kRowCoarseBins == 4 * kWave && kSelThreads == 16 * kWave, "coarse layout: 4 bins per lane, 16 splits per pass");
    const int tid = threadIdx.x, l = tid & 63, wv = tid >> 6;
    uint32_t *flat = &sh.hist[0][0];
    // level 1: thread tid sums coarse bins 4 l .. 4 l + 3 of splits wv, wv + 16, ...
    uint4 c = {0u, 0u, 0u, 0u};
    for (int sp = wv; sp < splits; sp += kSelWaves) {
        const uint4 v = *reinterpret_cast<const uint4 *>(h + static_cast<int64_t>(sp) * kRowHistWords + kRowHistBins + 4 * l);
        c.x += v.x;
        c.y += v.y;
        c.z += v.z;
        c.w += v.w;
    }
    *reinterpret_cast<uint4 *>(flat + wv * kRowCoarseBins + 4 * l) = c;
    __syncthreads();
    if (wv == 0) {
        uint32_t c4[4] = {0u, 0u, 0u, 0u};
        for (int r = 0; r < kSelWaves; ++r) {
            const uint4 v = *reinterpret_cast<const uint4 *>(flat + r * kRowCoarseBins + 4 * l);
            c4[0] += v.x;
            c4[1] += v.y;
            c4[2] += v.z;
            c4[3] += v.w;
        }
        const uint32_t tot = c4[0] + c4[1] + c4[2] + c4[3];
        const uint32_t suf = wave_suffix_sum(tot);  // lanes l and above (higher bins)
        uint32_t above = suf - tot;
        const uint32_t Ku = static_cast<uint32_t>(K);
        if (l == 0) sh.bcast[3] = 0u;  // not found unless a lane finds it
        if (above < Ku && above + tot >= Ku) {
            int bsel = 3;
            while (above + c4[bsel] < Ku) above += c4[bsel--];
            sh.bcast[0] = static_cast<uint32_t>(4 * l + bsel);  // the coarse bin
            sh.bcast[1] = above;                                // entries in higher coarse bins
            sh.bcast[3] = 1u;
        }
    }
    __syncthreads();
    RowBin r{};
    r.found = sh.bcast[3] != 0u;
    if (!r.found) {
        __syncthreads();
        return r;
    }
    const uint32_t cb = sh.bcast[0];
    // level 2: the sixteen fine counts of the coarse bin, summed over the
    // splits (thread tid: fine bin tid % 16 of splits tid / 16, + 64, ...)
    uint32_t f = 0u;
    for (int sp = tid >> 4; sp < splits; sp += kSelThreads / 16)
        f += h[static_cast<int64_t>(sp) * kRowHistWords + 16 * cb + (tid & 15)];
    // the 64 partial sums of each fine bin: lanes of equal tid % 16 in a
    // wave hold the same bin, so four lanes add (two lane swaps), then wave
    // 0 adds the 16 waves' sums (lane i: bin i)
    f += __shfl_xor(f, 16);
    f += __shfl_xor(f, 32);
    __syncthreads();  // level 1's counts are read
    if (l < 16) flat[wv * 16 + l] = f;
    __syncthreads();
    if (wv == 0) {
        uint32_t fi = 0u;
        if (l < 16)
            for (int r2 = 0; r2 < kSelWaves; ++r2) fi += flat[16 * r2 + l];
        // lane i holds fine bin i; the bin where the count from above first
        // reaches K (bins above it: lanes above)
        const uint32_t suf = wave_suffix_sum(l < 16 ? fi : 0u);
        const uint32_t above = sh.bcast[1] + suf - fi;
        const uint32_t Ku = static_cast<uint32_t>(K);
        const bool here = l < 16 && above < Ku && (above + fi >= Ku || l == 0);
        const uint64_t hm = ballot(here);
        const int src = hm ? 63 - __clzll(static_cast<long long>(hm)) : 0;  // the highest such bin
        if (l == src) {
            sh.bcast[0] = 16 * cb + static_cast<uint32_t>(l);
            sh.bcast[1] = above;
            sh.bcast[2] = fi;
        }
    }
    __syncthreads();
    r.bin = sh.bcast[0];
    r.above = sh.bcast[1];
    r.inbin = sh.bcast[2];
    __syncthreads();  // bcast read before a next use rewrites it
    return r;
}

// The K-th largest of the n scores in sc (LDS), each at or above bin (the
// leading kRowHistBits bits of its order-preserving key), every one above
// the bin taken: a radix select over the remaining 20 key bits of the bin's
// keys (digits of 8, 8 and 4 bits) by the whole workgroup; per digit every
// thread counts its keys into one 256-bin LDS histogram and wave 0 picks
// the digit (three barriers per digit). The first digit's counts give the
// bin's size, hence the rank of the K-th largest within it. found: that
// rank lies in the bin (else the caller selects otherwise).
__device__ __forceinline__ Sel block_select_bin(const float *sc, int n, int K, uint32_t bin, BlockShared &sh,
                                                bool *found)
{
    const int tid = threadIdx.x, l = tid & 63;
    uint32_t *hist = sh.digit_hist;
    uint32_t prefix = bin << (32 - kRowHistBits), pmask = ~0u << (32 - kRowHistBits);
    int remaining = 0;
    Sel r;
    r.all = false;
    r.kth = 0u;
    r.quota = 0;
    for (int p = 0; p < 3; ++p) {
        const int shift = p == 0 ? 12 : (p == 1 ? 4 : 0);
        const uint32_t dmask = p == 2 ? 0xFu : 0xFFu;
        if (tid < 256) hist[tid] = 0u;
        __syncthreads();
        for (int j = tid; j < n; j += kSelThreads) {
            const uint32_t k = ord_key(load_as<kLds>(sc, j));
            if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & dmask], 1u);
        }
        __syncthreads();
        if (tid < kWave) {
            const uint32_t c0 = hist[4 * l], c1 = hist[4 * l + 1], c2 = hist[4 * l + 2], c3 = hist[4 * l + 3];
            const uint32_t tot = c0 + c1 + c2 + c3;
            const uint32_t suf = wave_suffix_sum(tot);
            int rem = remaining;
            if (p == 0) {
                // the bin holds suf(lane 0) keys; the n - that many above it are all taken
                const int nb = static_cast<int>(lane_value(suf, 0));
                rem = K - (n - nb);
                if (tid == 0) sh.bcast[2] = rem >= 1 && rem <= nb ? 1u : 0u;
            }
            const uint32_t ru = static_cast<uint32_t>(rem);
            const uint32_t above = suf - tot;
            if (rem >= 1 && above < ru && ru <= suf) {
                uint32_t cum = above, dig;
                if (cum + c3 >= ru) {
                    dig = 4 * l + 3;
                } else {
                    cum += c3;
                    if (cum + c2 >= ru) {
                        dig = 4 * l + 2;
                    } else {
                        cum += c2;
                        if (cum + c1 >= ru) {
                            dig = 4 * l + 1;
                        } else {
                            cum += c1;
                            dig = 4 * l;
                        }
                    }
                }
                sh.bcast[0] = dig;
                sh.bcast[1] = static_cast<uint32_t>(rem) - cum;  // remaining after this digit
            }
        }
        __syncthreads();
        if (sh.bcast[2] == 0u) {  // uniform: the rank is not in the bin
            __syncthreads();
            *found = false;
            return r;
        }
        remaining = static_cast<int>(sh.bcast[1]);
        prefix |= sh.bcast[0] << shift;
        pmask |= dmask << shift;
        __syncthreads();  // bcast read before the next digit rewrites it
    }
    *found = true;
    r.kth = prefix;
    r.quota = remaining;
    return r;
}

// Stable compaction of the entries of sc[0, n) whose score is above tau into
// out_v / out_p (score, position; LDS) in ascending position; returns their
// number (entries past cap are counted, not written). The row is read in
// segments of kSelWaves * 4096 entries, a whole segment in registers at once
// (wave w: entries 4096 w .. + 4096, sixteen 16-byte loads per lane), so a
// segment costs one memory latency. A float comparison: the kept set is
// {key > ord_key(tau)} (or {score > 0} when tau is -0), a threshold set either
// way.
__device__ __forceinline__ int block_filter_regs(const float *sc, int n, float tau, float *out_v, int32_t *out_p, int cap,
                                                 BlockShared &sh)
{
    constexpr int E = 16, PER_WAVE = E * 4 * kWave, SEG = kSelWaves * PER_WAVE;
    const int tid = threadIdx.x, l = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    // entries past n read as zero through the buffer's bounds and are
    // masked below. The bound is rounded up to whole 16-byte groups: the
    // rows are the split scan's [B*G, Lk] floats in the workspace, whose
    // regions are padded to 256 bytes, so the up to three floats read past
    // a row end (the next row's, or the padding after the last row) lie
    // inside the workspace.
    const __amdgpu_buffer_rsrc_t rs = row_buffer(sc, (n + 3) & ~3);
    int base = 0;
    for (int s0 = 0; s0 < n; s0 += SEG) {
        const int w0 = s0 + wv * PER_WAVE;  // wave-uniform
        uint32_t v[E][4];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * l, 4 * (w0 + e * 4 * kWave), 0);
            v[e][0] = x[0];
            v[e][1] = x[1];
            v[e][2] = x[2];
            v[e][3] = x[3];
        }
        // entry w0 + 256 e + 4 l + u is kept when 4 l + u < n - w0 - 256 e
        // (a wave-uniform bound per group, so no per-entry position is held)
        uint32_t km[E];  // kept sub-entries of each group (bits 0..3)
        uint32_t tot = 0u;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int lim = n - w0 - e * 4 * kWave;
            uint32_t m = 0u;
#pragma unroll
            for (int u = 0; u < 4; ++u) m |= (4 * l + u < lim && __uint_as_float(v[e][u]) > tau) ? (1u << u) : 0u;
            km[e] = m;
            tot += static_cast<uint32_t>(__builtin_popcount(m));
        }
        const uint32_t wt = wave_sum(tot);
        if (l == 0) sh.wave_sum[0][wv] = static_cast<int>(wt);
        __syncthreads();
        int woff = 0, stot = 0;
        for (int x = 0; x < kSelWaves; ++x) {
            const int c = sh.wave_sum[0][x];
            woff += x < wv ? c : 0;
            stot += c;
        }
        __syncthreads();  // wave_sum read before the next segment rewrites it
        int off = base + woff;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const uint32_t c = static_cast<uint32_t>(__builtin_popcount(km[e]));
            const uint32_t incl = wave_incl_sum(c);
            int slot = off + static_cast<int>(incl - c);
            const int g0 = w0 + e * 4 * kWave;  // wave-uniform
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if ((km[e] >> u) & 1u) {
                    if (slot < cap) {
                        store_as<kLds>(out_v, slot, __uint_as_float(v[e][u]));
                        store_as<kLds>(out_p, slot, g0 + 4 * l + u);
                    }
                    ++slot;
                }
            }
            off += static_cast<int>(lane_value(incl, kWave - 1));
        }
        base += stot;
    }
    __syncthreads();  // the compacted entries are visible to the block
    return base;
}

__global__ __launch_bounds__(kSelThreads) void k_select_rows(RowSelectArgs a)
{
    __shared__ BlockShared sh;
    __shared__ float sel_scores[kSurvivors];
    __shared__ int32_t sel_pos[kSurvivors];
    const Geo &geo = a.geo;
    const int tid = threadIdx.x;
    if (a.kind == 0) {
        const int64_t gid = blockIdx.x;
        const int64_t b = gid / geo.G, m = gid % geo.G;
        const int64_t tl1 = geo.t_last(b, m) + 1;
        int n = static_cast<int>(tl1 > 0 ? tl1 : 0);
        const float *row = a.rows + gid * geo.Lk;
        const int64_t r0 = geo.first_row(m), r1 = geo.end_row(m);
        const int64_t stride = a.out_stride;
        int32_t *ci = a.out_idx + gid * a.out_stride;
        float *cs = a.out_sc ? a.out_sc + gid * a.out_stride : nullptr;
        auto emit = [&](int slot, int32_t p, float v) {
            if (a.to_candidates) {
                ci[slot] = p;
                if (cs) cs[slot] = v;
            } else {
                for (int64_t r = r0; r < r1; ++r) {
                    a.out_idx[(b * geo.Lq + r) * stride + slot] = p;
                    if (a.out_sc) a.out_sc[(b * geo.Lq + r) * stride + slot] = v;
                }
            }
        };
        auto finish = [&](int got) {
            if (a.to_candidates) {
                for (int t = got + tid; t < a.out_stride; t += kSelThreads) {
                    ci[t] = -1;
                    if (cs) cs[t] = -INFINITY;
                }
                if (a.out_count && tid == 0) a.out_count[gid] = got;
                return;
            }
            for (int64_t r = r0; r < r1; ++r) {
                for (int t = got + tid; t < a.out_stride; t += kSelThreads) {
                    a.out_idx[(b * geo.Lq + r) * stride + t] = -1;
                    if (a.out_sc) a.out_sc[(b * geo.Lq + r) * stride + t] = -INFINITY;
                }
            }
        };

        // The split scan's counts of the row's scores by their leading key
        // bits give the bin holding the K-th largest score (coarse counts
        // first, then the chosen coarse bin's sixteen fine ones); the scores
        // at or above that bin are compacted into LDS, every one above the
        // bin is taken, and the exact select runs over the bin's keys alone.
        // Falls back to the full row when the survivors overflow LDS.
        bool in_lds = false, in_bin = false;
        uint32_t bin = 0u;
        if (n > 2 * a.K && a.hist) {
            const RowBin rb = row_bin(a.hist + gid * a.splits * kRowHistWords, a.splits, a.K, sh);
            if (rb.found && rb.above + rb.inbin <= static_cast<uint32_t>(kSurvivors) && rb.bin > 0u) {
                bin = rb.bin;
                // keys >= bin << 20, i.e. scores above the float of the key just below
                const float tau = key_float((bin << (32 - kRowHistBits)) - 1u);
                const int kept = block_filter_regs(row, n, tau, sel_scores, sel_pos, kSurvivors, sh);
                if (kept >= a.K && kept <= kSurvivors) {
                    n = kept;
                    in_lds = in_bin = true;
                }
            }
        }
        Sel s;
        bool have_s = false;
        if (in_bin) {
            // every kept key above the chosen bin is taken; the K-th
            // largest is found among the bin's keys
            bool found = false;
            s = block_select_bin(sel_scores, n, a.K, bin, sh, &found);
            have_s = found;
        }
        if (!have_s) {
            uint32_t key[kSelRegs];
            if (n <= kSelRegs * kSelThreads) {
                if (in_lds)
                    block_load_keys<kLds>(sel_scores, n, key);
                else
                    block_load_keys<kGlobal>(row, n, key);
                s = block_select_regs(key, n, a.K, sh);
            } else {
                s = block_select(row, n, a.K, sh);
            }
        }
        const int got = in_lds ? block_emit<kLds>(sel_scores, sel_pos, n, s, sh, emit)
                               : block_emit<kGlobal>(row, nullptr, n, s, sh, emit);
        finish(got);
        return;
    }
    // kind 1: member row = blockIdx.x over flat query rows
    const int64_t row = blockIdx.x;
    const int64_t b = row / geo.Lq, r = row % geo.Lq;
    const int64_t m = r / geo.g;
    const int64_t gid = b * geo.G + m;
    const int mi = static_cast<int>(r - geo.first_row(m));
    const int64_t t = geo.pos(b, r);
    const int nc = a.cand_n[gid];
    const int32_t *C = a.cand + gid * a.c;
    const float *sc = a.rows + (gid * geo.g + mi) * static_cast<int64_t>(a.c);
    int32_t *oi = a.out_idx + row * a.out_stride;
    float *os = a.out_sc ? a.out_sc + row * a.out_stride : nullptr;
    int got;
    if (a.c <= kVec * kSelThreads) {
        // the whole row in registers, entries 4 tid .. 4 tid + 3: loaded
        // once, counted, selected and emitted without another pass
        int32_t cp[kVec];
        float cv[kVec];
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            const int j = kVec * tid + e;
            const int jc = j < a.c ? j : a.c - 1;
            cp[e] = load_as<kGlobal>(C, jc);
            cv[e] = load_as<kGlobal>(sc, jc);
        }
        // candidates s <= t are a prefix of C (ascending): count them
        int cnt_le = 0;
#pragma unroll
        for (int e = 0; e < kVec; ++e) cnt_le += (kVec * tid + e < nc && cp[e] <= t) ? 1 : 0;
        cnt_le = static_cast<int>(wave_sum(static_cast<uint32_t>(cnt_le)));
        if ((tid & 63) == 0) sh.wave_sum[0][tid >> 6] = cnt_le;
        __syncthreads();
        const int nvalid =
            static_cast<int>(row0_sum(static_cast<uint32_t>(sh.wave_sum[0][tid & (kSelWaves - 1)])));
        __syncthreads();
        uint32_t key[kVec];
#pragma unroll
        for (int e = 0; e < kVec; ++e) key[e] = ord_key(cv[e]);
        const Sel s = block_select_keys(
            key, [&](int e) { return kVec * tid + e < nvalid; }, [](int) { return true; }, nvalid, a.K, sh);
        bool ab[kVec], eq[kVec];
        int nab = 0, neq = 0;
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            const bool in = kVec * tid + e < nvalid;
            ab[e] = in && (s.all || key[e] > s.kth);
            eq[e] = in && !s.all && key[e] == s.kth;
            nab += ab[e];
            neq += eq[e];
        }
        int pab, peq, tab, teq;
        block_prefix2(nab, neq, &pab, &peq, &tab, &teq, sh);
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            int slot = -1;
            if (ab[e]) slot = pab + (peq < s.quota ? peq : s.quota), ++pab;
            else if (eq[e]) slot = peq < s.quota ? pab + peq : -1, ++peq;
            if (slot >= 0) {
                oi[slot] = cp[e];
                if (os) os[slot] = cv[e];
            }
        }
        got = tab + (teq < s.quota ? teq : s.quota);
    } else {
        // candidates s <= t are a prefix of C (ascending): count them
        int cnt_le = 0;
        for (int j0 = 0; j0 < nc; j0 += kSelThreads) {
            const int j = j0 + tid;
            cnt_le += (j < nc && C[j] <= t) ? 1 : 0;
        }
        cnt_le = static_cast<int>(wave_sum(static_cast<uint32_t>(cnt_le)));
        if ((tid & 63) == 0) sh.wave_sum[0][tid >> 6] = cnt_le;
        __syncthreads();
        const int nvalid =
            static_cast<int>(row0_sum(static_cast<uint32_t>(sh.wave_sum[0][tid & (kSelWaves - 1)])));
        __syncthreads();
        Sel s;
        if (nvalid <= kSelRegs * kSelThreads) {
            uint32_t key[kSelRegs];
            block_load_keys<kGlobal>(sc, nvalid, key);
            s = block_select_regs(key, nvalid, a.K, sh);
        } else {
            s = block_select(sc, nvalid, a.K, sh);
        }
        got = block_emit<kGlobal>(sc, C, nvalid, s, sh, [&](int slot, int32_t p, float v) {
            oi[slot] = p;
            if (os) os[slot] = v;
        });
    }
    for (int x = got + tid; x < a.out_stride; x += kSelThreads) {
        oi[x] = -1;
        if (os) os[x] = -INFINITY;
    }
}

// ------------------------------------------------ member select (registers)
// Eq. (9) for the rows of the MFMA refine: one wave per query row. The
// member's re-scored candidates (at most 64 * NV of them) are held in
// registers, entry j = 64 i + lane in kv[i] (kv = ord_key of the score).
// The K-th largest key kth is found by bisection over the key bits: after
// each bit the bracket [T, T + 2^bit) that holds kth is known together with
// the number of keys inside it; once that number fits a small LDS buffer
// those keys are compacted there and the remaining bits are resolved over
// them alone, so the full register array is swept only for the leading
// bits. The chosen entries are written in ascending candidate order, which
// is ascending position because C is ascending.
struct MemberSelectArgs {
    Geo geo;
    int topk, c;
    const int32_t *cand;        // [B*G, c], ascending, -1 pad
    const int32_t *cand_n;      // [B*G] |C|; read only when row_nvalid is null
    const int32_t *row_nvalid;  // [B, Lq] entries of C at or before the row's position, or null:
                                // counted here from C
    const float *scores;        // [B*G, g, c] member scores over C, or [B*G, c] shared by the members
    int shared;                 // 1: one score row per group (member-causal Reuse)
    int32_t *out_idx;           // [B, Lq, topk]
    float *out_sc;              // nullable
};

constexpr int kMsWaves = 4;     // rows (one per wave) per workgroup
constexpr int kMsChunk = 16;    // slabs of positions loaded at a time
#ifndef PIVOT_HIST_BINS
#define PIVOT_HIST_BINS 512
#endif
constexpr int kHistBins = PIVOT_HIST_BINS;  // value-range bins of the one-pass histogram
static_assert(kHistBins % kWave == 0, "whole bins per lane");

// Wave-uniform max / min: the prefix-scan pattern of wave_incl_sum, read
// from the last lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    uint32_t t;
    t = dpp_move<0x111>(v, 0u), v = t > v ? t : v;
    t = dpp_move<0x112>(v, 0u), v = t > v ? t : v;
    t = dpp_move<0x114>(v, 0u), v = t > v ? t : v;
    t = dpp_move<0x118>(v, 0u), v = t > v ? t : v;
    t = dpp_move<0x142, 0xA>(v, 0u), v = t > v ? t : v;
    t = dpp_move<0x143, 0xC>(v, 0u), v = t > v ? t : v;
    return lane_value(v, kWave - 1);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v)
{
    constexpr uint32_t kTop = 0xFFFFFFFFu;
    uint32_t t;
    t = dpp_move<0x111>(v, kTop), v = t < v ? t : v;
    t = dpp_move<0x112>(v, kTop), v = t < v ? t : v;
    t = dpp_move<0x114>(v, kTop), v = t < v ? t : v;
    t = dpp_move<0x118>(v, kTop), v = t < v ? t : v;
    t = dpp_move<0x142, 0xA>(v, kTop), v = t < v ? t : v;
    t = dpp_move<0x143, 0xC>(v, kTop), v = t < v ? t : v;
    return lane_value(v, kWave - 1);
}

// The best K of n entries (score desc, then lower entry index), emitted in
// entry order. Entry j's score is the 32-bit float at byte 4 j of rs and its
// position the int32 at byte 4 j of rc (both raw buffers, so loads past
// their ends read 0 without a branch); n <= 64 NV. Keys (ord_key) sit in
// registers, 64 NV per wave; the K-th largest is found by bisection over the
// 32 key bits with wave-uniform counts (v_cmp + s_bcnt1). Once the bracket
// holding it has at most kMsMid keys they are compacted into `mid` (kMsMid
// words of LDS, wave-private) and the remaining bits are resolved over them
// alone. A bracket that stays crowded is checked every 8 bits for a single
// repeated key (many exact zeros), which ends the search. emit(slot,
// position, score) is called for every selected entry, slots dense and
// ascending; positions are loaded a chunk ahead. Returns the count.
// Slot passed for the entries not selected when the emitter drops
// out-of-range slots (its stores go through a buffer resource of the row).
constexpr int kNoSlot = 0x1FFFFFFF;  // times 4 bytes: past any row, still a positive int

// SKIP: rows often fill only part of the NV slabs (the scan's survivor
// buffers), so the passes stop at the last non-empty slab, checked once per
// kMsChunk slabs; full rows (member scores) leave the checks out.
template <int NV, bool DROPS = false, bool SKIP = false, class Emit>
__device__ __forceinline__ int wave_topk_emit(__amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t rc, int n, int K,
                                              uint32_t *mid, Emit &&emit)
{
    static_assert(NV >= 1 && NV <= 2 * kWave, "slab count");
    constexpr int CH = NV < kMsChunk ? NV : kMsChunk;
    static_assert(NV % CH == 0, "whole chunks");
    const int l = lane_id();
    // Keys: 0 marks an empty slot (every float maps to a key >= 0x007FFFFF).
    uint32_t kv[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) kv[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, (kWave * i + l) * 4, 0, 0);
#pragma unroll
    for (int i = 0; i < NV; ++i) kv[i] = l < n - kWave * i ? ord_key(__uint_as_float(kv[i])) : 0u;

    // selected: key > kth, plus the first `quota` keys equal to kth;
    // ties_all: every key equal to kth is selected
    uint32_t kth = 1u;
    int quota = 0;
    bool ties_all = true;
    if (n > K) {
        uint32_t T = 0;
        bool found = false;
        BinKth bin{};
        {
            // One pass into kHistBins bins of equal width 2^shift over the
            // keys' range [lo, hi] (LDS atomics) finds the bin holding the
            // K-th largest key and the count above it; that bin's keys are
            // compacted into `mid` and the key is resolved by bisection over
            // the bin's values. A bin too crowded (many equal keys) falls
            // back to the bisection over all keys below.
            // the smallest non-empty key: empty (0) wraps to the largest
            // value under key - 1, so one unsigned min covers both
            uint32_t lo1 = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                if (SKIP && i % kMsChunk == 0 && kWave * i >= n) break;
                lo1 = min(lo1, kv[i] - 1u);
                hi = max(hi, kv[i]);
            }
            uint32_t lo = wave_min_u32(lo1) + 1u;
            hi = wave_max_u32(hi);
            int shift = 0;
            while (((hi - lo) >> shift) >= static_cast<uint32_t>(kHistBins)) ++shift;
            uint32_t *hist = mid + kMsMid;
            for (int j = l; j < kHistBins; j += kWave) hist[j] = 0u;
            wave_fence();
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                if (SKIP && i % kMsChunk == 0 && kWave * i >= n) break;
                // empty slots count into this lane's spare word past the bins
                // (no branch around the atomic)
                atomicAdd(&hist[kv[i] != 0u ? (kv[i] - lo) >> shift : kHistBins + l], 1u);
            }
            wave_fence();
            // lane l holds bins BPL l .. BPL l + BPL - 1; suffix counts run
            // from the top bin
            constexpr int BPL = kHistBins / kWave;
            uint32_t cb[BPL];
            uint32_t tot = 0;
#pragma unroll
            for (int j = 0; j < BPL; ++j) {
                cb[j] = hist[BPL * l + j];
                tot += cb[j];
            }
            const uint32_t suf = wave_suffix_sum(tot);
            const uint32_t above_lane = suf - tot;
            const bool here = above_lane < static_cast<uint32_t>(K) && static_cast<uint32_t>(K) <= suf;
            const int src = __ffsll(static_cast<long long>(ballot(here))) - 1;
            int bb = 0;
            uint32_t abv = 0, cnt = 0;
            if (here) {
                // the highest of this lane's bins whose count reaches K
                uint32_t cum = above_lane;
                bool done = false;
#pragma unroll
                for (int j = BPL - 1; j >= 0; --j) {
                    if (!done && cum + cb[j] >= static_cast<uint32_t>(K)) {
                        bb = BPL * l + j;
                        cnt = cb[j];
                        abv = cum;
                        done = true;
                    }
                    if (!done) cum += cb[j];
                }
            }
            bb = static_cast<int>(lane_value(static_cast<uint32_t>(bb), src));
            abv = lane_value(abv, src);
            cnt = lane_value(cnt, src);
            wave_fence();
            if (cnt <= static_cast<uint32_t>(kMsMid)) {
                const uint32_t blo = lo + (static_cast<uint32_t>(bb) << shift);
                const uint32_t bw = (1u << shift) - 1u;
                const uint32_t bhi = hi - blo < bw ? hi : blo + bw;
                int nm = 0;
#pragma unroll
                for (int i = 0; i < NV; ++i) {
                    if (SKIP && i % kMsChunk == 0 && kWave * i >= n) break;
                    const bool in = kv[i] >= blo && kv[i] <= bhi;
                    const uint64_t im = ballot(in);
                    // lanes outside the bin write their spare word past the bins
                    mid[in ? nm + mbcnt(im) : kMsMid + kHistBins + l] = kv[i];
                    nm += popc(im);
                }
                wave_fence();
                // counted over as few registers as the bin needs
                bin = bisect_bin_any(mid, nm, blo, bhi, static_cast<int>(abv), K);
                T = bin.kth;
                found = true;
            }
            wave_fence();
        }
        // invariant: kth in [T, T + 2^bit); n_lo = #{key >= T} >= K,
        // n_hi = #{key >= T + 2^bit} < K
        int n_lo = n, n_hi = 0;
        int bit = found ? 0 : 32;
        while (bit > 0 && n_lo - n_hi > kMsMid) {
            --bit;
            const uint32_t x = T | (1u << bit);
            const int c = count_ge(kv, x);
            if (c >= K) {
                T = x;
                n_lo = c;
            } else {
                n_hi = c;
            }
            if ((bit & 7) == 0 && bit > 0 && n_lo - n_hi > kMsMid) {
                // a bracket that stays crowded may hold one repeated key
                // (e.g. many exact zeros): if its largest key has every
                // bracket key at or above it, that key is kth
                uint32_t top = 0;
#pragma unroll
                for (int i = 0; i < NV; ++i) {
                    const bool in = kv[i] != 0u && (kv[i] >> bit) == (T >> bit);
                    top = in && kv[i] > top ? kv[i] : top;
                }
                top = wave_max_u32(top);
                if (count_ge(kv, top) == n_lo) {
                    T = top;
                    bit = 0;
                }
            }
        }
        if (bit > 0) {
            // compact the keys of the bracket into LDS, then finish there
            int nm = 0;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const bool in = kv[i] != 0u && (bit == 32 || (kv[i] >> bit) == (T >> bit));
                const uint64_t im = ballot(in);
                if (in) mid[nm + mbcnt(im)] = kv[i];
                nm += popc(im);
            }
            wave_fence();
            uint32_t mv[kMsMid / kWave];
#pragma unroll
            for (int q = 0; q < kMsMid / kWave; ++q) {
                const int j = kWave * q + l;
                mv[q] = j < nm ? mid[j] : 0u;
            }
            // n_hi counts the keys above the compacted bracket
            while (bit > 0) {
                --bit;
                const uint32_t x = T | (1u << bit);
                if (n_hi + count_ge(mv, x) >= K) T = x;
            }
        }
        kth = T;
        // found in a bin: every key above the bin exceeds T, every key
        // below it is less, so the bin's counts are the row's
        const int n_gt = found ? bin.n_gt : (T == 0xFFFFFFFFu ? 0 : count_ge(kv, T + 1u));
        const int n_eq = found ? bin.n_eq : count_ge(kv, T) - n_gt;
        quota = K - n_gt;
        ties_all = quota == n_eq;
    }

    // ordered emission; the next chunk of positions is loaded while the
    // current one is written
    int out = 0, eq_seen = 0;
    int32_t cv[CH];
#pragma unroll
    for (int e = 0; e < CH; ++e) cv[e] = static_cast<int32_t>(__builtin_amdgcn_raw_buffer_load_b32(rc, (kWave * e + l) * 4, 0, 0));
#pragma unroll
    for (int i0 = 0; i0 < NV; i0 += CH) {
        if (kWave * i0 >= n) break;
        int32_t cn[CH];
        if (i0 + CH < NV) {
#pragma unroll
            for (int e = 0; e < CH; ++e)
                cn[e] = static_cast<int32_t>(
                    __builtin_amdgcn_raw_buffer_load_b32(rc, (kWave * (i0 + CH + e) + l) * 4, 0, 0));
        }
#pragma unroll
        for (int e = 0; e < CH; ++e) {
            const uint32_t key = kv[i0 + e];
            bool take = key >= kth;  // kth >= 1, so empty slots never qualify
            if (!ties_all) {
                const bool eq = key == kth;
                const uint64_t em = ballot(eq);
                const int rank = eq_seen + mbcnt(em);
                eq_seen += popc(em);
                take = key > kth || (eq && rank < quota);
            }
            const uint64_t tm = ballot(take);
            if constexpr (DROPS)
                emit(take ? out + mbcnt(tm) : kNoSlot, cv[e], key_float(key));
            else if (take)
                emit(out + mbcnt(tm), cv[e], key_float(key));
            out += popc(tm);
        }
        if (i0 + CH < NV) {
#pragma unroll
            for (int e = 0; e < CH; ++e) cv[e] = cn[e];
        }
    }
    return out;
}

template <int NV>
__global__ __launch_bounds__(kMsWaves * kWave) void k_select_members(MemberSelectArgs a)
{
    __shared__ uint32_t mid_all[kMsWaves][kMsMid + kHistBins + kWave];
    const Geo &geo = a.geo;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar row addressing
    const int l = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * kMsWaves + wv;
    if (row >= geo.B * geo.Lq) return;  // wave-uniform; the waves never synchronise
    const int64_t b = row / geo.Lq, r = row - b * geo.Lq;
    const int64_t m = r / geo.g;
    const int64_t gid = b * geo.G + m;
    const int mi = static_cast<int>(r - geo.first_row(m));
    const int32_t *C = a.cand + gid * a.c;
    const float *sc = a.scores + (a.shared ? gid : gid * geo.g + mi) * static_cast<int64_t>(a.c);

    // The candidates a member may take are the prefix of C at or before its
    // position (nvalid entries).
    int nvalid;
    if (a.row_nvalid) {
        nvalid = a.row_nvalid[row];
    } else {
        // the candidates s <= t are a prefix of C (ascending): the last
        // 64-entry slab whose first entry is <= t holds its end
        const int64_t t = geo.pos(b, r);
        const int nc = a.cand_n[gid];
        const int jh = kWave * l;
        const bool head = l < NV && jh < nc && C[jh] <= t;
        const int nh = popc(ballot(head));
        nvalid = 0;
        if (nh > 0) {
            const int j = kWave * (nh - 1) + l;
            nvalid = kWave * (nh - 1) + popc(ballot(j < nc && C[j] <= t));
        }
    }
    int32_t *oi = a.out_idx + row * a.topk;
    float *os = a.out_sc ? a.out_sc + row * a.topk : nullptr;
    // the row's outputs as buffer resources: a store is one offset, not a
    // 64-bit address computation
    const __amdgpu_buffer_rsrc_t ri = row_buffer(oi, a.topk), rsc = row_buffer(os, os ? a.topk : 0);
    const int out = wave_topk_emit<NV, true>(row_buffer(sc, a.c), row_buffer(C, a.c), nvalid, a.topk, mid_all[wv],
                                       [&](int slot, int32_t pos, float v) {
                                           __builtin_amdgcn_raw_buffer_store_b32(static_cast<uint32_t>(pos), ri,
                                                                                 slot * 4, 0, 0);
                                           if (os) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rsc,
                                                                                          slot * 4, 0, 0);
                                       });
    for (int x = out + l; x < a.topk; x += kWave) {
        oi[x] = -1;
        if (os) os[x] = -INFINITY;
    }
}

// Final selection of the fused scan's groups: one wave per group selects
// the best K of the group's survivor buffer (cnt entries in ascending
// position, written by k_scan_mfma) and writes the group's candidate set
// (Refine) or the row of every member (Reuse, dense). NV > 0: the register
// select above (cnt <= 64 NV); NV == 0: the streaming radix select over the
// buffer in global memory, for any size. Two waves per SIMD at least: at NV =
// 128 the compiler would otherwise take 269 registers (one wave per SIMD);
// capped at 256 it spills 13 loop-invariant values once (0.41 -> 0.25 ms at
// 128K Refine g=8; the same cap on the member select, four waves at 128
// registers, made it slower, 0.80 -> 0.86 ms).
struct GroupSelectArgs {
    Geo geo;
    int K, cap;
    const float *buf;     // [B*G][2*cap]: cap scores, then cap int32 positions
    const int32_t *cnt;   // [B*G] buffered entries
    SelectionOut out;
};

template <int NV>
__global__ __launch_bounds__(kMsWaves * kWave, 2) void k_select_groups(GroupSelectArgs a)
{
    __shared__ uint32_t lds[kMsWaves][NV > 0 ? kMsMid + kHistBins + kWave : 256];
    const Geo &geo = a.geo;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = threadIdx.x & 63;
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * kMsWaves + wv;
    if (gid >= geo.B * geo.G) return;  // wave-uniform; the waves never synchronise
    const int64_t b = gid / geo.G, m = gid - b * geo.G;
    const float *bs = a.buf + gid * 2 * static_cast<int64_t>(a.cap);
    const int32_t *bi = reinterpret_cast<const int32_t *>(bs + a.cap);
    const int n = a.cnt[gid];
    if (NV == 0) {
        Filter f;
        f.set_buffer(const_cast<float *>(bs), a.cap);
        f.K = a.K;
        f.cnt = n;
        f.tau = -INFINITY;
        f.hist = lds[wv];
        finish_group(geo, a.out, b, m, f);
        return;
    }
    const SelectionOut &o = a.out;
    const __amdgpu_buffer_rsrc_t rs = row_buffer(bs, n), rp = row_buffer(bi, n);
    if (o.to_candidates) {
        int32_t *ci = o.idx + gid * o.stride;
        float *cs = o.sc ? o.sc + gid * o.stride : nullptr;
        const __amdgpu_buffer_rsrc_t rci = row_buffer(ci, o.stride), rcs = row_buffer(cs, cs ? o.stride : 0);
        const int got = wave_topk_emit<(NV > 0 ? NV : 1), true, true>(rs, rp, n, a.K, lds[wv], [&](int slot, int32_t p, float v) {
            __builtin_amdgcn_raw_buffer_store_b32(static_cast<uint32_t>(p), rci, slot * 4, 0, 0);
            if (cs) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rcs, slot * 4, 0, 0);
        });
        for (int t = got + l; t < o.stride; t += kWave) {
            ci[t] = -1;
            if (cs) cs[t] = -INFINITY;
        }
        if (o.count && l == 0) o.count[gid] = got;
        return;
    }
    const int64_t r0 = geo.first_row(m), r1 = geo.end_row(m);
    const int64_t stride = o.stride;
    const int got = wave_topk_emit<(NV > 0 ? NV : 1), false, true>(rs, rp, n, a.K, lds[wv], [&](int slot, int32_t p, float v) {
        for (int64_t r = r0; r < r1; ++r) {
            const int64_t off = (b * geo.Lq + r) * stride + slot;
            o.idx[off] = p;
            if (o.sc) o.sc[off] = v;
        }
    });
    for (int64_t r = r0; r < r1; ++r) {
        for (int t = got + l; t < o.stride; t += kWave) {
            const int64_t off = (b * geo.Lq + r) * stride + t;
            o.idx[off] = -1;
            if (o.sc) o.sc[off] = -INFINITY;
        }
    }
}

// ------------------------------------------------- exact-order scan (any)
// One wave per group; lane l scores key base + l with the definition's exact
// fp32 order: for each head, dot = sum_i q_i k_i (one rounding per product
// and per sum, dims ascending); term = w * max(dot, 0); acc += term.
template <typename T>
__device__ __forceinline__ float exact_score(const T *__restrict__ qv, const float *__restrict__ wv,
                                             const T *__restrict__ key, int H, int D)
{
#pragma clang fp contract(off)  // one rounding per product and per sum: no fused multiply-add
    float acc = 0.0f;
    for (int j = 0; j < H; ++j) {
        float dot = 0.0f;
        for (int i = 0; i < D; ++i) {
            const float prod = widen<T>(qv[j * D + i]) * widen<T>(key[i]);
            dot = dot + prod;
        }
        const float relu = dot > 0.0f ? dot : 0.0f;
        const float term = wv[j] * relu;
        acc = acc + term;
    }
    if (acc == 0.0f) acc = 0.0f;
    return acc;
}

template <typename T, int Mode>
__global__ __launch_bounds__(256) void k_scan_exact(ScanArgs a)
{
    __shared__ uint32_t hist[4][256];
    const Geo &geo = a.geo;
    const int wv = threadIdx.x >> 6;
    const int l = threadIdx.x & 63;
    const int64_t nblk = (geo.G + 3) >> 2;
    const int64_t b = blockIdx.x % geo.B;
    const int64_t blk = nblk - 1 - blockIdx.x / geo.B;
    const int64_t m = blk * 4 + wv;
    if (m >= geo.G) return;  // no workgroup barriers below
    const int64_t tl = geo.t_last(b, m);
    const int64_t gid = b * geo.G + m;
    const T *qv = static_cast<const T *>(a.qsrc) + gid * a.H * a.D;
    const float *wv_ = a.wsrc + gid * a.H;
    const T *kbase = static_cast<const T *>(a.keys.base);

    Filter f;
    f.K = a.K;
    f.cap = a.cap;
    f.cnt = 0;
    f.tau = -INFINITY;
    f.hist = hist[wv];
    if (Mode == kFilter) f.set_buffer(a.buf_s + gid * 2 * static_cast<int64_t>(a.cap), a.cap);  // [cap scores | cap positions]
    float *row = (Mode == kRows) ? a.rows + gid * geo.Lk : nullptr;

    for (int64_t base = 0; base <= tl; base += kWave) {
        const int64_t s = base + l;
        const bool valid = s <= tl;
        const float score = valid ? exact_score<T>(qv, wv_, kbase + a.keys.row(b, s) * a.D, a.H, a.D) : 0.0f;
        if (Mode == kFilter) {
            f.push(valid, score, static_cast<int32_t>(s));
        } else if (valid) {
            row[s] = score;
        }
    }
    if (Mode == kFilter) {
        finish_group(geo, a.out, b, m, f);
    } else {
        for (int64_t s = tl + 1 + l; s < geo.Lk; s += kWave) row[s] = -INFINITY;
    }
}

// --------------------------------------------------------------- refine
struct RefineArgs {
    const void *q;   // [B, Lq, H, D]
    const float *w;  // [B, Lq, H]
    Keys keys;       // [B, Lk, D] contiguous, or paged
    Geo geo;
    int H, D;
    int topk, c;
    const int32_t *cand;    // [B*G, c], ascending, -1 pad
    const int32_t *cand_n;  // [B*G]
    float *scratch;         // [B*G, g, c]
    int32_t *out_idx;       // [B, Lq, topk]
    float *out_sc;          // nullable
    int splits;             // > 1: workgroup (gid, split) scores one slice of C
    int finish;             // select each member's top-k in this kernel (splits == 1 only);
                            // otherwise k_select_members / k_select_rows does it
    int32_t *row_nvalid;    // [B, Lq], nullable (splits == 1): #{j : C[j] <= t} per row
};

// Member selection from its scratch row; candidates s <= t are exactly the
// first nvalid entries of C (C is ascending).
__device__ void finish_member(const RefineArgs &a, int64_t b, int64_t r, const int32_t *C, const float *srow,
                              int nvalid, uint32_t *hist)
{
    wave_fence();
    const Sel s = wave_select(srow, nvalid, a.topk, hist);
    const int l = lane_id();
    int32_t *oi = a.out_idx + (b * a.geo.Lq + r) * a.topk;
    float *os = a.out_sc ? a.out_sc + (b * a.geo.Lq + r) * a.topk : nullptr;
    const int n = wave_emit(srow, C, nvalid, s, [&](int slot, int32_t p, float v) {
        oi[slot] = p;
        if (os) os[slot] = v;
    });
    for (int t = n + l; t < a.topk; t += kWave) {
        oi[t] = -1;
        if (os) os[t] = -INFINITY;
    }
}

// Number of entries of the ascending list C[0..n) at or below t (one wave;
// a ballot over 64 slab heads per step finds the slab holding the end).
__device__ __forceinline__ int prefix_le(const int32_t *C, int n, int64_t t)
{
    const int l = lane_id();
    int done = 0;
    for (int s0 = 0; s0 < n; s0 += kWave * kWave) {
        const int jh = s0 + kWave * l;
        const int nh = popc(ballot(jh < n && C[jh] <= t));
        if (nh == 0) break;
        const int j = s0 + kWave * (nh - 1) + l;
        const int last = kWave * (nh - 1) + popc(ballot(j < n && C[j] <= t));
        done = s0 + last;
        if (nh < kWave) break;
    }
    return done;
}

// Candidates per refine tile (two tiles in LDS: 2 x 32 KiB at 128).
#ifndef PIVOT_REFINE_TILE
#define PIVOT_REFINE_TILE 128
#endif
constexpr int kRefineTile = PIVOT_REFINE_TILE;
static_assert(kRefineTile % 64 == 0, "whole 64-candidate quarters");

// XCD-aware order: workgroups are dealt round-robin to the 8 XCDs, so
// workgroup i is given unit (i % 8) * (n / 8) + i / 8 and each XCD's L2
// serves a contiguous run of units (the tail beyond a multiple of 8 keeps
// its index).
__device__ __forceinline__ int64_t xcd_unit(int64_t i, int64_t n)
{
    constexpr int kXcds = 8;
    const int64_t full = n / kXcds * kXcds;
    if (i >= full) return i;
    return (i % kXcds) * (n / kXcds) + i / kXcds;
}

// One workgroup of NW waves (4 or 8) per group (or per slice of C when
// splits > 1); wave w re-scores member (round * NW + w), and a wave without
// a member in the last round only helps gather. Each 128-candidate tile of
// key rows is gathered once into LDS (global_load_lds, the scan's swizzle)
// and shared by every member wave; candidate positions are prefetched a tile
// ahead, and the scoring is the scan's pipelined tile_step. Groups are
// ordered per XCD, so neighbouring groups (whose candidate sets overlap)
// share an L2.
template <int H, int D, int NW, bool PAGED>
__global__ __launch_bounds__(NW * 64) void k_refine_mfma(RefineArgs a)
{
    static_assert(H % 16 == 0 && D == 128, "tile layout assumes 128-dim keys (16 chunks of 8 bf16 per row)");
    constexpr int RB = H / 16;
    constexpr int NT = kRefineTile;            // candidates per tile
    constexpr int NQ = NT / kWave;             // 64-candidate quarters per tile
    constexpr int kSlices = NT * D * 2 / 1024; // 1 KiB slices per tile (32)
    constexpr int kMaxSlices = kSlices / NW;   // per wave
    static_assert(kSlices % NW == 0, "each wave gathers the same number of slices");

    __shared__ __attribute__((aligned(1024))) uint16_t tile0[NT * D];
    __shared__ __attribute__((aligned(1024))) uint16_t tile1[NT * D];
    __shared__ uint32_t hist[8][256];

    const Geo &geo = a.geo;
    constexpr int nwaves = NW;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = threadIdx.x & 63;
    const int64_t unit = xcd_unit(blockIdx.x, static_cast<int64_t>(gridDim.x));
    const int64_t gid = unit / a.splits;
    const int split = static_cast<int>(unit % a.splits);
    const int64_t b = gid / geo.G, m = gid % geo.G;
    const int64_t r0 = geo.first_row(m), r1 = geo.end_row(m);
    const int gm = static_cast<int>(r1 - r0);
    const int nc = a.cand_n[gid];
    const int32_t *C = a.cand + gid * a.c;
    const uint16_t *kbase = static_cast<const uint16_t *>(a.keys.base);
    // this workgroup's tiles of C: [tile_lo, tile_hi)
    const int ntiles_all = (nc + NT - 1) / NT;
    if (ntiles_all == 0) {
        // an empty C (every member precedes its sequence's keys): each
        // member row still gets its causal count (0) or its -1 padding
        if (split == 0) {
            for (int mi = wv; mi < gm; mi += nwaves) {
                const int64_t r = r0 + mi;
                if (a.row_nvalid && l == 0) a.row_nvalid[b * geo.Lq + r] = 0;
                if (a.finish) finish_member(a, b, r, C, a.scratch + (gid * geo.g + mi) * a.c, 0, hist[wv]);
            }
        }
        return;  // uniform over the workgroup
    }
    const int per_split = (ntiles_all + a.splits - 1) / a.splits;
    const int tile_lo = split * per_split;
    const int tile_hi = tile_lo + per_split < ntiles_all ? tile_lo + per_split : ntiles_all;
    if (tile_lo >= tile_hi) return;  // uniform over the workgroup
    const int ntiles = tile_hi - tile_lo;

    // positions of the key rows this lane gathers for a tile (slices
    // wv + nwaves j, tile rows slice_row(slice, l)), loaded a tile ahead and
    // consumed raw by the DMA issue, so the loads never stall the MFMAs.
    // Paged keys add a step: positions are loaded two tiles ahead, and one
    // tile ahead become page offsets plus table entries (loaded), which the
    // issue combines; every array is written once per tile, so no loaded
    // value is copied (a copy would wait for the loads in flight).
    auto load_pos = [&](int tile_idx, int32_t (&pos)[kMaxSlices]) {
#pragma unroll
        for (int j = 0; j < kMaxSlices; ++j) {
            const int cj = tile_idx * NT + slice_row(wv + nwaves * j, l);
            pos[j] = cj < nc ? C[cj] : 0;  // row 0: any valid key (masked)
        }
    };
    auto load_entries = [&](const int32_t (&pos)[kMaxSlices], int32_t (&off)[kMaxSlices],
                            int32_t (&ent)[kMaxSlices]) {
        if constexpr (PAGED) {
#pragma unroll
            for (int j = 0; j < kMaxSlices; ++j) {
                const uint32_t sp = static_cast<uint32_t>(pos[j]);
                off[j] = static_cast<int32_t>(a.keys.page_offset(sp));
                // computed here, not sunk below the reload of pos (which
                // would then need other registers and a waited copy)
                asm volatile("" : "+v"(off[j]));
                ent[j] = a.keys.entry(b, sp);
            }
        }
    };
    // key = positions (contiguous) or page offsets (paged)
    auto issue_tile = [&](int buf, const int32_t (&key)[kMaxSlices], const int32_t (&ent)[kMaxSlices]) {
        uint16_t *dst = buf ? tile1 : tile0;
#pragma unroll
        for (int j = 0; j < kMaxSlices; ++j) {
            const int slice = wv + nwaves * j;
            const int64_t r = PAGED ? a.keys.paged_row(ent[j], static_cast<uint32_t>(key[j])) : a.keys.flat(b, key[j]);
            const uint16_t *src = kbase + r * D + slice_col(slice, l);
            __builtin_amdgcn_global_load_lds((global_cptr)src, (lds_ptr)(dst + slice * 512), 16, 0, 0);
        }
    };

    for (int round = 0; round * nwaves < gm; ++round) {
        const int mi = round * nwaves + wv;
        const bool active = mi < gm;
        const int64_t r = r0 + (active ? mi : 0);
        const int64_t t = geo.pos(b, r);
        float *srow = a.scratch + (gid * geo.g + (active ? mi : 0)) * a.c;

        bf16x8 afr[RB][4];
        float wr[RB][4];
        load_a<H>(static_cast<const uint16_t *>(a.q) + (b * geo.Lq + r) * H * D, l, afr);
        load_w<H>(a.w + (b * geo.Lq + r) * H, l, wr);

        int32_t pos[kMaxSlices], off[kMaxSlices] = {}, ent[kMaxSlices] = {};
        load_pos(tile_lo, pos);
        if constexpr (PAGED) {
            load_entries(pos, off, ent);
            issue_tile(0, off, ent);
            if (ntiles > 1) {
                load_pos(tile_lo + 1, pos);
                load_entries(pos, off, ent);
            }
            if (ntiles > 2) load_pos(tile_lo + 2, pos);
        } else {
            issue_tile(0, pos, ent);
            if (ntiles > 1) load_pos(tile_lo + 1, pos);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        tile_barrier();

        f32x4 carry[RB];
        float pc[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) carry[rb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        auto store = [&](int tile_idx, int qt, float score) {
            const int j = tile_idx * NT + qt * kWave + l;
            if (active && j < nc) srow[j] = score;
        };
        for (int it = 0; it < ntiles; ++it) {
            const int cur = it & 1;
            // the buffer of tile it + 1 held tile it - 1, which every wave
            // finished reading before the last barrier
            if (it + 1 < ntiles) {
                if constexpr (PAGED) {
                    issue_tile(cur ^ 1, off, ent);
                    if (it + 2 < ntiles) {
                        load_entries(pos, off, ent);
                        // the positions are read before they are reloaded
                        __builtin_amdgcn_sched_barrier(0);
                        if (it + 3 < ntiles) load_pos(tile_lo + it + 3, pos);
                    }
                } else {
                    issue_tile(cur ^ 1, pos, ent);
                    if (it + 2 < ntiles) load_pos(tile_lo + it + 2, pos);
                }
            }
            const int ti = tile_lo + it;
            auto emit = [&](int qt, float score) {
                if (qt < 0)
                    store(ti - 1, NQ - 1, score);
                else
                    store(ti, qt, score);
            };
            if (!active) {
            } else if (cur == 0) {
                tile_step<RB, NT / 16>(afr, wr, tile0, l, carry, pc, it > 0, emit);
            } else {
                tile_step<RB, NT / 16>(afr, wr, tile1, l, carry, pc, it > 0, emit);
            }
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next tile is in LDS
            tile_barrier();
        }
        if (active) {
            const float q4[4] = {pc[0], pc[1], pc[2], relu_weighted<RB>(carry, wr)};
            store(tile_hi - 1, NQ - 1, quarter_transpose_sum(q4));
        }
        if (active && (a.row_nvalid || a.finish)) {
            const int nvalid = prefix_le(C, nc, t);
            if (a.row_nvalid && l == 0) a.row_nvalid[b * geo.Lq + r] = nvalid;
            if (a.finish) finish_member(a, b, r, C, srow, nvalid, hist[wv]);
        }
    }
}

// Exact-order refine: one workgroup of 4 waves per group; lane l scores
// candidate tile*64 + l for the wave's member.
template <typename T>
__global__ __launch_bounds__(256) void k_refine_exact(RefineArgs a)
{
    __shared__ uint32_t hist[4][256];
    const Geo &geo = a.geo;
    const int wv = threadIdx.x >> 6;
    const int l = threadIdx.x & 63;
    const int64_t gid = blockIdx.x;
    const int64_t b = gid / geo.G, m = gid % geo.G;
    const int64_t r0 = geo.first_row(m), r1 = geo.end_row(m);
    const int gm = static_cast<int>(r1 - r0);
    const int nc = a.cand_n[gid];
    const int32_t *C = a.cand + gid * a.c;
    const T *kbase = static_cast<const T *>(a.keys.base);
    for (int mi = wv; mi < gm; mi += 4) {
        const int64_t r = r0 + mi;
        const int64_t t = geo.pos(b, r);
        const T *qv = static_cast<const T *>(a.q) + (b * geo.Lq + r) * a.H * a.D;
        const float *wv_ = a.w + (b * geo.Lq + r) * a.H;
        float *srow = a.scratch + (gid * geo.g + mi) * a.c;
        int nvalid = 0;
        for (int jb = 0; jb < nc; jb += kWave) {
            const int j = jb + l;
            const bool in = j < nc;
            const int32_t pos = in ? C[j] : 0;
            if (in) srow[j] = exact_score<T>(qv, wv_, kbase + a.keys.row(b, pos) * a.D, a.H, a.D);
            nvalid += popc(ballot(in && pos <= t));
        }
        finish_member(a, b, r, C, srow, nvalid, hist[wv]);
    }
}

}  // namespace

// --------------------------------------------------------------- launchers
hipError_t launch_pool(const LaunchShape &sh, int g, int64_t G, const void *q, const float *w, void *qbar,
                       float *wbar, int agg, hipStream_t st)
{
    hipError_t e = hipSuccess;
    Geo geo{sh.B, G, sh.Lq, sh.Lk, g, sh.lens};
    const int vec = sh.bf16 ? 8 : 4;
    const int64_t total = sh.B * G * sh.H * (sh.D / vec);
    const int64_t blocks = (total + 255) / 256;
    if (sh.bf16) {
        e = launch(&k_pool<uint16_t>, dim3(static_cast<uint32_t>(blocks)), dim3(256), st, static_cast<const uint16_t *>(q), w, static_cast<uint16_t *>(qbar), wbar, geo, sh.H, sh.D, agg);
    } else {
        e = launch(&k_pool<float>, dim3(static_cast<uint32_t>(blocks)), dim3(256), st, static_cast<const float *>(q), w, static_cast<float *>(qbar), wbar, geo, sh.H, sh.D, agg);
    }
    return e;
}

bool mfma_shape(const LaunchShape &sh) { return sh.bf16 && (sh.H == 32 || sh.H == 64) && sh.D == 128; }

hipError_t launch_scan(const LaunchShape &sh, const ScanLaunch &L, hipStream_t st)
{
    hipError_t e = hipSuccess;
    ScanArgs a{};
    a.qsrc = L.qsrc;
    a.wsrc = L.wsrc;
    a.keys = Keys{L.k, sh.pages, sh.Lk};
    a.geo = Geo{sh.B, L.G, sh.Lq, sh.Lk, L.g, sh.lens};
    a.H = sh.H;
    a.D = sh.D;
    a.K = L.K;
    a.cap = L.cap;
    a.buf_s = L.buf;
    a.buf_n = L.buf_n;
    a.smp = L.smp;
    a.pool_inline = L.pool_inline;
    a.agg = L.agg;
    a.out = SelectionOut{L.out_idx, L.out_sc, L.out_count, L.out_stride, L.to_candidates};
    a.rows = L.rows;
    const int64_t blocks = sh.B * ((L.G + 3) / 4);
    const dim3 grid(static_cast<uint32_t>(blocks)), block(256);
    const bool rows = L.rows != nullptr;
    if (mfma_shape(sh)) {
        const dim3 mgrid(static_cast<uint32_t>(sh.B * ((L.G + kScanWaves - 1) / kScanWaves)));
        const dim3 mblock(kScanWaves * 64);
        const bool paged = sh.pages.table != nullptr;
        if (sh.H == 64) {
            if (rows && paged)
                e = launch(&k_scan_mfma<64, 128, kRows, true>, mgrid, mblock, st, a);
            else if (rows)
                e = launch(&k_scan_mfma<64, 128, kRows, false>, mgrid, mblock, st, a);
            else if (paged)
                e = launch(&k_scan_mfma<64, 128, kFilter, true>, mgrid, mblock, st, a);
            else
                e = launch(&k_scan_mfma<64, 128, kFilter, false>, mgrid, mblock, st, a);
        } else {
            if (rows && paged)
                e = launch(&k_scan_mfma<32, 128, kRows, true>, mgrid, mblock, st, a);
            else if (rows)
                e = launch(&k_scan_mfma<32, 128, kRows, false>, mgrid, mblock, st, a);
            else if (paged)
                e = launch(&k_scan_mfma<32, 128, kFilter, true>, mgrid, mblock, st, a);
            else
                e = launch(&k_scan_mfma<32, 128, kFilter, false>, mgrid, mblock, st, a);
        }
    } else if (sh.bf16) {
        if (rows)
            e = launch(&k_scan_exact<uint16_t, kRows>, grid, block, st, a);
        else
            e = launch(&k_scan_exact<uint16_t, kFilter>, grid, block, st, a);
    } else {
        if (rows)
            e = launch(&k_scan_exact<float, kRows>, grid, block, st, a);
        else
            e = launch(&k_scan_exact<float, kFilter>, grid, block, st, a);
    }
    return e;
}

hipError_t launch_refine(const LaunchShape &sh, const RefineLaunch &L, hipStream_t st)
{
    hipError_t e = hipSuccess;
    RefineArgs a{};
    a.q = L.q;
    a.w = L.w;
    a.keys = Keys{L.k, sh.pages, sh.Lk};
    a.geo = Geo{sh.B, L.G, sh.Lq, sh.Lk, L.g, sh.lens};
    a.H = sh.H;
    a.D = sh.D;
    a.topk = L.topk;
    a.c = L.c;
    a.cand = L.cand;
    a.cand_n = L.cand_n;
    a.scratch = L.scratch;
    a.out_idx = L.out_idx;
    a.out_sc = L.out_sc;
    a.splits = L.splits > 1 ? L.splits : 1;
    a.finish = a.splits == 1 && L.finish;
    a.row_nvalid = a.splits == 1 ? L.row_nvalid : nullptr;
    const dim3 grid(static_cast<uint32_t>(sh.B * L.G * a.splits));
    if (mfma_shape(sh)) {
        // 4 or 8 member waves; more members loop in rounds
        const bool paged = sh.pages.table != nullptr;
        if (sh.H == 64) {
            if (L.g <= 4 && paged)
                e = launch(&k_refine_mfma<64, 128, 4, true>, grid, dim3(64 * 4), st, a);
            else if (L.g <= 4)
                e = launch(&k_refine_mfma<64, 128, 4, false>, grid, dim3(64 * 4), st, a);
            else if (paged)
                e = launch(&k_refine_mfma<64, 128, 8, true>, grid, dim3(64 * 8), st, a);
            else
                e = launch(&k_refine_mfma<64, 128, 8, false>, grid, dim3(64 * 8), st, a);
        } else {
            if (L.g <= 4 && paged)
                e = launch(&k_refine_mfma<32, 128, 4, true>, grid, dim3(64 * 4), st, a);
            else if (L.g <= 4)
                e = launch(&k_refine_mfma<32, 128, 4, false>, grid, dim3(64 * 4), st, a);
            else if (paged)
                e = launch(&k_refine_mfma<32, 128, 8, true>, grid, dim3(64 * 8), st, a);
            else
                e = launch(&k_refine_mfma<32, 128, 8, false>, grid, dim3(64 * 8), st, a);
        }
    } else if (sh.bf16) {
        e = launch(&k_refine_exact<uint16_t>, grid, dim3(256), st, a);
    } else {
        e = launch(&k_refine_exact<float>, grid, dim3(256), st, a);
    }
    return e;
}

}  // namespace pivot

namespace pivot {

hipError_t launch_scan_split(const LaunchShape &sh, const ScanLaunch &L, int splits, hipStream_t st)
{
    hipError_t e = hipSuccess;
    if (!mfma_shape(sh) || !L.rows || splits < 1) return hipErrorInvalidValue;
    ScanArgs a{};
    a.qsrc = L.qsrc;
    a.wsrc = L.wsrc;
    a.keys = Keys{L.k, sh.pages, sh.Lk};
    a.geo = Geo{sh.B, L.G, sh.Lq, sh.Lk, L.g, sh.lens};
    a.H = sh.H;
    a.D = sh.D;
    a.pool_inline = L.pool_inline;
    a.agg = L.agg;
    a.rows = L.rows;
    a.hist = L.hist;
    const dim3 grid(static_cast<uint32_t>(sh.B * L.G * splits));
    if (sh.H == 64 && sh.pages.table)
        e = launch(&k_scan_split<64, 128, true>, grid, dim3(kSplitWaves * 64), st, a, splits);
    else if (sh.H == 64)
        e = launch(&k_scan_split<64, 128, false>, grid, dim3(kSplitWaves * 64), st, a, splits);
    else if (sh.pages.table)
        e = launch(&k_scan_split<32, 128, true>, grid, dim3(kSplitWaves * 64), st, a, splits);
    else
        e = launch(&k_scan_split<32, 128, false>, grid, dim3(kSplitWaves * 64), st, a, splits);
    return e;
}

int scan_sample_slots() { return kSampleSlots; }
int row_hist_bins() { return kRowHistWords; }
int refine_tile() { return kRefineTile; }

int group_select_slabs(int cap)
{
    for (int nv : {8, 16, 32, 64, 128})
        if (cap <= kWave * nv) return nv;
    return 0;
}

hipError_t launch_select_groups(const LaunchShape &sh, const ScanLaunch &L, hipStream_t st)
{
    hipError_t e = hipSuccess;
    if (!mfma_shape(sh) || L.rows || !L.buf_n) return hipErrorInvalidValue;
    GroupSelectArgs a{};
    a.geo = Geo{sh.B, L.G, sh.Lq, sh.Lk, L.g, sh.lens};
    a.K = L.K;
    a.cap = L.cap;
    a.buf = L.buf;
    a.cnt = L.buf_n;
    a.out = SelectionOut{L.out_idx, L.out_sc, L.out_count, L.out_stride, L.to_candidates};
    const dim3 grid(static_cast<uint32_t>((sh.B * L.G + kMsWaves - 1) / kMsWaves)), block(kMsWaves * kWave);
    switch (group_select_slabs(L.cap)) {
    case 8: e = launch(&k_select_groups<8>, grid, block, st, a); break;
    case 16: e = launch(&k_select_groups<16>, grid, block, st, a); break;
    case 32: e = launch(&k_select_groups<32>, grid, block, st, a); break;
    case 64: e = launch(&k_select_groups<64>, grid, block, st, a); break;
    case 128: e = launch(&k_select_groups<128>, grid, block, st, a); break;
    default: e = launch(&k_select_groups<0>, grid, block, st, a); break;
    }
    return e;
}

int member_select_slabs(int c)
{
    for (int nv : {8, 16, 32, 64})
        if (c <= kWave * nv) return nv;
    return 0;
}

hipError_t launch_select_members(const LaunchShape &sh, const MemberSelectLaunch &L, hipStream_t st)
{
    hipError_t e = hipSuccess;
    MemberSelectArgs a{};
    a.geo = Geo{sh.B, L.G, sh.Lq, sh.Lk, L.g, sh.lens};
    a.topk = L.topk;
    a.c = L.c;
    a.cand = L.cand;
    a.cand_n = L.cand_n;
    a.row_nvalid = L.row_nvalid;
    a.scores = L.scores;
    a.shared = L.shared;
    a.out_idx = L.out_idx;
    a.out_sc = L.out_sc;
    const int64_t rows = sh.B * sh.Lq;
    const dim3 grid(static_cast<uint32_t>((rows + kMsWaves - 1) / kMsWaves)), block(kMsWaves * kWave);
    switch (member_select_slabs(L.c)) {
    case 8: e = launch(&k_select_members<8>, grid, block, st, a); break;
    case 16: e = launch(&k_select_members<16>, grid, block, st, a); break;
    case 32: e = launch(&k_select_members<32>, grid, block, st, a); break;
    case 64: e = launch(&k_select_members<64>, grid, block, st, a); break;
    default: return hipErrorInvalidValue;
    }
    return e;
}

hipError_t launch_select_rows(const LaunchShape &sh, const RowSelectLaunch &L, hipStream_t st)
{
    hipError_t e = hipSuccess;
    RowSelectArgs a{};
    a.geo = Geo{sh.B, L.G, sh.Lq, sh.Lk, L.g, sh.lens};
    a.kind = L.kind;
    a.rows = L.rows;
    a.K = L.K;
    a.to_candidates = L.to_candidates;
    a.out_idx = L.out_idx;
    a.out_sc = L.out_sc;
    a.out_count = L.out_count;
    a.out_stride = L.out_stride;
    a.cand = L.cand;
    a.cand_n = L.cand_n;
    a.c = L.c;
    a.hist = L.hist;
    a.splits = L.hist_splits;
    const int64_t jobs = L.kind == 0 ? sh.B * L.G : sh.B * sh.Lq;
    e = launch(&k_select_rows, dim3(static_cast<uint32_t>(jobs)), dim3(kSelThreads), st, a);
    return e;
}

}  // namespace pivot
