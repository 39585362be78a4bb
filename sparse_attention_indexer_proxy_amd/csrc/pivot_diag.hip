// O1-O3 diagnostics of selected index rows (PIVOT paper summary, "Key
// observations", Figure 2): how much adjacent queries' top-k sets overlap,
// how large a group's union and intersection are, and how fast each row's
// indexer-score mass saturates. Rows are the indexer's outputs: the selected
// positions in ascending order, then -1.
//
//   k_row_overlap   one wave per row t: |T_t ∩ T_{t+d}|; the partner row is
//                   a bitmap in LDS (positions below 2^17) probed once per
//                   entry of T_t, else a sorted array searched by bisection.
//   k_group_bits    one workgroup per group whose positions are below 2^17:
//                   the union is the OR of the rows' bitmaps, the
//                   intersection their AND.
//   k_group_sets    the other groups: rows merged pairwise in LDS into one
//                   sorted multiset; distinct values = union, values
//                   occurring in every row = intersection.
//   k_row_mass      one wave per row: the row's scores as ordered keys in
//                   registers; the j-th largest (three j at once) by bisection
//                   over the key bits; the mass of the best j = the sum above
//                   it plus its ties.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "pivot_kernels.h"
#include "pivot_launch.h"

namespace pivot {
namespace {

constexpr int kW = 64;            // wavefront
constexpr int kRowMax = 4096;     // row width limit (LDS / registers)
constexpr int kGroupMax = 16384;  // padded g * k limit of the group kernel (LDS)
constexpr int kDiagWaves = 4;
constexpr int kBitWords = 4096;   // bitmaps of positions below 32 * 4096 = 2^17
constexpr int32_t kNotHere = -2;  // group result left to the merge kernel

__device__ __forceinline__ int lane() { return threadIdx.x & (kW - 1); }
__device__ __forceinline__ int popc64(uint64_t x) { return __popcll(x); }

// Wave reductions on DPP lane moves (gfx9: row_shr:n = 0x110 + n,
// row_bcast:15 = 0x142, row_bcast:31 = 0x143; lanes without a source take
// `fill`): a Hillis-Steele scan whose last lane holds the result.
template <int Ctrl, int RowMask = 0xF>
__device__ __forceinline__ int32_t dpp_move(int32_t v, int32_t fill)
{
    return __builtin_amdgcn_update_dpp(fill, v, Ctrl, RowMask, 0xF, false);
}

template <class Op>
__device__ __forceinline__ int32_t wave_reduce(int32_t v, int32_t fill, Op op)
{
    v = op(v, dpp_move<0x111>(v, fill));
    v = op(v, dpp_move<0x112>(v, fill));
    v = op(v, dpp_move<0x114>(v, fill));
    v = op(v, dpp_move<0x118>(v, fill));
    v = op(v, dpp_move<0x142, 0xA>(v, fill));
    v = op(v, dpp_move<0x143, 0xC>(v, fill));
    return __builtin_amdgcn_readlane(v, kW - 1);
}

// Inclusive prefix sum over the lanes (every lane's own result).
__device__ __forceinline__ int32_t wave_reduce_scan(int32_t v)
{
    v += dpp_move<0x111>(v, 0);
    v += dpp_move<0x112>(v, 0);
    v += dpp_move<0x114>(v, 0);
    v += dpp_move<0x118>(v, 0);
    v += dpp_move<0x142, 0xA>(v, 0);
    v += dpp_move<0x143, 0xC>(v, 0);
    return v;
}

__device__ __forceinline__ int32_t wave_min_i32(int32_t v)
{
    return wave_reduce(v, INT32_MAX, [](int32_t x, int32_t y) { return x < y ? x : y; });
}
__device__ __forceinline__ int32_t wave_max_i32(int32_t v)
{
    return wave_reduce(v, INT32_MIN, [](int32_t x, int32_t y) { return x > y ? x : y; });
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v)
{
    return static_cast<uint32_t>(
        wave_reduce(static_cast<int32_t>(v), 0, [](int32_t x, int32_t y) { return static_cast<int32_t>(static_cast<uint32_t>(x) + static_cast<uint32_t>(y)); }));
}
__device__ __forceinline__ uint32_t wave_and_u32(uint32_t v)
{
    return static_cast<uint32_t>(wave_reduce(static_cast<int32_t>(v), -1, [](int32_t x, int32_t y) { return x & y; }));
}
__device__ __forceinline__ uint32_t wave_or_u32(uint32_t v)
{
    return static_cast<uint32_t>(wave_reduce(static_cast<int32_t>(v), 0, [](int32_t x, int32_t y) { return x | y; }));
}

// A row's entries, lane l holding entries 64 i + l (all loads issued at once;
// past k reads as -1), and its valid length: the prefix before the first -1.
template <int NV>
__device__ __forceinline__ int load_row(const int32_t *row, int k, int32_t (&v)[NV])
{
    const int l = lane();
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = kW * i + l < k ? row[kW * i + l] : -1;
    int n = NV * kW < k ? NV * kW : k;
#pragma unroll
    for (int i = NV - 1; i >= 0; --i) n = v[i] < 0 ? kW * i + l : n;  // this lane's first pad
    return wave_min_i32(n);
}

// Whether x is among the n ascending entries p[0..n).
__device__ __forceinline__ bool sorted_has(const int32_t *p, int n, int32_t x)
{
    int pos = 0;
    for (int step = 1 << 12; step > 0; step >>= 1)
        if (pos + step <= n && p[pos + step - 1] < x) pos += step;
    return pos < n && p[pos] == x;
}

template <int NV>
__global__ __launch_bounds__(kDiagWaves * kW) void k_row_overlap(StatsArgs a)
{
    // per wave: the partner row as a bitmap (positions < 32 * kBitWords) or
    // as a sorted array (k <= kRowMax = kBitWords entries)
    __shared__ uint32_t lds[kDiagWaves][kBitWords];
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = lane();
    const int64_t row = static_cast<int64_t>(blockIdx.x) * kDiagWaves + wv;
    if (row >= a.B * a.Lq) return;  // wave-uniform; no workgroup barrier below
    const int64_t b = row / a.Lq, t = row - b * a.Lq;
    if (t + a.d >= a.Lq) {
        if (l == 0) a.overlap[row] = -1;
        return;
    }
    int32_t v0[NV], v1[NV];
    const int n0 = load_row(a.idx + row * a.k, a.k, v0);
    const int n1 = load_row(a.idx + (row + a.d) * a.k, a.k, v1);
    uint32_t *bm = lds[wv];
    int32_t mx = INT32_MIN;  // the partner row's largest entry (its last valid one)
#pragma unroll
    for (int i = 0; i < NV; ++i) mx = kW * i + l < n1 && v1[i] > mx ? v1[i] : mx;
    mx = wave_max_i32(mx);
    int cnt = 0;
    if (mx < 32 * kBitWords) {
        // bitmap: clear the words in use, set the partner's bits, probe
        const int words = mx < 0 ? 0 : (mx >> 5) + 1;
        for (int w = l; w < words; w += kW) bm[w] = 0u;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (kW * i + l < n1) atomicOr(&bm[v1[i] >> 5], 1u << (v1[i] & 31));
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int32_t x = v0[i];
            const bool in = kW * i + l < n0 && x <= mx;  // valid entries are >= 0
            const bool hit = in && ((bm[in ? x >> 5 : 0] >> (x & 31)) & 1u);
            cnt += popc64(__ballot(hit));
        }
    } else {
        int32_t *p = reinterpret_cast<int32_t *>(bm);
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (kW * i + l < n1) p[kW * i + l] = v1[i];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int j = kW * i + l;
            cnt += popc64(__ballot(j < n0 && sorted_has(p, n1, v0[i])));
        }
    }
    if (l == 0) a.overlap[row] = cnt;
}

// Groups whose positions are all below 32 * kBitWords: the union is the OR
// of the rows' bitmaps, the intersection their AND, built row by row in LDS
// (rows are sets; each thread holds up to kSeg of the group's entries). A
// group with a larger position is marked kNotHere in its first requested
// output for k_group_sets.
constexpr int kSetThreads = 512;
constexpr int kSeg = kGroupMax / kSetThreads;  // entries per thread (32)

__global__ __launch_bounds__(kSetThreads) void k_group_bits(StatsArgs a)
{
    __shared__ uint32_t U[kBitWords], A[kBitWords], T[kBitWords];
    __shared__ int32_t red[kSetThreads / kW][2];
    const int64_t gid = blockIdx.x;
    const int64_t b = gid / a.G, m = gid - b * a.G;
    const int64_t t0 = m * a.g;
    const int gm = static_cast<int>((t0 + a.g < a.Lq ? t0 + a.g : a.Lq) - t0);
    const int N = gm * a.k;  // <= kGroupMax (checked by the caller)
    const int tid = threadIdx.x, l = lane(), wv = tid >> 6;
    const int32_t *g0 = a.idx + (b * a.Lq + t0) * a.k;
    int32_t ld[kSeg];
    int32_t mx = INT32_MIN;
#pragma unroll
    for (int q = 0; q < kSeg; ++q) {
        const int e = tid + q * kSetThreads;
        ld[q] = e < N ? g0[e] : -1;  // -1: padding (rows are their valid prefix, then -1)
        mx = ld[q] > mx ? ld[q] : mx;
    }
    mx = wave_max_i32(mx);
    if (l == 0) red[wv][0] = mx;
    __syncthreads();
    mx = wave_max_i32(red[l & (kSetThreads / kW - 1)][0]);
    if (mx >= 32 * kBitWords) {
        if (tid == 0) {
            if (a.group_union) a.group_union[gid] = kNotHere;
            else a.group_inter[gid] = kNotHere;
        }
        return;  // uniform
    }
    const int words = mx < 0 ? 0 : (mx >> 5) + 1;
    for (int w = tid; w < words; w += kSetThreads) U[w] = A[w] = T[w] = 0u;
    __syncthreads();
    // every row into U, row 0 into A
#pragma unroll
    for (int q = 0; q < kSeg; ++q) {
        const int e = tid + q * kSetThreads;
        if (ld[q] >= 0) {
            const uint32_t bit = 1u << (ld[q] & 31);
            atomicOr(&U[ld[q] >> 5], bit);
            if (e < a.k) atomicOr(&A[ld[q] >> 5], bit);
        }
    }
    __syncthreads();
    for (int r = 1; r < gm; ++r) {
#pragma unroll
        for (int q = 0; q < kSeg; ++q) {
            const int e = tid + q * kSetThreads;
            if (ld[q] >= 0 && e >= r * a.k && e < (r + 1) * a.k) atomicOr(&T[ld[q] >> 5], 1u << (ld[q] & 31));
        }
        __syncthreads();
        for (int w = tid; w < words; w += kSetThreads) {
            A[w] &= T[w];
            T[w] = 0u;
        }
        __syncthreads();
    }
    uint32_t nu = 0, ni = 0;
    for (int w = tid; w < words; w += kSetThreads) {
        nu += __popc(U[w]);
        ni += __popc(A[w]);
    }
    nu = wave_sum_u32(nu);
    ni = wave_sum_u32(ni);
    if (l == 0) {
        red[wv][0] = static_cast<int32_t>(nu);
        red[wv][1] = static_cast<int32_t>(ni);
    }
    __syncthreads();
    if (wv == 0) {
        const int i = l & (kSetThreads / kW - 1);
        const uint32_t su = wave_sum_u32(l < kSetThreads / kW ? static_cast<uint32_t>(red[i][0]) : 0u);
        const uint32_t si = wave_sum_u32(l < kSetThreads / kW ? static_cast<uint32_t>(red[i][1]) : 0u);
        if (l == 0) {
            if (a.group_union) a.group_union[gid] = static_cast<int32_t>(su);
            if (a.group_inter) a.group_inter[gid] = static_cast<int32_t>(si);
        }
    }
}

// A group's rows are merged into one sorted multiset (rows are sets, so a
// value occurs at most once per row): the union is the number of distinct
// values, the intersection the number of values occurring in every row
// (v[p] == v[p + gm - 1]). The rows, padded with a sentinel to kp entries
// (a multiple of the per-thread segment) and to a power-of-two count P,
// are merged pairwise in LDS, log2 P levels, each output segment found by a
// merge-path search (equal values: the left run first).
constexpr int32_t kSentinel = 0x7FFFFFFF;

__global__ __launch_bounds__(kSetThreads) void k_group_sets(StatsArgs a)
{
    __shared__ int32_t buf[2][kGroupMax];
    __shared__ int32_t cnt[2];
    const int64_t gid = blockIdx.x;
    // only the groups k_group_bits left (uniform)
    if ((a.group_union ? a.group_union[gid] : a.group_inter[gid]) != kNotHere) return;
    const int64_t b = gid / a.G, m = gid - b * a.G;
    const int64_t t0 = m * a.g;
    const int gm = static_cast<int>((t0 + a.g < a.Lq ? t0 + a.g : a.Lq) - t0);
    const int kp = (a.k + kSeg - 1) / kSeg * kSeg;  // padded run length
    int P = 1;
    while (P < gm) P <<= 1;
    const int N = P * kp;  // <= kGroupMax (checked by the caller)
    const int tid = threadIdx.x;
    if (tid < 2) cnt[tid] = 0;
    // every thread loads its (at most kSeg) entries with all loads in flight
    const int32_t *g0 = a.idx + (b * a.Lq + t0) * a.k;
    int32_t ld[kSeg];
#pragma unroll
    for (int q = 0; q < kSeg; ++q) {
        const int e = tid + q * kSetThreads;
        const int r = e / kp, j = e - r * kp;
        ld[q] = (e < N && r < gm && j < a.k) ? g0[r * a.k + j] : -1;
    }
#pragma unroll
    for (int q = 0; q < kSeg; ++q) {
        const int e = tid + q * kSetThreads;
        if (e < N) buf[0][e] = ld[q] < 0 ? kSentinel : ld[q];
    }
    __syncthreads();
    int src = 0;
    for (int L = kp; L < N; L <<= 1) {
        const int32_t *in = buf[src];
        int32_t *out = buf[src ^ 1];
        for (int o0 = tid * kSeg; o0 < N; o0 += kSetThreads * kSeg) {
            const int pair = o0 / (2 * L), d = o0 - pair * 2 * L;
            const int32_t *A = in + pair * 2 * L, *Bv = A + L;
            int lo = d > L ? d - L : 0, hi = d < L ? d : L;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (A[mid] <= Bv[d - 1 - mid]) lo = mid + 1;
                else hi = mid;
            }
            int i = lo, j = d - lo;
            for (int e = 0; e < kSeg; ++e) {
                const bool take_a = j >= L || (i < L && A[i] <= Bv[j]);
                out[o0 + e] = take_a ? A[i] : Bv[j];
                i += take_a ? 1 : 0;
                j += take_a ? 0 : 1;
            }
        }
        __syncthreads();
        src ^= 1;
    }
    const int32_t *v = buf[src];
    int nu = 0, ni = 0;
    for (int p = tid; p < N; p += kSetThreads) {
        const int32_t x = v[p];
        if (x == kSentinel) continue;
        nu += (p == 0 || v[p - 1] != x) ? 1 : 0;
        ni += (p + gm - 1 < N && v[p + gm - 1] == x) ? 1 : 0;
    }
    for (int o = kW / 2; o > 0; o >>= 1) {
        nu += __shfl_xor(nu, o);
        ni += __shfl_xor(ni, o);
    }
    if (lane() == 0) {
        atomicAdd(&cnt[0], nu);
        atomicAdd(&cnt[1], ni);
    }
    __syncthreads();
    if (tid == 0) {
        if (a.group_union) a.group_union[gid] = cnt[0];
        if (a.group_inter) a.group_inter[gid] = cnt[1];
    }
}

// Orderable key of a float: larger floats give larger keys, and every float
// maps to a key >= 0x007FFFFF (0 marks an empty slot).
__device__ __forceinline__ uint32_t okey(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float wave_sum(float v)
{
    return __int_as_float(wave_reduce(__float_as_int(v), 0, [](int32_t x, int32_t y) {
        return __float_as_int(__int_as_float(x) + __int_as_float(y));
    }));
}

template <int NV>
__device__ __forceinline__ int wave_count_ge(const uint32_t (&kv)[NV], uint32_t x)
{
    int n = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) n += popc64(__ballot(kv[i] >= x));
    return n;
}

__device__ __forceinline__ float okey_float(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

template <int NV>
__global__ __launch_bounds__(kDiagWaves * kW) void k_row_mass(StatsArgs a)
{
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = lane();
    const int64_t row = static_cast<int64_t>(blockIdx.x) * kDiagWaves + wv;
    if (row >= a.B * a.Lq) return;  // wave-uniform
    const int32_t *ri = a.idx + row * a.k;
    const float *rs = a.scores + row * a.k;
    uint32_t kv[NV];
    float part = 0.0f;
    int n;
    {
        int32_t iv[NV];
        float sv[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) sv[i] = kW * i + l < a.k ? rs[kW * i + l] : 0.0f;
        n = load_row(ri, a.k, iv);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const bool in = kW * i + l < n;
            kv[i] = in ? okey(sv[i]) : 0u;
            part += in ? sv[i] : 0.0f;
        }
    }
    const float total = wave_sum(part);
    // floor(f k) for f = 1/4, 1/2, 3/4 (exact integer arithmetic)
    const int jsel[3] = {a.k / 4, a.k / 2, 3 * a.k / 4};
    // the jsel-th largest key of each: the largest T with #{key >= T} >= jsel;
    // the three searches share each pass over the keys, which starts below
    // the leading bits every valid key shares (each answer is a valid key)
    uint32_t kand = ~0u, kor = 0u;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        kand &= kv[i] != 0u ? kv[i] : ~0u;
        kor |= kv[i];
    }
    kand = wave_and_u32(kand);
    kor = wave_or_u32(kor);
    const uint32_t diff = kand ^ kor;
    const int topbit = diff == 0u ? -1 : 31 - __builtin_clz(diff);
    const uint32_t shared = topbit < 0 ? kand : (topbit == 31 ? 0u : (kand & ~((2u << topbit) - 1u)));
    uint32_t T[3] = {shared, shared, shared};
    // One pass of the 8 bits below the shared ones into 256 bins (LDS) gives
    // each search its bin, and with it 8 more bits of T; the bisection then
    // covers the bits below the bin only: over the bins' own keys, compacted
    // to LDS, when each of the three bins holds at most kMassSmall keys, else
    // over all keys.
    constexpr int kMassSmall = 2 * kW;
    int lowbit = topbit;
    bool small = false;
    uint32_t need[3] = {0u, 0u, 0u};  // small path: the rank sought within each bin
    uint32_t sv[3][kMassSmall / kW];  // small path: each bin's keys, 0 = empty
    if (topbit >= 0) {
        __shared__ uint32_t hist_all[kDiagWaves][256];
        uint32_t *hist = hist_all[wv];
        const int shift = topbit >= 7 ? topbit - 7 : 0;
        for (int j = l; j < 256; j += kW) hist[j] = 0u;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (kv[i] != 0u) atomicAdd(&hist[(kv[i] >> shift) & 0xFFu], 1u);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // lane l holds bins 4l .. 4l + 3; counts of the keys in higher bins
        const uint32_t c0 = hist[4 * l], c1 = hist[4 * l + 1], c2 = hist[4 * l + 2], c3 = hist[4 * l + 3];
        const uint32_t tot = c0 + c1 + c2 + c3;
        const uint32_t incl = static_cast<uint32_t>(
            wave_reduce_scan(static_cast<int32_t>(tot)));  // inclusive prefix over lanes
        const uint32_t all = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int32_t>(incl), kW - 1));
        const uint32_t above_lane = all - incl;  // keys in the bins of higher lanes
#pragma unroll
        for (int f = 0; f < 3; ++f) {
            const uint32_t j = static_cast<uint32_t>(jsel[f]);
            if (jsel[f] == 0 || jsel[f] >= n) continue;  // uniform; T unused
            const bool here = above_lane < j && j <= above_lane + tot;
            const int src = __ffsll(static_cast<long long>(__ballot(here))) - 1;
            uint32_t dig = 0;
            if (here) {
                uint32_t cum = above_lane;
                if (cum + c3 >= j) {
                    dig = 4 * l + 3;
                } else if ((cum += c3) + c2 >= j) {
                    dig = 4 * l + 2;
                } else if ((cum += c2) + c1 >= j) {
                    dig = 4 * l + 1;
                } else {
                    dig = 4 * l;
                }
            }
            dig = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int32_t>(dig), src));
            T[f] = (T[f] & ~(0xFFu << shift)) | (dig << shift);
        }
        lowbit = shift - 1;
        // whether every searched bin is small
        bool fits = lowbit >= 0;
#pragma unroll
        for (int f = 0; f < 3; ++f) {
            if (jsel[f] == 0 || jsel[f] >= n) continue;
            fits = fits && hist[(T[f] >> shift) & 0xFFu] <= static_cast<uint32_t>(kMassSmall);
        }
        if (fits) {
            small = true;
            // compact each bin's keys into LDS, then into registers
            __shared__ uint32_t lists[kDiagWaves][3][kMassSmall];
#pragma unroll
            for (int f = 0; f < 3; ++f) {
                if (jsel[f] == 0 || jsel[f] >= n) continue;
                const uint32_t lo = T[f], hi = T[f] | ((1u << shift) - 1u);  // the bin's keys
                int base = 0;
#pragma unroll
                for (int i = 0; i < NV; ++i) {
                    const bool in = kv[i] >= lo && kv[i] <= hi;
                    const uint64_t bm = __ballot(in);
                    if (in) lists[wv][f][base + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bm >> 32),
                                                      __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bm), 0u))] = kv[i];
                    base += popc64(bm);
                }
                // the rank sought within the bin: jsel minus the keys above it
                int above = 0;
#pragma unroll
                for (int i = 0; i < NV; ++i) above += popc64(__ballot(kv[i] > hi));
                need[f] = static_cast<uint32_t>(jsel[f] - above);
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
                for (int q = 0; q < kMassSmall / kW; ++q) sv[f][q] = kW * q + l < base ? lists[wv][f][kW * q + l] : 0u;
            }
        }
    }
    if (small) {
        // each search over its bin's keys alone: the largest T with
        // #{bin key >= T} >= the rank left
#pragma unroll
        for (int f = 0; f < 3; ++f) {
            if (jsel[f] == 0 || jsel[f] >= n) continue;
            for (int bit = lowbit; bit >= 0; --bit) {
                const uint32_t x = T[f] | (1u << bit);
                int c = 0;
#pragma unroll
                for (int q = 0; q < kMassSmall / kW; ++q) c += popc64(__ballot(sv[f][q] >= x));
                T[f] = c >= static_cast<int>(need[f]) ? x : T[f];
            }
        }
        lowbit = -1;  // done
    }
    for (int bit = lowbit; bit >= 0; --bit) {
        const uint32_t x0 = T[0] | (1u << bit), x1 = T[1] | (1u << bit), x2 = T[2] | (1u << bit);
        // per-lane counts, packed 3 x 10 bits (<= NV <= 64 each), summed over
        // the wave as two 16-bit pairs and one word (totals <= 4096)
        uint32_t c = 0;
#pragma unroll
        for (int i = 0; i < NV; ++i)
            c += (kv[i] >= x0 ? 1u : 0u) | (kv[i] >= x1 ? 1u << 10 : 0u) | (kv[i] >= x2 ? 1u << 20 : 0u);
        const uint32_t s01 = wave_sum_u32((c & 0x3FFu) | (((c >> 10) & 0x3FFu) << 16));
        const int c0 = static_cast<int>(s01 & 0xFFFFu), c1 = static_cast<int>(s01 >> 16),
                  c2 = static_cast<int>(wave_sum_u32(c >> 20));
        T[0] = c0 >= jsel[0] ? x0 : T[0];
        T[1] = c1 >= jsel[1] ? x1 : T[1];
        T[2] = c2 >= jsel[2] ? x2 : T[2];
    }
    for (int f = 0; f < 3; ++f) {
        float top = total;
        if (jsel[f] == 0) {
            top = 0.0f;
        } else if (jsel[f] < n) {
            const uint32_t t = T[f];
            int above = 0;
            float sabove = 0.0f;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                above += popc64(__ballot(kv[i] > t));
                sabove += kv[i] > t ? okey_float(kv[i]) : 0.0f;
            }
            top = wave_sum(sabove) + static_cast<float>(jsel[f] - above) * okey_float(t);
        }
        a.mass[row * 3 + f] = total > 0.0f ? top / total : NAN;
    }
}

}  // namespace

hipError_t launch_stats(const StatsArgs &a, hipStream_t st)
{
    const int64_t rows = a.B * a.Lq;
    const dim3 block(kDiagWaves * kW);
    const dim3 rgrid(static_cast<uint32_t>((rows + kDiagWaves - 1) / kDiagWaves));
    hipError_t e = hipSuccess;
    if (a.overlap) {
        if (a.k <= 1024)
            e = launch(&k_row_overlap<16>, rgrid, block, st, a);
        else if (a.k <= 2048)
            e = launch(&k_row_overlap<32>, rgrid, block, st, a);
        else
            e = launch(&k_row_overlap<64>, rgrid, block, st, a);
        if (e != hipSuccess) return e;
    }
    if (a.group_union || a.group_inter) {
        const dim3 ggrid(static_cast<uint32_t>(a.B * a.G));
        e = launch(&k_group_bits, ggrid, dim3(kSetThreads), st, a);
        if (e != hipSuccess) return e;
        e = launch(&k_group_sets, ggrid, dim3(kSetThreads), st, a);
        if (e != hipSuccess) return e;
    }
    if (a.mass) {
        if (a.k <= 1024)
            e = launch(&k_row_mass<16>, rgrid, block, st, a);
        else if (a.k <= 2048)
            e = launch(&k_row_mass<32>, rgrid, block, st, a);
        else
            e = launch(&k_row_mass<64>, rgrid, block, st, a);
    }
    return e;
}

int stats_row_max() { return kRowMax; }

int stats_group_fits(int g, int k)
{
    int P = 1;
    while (P < g) P <<= 1;
    const int64_t kp = (int64_t(k) + kSeg - 1) / kSeg * kSeg;
    return P * kp <= kGroupMax;
}

}  // namespace pivot
