// Rank order of finished index rows: each row's selected entries reordered
// by score, highest first, equal scores by lower position, padding (-1) last.
//
// The pages define T_t = TopK(I_{t,:}, k) (PIVOT paper summary, eq. (1) and
// eqs. (6), (9)) without fixing the order inside a row; the indexer kernels
// emit the set in ascending position, and this pass gives callers that want
// the ranking the order TopK's own selection rule defines (higher score
// first, equal scores by lower position). It is a permutation of each row:
// no score is recomputed.
//
// One workgroup sorts one row: every entry becomes a 64-bit key whose
// ascending order is the rank order (high word: the complement of the
// score's order-preserving bit pattern; low word: the position; padding: all
// ones), the row is padded with all-ones keys to a power of two P and sorted
// by a bitonic network held in registers, then the keys are written back as
// (position, score). The pass reads and writes the row once (8 bytes per
// entry each way); its algorithmic traffic is 16 bytes per entry.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>
#include <utility>

#include "pivot_kernels.h"
#include "pivot_launch.h"

namespace pivot {
namespace {

constexpr int kRankMaxLog = 13;  // rows of up to 8192 entries (64 KiB of keys)

// Ascending keys = rank order. ord is the usual order-preserving map of the
// float bits (negative values complemented, non-negative ones with the sign
// bit set), so ~ord ascends as the score descends. A valid entry's high word
// is never all ones unless the score is a NaN with every bit set, and even
// then its low word (a position below 2^31) keeps it below the padding key.
__device__ __forceinline__ uint64_t rank_key(int32_t pos, float score)
{
    if (pos < 0) return ~0ull;
    const uint32_t b = __float_as_uint(score);
    const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return (static_cast<uint64_t>(~ord) << 32) | static_cast<uint32_t>(pos);
}

__device__ __forceinline__ float rank_score(uint64_t key)
{
    const uint32_t ord = ~static_cast<uint32_t>(key >> 32);
    return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

// The key of lane l ^ M (M < 64): quad permutes (DPP) for M = 1, 2, the
// bit-mask swizzle within 32 lanes for M < 32, a lane permute for M = 32.
template <int M>
__device__ __forceinline__ uint32_t xor_lane32(uint32_t v)
{
    if constexpr (M == 1) {
        return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, false));
    } else if constexpr (M == 2) {
        return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, false));
    } else if constexpr (M < 32) {
        return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(v), 0x1F | (M << 10)));
    } else {
        static_assert(M == 32, "lanes of one wave");
        return static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), 32));
    }
}

template <int M>
__device__ __forceinline__ uint64_t xor_lane64(uint64_t v)
{
    const uint32_t lo = xor_lane32<M>(static_cast<uint32_t>(v));
    const uint32_t hi = xor_lane32<M>(static_cast<uint32_t>(v >> 32));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Entry e of a bitonic step keeps the smaller key of its pair (e, e ^ dist)
// when it is the pair's low entry of an ascending merge (bit `size` of e
// clear) or the high entry of a descending one.
__device__ __forceinline__ uint64_t keep(uint64_t mine, uint64_t other, int e, int size, int dist)
{
    const bool low = (e & dist) == 0, up = (e & size) == 0;
    const bool small = low == up;
    return (mine < other) == small ? mine : other;
}

// Compile-time loop: f(integral_constant<int, 0>) .. f(integral_constant<int, N - 1>).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Threads sorting one row of P = 2^LOGP keys: one per key up to 256 keys,
// then 256 threads (8 keys each at 2048), 512 for 8192 keys.
constexpr int rank_threads(int logp) { return logp >= 13 ? 512 : (logp >= 8 ? 256 : 1 << logp); }

// One row per workgroup of NT threads (rows [gridDim.x, k] of idx and sc, in
// place). Thread t holds the E = P / NT consecutive entries t E .. t E + E -
// 1 in registers, so the steps of the bitonic network with dist < E run
// inside a thread, those with dist < 64 E between the lanes of a wave (DPP,
// swizzles), and only the widest (dist >= 64 E, a partner in another wave)
// go through LDS, two barriers each. Every step is unrolled at compile time
// (register indices are constants). Many small workgroups per CU hide the
// latency of the lane exchanges.
template <int LOGP>
__global__ __launch_bounds__(rank_threads(LOGP)) void k_rank_rows(int32_t *__restrict__ idx,
                                                                  float *__restrict__ sc, int k)
{
    constexpr int P = 1 << LOGP;
    constexpr int NT = rank_threads(LOGP);
    constexpr int E = P / NT;  // entries per thread
    constexpr bool kWaves = NT > 64;
    __shared__ uint64_t xch[kWaves ? P : 1];
    const int t = threadIdx.x;
    const int64_t row = blockIdx.x;
    int32_t *ir = idx + row * k;
    float *sr = sc + row * k;

    uint64_t r[E];
#pragma unroll
    for (int i = 0; i < E; ++i) {
        const int e = t * E + i;
        r[i] = e < k ? rank_key(ir[e], sr[e]) : ~0ull;
    }

    static_for<LOGP>([&](auto sl) {
        constexpr int size = 2 << decltype(sl)::value;
        static_for<decltype(sl)::value + 1>([&](auto dl) {
            constexpr int dist = (size >> 1) >> decltype(dl)::value;
            if constexpr (dist < E) {
#pragma unroll
                for (int i = 0; i < E; ++i) {
                    if (i & dist) continue;
                    const uint64_t a = r[i], b = r[i + dist];
                    const bool up = ((t * E + i) & size) == 0;
                    const bool sw = (a > b) == up;
                    r[i] = sw ? b : a;
                    r[i + dist] = sw ? a : b;
                }
            } else if constexpr (dist < 64 * E) {
#pragma unroll
                for (int i = 0; i < E; ++i) r[i] = keep(r[i], xor_lane64<dist / E>(r[i]), t * E + i, size, dist);
            } else {
                __syncthreads();  // every read of the previous exchange is done
#pragma unroll
                for (int i = 0; i < E; ++i) xch[i * NT + t] = r[i];
                __syncthreads();
                const int tp = t ^ (dist / E);
#pragma unroll
                for (int i = 0; i < E; ++i) r[i] = keep(r[i], xch[i * NT + tp], t * E + i, size, dist);
            }
        });
    });

#pragma unroll
    for (int i = 0; i < E; ++i) {
        const int e = t * E + i;
        if (e < k) {
            const uint64_t v = r[i];
            const bool pad = v == ~0ull;
            ir[e] = pad ? -1 : static_cast<int32_t>(static_cast<uint32_t>(v));
            sr[e] = pad ? -INFINITY : rank_score(v);
        }
    }
}

template <int LOGP>
hipError_t launch_rank_p(int32_t *idx, float *sc, int64_t rows, int k, hipStream_t st)
{
    return launch(k_rank_rows<LOGP>, dim3(static_cast<unsigned>(rows)), dim3(rank_threads(LOGP)), st, idx, sc, k);
}

}  // namespace

int rank_rows_max() { return 1 << kRankMaxLog; }

hipError_t launch_rank_rows(int32_t *idx, float *sc, int64_t rows, int k, hipStream_t st)
{
    if (rows <= 0) return hipSuccess;
    if (k < 1 || k > rank_rows_max() || rows > 0x7FFFFFFF) return hipErrorInvalidValue;
    int logp = 0;
    while ((1 << logp) < k) ++logp;
    switch (logp) {
    case 0: return launch_rank_p<0>(idx, sc, rows, k, st);
    case 1: return launch_rank_p<1>(idx, sc, rows, k, st);
    case 2: return launch_rank_p<2>(idx, sc, rows, k, st);
    case 3: return launch_rank_p<3>(idx, sc, rows, k, st);
    case 4: return launch_rank_p<4>(idx, sc, rows, k, st);
    case 5: return launch_rank_p<5>(idx, sc, rows, k, st);
    case 6: return launch_rank_p<6>(idx, sc, rows, k, st);
    case 7: return launch_rank_p<7>(idx, sc, rows, k, st);
    case 8: return launch_rank_p<8>(idx, sc, rows, k, st);
    case 9: return launch_rank_p<9>(idx, sc, rows, k, st);
    case 10: return launch_rank_p<10>(idx, sc, rows, k, st);
    case 11: return launch_rank_p<11>(idx, sc, rows, k, st);
    case 12: return launch_rank_p<12>(idx, sc, rows, k, st);
    default: return launch_rank_p<13>(idx, sc, rows, k, st);
    }
}

}  // namespace pivot
