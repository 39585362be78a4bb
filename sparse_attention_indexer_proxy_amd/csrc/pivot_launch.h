// Kernel launch that reports its own status.
#pragma once

#include <hip/hip_runtime.h>

#include <tuple>
#include <type_traits>
#include <utility>

namespace pivot {

// Enqueues kernel k on st and returns the status of this launch alone.
// (hipLaunchKernelGGL + hipGetLastError would return the thread's sticky
// last error, which an earlier, unrelated failure may still hold.) The
// arguments are converted to the kernel's parameter types and passed by
// address, as hipLaunchKernel expects.
template <class... P, class... A>
inline hipError_t launch(void (*k)(P...), dim3 grid, dim3 block, hipStream_t st, A &&...args)
{
    static_assert(sizeof...(P) == sizeof...(A), "one argument per kernel parameter");
    std::tuple<std::decay_t<P>...> vals(std::forward<A>(args)...);
    return std::apply(
        [&](auto &...v) {
            void *ptrs[] = {static_cast<void *>(&v)...};
            return hipLaunchKernel(reinterpret_cast<const void *>(k), grid, block, ptrs, 0, st);
        },
        vals);
}

}  // namespace pivot
