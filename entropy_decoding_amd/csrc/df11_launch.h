// Kernel launch returning the launch's own status.
//
// hipLaunchKernelGGL returns nothing, and hipGetLastError after it would also
// report an earlier failure of any HIP call on the calling thread (the
// caller's, say).  launch() converts the arguments to the kernel's parameter
// types, keeps them alive for the call and returns hipLaunchKernel's result.
#pragma once

#include <hip/hip_runtime.h>

#include "df11.h"

#include <cstddef>
#include <tuple>
#include <utility>

namespace df11_detail {

template <class... P, std::size_t... I>
hipError_t launch_tuple(void (*k)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t st,
                        std::tuple<P...> &args, std::index_sequence<I...>) {
    void *p[] = {static_cast<void *>(&std::get<I>(args))...};
    return hipLaunchKernel(reinterpret_cast<const void *>(k), grid, block, p, lds, st);
}

template <class... P, class... A>
hipError_t launch(void (*k)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t st,
                  A &&...args) {
    static_assert(sizeof...(P) == sizeof...(A), "one argument per kernel parameter");
    std::tuple<P...> t(std::forward<A>(args)...);
    return launch_tuple(k, grid, block, lds, st, t, std::index_sequence_for<P...>{});
}

// df11_decompress_block with the grid capped at workgroups_per_cu resident
// workgroups per compute unit (0: the default grid).  Each wave loops over
// the tiles with the grid's stride, so any grid decodes every tile; a capped
// grid leaves the other workgroup slots of every compute unit to kernels on
// other streams.
int decompress_block_capped(const df11_device_stream *s, void *out, int32_t *d_status,
                            hipStream_t st, uint32_t workgroups_per_cu);

}  // namespace df11_detail
