// focus_launch.h -- kernel launches that report their own status.
//
// hipLaunchKernel returns the status of the launch it makes.  Reading the
// thread's last error after a triple-chevron launch instead (hipGetLastError)
// would report, and clear, an error left by any earlier HIP call of the same
// thread, including calls that have nothing to do with this library.
#pragma once
#include <hip/hip_runtime.h>

#include <tuple>
#include <utility>

namespace focus {

// Launch `kernel` on `stream` with no dynamic LDS.  The arguments are
// converted to the kernel's parameter types first, so each entry of the
// argument array points at a value of exactly the type the kernel expects.
template <typename... P, typename... A>
inline hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream, A&&... args) {
    static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
    static_assert(sizeof...(P) > 0, "kernels here take arguments");
    std::tuple<P...> vals(std::forward<A>(args)...);
    return std::apply(
        [&](auto&... v) {
            void* argv[] = {static_cast<void*>(&v)...};
            return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, stream);
        },
        vals);
}

}  // namespace focus
