// count.h -- dispatch on a small wave-uniform count, so that the last
// passes of a software pipeline can run as straight-line code specialised
// on how many remain (loads only for passes that exist, exact waits for
// those in flight).
#pragma once
#include <hip/hip_runtime.h>

namespace qmv {

template <int V>
struct Int {
    static constexpr int value = V;
};

// Calls f(Int<R>{}) for the R in [R0, RMAX] equal to r; no call for r
// outside that range.
template <int R0, int RMAX, class F>
__device__ __forceinline__ void with_count(int r, F &&f) {
    if constexpr (R0 <= RMAX) {
        if (r == R0)
            f(Int<R0>{});
        else
            with_count<R0 + 1, RMAX>(r, f);
    }
}

}  // namespace qmv
