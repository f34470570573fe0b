// Split-K reduction helper shared by the finish kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>

namespace qe {

// sum_k p[k * stride] for k = 0 .. n-1, added in order; the loads are issued in independent
// batches of B (a chain of dependent loads would cost one memory latency per term, a batch one
// latency for B terms)
template <int B = 16>
__device__ inline float sum_splits(const float* __restrict__ p, size_t stride, int n) {
    float sum = 0.0f;
    for (int k = 0; k < n; k += B) {
        float a[B];
#pragma unroll
        for (int q = 0; q < B; ++q) a[q] = k + q < n ? p[(size_t)(k + q) * stride] : 0.0f;
#pragma unroll
        for (int q = 0; q < B; ++q)
            if (k + q < n) sum += a[q];
    }
    return sum;
}

// The same for exact int32 partial sums (integer adds: any order gives the same result)
__device__ inline int32_t sum_splits_i32(const int32_t* __restrict__ p, size_t stride, int n) {
    constexpr int B = 16;
    int32_t sum = 0;
    for (int k = 0; k < n; k += B) {
        int32_t a[B];
#pragma unroll
        for (int q = 0; q < B; ++q) a[q] = k + q < n ? p[(size_t)(k + q) * stride] : 0;
#pragma unroll
        for (int q = 0; q < B; ++q) sum += a[q];
    }
    return sum;
}

}  // namespace qe
