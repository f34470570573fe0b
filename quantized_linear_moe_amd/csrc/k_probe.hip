// Measurement aids, not part of the QE computation: kernels whose duration, taken by the
// caller with events on the launch stream, gives the rates this device sustains, to set
// beside the published peaks in the roofline of the hot path's kernels.
//
//   probe_mfma_i8_kernel : int8 matrix-core throughput (v_mfma_i32_16x16x64_i8, the main
//                          GEMM's instruction), a loop on register operands
//   probe_mfma_bf16_kernel: bf16 matrix-core throughput (v_mfma_f32_16x16x32_bf16, the
//                          weight-only GEMM's instruction), the same loop
//   probe_copy_kernel    : streaming HBM copy (16-byte loads and stores)
//   probe_read_kernel    : streaming HBM read (16-byte loads folded into one word per thread)

#include "qe_internal.h"

namespace qe {

typedef int32_t v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int PM_ACC = 8;  // independent accumulators per wave: cover the MFMA latency

// Each wave issues PM_ACC * iters MFMAs on register operands fixed through the loop.  The
// matrix cores of this part are power-limited, so the rate depends on the operand values:
//   operands 0: small constant bytes (1 .. 11): the highest rate the part sustains
//   operands 1: random per lane in the main GEMM's value ranges: A6 codes in [-31, 31] times
//               4-bit weight codes scaled by 16 (the GEMM's int4-in-int8 encoding)
__global__ __launch_bounds__(256) void probe_mfma_i8_kernel(int32_t* __restrict__ out, int iters, int operands) {
    const uint32_t lane_id = blockIdx.x * 256u + threadIdx.x;
    uint32_t h = (lane_id + 1u) * 0x9E3779B9u;
    auto rnd = [&h]() {
        h = h * 1664525u + 1013904223u;
        return h >> 8;
    };
    v4i a, b;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (operands == 0) {
            a[q] = q + 1;
            b[q] = 2 * q + 5;
        } else {
            uint32_t wa = 0, wb = 0;
#pragma unroll
            for (int y = 0; y < 4; ++y) {
                const int ca = (int)(rnd() % 63u) - 31, cb = ((int)(rnd() % 15u) - 7) * 16;
                wa |= (uint32_t)(ca & 0xFF) << (8 * y);
                wb |= (uint32_t)(cb & 0xFF) << (8 * y);
            }
            a[q] = (int32_t)wa;
            b[q] = (int32_t)wb;
        }
    }
    v4i acc[PM_ACC];
#pragma unroll
    for (int j = 0; j < PM_ACC; ++j) acc[j] = v4i{0, 0, 0, 0};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < PM_ACC; ++j) acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[j], 0, 0, 0);
    }
    v4i sum = acc[0];
#pragma unroll
    for (int j = 1; j < PM_ACC; ++j) sum += acc[j];
    *reinterpret_cast<v4i*>(out + (size_t)lane_id * 4) = sum;
}

// The bf16 counterpart: operands 0 holds small constants (1, 2, 3, 4 as bf16), operands 1
// random values in the weight-only GEMM's ranges: activations of about unit scale with a
// random sign and exponent, and weights that are 3-bit codes times a scale near 2^-7.
__global__ __launch_bounds__(256) void probe_mfma_bf16_kernel(float* __restrict__ out, int iters, int operands) {
    const uint32_t lane_id = blockIdx.x * 256u + threadIdx.x;
    uint32_t h = (lane_id + 1u) * 0x9E3779B9u;
    auto rnd = [&h]() {
        h = h * 1664525u + 1013904223u;
        return h >> 8;
    };
    v8bf a, b;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        if (operands == 0) {
            a[q] = (__bf16)(float)(q % 4 + 1);
            b[q] = (__bf16)(float)(q % 2 + 1);
        } else {
            const uint32_t r = rnd();
            const float xa = (1.0f + (r & 127) / 128.0f) * (float)(1 << ((r >> 7) & 3)) * 0.25f;
            a[q] = (__bf16)((r >> 9) & 1 ? -xa : xa);
            b[q] = (__bf16)(((int)((r >> 10) & 7) - 4) * 0.0078125f);
        }
    }
    v4f acc[PM_ACC];
#pragma unroll
    for (int j = 0; j < PM_ACC; ++j) acc[j] = v4f{0, 0, 0, 0};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < PM_ACC; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    }
    v4f sum = acc[0];
#pragma unroll
    for (int j = 1; j < PM_ACC; ++j) sum += acc[j];
    *reinterpret_cast<v4f*>(out + (size_t)lane_id * 4) = sum;
}

__global__ __launch_bounds__(256) void probe_copy_kernel(const v4u* __restrict__ src, v4u* __restrict__ dst,
                                                         size_t n16) {
    const size_t stride = (size_t)gridDim.x * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {  // four independent 16-byte loads in flight
        const v4u v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
        dst[i] = v0;
        dst[i + stride] = v1;
        dst[i + 2 * stride] = v2;
        dst[i + 3 * stride] = v3;
    }
    for (; i < n16; i += stride) dst[i] = src[i];
}

// Reads every 16-byte chunk once (four independent loads in flight per thread) and folds the
// words with XOR, so no load can be dropped; one word per thread goes to `sink`.
__global__ __launch_bounds__(256) void probe_read_kernel(const v4u* __restrict__ src, size_t n16,
                                                         uint32_t* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t h = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const v4u v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
        h ^= v0[0] ^ v0[1] ^ v0[2] ^ v0[3] ^ v1[0] ^ v1[1] ^ v1[2] ^ v1[3];
        h ^= v2[0] ^ v2[1] ^ v2[2] ^ v2[3] ^ v3[0] ^ v3[1] ^ v3[2] ^ v3[3];
    }
    for (; i < n16; i += stride) {
        const v4u v = src[i];
        h ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    sink[(size_t)blockIdx.x * 256 + threadIdx.x] = h;
}

hipError_t launch_probe_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t st) {
    hipLaunchKernelGGL(probe_read_kernel, dim3(256 * 16), dim3(256), 0, st, reinterpret_cast<const v4u*>(src),
                       bytes / 16, sink);
    return hipGetLastError();
}

size_t probe_read_sink_words() { return (size_t)256 * 16 * 256; }

hipError_t launch_probe_mfma_i8(int32_t* out, int blocks, int iters, int operands, hipStream_t st) {
    hipLaunchKernelGGL(probe_mfma_i8_kernel, dim3(blocks), dim3(256), 0, st, out, iters, operands);
    return hipGetLastError();
}

double probe_mfma_i8_ops(int blocks, int iters) {
    return 2.0 * 16 * 16 * 64 * (double)PM_ACC * iters * 4.0 * blocks;  // 4 waves per workgroup
}

hipError_t launch_probe_mfma_bf16(float* out, int blocks, int iters, int operands, hipStream_t st) {
    hipLaunchKernelGGL(probe_mfma_bf16_kernel, dim3(blocks), dim3(256), 0, st, out, iters, operands);
    return hipGetLastError();
}

double probe_mfma_bf16_flops(int blocks, int iters) {
    return 2.0 * 16 * 16 * 32 * (double)PM_ACC * iters * 4.0 * blocks;
}

hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t st) {
    const size_t n16 = bytes / 16;
    hipLaunchKernelGGL(probe_copy_kernel, dim3(256 * 16), dim3(256), 0, st, reinterpret_cast<const v4u*>(src),
                       reinterpret_cast<v4u*>(dst), n16);
    return hipGetLastError();
}

}  // namespace qe
