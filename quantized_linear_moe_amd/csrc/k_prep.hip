// Load-time re-layout of a QE linear's parameters into the kernels' formats.
//
//   * W4 main weights: canonical bytes [d_out][d_in/2] (code 2m low nibble, 2m+1
//     high nibble) -> tiles of 16 channels x 64 K, 512 bytes each, ordered
//     (channel block, K step, lane): lane l owns channel 16*nb + l%16 and codes
//     k = 64*ks + 16*(l/16) + [0, 16) in 8 bytes; each 8-code half is stored so
//     byte b = code b | code b+4 << 4.
//   * W3 main weights: canonical 96-bit groups -> tiles of 16 channels x 128 K,
//     12 bytes per lane: lane l owns channel 16*nb + l%16 and codes
//     k = 128*kb + 32*s + 8*(l/16) + p (s = 0..3, p = 0..7) in sign/magnitude form:
//     |c| of code 8s+p at bits 4p + 2(s&1) of dword s>>1, its sign at bit 4p + 3 - s
//     of dword 2 (the weight-streaming kernel turns 8 codes into one fp4 word).
//   * Adapter/router matrices are transposed so every MFMA operand fragment is
//     16 contiguous bytes, and padded with zeros to whole MFMA steps.

#include "qe_internal.h"

namespace qe {

__device__ inline int canon_w4_code(const uint8_t* row, int k) {
    const uint32_t b = row[k >> 1];
    const int nib = (k & 1) ? (b >> 4) : (b & 15);
    return nib;  // 4-bit two's complement pattern
}

__global__ void prep_w4_kernel(const uint8_t* __restrict__ packed, int d_out, int d_in, uint32_t* __restrict__ tiled) {
    const int KS = d_in / 64, NB = d_out / 16;
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;  // (nb, ks, lane)
    if (idx >= (size_t)NB * KS * 64) return;
    const int lane = (int)(idx % 64);
    const size_t nk = idx / 64;
    const int ks = (int)(nk % KS), nb = (int)(nk / KS);
    const int n = nb * 16 + (lane & 15), g = lane >> 4;
    const uint8_t* row = packed + (size_t)n * (d_in / 2);
    uint32_t out[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int kbase = ks * 64 + g * 16 + h * 8;
        uint32_t d = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t lo = (uint32_t)canon_w4_code(row, kbase + b);
            const uint32_t hi = (uint32_t)canon_w4_code(row, kbase + b + 4);
            d |= (lo | (hi << 4)) << (8 * b);
        }
        out[h] = d;
    }
    tiled[idx * 2] = out[0];
    tiled[idx * 2 + 1] = out[1];
}

hipError_t launch_prep_w4(const uint8_t* packed, int d_out, int d_in, uint8_t* tiled, hipStream_t st) {
    const size_t n = (size_t)(d_out / 16) * (d_in / 64) * 64;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(prep_w4_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, packed, d_out, d_in,
                       reinterpret_cast<uint32_t*>(tiled));
    return hipGetLastError();
}

__device__ inline uint32_t canon_w3_code(const uint32_t* row, int k) {
    const uint32_t* grp = row + (size_t)(k >> 5) * 3;
    const int bit = 3 * (k & 31);
    const uint64_t lo = (uint64_t)grp[0] | ((uint64_t)grp[1] << 32);
    if (bit + 3 <= 64) return (uint32_t)(lo >> bit) & 7u;
    if (bit >= 64) return (grp[2] >> (bit - 64)) & 7u;
    return (uint32_t)((lo >> bit) | ((uint64_t)grp[2] << (64 - bit))) & 7u;
}

__global__ void prep_w3_kernel(const uint32_t* __restrict__ packed, int d_out, int d_in, uint32_t* __restrict__ tiled) {
    const int KB = d_in / 128, NB = d_out / 16;
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)NB * KB * 64) return;
    const int lane = (int)(idx % 64);
    const size_t nk = idx / 64;
    const int kb = (int)(nk % KB), nb = (int)(nk / KB);
    const int n = nb * 16 + (lane & 15), g = lane >> 4;
    const uint32_t* row = packed + (size_t)n * (d_in / 32) * 3;
    uint32_t w[3] = {0, 0, 0};
    for (int s = 0; s < 4; ++s) {
        for (int p = 0; p < 8; ++p) {
            const uint32_t c = canon_w3_code(row, kb * 128 + s * 32 + g * 8 + p);  // 3-bit two's complement
            const int v = (c & 4u) ? (int)c - 8 : (int)c;
            const uint32_t mag = (uint32_t)(v < 0 ? -v : v), sign = v < 0 ? 1u : 0u;
            w[s >> 1] |= mag << (4 * p + 2 * (s & 1));
            w[2] |= sign << (4 * p + 3 - s);
        }
    }
    uint32_t* o = tiled + idx * 3;
    o[0] = w[0];
    o[1] = w[1];
    o[2] = w[2];
}

hipError_t launch_prep_w3(const uint32_t* packed, int d_out, int d_in, uint32_t* tiled, hipStream_t st) {
    const size_t n = (size_t)(d_out / 16) * (d_in / 128) * 64;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(prep_w3_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, packed, d_out, d_in, tiled);
    return hipGetLastError();
}

// dst[c][r] = src[r][c] for r < rows, c < cols; zeros elsewhere in [dst_rows][dst_ld]
__global__ void transpose_kernel(const uint16_t* __restrict__ src, int rows, int cols, uint16_t* __restrict__ dst,
                                 int dst_ld, int dst_rows) {
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)dst_rows * dst_ld) return;
    const int c = (int)(idx / dst_ld), r = (int)(idx % dst_ld);
    dst[idx] = (src && r < rows && c < cols) ? src[(size_t)r * cols + c] : (uint16_t)0;
}

hipError_t launch_prep_transpose(const uint16_t* src, int rows, int cols, uint16_t* dst, int dst_ld, int dst_rows,
                                 hipStream_t st) {
    const size_t n = (size_t)dst_rows * dst_ld;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(transpose_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, src, rows, cols, dst,
                       dst_ld, dst_rows);
    return hipGetLastError();
}

__global__ void smooth_kernel(const float* __restrict__ s, int d_in, float* __restrict__ s_out,
                              float* __restrict__ inv_out) {
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= d_in) return;
    const float v = s ? s[j] : 1.0f;
    s_out[j] = v;
    inv_out[j] = 1.0f / v;  // IEEE division: the correctly rounded reciprocal
}

hipError_t launch_prep_smooth(const float* s, int d_in, float* s_out, float* inv_out, hipStream_t st) {
    hipLaunchKernelGGL(smooth_kernel, dim3((d_in + 255) / 256), dim3(256), 0, st, s, d_in, s_out, inv_out);
    return hipGetLastError();
}

__global__ void fill_zero_kernel(uint32_t* __restrict__ p, size_t n_words) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n_words) p[i] = 0u;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
    const size_t n = bytes / 4;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       reinterpret_cast<uint32_t*>(p), n);
    return hipGetLastError();
}

}  // namespace qe
