// Calibration statistic of Quant Experts: per-token important channels
//   S_t = Top-k(|x_t| * w),  w = Mean_row(|W_f|)
// and the frequency with which every channel is selected (MCISLAB DeepRead
// summary, "Method", first paragraph; thelatestinai.com listing, Figure 3).
//
// Top-k: one workgroup per token.  Scores are non-negative float32, so their bit
// patterns order like unsigned integers; an exact MSB-first radix select (four
// 8-bit digit passes over the keys held in LDS) finds the k-th largest key tau.
// All keys > tau are taken, then the lowest channel indices among keys == tau
// (an ordered block scan), which implements the (score desc, index asc) order
// exactly.  The k selected channels are ordered by rank counting and the
// histogram is accumulated with integer atomics (deterministic).

#include "qe_internal.h"

namespace qe {

// ----------------------------------------------------------------- column mean
// w[j] = (sum_i |W[i][j]|) / d_out in float64, rounded once to float32.
// 64 columns per workgroup; the 4 waves sum interleaved rows, combined in a fixed order.
__global__ __launch_bounds__(256) void colmean_kernel(const void* __restrict__ W, int dtype, int d_out, int d_in,
                                                      float* __restrict__ w) {
    __shared__ double part[4][64];
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int j = blockIdx.x * 64 + lane;
    double s = 0.0;
    if (j < d_in) {
        for (int i = wid; i < d_out; i += 4) {
            const size_t idx = (size_t)i * d_in + j;
            float f = dtype == QE_BF16 ? __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(W)[idx] << 16)
                                       : reinterpret_cast<const float*>(W)[idx];
            s += (double)__builtin_fabsf(f);
        }
    }
    part[wid][lane] = s;
    __syncthreads();
    if (wid == 0 && j < d_in) {
        double tot = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
        w[j] = (float)(tot / (double)d_out);
    }
}

hipError_t launch_colmean(const void* W, int dtype, int d_out, int d_in, float* w, hipStream_t st) {
    hipLaunchKernelGGL(colmean_kernel, dim3((d_in + 63) / 64), dim3(256), 0, st, W, dtype, d_out, d_in, w);
    return hipGetLastError();
}

// ----------------------------------------------------------------------- top-k
constexpr int TK_THREADS = 256;  // one thread per radix bin in the digit search
constexpr int TK_MAX_K = 1024;
constexpr int TK_MAX_D = 32768;

__device__ inline uint32_t block_excl_scan(uint32_t v, uint32_t* wave_tot, uint32_t* total) {
    const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
    uint32_t incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        uint32_t o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    if (lane == 63) wave_tot[wid] = incl;
    __syncthreads();
    uint32_t base = 0, tot = 0;
    for (int w2 = 0; w2 < TK_THREADS / 64; ++w2) {
        if (w2 < wid) base += wave_tot[w2];
        tot += wave_tot[w2];
    }
    *total = tot;
    __syncthreads();
    return base + incl - v;
}

__global__ __launch_bounds__(TK_THREADS) void topk_kernel(const void* __restrict__ x, int x_dtype,
                                                          const float* __restrict__ w, int T, int d_in, int k,
                                                          int32_t* __restrict__ topk, uint32_t* __restrict__ hist) {
    extern __shared__ __attribute__((aligned(16))) uint32_t keys[];  // [d_in]
    __shared__ uint32_t bins[256];
    __shared__ uint32_t sel_key[TK_MAX_K];
    __shared__ int32_t sel_idx[TK_MAX_K];
    __shared__ uint32_t wave_tot[TK_THREADS / 64];
    __shared__ uint32_t s_prefix, s_remaining, s_ngt;
    const int t = blockIdx.x;
    const int tid = threadIdx.x;
    const size_t row = (size_t)t * d_in;

    for (int j = tid; j < d_in; j += TK_THREADS) {
        const float xv = x_dtype == QE_BF16 ? __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(x)[row + j] << 16)
                                            : reinterpret_cast<const float*>(x)[row + j];
        uint32_t key = __float_as_uint(__builtin_fabsf(xv) * w[j]);
        keys[j] = (key == 0x80000000u) ? 0u : key;  // -0 orders as +0
    }
    if (tid == 0) {
        s_prefix = 0;
        s_remaining = (uint32_t)k;
        s_ngt = 0;
    }
    __syncthreads();

    uint32_t prefix = 0, mask = 0;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        bins[tid] = 0;
        __syncthreads();
        for (int j = tid; j < d_in; j += TK_THREADS) {
            const uint32_t key = keys[j];
            if ((key & mask) == prefix) atomicAdd(&bins[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        // digit of the k-th largest: bins in descending order, one per thread; the thread
        // whose inclusive prefix first reaches the remaining count owns it (exactly one does,
        // as the bins hold every key still matching the prefix)
        {
            const uint32_t rem = s_remaining;
            const uint32_t cnt = bins[255 - tid];
            uint32_t total;
            const uint32_t excl = block_excl_scan(cnt, wave_tot, &total);
            if (excl < rem && excl + cnt >= rem) {
                s_remaining = rem - excl;
                s_prefix = prefix | ((uint32_t)(255 - tid) << shift);
            }
        }
        __syncthreads();
        prefix = s_prefix;
        mask |= 255u << shift;
    }
    const uint32_t tau = prefix;
    const uint32_t need_eq = s_remaining;  // keys equal to tau to take, lowest indices first

    // keys strictly above tau (any order; ranked below)
    for (int j = tid; j < d_in; j += TK_THREADS) {
        const uint32_t key = keys[j];
        if (key > tau) {
            const uint32_t pos = atomicAdd(&s_ngt, 1u);
            if (pos < (uint32_t)k) {
                sel_key[pos] = key;
                sel_idx[pos] = j;
            }
        }
    }
    __syncthreads();
    const uint32_t ngt = s_ngt;
    // keys equal to tau: contiguous chunks per thread, ordered by an exclusive scan
    const int chunk = (d_in + TK_THREADS - 1) / TK_THREADS;
    const int jb = min(d_in, tid * chunk), je = min(d_in, jb + chunk);
    uint32_t cnt = 0;
    for (int j = jb; j < je; ++j) cnt += keys[j] == tau;
    uint32_t total;
    uint32_t r = block_excl_scan(cnt, wave_tot, &total);
    for (int j = jb; j < je && r < need_eq; ++j) {
        if (keys[j] == tau && ngt + r < (uint32_t)k) {
            sel_key[ngt + r] = tau;
            sel_idx[ngt + r] = j;
            ++r;
        }
    }
    __syncthreads();
    // order by (key desc, index asc) and emit
    for (int i = tid; i < k; i += TK_THREADS) {
        const uint32_t ki = sel_key[i];
        const int ii = sel_idx[i];
        int rank = 0;
        for (int m = 0; m < k; ++m) {
            const uint32_t km = sel_key[m];
            rank += (km > ki) || (km == ki && sel_idx[m] < ii);
        }
        if (topk) topk[(size_t)t * k + rank] = ii;
        atomicAdd(&hist[ii], 1u);
    }
}

hipError_t launch_topk(const void* x, int x_dtype, const float* w, int T, int d_in, int k, int32_t* topk,
                       uint32_t* hist, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    const size_t lds = (size_t)d_in * sizeof(uint32_t);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(topk_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)(TK_MAX_D * sizeof(uint32_t)));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_kernel, dim3(T), dim3(TK_THREADS), lds, st, x, x_dtype, w, T, d_in, k, topk, hist);
    return hipGetLastError();
}

}  // namespace qe
