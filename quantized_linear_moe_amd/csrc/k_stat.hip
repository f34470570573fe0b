// Calibration statistic of Quant Experts: per-token important channels
//   S_t = Top-k(|x_t| * w),  w = Mean_row(|W_f|)
// and the frequency with which every channel is selected (MCISLAB DeepRead
// summary, "Method", first paragraph; thelatestinai.com listing, Figure 3).
//
// Top-k: one workgroup per token.  Scores are non-negative float32, so their bit patterns
// order like unsigned integers.  A threshold below the k-th largest key (from the
// per-thread maxima of keys held in registers) leaves a short list that is ranked exactly
// under (score desc, index asc); mass ties or large k take an exact radix select.  The
// histogram is accumulated with integer atomics (deterministic counts).

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
// One workgroup of 512 threads per token.  Keys are the float32 bit patterns of |x| * |w|
// (non-negative floats order like unsigned integers; |w| makes w = -0 give +0, which compares
// equal to -0 as the definition's float comparison does), stored as key + 1 so that 0 marks
// "no channel".
//
// Fast path (k <= TK_FAST_K), keys in registers: thread tid holds channels
// (i * 512 + tid) * 8 + e, e < 8 (16-byte loads of x and w).  Each wave sorts its 64
// per-thread maxima (a bitonic network of lane shuffles) and takes the ceil(k/8)-th largest;
// tau = the smallest of the 8 waves' values.  At least 8 * ceil(k/8) >= k threads hold a key
// >= tau, so every top-k key is >= tau.  The keys >= tau are listed in LDS (one ballot, and
// one LDS atomic per wave and register that has any) and each listed key's rank under
// (key desc, channel asc) is counted against the list: for the top k these are their ranks
// among all keys, as every other key is below tau.
// Exact path (mass ties at tau overflow the list, or k is large), keys recomputed from
// memory in 512-channel chunks: an MSB-first radix select gives the k-th largest key tau*,
// every key > tau* is listed, then the lowest channels among the keys == tau* in channel
// order, and the k listed are ranked the same way.
constexpr int TK_THREADS = 512;
constexpr int TK_MAX_K = 1024;
constexpr int TK_MAX_D = 32768;
constexpr int TK_FAST_K = 256;
constexpr int TK_CAND = 1024;  // list length; holds any k <= TK_MAX_K for the exact path

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

struct TkShared {
    uint32_t bins[256];
    uint32_t wave_tot[TK_THREADS / 64];
    v2u cand[TK_CAND];  // (key + 1, channel)
    uint32_t prank[TK_THREADS / 64][128];  // partial ranks of short lists, one row per wave
    uint32_t count, prefix, remaining;
};

// key + 1 of channel j (0 when j is past the row)
__device__ inline uint32_t tk_key(const void* __restrict__ x, int x_dtype, const float* __restrict__ w, size_t row,
                                  int d_in, int j) {
    if (j >= d_in) return 0u;
    const float xv = x_dtype == QE_BF16 ? __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(x)[row + j] << 16)
                                        : reinterpret_cast<const float*>(x)[row + j];
    return __float_as_uint(__builtin_fabsf(xv) * __builtin_fabsf(w[j])) + 1u;
}

// Append (key, channel) to the list for the lanes with `take` set (list order: any).
__device__ inline void tk_append(TkShared& S, bool take, uint32_t key, int ch) {
    const int lane = threadIdx.x & 63;
    const uint64_t b = __ballot(take);
    if (b == 0) return;  // wave-uniform
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(&S.count, (uint32_t)__popcll(b));
    base = __shfl(base, 0, 64);
    if (take) {
        const uint32_t pos = base + (uint32_t)__popcll(b & ((1ull << lane) - 1ull));
        if (pos < TK_CAND) S.cand[pos] = v2u{key, (uint32_t)ch};
    }
}

// Rank every listed key under (key desc, channel asc); those ranked below k are the token's
// top k: written in rank order and counted in the histogram.  A list of up to 128 is split in
// 8 slices of 16: wave p counts, for every entry, the entries of slice p ahead of it, and the
// 8 partial counts are summed.  Longer lists: each entry counts the entries ahead of it,
// reading the list in batches of 16.
__device__ inline void tk_emit(TkShared& S, uint32_t n, int k, int t, int32_t* __restrict__ topk,
                               uint32_t* __restrict__ hist) {
    constexpr int B = 16;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    auto ahead = [](v2u o, v2u me) { return (o[0] > me[0]) || (o[0] == me[0] && o[1] < me[1]); };
    if (n <= 128) {
        v2u sl[B];
#pragma unroll
        for (int q = 0; q < B; ++q) {
            const uint32_t m = wid * B + q;
            sl[q] = m < n ? S.cand[m] : v2u{0u, 0u};  // listed keys are >= 1
        }
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const uint32_t c = lane + 64 * r;
            if (c < n) {
                const v2u me = S.cand[c];
                uint32_t cnt = 0;
#pragma unroll
                for (int q = 0; q < B; ++q) cnt += ahead(sl[q], me);
                S.prank[wid][c] = cnt;
            }
        }
        __syncthreads();
        if ((uint32_t)tid < n) {
            uint32_t rank = 0;
#pragma unroll
            for (int p = 0; p < TK_THREADS / 64; ++p) rank += S.prank[p][tid];
            if (rank < (uint32_t)k) {
                const uint32_t ic = S.cand[tid][1];
                if (topk) topk[(size_t)t * k + rank] = (int32_t)ic;
                atomicAdd(&hist[ic], 1u);
            }
        }
        return;
    }
    for (uint32_t c = tid; c < n; c += TK_THREADS) {
        const v2u me = S.cand[c];
        uint32_t rank = 0;
        for (uint32_t m0 = 0; m0 < n; m0 += B) {
            v2u o[B];
#pragma unroll
            for (int q = 0; q < B; ++q) o[q] = m0 + q < n ? S.cand[m0 + q] : v2u{0u, 0u};
#pragma unroll
            for (int q = 0; q < B; ++q) rank += ahead(o[q], me);
        }
        if (rank < (uint32_t)k) {
            if (topk) topk[(size_t)t * k + rank] = (int32_t)me[1];
            atomicAdd(&hist[me[1]], 1u);
        }
    }
}

// Largest-first order of one value per lane across the wave (bitonic network, lane shuffles).
__device__ inline uint32_t wave_sort_desc(uint32_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const uint32_t o = __shfl_xor(v, stride, 64);
            const bool keep_max = ((lane & stride) == 0) == ((lane & size) == 0);
            v = keep_max ? max(v, o) : min(v, o);
        }
    }
    return v;
}

// Exact selection of the token's top k from keys recomputed from memory (see above).
__device__ __attribute__((noinline)) void tk_exact(TkShared& S, const void* __restrict__ x, int x_dtype,
                                                   const float* __restrict__ w, int t, int d_in, int k,
                                                   int32_t* __restrict__ topk, uint32_t* __restrict__ hist) {
    const int tid = threadIdx.x;
    const size_t row = (size_t)t * d_in;
    // radix select of the k-th largest key
    uint32_t prefix = 0, mask = 0;
    if (tid == 0) S.remaining = (uint32_t)k;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        if (tid < 256) S.bins[tid] = 0;
        __syncthreads();
        for (int j = tid; j < d_in; j += TK_THREADS) {
            const uint32_t key = tk_key(x, x_dtype, w, row, d_in, j);
            if ((key & mask) == prefix) atomicAdd(&S.bins[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        // digit of the k-th largest: bins in descending order, one per thread; the thread whose
        // inclusive prefix first reaches the remaining count owns it (exactly one does)
        const uint32_t r = S.remaining;
        const uint32_t cnt = tid < 256 ? S.bins[255 - tid] : 0u;
        uint32_t total;
        const uint32_t excl = block_excl_scan(cnt, S.wave_tot, &total);
        if (tid < 256 && excl < r && excl + cnt >= r) {
            S.remaining = r - excl;
            S.prefix = prefix | ((uint32_t)(255 - tid) << shift);
        }
        __syncthreads();
        prefix = S.prefix;
        mask |= 255u << shift;
    }
    const uint32_t tau = prefix, need_eq = S.remaining;
    if (tid == 0) S.count = 0;
    __syncthreads();
    // keys above tau* (fewer than k), then the lowest channels among the keys equal to it
    for (int j0 = 0; j0 < d_in; j0 += TK_THREADS) {
        const uint32_t key = tk_key(x, x_dtype, w, row, d_in, j0 + tid);
        tk_append(S, key > tau, key, j0 + tid);
    }
    __syncthreads();
    const uint32_t ngt = S.count;
    uint32_t taken = 0;
    for (int j0 = 0; j0 < d_in && taken < need_eq; j0 += TK_THREADS) {  // block-uniform condition
        const uint32_t key = tk_key(x, x_dtype, w, row, d_in, j0 + tid);
        const uint32_t eq = key == tau ? 1u : 0u;
        uint32_t total;
        const uint32_t r = taken + block_excl_scan(eq, S.wave_tot, &total);
        if (eq && r < need_eq) S.cand[ngt + r] = v2u{tau, (uint32_t)(j0 + tid)};
        taken += total;
    }
    __syncthreads();
    tk_emit(S, (uint32_t)k, k, t, topk, hist);
}

template <int KPT>
__global__ __launch_bounds__(TK_THREADS, KPT >= 64 ? 2 : 4) void topk_kernel(
    const void* __restrict__ x, int x_dtype, const float* __restrict__ w, int T, int d_in, int k,
    int32_t* __restrict__ topk, uint32_t* __restrict__ hist) {
    __shared__ TkShared S;
    const int t = blockIdx.x, tid = threadIdx.x;
    if (k > TK_FAST_K) {
        tk_exact(S, x, x_dtype, w, t, d_in, k, topk, hist);
        return;
    }
    constexpr int NV = KPT / 8;  // 8-channel groups per thread
    const size_t row = (size_t)t * d_in;
    const bool vec = (d_in & 7) == 0;  // rows start 16-byte aligned

    uint32_t key[KPT];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int j0 = (i * TK_THREADS + tid) * 8;
        if (vec && j0 + 8 <= d_in) {
            const v4f w0 = *reinterpret_cast<const v4f*>(w + j0), w1 = *reinterpret_cast<const v4f*>(w + j0 + 4);
            float xv[8];
            if (x_dtype == QE_BF16) {
                const v4u q = *reinterpret_cast<const v4u*>(reinterpret_cast<const uint16_t*>(x) + row + j0);
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    xv[2 * h] = __uint_as_float(q[h] << 16);
                    xv[2 * h + 1] = __uint_as_float(q[h] & 0xFFFF0000u);
                }
            } else {
                const float* xr = reinterpret_cast<const float*>(x) + row + j0;
                const v4f a = *reinterpret_cast<const v4f*>(xr), b = *reinterpret_cast<const v4f*>(xr + 4);
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    xv[h] = a[h];
                    xv[4 + h] = b[h];
                }
            }
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                key[8 * i + h] = __float_as_uint(__builtin_fabsf(xv[h]) * __builtin_fabsf(w0[h])) + 1u;
                key[8 * i + 4 + h] = __float_as_uint(__builtin_fabsf(xv[4 + h]) * __builtin_fabsf(w1[h])) + 1u;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) key[8 * i + e] = tk_key(x, x_dtype, w, row, d_in, j0 + e);
        }
    }
    uint32_t m = 0u;
#pragma unroll
    for (int q = 0; q < KPT; ++q) m = max(m, key[q]);
    const uint32_t wtau = __shfl(wave_sort_desc(m), (k + 7) / 8 - 1, 64);
    if ((tid & 63) == 0) S.wave_tot[tid >> 6] = wtau;
    if (tid == 0) S.count = 0;
    __syncthreads();
    uint32_t tau = S.wave_tot[0];
#pragma unroll
    for (int w2 = 1; w2 < TK_THREADS / 64; ++w2) tau = min(tau, S.wave_tot[w2]);
    tau = max(tau, 1u);  // never list the padding
    // list the keys >= tau: per-thread counts, a wave scan, one LDS atomic per wave
    uint32_t cnt = 0;
#pragma unroll
    for (int q = 0; q < KPT; ++q) cnt += key[q] >= tau ? 1u : 0u;
    const int lane = tid & 63;
    uint32_t incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    const uint32_t wsum = __shfl(incl, 63, 64);
    uint32_t base = 0;
    if (lane == 0 && wsum) base = atomicAdd(&S.count, wsum);
    uint32_t pos = __shfl(base, 0, 64) + incl - cnt;
    if (cnt) {
#pragma unroll
        for (int q = 0; q < KPT; ++q)
            if (key[q] >= tau) {
                if (pos < TK_CAND) S.cand[pos] = v2u{key[q], (uint32_t)(((q >> 3) * TK_THREADS + tid) * 8 + (q & 7))};
                ++pos;
            }
    }
    __syncthreads();
    const uint32_t n = S.count;
    if (n <= TK_CAND) {  // block-uniform
        tk_emit(S, n, k, t, topk, hist);
        return;
    }
    __syncthreads();
    tk_exact(S, x, x_dtype, w, t, d_in, k, topk, hist);
}

hipError_t launch_topk(const void* x, int x_dtype, const float* w, int T, int d_in, int k, int32_t* topk,
                       uint32_t* hist, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if (d_in > TK_MAX_D || k > TK_MAX_K || k > d_in || k < 1) return hipErrorInvalidValue;
    const int per = (d_in + TK_THREADS * 8 - 1) / (TK_THREADS * 8);  // 8-channel groups per thread
    if (per <= 1) {
        hipLaunchKernelGGL(topk_kernel<8>, dim3(T), dim3(TK_THREADS), 0, st, x, x_dtype, w, T, d_in, k, topk, hist);
    } else if (per <= 2) {
        hipLaunchKernelGGL(topk_kernel<16>, dim3(T), dim3(TK_THREADS), 0, st, x, x_dtype, w, T, d_in, k, topk, hist);
    } else if (per <= 4) {
        hipLaunchKernelGGL(topk_kernel<32>, dim3(T), dim3(TK_THREADS), 0, st, x, x_dtype, w, T, d_in, k, topk, hist);
    } else {
        hipLaunchKernelGGL(topk_kernel<64>, dim3(T), dim3(TK_THREADS), 0, st, x, x_dtype, w, T, d_in, k, topk, hist);
    }
    return hipGetLastError();
}

}  // namespace qe
