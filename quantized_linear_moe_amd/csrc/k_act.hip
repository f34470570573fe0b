// Activation-side kernels of the QE linear:
//   * smoothing + per-token symmetric RTN quantization (step a1),
//   * the x-projection  P = bf16(x) . [A_s | A_1..A_N | R]  on bf16 MFMA
//     (inputs of the shared expert, the routed experts and the router),
//   * its reduction, the argmin router and the bf16 adapter inputs (a5, a4/a6),
//   * token bucketing by routed expert (counts, offsets, stable permutation).
//
// Method sources: MCISLAB DeepRead summary of Quant Experts, "Method" (scaling
// before activation quantization; shared expert on every token; router choosing
// the routed expert with the smallest predicted error); thelatestinai.com
// listing, Table 7 (dense adapters, one d x N_r router map per token).

#include <algorithm>

#include "qe_dma.h"
#include "qe_internal.h"

namespace qe {

// ---------------------------------------------------------------- helpers
__device__ inline float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// float32 -> bf16 bits, round to nearest even (inputs finite)
__device__ inline uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// a / b correctly rounded, given inv_b = RN(1/b).  One multiply and two fused
// multiply-adds (Markstein's correction).  Exact for |a| in [2^-100, 2^100] and b
// in [2^-90, 2^90] with quotients of magnitude >= 2^-3; callers fall back to the
// IEEE division outside that domain.
__device__ inline float div_markstein(float a, float b, float inv_b) {
    float q0 = a * inv_b;
    float r = __builtin_fmaf(-b, q0, a);
    return __builtin_fmaf(r, inv_b, q0);
}

__device__ inline bool in_markstein_range(float a) {
    float m = __builtin_fabsf(a);
    return (m >= 0x1p-100f && m <= 0x1p100f) || m == 0.0f;
}

// x / s exactly as IEEE float32 division
__device__ inline float smooth_div(float x, float s, float inv_s) {
    return in_markstein_range(x) ? div_markstein(x, s, inv_s) : x / s;
}

// load 8 consecutive activations as float
__device__ inline void load8(const void* x, int x_dtype, size_t idx, float out[8]) {
    if (x_dtype == QE_BF16) {
        v4u p = *reinterpret_cast<const v4u*>(reinterpret_cast<const uint16_t*>(x) + idx);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = __uint_as_float(p[i] << 16);
            out[2 * i + 1] = __uint_as_float(p[i] & 0xFFFF0000u);
        }
    } else {
        const v4f* p = reinterpret_cast<const v4f*>(reinterpret_cast<const float*>(x) + idx);
        v4f a = p[0], b = p[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[i] = a[i];
            out[4 + i] = b[i];
        }
    }
}

__device__ inline float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// ---------------------------------------------------------------- a1: quant
// One workgroup per token; each thread owns up to QA_IT groups of 8 consecutive
// channels, whose x' = x / s stays in registers between the two passes.
// Pass 1: x' and the token's max |x'|.  Pass 2: codes = clamp(rint(x' / s_x), +-qmax)
// with s_x = amax / qmax.  All float32 with IEEE division semantics (Markstein's
// correction, with the exact division as a wave-uniform fallback outside its
// verified domain) and round half to even.
constexpr int QA_IT = 4;

template <bool kHasInv>
__device__ inline void smooth8(const float* __restrict__ smooth, const float* __restrict__ inv_smooth, int j,
                               float v[8]) {
    const v4f s0 = *reinterpret_cast<const v4f*>(smooth + j), s1 = *reinterpret_cast<const v4f*>(smooth + j + 4);
    float s[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    float is[8];
    if (kHasInv) {
        const v4f i0 = *reinterpret_cast<const v4f*>(inv_smooth + j), i1 = *reinterpret_cast<const v4f*>(inv_smooth + j + 4);
        is[0] = i0[0]; is[1] = i0[1]; is[2] = i0[2]; is[3] = i0[3];
        is[4] = i1[0]; is[5] = i1[1]; is[6] = i1[2]; is[7] = i1[3];
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) is[i] = 1.0f / s[i];
    }
    bool ok = true;
    float r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        r[i] = div_markstein(v[i], s[i], is[i]);
        ok = ok && in_markstein_range(v[i]);
    }
    if (__builtin_expect(__any(!ok), 0)) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (!in_markstein_range(v[i])) r[i] = v[i] / s[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = r[i];
}

template <bool kHasInv>
__global__ __launch_bounds__(1024) void quant_act_kernel(const void* __restrict__ x, int x_dtype,
                                                         const float* __restrict__ smooth,
                                                         const float* __restrict__ inv_smooth, int T, int d_in,
                                                         int qmax, int8_t* __restrict__ codes,
                                                         float* __restrict__ s_x) {
    const int t = blockIdx.x;
    if (t >= T) return;
    const size_t row = (size_t)t * d_in;
    const int nthr = blockDim.x;
    __shared__ float red[1024 / kWave];
    __shared__ float s_bcast[2];

    float xv[QA_IT][8];
    float amax = 0.0f;
#pragma unroll
    for (int it = 0; it < QA_IT; ++it) {
        const int j = (it * nthr + threadIdx.x) * 8;
        if (j < d_in) {
            load8(x, x_dtype, row + j, xv[it]);
            if (smooth) smooth8<kHasInv>(smooth, inv_smooth, j, xv[it]);
#pragma unroll
            for (int i = 0; i < 8; ++i) amax = fmaxf(amax, __builtin_fabsf(xv[it][i]));
        }
    }
    amax = wave_max(amax);
    const int wid = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    if (lane == 0) red[wid] = amax;
    __syncthreads();
    if (threadIdx.x == 0) {
        float m = red[0];
        for (int i = 1; i < nthr / kWave; ++i) m = fmaxf(m, red[i]);
        const float sx = m / (float)qmax;
        s_bcast[0] = sx;
        s_bcast[1] = (sx != 0.0f) ? 1.0f / sx : 0.0f;
        s_x[t] = sx;
    }
    __syncthreads();
    const float sx = s_bcast[0], inv_sx = s_bcast[1];
    const bool fast = (sx >= 0x1p-90f && sx <= 0x1p90f);
    const float fq = (float)qmax;

#pragma unroll
    for (int it = 0; it < QA_IT; ++it) {
        const int j = (it * nthr + threadIdx.x) * 8;
        if (j >= d_in) continue;
        float r[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = div_markstein(xv[it][i], sx, inv_sx);
        if (!fast) {  // uniform over the workgroup
#pragma unroll
            for (int i = 0; i < 8; ++i) r[i] = xv[it][i] / sx;
        }
        uint32_t packed[2] = {0u, 0u};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float q = sx != 0.0f ? fminf(fmaxf(__builtin_rintf(r[i]), -fq), fq) : 0.0f;
            packed[i >> 2] |= ((uint32_t)(int32_t)q & 0xFFu) << (8 * (i & 3));
        }
        *reinterpret_cast<v2u*>(codes + row + j) = v2u{packed[0], packed[1]};
    }
}

hipError_t launch_quant_act(const void* x, int x_dtype, const float* smooth, const float* inv_smooth, int T,
                            int d_in, int a_bits, int8_t* codes, float* s_x, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    const int qmax = (1 << (a_bits - 1)) - 1;
    // enough threads that every channel group fits in QA_IT register slots
    const int groups = (d_in + 7) / 8;
    const int threads = ((groups + QA_IT - 1) / QA_IT + kWave - 1) / kWave * kWave;
    if (threads > 1024) return hipErrorInvalidValue;  // d_in > 32768: rejected by the caller
    if (inv_smooth || !smooth) {
        hipLaunchKernelGGL(quant_act_kernel<true>, dim3(T), dim3(threads), 0, st, x, x_dtype, smooth, inv_smooth, T,
                           d_in, qmax, codes, s_x);
    } else {
        hipLaunchKernelGGL(quant_act_kernel<false>, dim3(T), dim3(threads), 0, st, x, x_dtype, smooth, inv_smooth, T,
                           d_in, qmax, codes, s_x);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------- x-projection
// P[t][c] = sum_k bf16(x)[t][k] * Mt[col0 + c][k]  for c < ncols, as split-K
// partials part[ks][t][c] (float32).  bf16 MFMA 16x16x32, fp32 accumulation.
// Workgroup: 4 waves, 128 tokens x 320 columns (each wave all 128 tokens x 80
// columns).  The x tile (shared by the waves) is double-buffered through LDS in
// 128-wide K chunks; each wave streams its Mt rows (K-contiguous, 16 bytes per
// lane) straight into registers, one K step ahead of the MFMAs.
constexpr int XP_TOK = 128;      // tokens per workgroup
constexpr int XP_MB = XP_TOK / 16;
constexpr int XP_NBW = 5;        // 16-column blocks per wave
constexpr int XP_COLS = 4 * XP_NBW * 16;
constexpr int XP_KC = 64;        // K chunk staged in LDS
constexpr int XP_LDS_LD = XP_KC * 2 + 16;  // bytes per LDS row (padded against bank conflicts)

__device__ inline v4u load_x8_bf16(const void* x, int x_dtype, size_t idx) {
    if (x_dtype == QE_BF16) return *reinterpret_cast<const v4u*>(reinterpret_cast<const uint16_t*>(x) + idx);
    const v4f* p = reinterpret_cast<const v4f*>(reinterpret_cast<const float*>(x) + idx);
    const v4f a = p[0], b = p[1];
    v4u val;
    val[0] = f32_to_bf16_bits(a[0]) | (f32_to_bf16_bits(a[1]) << 16);
    val[1] = f32_to_bf16_bits(a[2]) | (f32_to_bf16_bits(a[3]) << 16);
    val[2] = f32_to_bf16_bits(b[0]) | (f32_to_bf16_bits(b[1]) << 16);
    val[3] = f32_to_bf16_bits(b[2]) | (f32_to_bf16_bits(b[3]) << 16);
    return val;
}

__global__ __launch_bounds__(256, 2) void xproj_kernel(const void* __restrict__ x, int x_dtype, int T, int d_in,
                                                       const uint16_t* __restrict__ mt, int col0, int ncols,
                                                       int ncols_pad, int ksplit, float* __restrict__ part) {
    __shared__ __attribute__((aligned(16))) uint8_t xs[2][XP_TOK * XP_LDS_LD];
    const int tile = blockIdx.x, ks = blockIdx.y, cgrp = blockIdx.z;
    const int tok0 = tile * XP_TOK;
    const int tid = threadIdx.x, wid = tid / kWave, lane = tid % kWave;
    const int lr = lane & 15, lg = lane >> 4;
    const int kb32 = d_in / 32;
    const int kbeg = (int)((long)ks * kb32 / ksplit) * 32;
    const int kend = (int)((long)(ks + 1) * kb32 / ksplit) * 32;
    const int cbase = cgrp * XP_COLS + wid * XP_NBW * 16;  // first column of this wave (relative to col0)

    // staging map: 4 x 16-byte loads per thread per chunk (128 rows x 8 chunks of 8 bf16)
    constexpr int XP_SL = XP_TOK * XP_KC / 8 / 256;
    auto stage = [&](int k0, v4u (&reg)[XP_SL]) {
#pragma unroll
        for (int p = 0; p < XP_SL; ++p) {
            const int i = p * 256 + tid, r = i / (XP_KC / 8), c8 = i % (XP_KC / 8);
            const int t = tok0 + r, k = k0 + c8 * 8;
            reg[p] = (t < T && k < kend) ? load_x8_bf16(x, x_dtype, (size_t)t * d_in + k) : v4u{0, 0, 0, 0};
        }
    };
    auto commit = [&](int buf, const v4u (&reg)[XP_SL]) {
#pragma unroll
        for (int p = 0; p < XP_SL; ++p) {
            const int i = p * 256 + tid, r = i / (XP_KC / 8), c8 = i % (XP_KC / 8);
            *reinterpret_cast<v4u*>(&xs[buf][r * XP_LDS_LD + c8 * 16]) = reg[p];
        }
    };
    const uint16_t* brow[XP_NBW];
    bool bok[XP_NBW];
#pragma unroll
    for (int n = 0; n < XP_NBW; ++n) {
        const int c = cbase + n * 16 + lr;
        bok[n] = c < ncols;
        brow[n] = mt + (size_t)(col0 + (bok[n] ? c : 0)) * d_in + lg * 8;
    }
    auto load_b = [&](int k, v8bf (&b)[XP_NBW]) {
#pragma unroll
        for (int n = 0; n < XP_NBW; ++n)
            b[n] = (bok[n] && k < kend) ? *reinterpret_cast<const v8bf*>(brow[n] + k) : v8bf{};
    };

    v4f acc[XP_MB][XP_NBW];
#pragma unroll
    for (int m = 0; m < XP_MB; ++m)
#pragma unroll
        for (int n = 0; n < XP_NBW; ++n) acc[m][n] = v4f{0, 0, 0, 0};

    v4u xr[XP_SL];
    v8bf bcur[XP_NBW], bnext[XP_NBW];
    stage(kbeg, xr);
    commit(0, xr);
    load_b(kbeg, bcur);
    __syncthreads();
    int buf = 0;
    for (int k0 = kbeg; k0 < kend; k0 += XP_KC) {
        const bool more = k0 + XP_KC < kend;
        if (more) stage(k0 + XP_KC, xr);
#pragma unroll
        for (int s = 0; s < XP_KC / 32; ++s) {
            const int k = k0 + s * 32;
            if (k >= kend) break;
            load_b(k + 32, bnext);
#pragma unroll
            for (int m = 0; m < XP_MB; ++m) {
                const v8bf a = *reinterpret_cast<const v8bf*>(&xs[buf][(m * 16 + lr) * XP_LDS_LD + (s * 32 + lg * 8) * 2]);
#pragma unroll
                for (int n = 0; n < XP_NBW; ++n)
                    acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bcur[n], acc[m][n], 0, 0, 0);
            }
#pragma unroll
            for (int n = 0; n < XP_NBW; ++n) bcur[n] = bnext[n];
        }
        if (more) commit(buf ^ 1, xr);
        __syncthreads();
        buf ^= 1;
    }
    // store partials: lane holds rows 4*lg + r, column lr of each 16x16 block
    float* out = part + (size_t)ks * T * ncols_pad;
#pragma unroll
    for (int m = 0; m < XP_MB; ++m)
#pragma unroll
        for (int n = 0; n < XP_NBW; ++n) {
            const int c = cbase + n * 16 + lr;
            if (c >= ncols_pad) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = tok0 + m * 16 + lg * 4 + r;
                if (t < T) out[(size_t)t * ncols_pad + c] = acc[m][n][r];
            }
        }
}

hipError_t launch_xproj(const void* x, int x_dtype, int T, int d_in, const uint16_t* mt, int col0, int ncols,
                        int ncols_pad, int ksplit, float* part, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    dim3 grid((T + XP_TOK - 1) / XP_TOK, ksplit, (ncols_pad + XP_COLS - 1) / XP_COLS);
    hipLaunchKernelGGL(xproj_kernel, grid, dim3(256), 0, st, x, x_dtype, T, d_in, mt, col0, ncols, ncols_pad, ksplit,
                       part);
    return hipGetLastError();
}

// ------------------------------------------------- x-projection reduction + router
// One workgroup per token: each thread reduces columns of the split-K partials in a
// fixed order, the router takes the argmin over its columns (lowest index on ties),
// and the bf16 adapter inputs of the shared and of the selected routed expert are written.
__global__ __launch_bounds__(1024) void xproj_finish_kernel(const float* __restrict__ part, int ksplit, int T,
                                                            int ncols_pad, int se_col, int r_s, int rs_pad, int re_col,
                                                            int n_r, int r_r, int rr_pad, int router_col,
                                                            const int32_t* __restrict__ expert_in,
                                                            float* __restrict__ scores, int32_t* __restrict__ expert_out,
                                                            uint16_t* __restrict__ u, uint16_t* __restrict__ v) {
    extern __shared__ float sums[];  // [4][ncols_pad]: quarter sums, then the total in row 0
    __shared__ int s_e;
    const int t = blockIdx.x;
    if (t >= T) return;
    const int q = threadIdx.x >> 8, c0 = threadIdx.x & 255;
    const int k0 = ksplit * q / 4, k1 = ksplit * (q + 1) / 4;
    const size_t stride = (size_t)T * ncols_pad;
    for (int c = c0; c < ncols_pad; c += 256) {
        const float* p = part + (size_t)t * ncols_pad + c;
        float s = 0.0f;
        int k = k0;
        for (; k + 4 <= k1; k += 4) {  // independent loads, summed in order
            const float a0 = p[(size_t)k * stride], a1 = p[(size_t)(k + 1) * stride];
            const float a2 = p[(size_t)(k + 2) * stride], a3 = p[(size_t)(k + 3) * stride];
            s += a0;
            s += a1;
            s += a2;
            s += a3;
        }
        for (; k < k1; ++k) s += p[(size_t)k * stride];
        sums[q * ncols_pad + c] = s;
    }
    __syncthreads();
    if (q == 0) {
        for (int c = c0; c < ncols_pad; c += 256)
            sums[c] = ((sums[c] + sums[ncols_pad + c]) + sums[2 * ncols_pad + c]) + sums[3 * ncols_pad + c];
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int e = 0;
        if (router_col >= 0) {
            float best = sums[router_col];
            for (int j = 1; j < n_r; ++j)
                if (sums[router_col + j] < best) {  // strict: the lowest index wins ties
                    best = sums[router_col + j];
                    e = j;
                }
            if (expert_out) expert_out[t] = e;
        } else if (expert_in) {
            e = min(max(expert_in[t], 0), max(n_r - 1, 0));
        }
        s_e = e;
    }
    if (scores && router_col >= 0 && threadIdx.x < n_r) scores[(size_t)t * n_r + threadIdx.x] = sums[router_col + threadIdx.x];
    __syncthreads();
    const int e = s_e;
    if (u && se_col >= 0) {
        for (int c = threadIdx.x; c < rs_pad; c += 1024)
            u[(size_t)t * rs_pad + c] = c < r_s ? (uint16_t)f32_to_bf16_bits(sums[se_col + c]) : (uint16_t)0;
    }
    if (v && re_col >= 0) {
        for (int c = threadIdx.x; c < rr_pad; c += 1024)
            v[(size_t)t * rr_pad + c] = c < r_r ? (uint16_t)f32_to_bf16_bits(sums[re_col + e * rr_pad + c]) : (uint16_t)0;
    }
}

hipError_t launch_xproj_finish(const float* part, int ksplit, int T, int ncols_pad, int col0, int se_col, int r_s,
                               int rs_pad, int re_col, int n_r, int r_r, int rr_pad, int router_col,
                               const int32_t* expert_in, float* scores, int32_t* expert_out, uint16_t* u,
                               uint16_t* v, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    // columns are relative to the projected block that starts at col0
    auto rel = [&](int c) { return c < 0 ? -1 : c - col0; };
    hipLaunchKernelGGL(xproj_finish_kernel, dim3(T), dim3(1024), 4 * (size_t)ncols_pad * sizeof(float), st, part, ksplit, T,
                       ncols_pad, rel(se_col), r_s, rs_pad, rel(re_col), n_r, r_r, rr_pad, rel(router_col), expert_in,
                       scores, expert_out, u, v);
    return hipGetLastError();
}

// ------------------------------------------------------- two-pass prologue (prefill)
// Pass 1 (route_pass): one read of x gives, per token and K split, the shared-expert and
// router projections (the first `ncols` rows of Mt: A_s^T, then R^T padded to 16 rows)
// and the partial max |x / s|.  route_finish turns them into the routed expert, u and
// s_x.  Pass 2 (expert_quant) walks the tokens in expert-sorted tiles and, in a second
// read of x, writes the activation codes and the selected routed expert's input v.

// raw storage of 8 consecutive activations, loaded ahead of use
template <int XDT>
struct Raw8;
template <>
struct Raw8<QE_BF16> {
    v4u b;
    __device__ void load(const void* x, size_t idx) { b = *reinterpret_cast<const v4u*>(reinterpret_cast<const uint16_t*>(x) + idx); }
    __device__ void zero() { b = v4u{0, 0, 0, 0}; }
    __device__ void get(float out[8]) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = __uint_as_float(b[i] << 16);
            out[2 * i + 1] = __uint_as_float(b[i] & 0xFFFF0000u);
        }
    }
};
template <>
struct Raw8<QE_F32> {
    v4f a, b;
    __device__ void load(const void* x, size_t idx) {
        const v4f* p = reinterpret_cast<const v4f*>(reinterpret_cast<const float*>(x) + idx);
        a = p[0];
        b = p[1];
    }
    __device__ void zero() { a = b = v4f{0, 0, 0, 0}; }
    __device__ void get(float out[8]) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[i] = a[i];
            out[4 + i] = b[i];
        }
    }
};

__device__ inline v4u pack_bf16x8(const float v[8]) {
    v4u r;
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = f32_to_bf16_bits(v[2 * q]) | (f32_to_bf16_bits(v[2 * q + 1]) << 16);
    return r;
}

constexpr int RP_TOK = 64;             // tokens per workgroup
constexpr int RP_KC = 64;              // K chunk staged in LDS
constexpr int RP_LD = RP_KC * 2 + 16;  // LDS row stride (bytes)
constexpr int RP_MAXN = 5;             // up to 80 projected columns
constexpr int RP_MCH = (RP_MAXN * 16 * 8 + 255) / 256;  // Mt chunks per thread

template <int XDT>
__global__ __launch_bounds__(256) void route_pass_kernel(const void* __restrict__ x, int T, int d_in,
                                                         const uint16_t* __restrict__ mt, int ncols,
                                                         const float* __restrict__ smooth,
                                                         const float* __restrict__ inv_smooth, int ksplit,
                                                         float* __restrict__ part, float* __restrict__ amax_part) {
    __shared__ __attribute__((aligned(16))) uint8_t xs[RP_TOK * RP_LD];
    __shared__ __attribute__((aligned(16))) uint8_t ms[RP_MAXN * 16 * RP_LD];
    const int tok0 = blockIdx.x * RP_TOK, ks = blockIdx.y;
    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int nch = d_in / RP_KC;
    const int kbeg = (int)((long)ks * nch / ksplit) * RP_KC, kend = (int)((long)(ks + 1) * nch / ksplit) * RP_KC;
    const int nbk = ncols / 16;
    const int c8 = tid & 7;
    int trow[2];
    bool tval[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        trow[p] = tok0 + (tid >> 3) + 32 * p;
        tval[p] = trow[p] < T;
    }

    v4f acc[RP_MAXN];
#pragma unroll
    for (int n = 0; n < RP_MAXN; ++n) acc[n] = v4f{0, 0, 0, 0};
    float amax[2] = {0.0f, 0.0f};

    // registers holding the next chunk: two x groups of 8, up to RP_MCH Mt groups of 8
    Raw8<XDT> xr[2];
    v4u mr[RP_MCH];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            if (tval[p]) xr[p].load(x, (size_t)trow[p] * d_in + k0 + c8 * 8);
            else xr[p].zero();
        }
#pragma unroll
        for (int j = 0; j < RP_MCH; ++j) {
            const int i = tid + 256 * j, r = i >> 3;
            if (r < ncols) mr[j] = *reinterpret_cast<const v4u*>(mt + (size_t)r * d_in + k0 + (i & 7) * 8);
        }
    };
    if (kbeg < kend) fetch(kbeg);
    for (int k0 = kbeg; k0 < kend; k0 += RP_KC) {
        __syncthreads();  // previous chunk's MFMAs are done with the LDS tiles
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            float v[8];
            xr[p].get(v);
            *reinterpret_cast<v4u*>(xs + ((tid >> 3) + 32 * p) * RP_LD + c8 * 16) = pack_bf16x8(v);
            if (tval[p]) {
                smooth8<true>(smooth, inv_smooth, k0 + c8 * 8, v);
#pragma unroll
                for (int i = 0; i < 8; ++i) amax[p] = fmaxf(amax[p], __builtin_fabsf(v[i]));
            }
        }
#pragma unroll
        for (int j = 0; j < RP_MCH; ++j) {
            const int i = tid + 256 * j, r = i >> 3;
            if (r < ncols) *reinterpret_cast<v4u*>(ms + r * RP_LD + (i & 7) * 16) = mr[j];
        }
        __syncthreads();
        if (k0 + RP_KC < kend) fetch(k0 + RP_KC);  // in flight during the MFMAs
#pragma unroll
        for (int s = 0; s < RP_KC / 32; ++s) {
            const v8bf a = *reinterpret_cast<const v8bf*>(xs + (wid * 16 + lr) * RP_LD + (s * 32 + lg * 8) * 2);
#pragma unroll
            for (int n = 0; n < RP_MAXN; ++n) {
                if (n >= nbk) break;
                const v8bf b = *reinterpret_cast<const v8bf*>(ms + (n * 16 + lr) * RP_LD + (s * 32 + lg * 8) * 2);
                acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[n], 0, 0, 0);
            }
        }
    }
    float* out = part + (size_t)ks * T * ncols;
#pragma unroll
    for (int n = 0; n < RP_MAXN; ++n) {
        if (n >= nbk) break;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = tok0 + wid * 16 + lg * 4 + r;
            if (t < T) out[(size_t)t * ncols + n * 16 + lr] = acc[n][r];
        }
    }
    // the 8 threads of a token row are 8 consecutive lanes
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        float m = amax[p];
        m = fmaxf(m, __shfl_xor(m, 1, 64));
        m = fmaxf(m, __shfl_xor(m, 2, 64));
        m = fmaxf(m, __shfl_xor(m, 4, 64));
        if (c8 == 0 && tval[p]) amax_part[(size_t)ks * T + trow[p]] = m;
    }
}

int route_pass_ksplit(int T, int d_in) {
    const int tiles = (T + RP_TOK - 1) / RP_TOK;
    const int ks = std::min((1024 + tiles - 1) / tiles, std::max(1, d_in / 256));
    return std::max(ks, 1);
}

hipError_t launch_route_pass(const void* x, int x_dtype, int T, int d_in, const uint16_t* mt, int ncols,
                             const float* smooth, const float* inv_smooth, int ksplit, float* part, float* amax_part,
                             hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if (ncols > RP_MAXN * 16 || ncols % 16 || d_in % RP_KC || !smooth || !inv_smooth) return hipErrorInvalidValue;
    const dim3 grid((T + RP_TOK - 1) / RP_TOK, ksplit);
    if (x_dtype == QE_BF16)
        hipLaunchKernelGGL(route_pass_kernel<QE_BF16>, grid, dim3(256), 0, st, x, T, d_in, mt, ncols, smooth,
                           inv_smooth, ksplit, part, amax_part);
    else
        hipLaunchKernelGGL(route_pass_kernel<QE_F32>, grid, dim3(256), 0, st, x, T, d_in, mt, ncols, smooth,
                           inv_smooth, ksplit, part, amax_part);
    return hipGetLastError();
}

// One wave per token: fixed-order split-K sums, router argmin (lowest index on ties),
// u = bf16(shared projection), s_x = max |x/s| / qmax (a max is exact in any order).
__global__ __launch_bounds__(256) void route_finish_kernel(const float* __restrict__ part,
                                                           const float* __restrict__ amax_part, int ksplit, int T,
                                                           int ncols, int r_s, int rs_pad, int router_col, int n_r,
                                                           int qmax, int32_t* __restrict__ expert,
                                                           uint16_t* __restrict__ u, float* __restrict__ s_x) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (t >= T) return;
    // columns lane and lane + 64 (ncols <= 80)
    float sum[2] = {0.0f, 0.0f};
    const size_t stride = (size_t)T * ncols;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int c = lane + 64 * j;
        if (c < ncols) {
            const float* p = part + (size_t)t * ncols + c;
            for (int k = 0; k < ksplit; ++k) sum[j] += p[(size_t)k * stride];
        }
    }
    if (router_col >= 0) {
        float best = __builtin_inff();
        int bi = 1 << 30;
#pragma unroll
        for (int j = 0; j < 2; ++j) {  // lane's own candidates, lower column first
            const int c = lane + 64 * j;
            if (c >= router_col && c < router_col + n_r && (sum[j] < best || bi == 1 << 30)) {
                best = sum[j];
                bi = c - router_col;
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float ob = __shfl_xor(best, off, 64);
            const int oi = __shfl_xor(bi, off, 64);
            if (ob < best || (ob == best && oi < bi)) {
                best = ob;
                bi = oi;
            }
        }
        if (lane == 0) expert[t] = bi;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int c = lane + 64 * j;
        if (u && c < rs_pad) u[(size_t)t * rs_pad + c] = c < r_s ? (uint16_t)f32_to_bf16_bits(sum[j]) : (uint16_t)0;
    }
    float m = 0.0f;
    for (int k = lane; k < ksplit; k += 64) m = fmaxf(m, amax_part[(size_t)k * T + t]);
    m = wave_max(m);
    if (lane == 0) s_x[t] = m / (float)qmax;
}

hipError_t launch_route_finish(const float* part, const float* amax_part, int ksplit, int T, int ncols, int r_s,
                               int rs_pad, int router_col, int n_r, int a_bits, int32_t* expert, uint16_t* u,
                               float* s_x, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(route_finish_kernel, dim3((T + 3) / 4), dim3(256), 0, st, part, amax_part, ksplit, T, ncols,
                       r_s, rs_pad, router_col, n_r, (1 << (a_bits - 1)) - 1, expert, u, s_x);
    return hipGetLastError();
}

// Pass 2.  A workgroup takes 128 token rows in `perm` order (tokens grouped by expert),
// one 16-row block per wave, and a K range walked in 32-wide steps by all 8 waves
// together.  Per step a lane owns 8 consecutive channels of one row: it writes their
// codes (x / s, then / s_x, round half to even, clamp -- the float32 operations of the
// activation quantization kernel) and feeds bf16(x) to the MFMAs of v = x . A_e.  The
// experts present in the tile are taken up to 8/NBR at a time; each MFMA sees only the
// rows of its expert (A masked), so one accumulator collects every row's own expert
// exactly.  x, the expert fragments (shared by the 8 row blocks) and the smoothing
// factors of each step reach LDS by DMA through a 4-stage ring, three steps ahead,
// with explicit waits and no staging registers.  With K split over workgroups the
// partial v go to `vpart` and vpart_finish adds them in K order.
constexpr int EQ_W = 8;              // waves per workgroup
constexpr int EQ_ROWS = 16 * EQ_W;   // token rows per workgroup
constexpr int EQ_NS = 4;             // ring stages

template <int XDT, int NBR>
__global__ __launch_bounds__(64 * EQ_W) void expert_quant_kernel(
    const void* __restrict__ x, int T, int d_in, const float* __restrict__ smooth,
    const float* __restrict__ inv_smooth, const float* __restrict__ s_x, int qmax, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ expert, int n_r, const uint16_t* __restrict__ mt_re, int r_r, int ksq,
    float* __restrict__ vpart, int8_t* __restrict__ codes, uint16_t* __restrict__ v) {
    constexpr int XOPS = XDT == QE_BF16 ? 1 : 2;  // 1 KB copies of x per wave and step
    constexpr int RR = NBR * 16;                  // padded routed rank
    constexpr int ESLOTS = NBR ? EQ_W / NBR : 1;  // experts per pass
    constexpr int X_STAGE = EQ_W * XOPS * 1024;
    constexpr int B_STAGE = NBR ? EQ_W * 1024 : 0;
    constexpr int S_STAGE = EQ_W * 256;
    constexpr int STAGE = X_STAGE + B_STAGE + S_STAGE;
    constexpr int OPS = XOPS + (NBR ? 1 : 0) + 1;  // DMA instructions per wave and step
    constexpr int ESZ = XDT == QE_BF16 ? 2 : 4;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[EQ_NS * STAGE];
    __shared__ uint32_t s_pres[EQ_W];

    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int tile = blockIdx.x, kq = blockIdx.y;
    const int pos0 = tile * EQ_ROWS;
    const int pos = pos0 + wid * 16 + lr;
    const bool valid = pos < T;
    const int t = valid ? (perm ? perm[pos] : pos) : 0;  // rows past T read row 0 and are never stored
    const int e_row = (NBR && valid && expert) ? min(max(expert[t], 0), n_r - 1) : -1;
    const float sx = valid ? s_x[t] : 0.0f;
    const float inv_sx = sx != 0.0f ? 1.0f / sx : 0.0f;
    const bool fast = sx >= 0x1p-90f && sx <= 0x1p90f;
    const float fq = (float)qmax;
    uint32_t pres = 0;
    if (NBR)
        for (int e = 0; e < n_r; ++e)
            if (__ballot(e_row == e)) pres |= 1u << e;
    if (lane == 0) s_pres[wid] = pres;
    __syncthreads();
    uint32_t present = 0;
#pragma unroll
    for (int w = 0; w < EQ_W; ++w) present |= s_pres[w];

    const int nsteps = d_in / 32;
    const int g0 = (int)((long)kq * nsteps / ksq), g1 = (int)((long)(kq + 1) * nsteps / ksq);
    const int nst = g1 - g0;  // >= 1: ksq <= nsteps
    const uint32_t lds0 = lds_addr(smem);
    const char* xsrc = reinterpret_cast<const char*>(x) + ((size_t)t * d_in + lg * 8) * ESZ;
    const float* ssrc = lane < 32 ? smooth + lane : inv_smooth + (lane - 32);
    int8_t* crow = codes + (size_t)t * d_in + lg * 8;

    v4f acc[NBR ? NBR : 1];
#pragma unroll
    for (int n = 0; n < (NBR ? NBR : 1); ++n) acc[n] = v4f{0, 0, 0, 0};

    uint32_t pm = present;
    bool first = true;
    do {  // passes over the present experts; the codes are written on the first
        int ex[ESLOTS];
#pragma unroll
        for (int j = 0; j < ESLOTS; ++j) {
            ex[j] = -1;
            if (NBR && pm) {
                ex[j] = __builtin_ctz(pm);
                pm &= pm - 1;
            }
        }
        // this wave's expert-fragment copy: slot wid / NBR, column block wid % NBR
        int my_e = max(ex[0], 0);  // empty slots repeat a present expert (never used)
#pragma unroll
        for (int j = 1; j < ESLOTS; ++j)
            if (j == wid / (NBR ? NBR : 1) && ex[j] >= 0) my_e = ex[j];
        const uint16_t* bsrc =
            NBR ? mt_re + ((size_t)my_e * RR + (wid % (NBR ? NBR : 1)) * 16 + lr) * d_in + lg * 8 : nullptr;
        auto issue = [&](int stage, int step) {
            const uint32_t base = lds0 + stage * STAGE;
            const size_t k = (size_t)step * 32;
#pragma unroll
            for (int o = 0; o < XOPS; ++o) dma16(xsrc + k * ESZ + o * 16, base + (wid * XOPS + o) * 1024);
            if (NBR) dma16(bsrc + k, base + X_STAGE + wid * 1024);
            dma4(ssrc + k, base + X_STAGE + B_STAGE + wid * 256);
        };
#pragma unroll
        for (int st = 0; st < EQ_NS - 1; ++st) issue(st, g0 + min(st, nst - 1));
        QE_WAIT_VMCNT_LDS((EQ_NS - 2) * OPS);
        QE_WG_BARRIER();

        for (int i = 0; i < nst; ++i) {
            // refill the slot consumed in the previous step (past the end: a harmless repeat)
            issue((i + EQ_NS - 1) % EQ_NS, g0 + min(i + EQ_NS - 1, nst - 1));
            const uint8_t* st = smem + (i % EQ_NS) * STAGE;
            float xc[8];
            if (XDT == QE_BF16) {
                Raw8<QE_BF16> r;
                r.b = *reinterpret_cast<const v4u*>(st + wid * 1024 + lane * 16);
                r.get(xc);
            } else {
                Raw8<QE_F32> r;
                r.a = *reinterpret_cast<const v4f*>(st + wid * 2048 + lane * 16);
                r.b = *reinterpret_cast<const v4f*>(st + wid * 2048 + 1024 + lane * 16);
                r.get(xc);
            }
            const uint8_t* sp = st + X_STAGE + B_STAGE + wid * 256 + lg * 32;
            const v4f s0 = *reinterpret_cast<const v4f*>(sp), s1 = *reinterpret_cast<const v4f*>(sp + 16);
            const v4f i0 = *reinterpret_cast<const v4f*>(sp + 128), i1 = *reinterpret_cast<const v4f*>(sp + 144);
            const v4u abits = pack_bf16x8(xc);
            if (first) {
                // codes: x' = x / s, q = clamp(rint(x' / s_x))
                float xs8[8];
                bool ok = true;
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const float sq = q < 4 ? s0[q] : s1[q - 4], iq = q < 4 ? i0[q] : i1[q - 4];
                    xs8[q] = div_markstein(xc[q], sq, iq);
                    ok = ok && in_markstein_range(xc[q]);
                }
                if (__builtin_expect(__any(!ok), 0)) {
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const float sq = q < 4 ? s0[q] : s1[q - 4];
                        if (!in_markstein_range(xc[q])) xs8[q] = xc[q] / sq;
                    }
                }
                uint32_t packed[2] = {0u, 0u};
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    float qv = 0.0f;
                    if (sx != 0.0f) {
                        const float r = fast ? div_markstein(xs8[q], sx, inv_sx) : xs8[q] / sx;
                        qv = fminf(fmaxf(__builtin_rintf(r), -fq), fq);
                    }
                    packed[q >> 2] |= ((uint32_t)(int32_t)qv & 0xFFu) << (8 * (q & 3));
                }
                if (valid) *reinterpret_cast<v2u*>(crow + (size_t)(g0 + i) * 32) = v2u{packed[0], packed[1]};
            }
            if (NBR) {
                const v4u zero4 = v4u{0, 0, 0, 0};
#pragma unroll
                for (int j = 0; j < ESLOTS; ++j) {
                    if (ex[j] < 0) break;  // uniform
                    const v4u am = e_row == ex[j] ? abits : zero4;
#pragma unroll
                    for (int n = 0; n < (NBR ? NBR : 1); ++n) {
                        const v8bf bq = *reinterpret_cast<const v8bf*>(st + X_STAGE + (j * NBR + n) * 1024 + lane * 16);
                        acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const v8bf*>(&am), bq,
                                                                         acc[n], 0, 0, 0);
                    }
                }
            }
            // the slot read here is the DMA target of the next step: every LDS read must
            // have completed (lgkmcnt 0); and step i+1 must have landed
            __builtin_amdgcn_sched_barrier(0);
            QE_WAIT_VMCNT_LDS((EQ_NS - 2) * OPS);
            QE_WG_BARRIER();
        }
        QE_WAIT_VMCNT(0);  // the repeated tail copies, before the ring is refilled or freed
        QE_WG_BARRIER();
        first = false;
    } while (pm);
    if (NBR == 0 || !v) return;

    // lane holds column n*16 + lr and rows 4*lg + r of the wave's block
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = lg * 4 + r;
        const int tt = __shfl(valid ? t : -1, row, 64);
        const int p = pos0 + wid * 16 + row;
#pragma unroll
        for (int n = 0; n < (NBR ? NBR : 1); ++n) {
            const int c = n * 16 + lr;
            if (ksq == 1) {
                if (tt >= 0) v[(size_t)tt * RR + c] = c < r_r ? (uint16_t)f32_to_bf16_bits(acc[n][r]) : (uint16_t)0;
            } else if (p < T) {
                vpart[((size_t)kq * T + p) * RR + c] = acc[n][r];
            }
        }
    }
}

// v[perm[pos]][c] = bf16(sum over q, in order, of vpart[q][pos][c])
__global__ __launch_bounds__(256) void vpart_finish_kernel(const float* __restrict__ vpart, int ksq, int T, int rr_pad,
                                                           int r_r, const int32_t* __restrict__ perm,
                                                           uint16_t* __restrict__ v) {
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)T * rr_pad) return;
    const int pos = (int)(idx / rr_pad), c = (int)(idx % rr_pad);
    float a = 0.0f;
    for (int q = 0; q < ksq; ++q) a += vpart[(size_t)q * T * rr_pad + idx];
    const int tt = perm ? perm[pos] : pos;
    v[(size_t)tt * rr_pad + c] = c < r_r ? (uint16_t)f32_to_bf16_bits(a) : (uint16_t)0;
}

int expert_quant_ksplit(int T, int d_in) {
    const int tiles = (T + EQ_ROWS - 1) / EQ_ROWS;
    const int ks = std::min((512 + tiles - 1) / tiles, std::max(1, d_in / 32 / 8));
    return std::max(ks, 1);
}

template <int XDT>
static hipError_t launch_eq(dim3 grid, hipStream_t st, int nbr, const void* x, int T, int d_in, const float* smooth,
                            const float* inv_smooth, const float* s_x, int qmax, const int32_t* perm,
                            const int32_t* expert, int n_r, const uint16_t* mt_re, int r_r, int ksq, float* vpart,
                            int8_t* codes, uint16_t* v) {
#define QE_EQ_LAUNCH(NB)                                                                                            \
    hipLaunchKernelGGL((expert_quant_kernel<XDT, NB>), grid, dim3(64 * EQ_W), 0, st, x, T, d_in, smooth,           \
                       inv_smooth, s_x, qmax, perm, expert, n_r, mt_re, r_r, ksq, vpart, codes, v)
    if (nbr == 0) QE_EQ_LAUNCH(0);
    else if (nbr == 2) QE_EQ_LAUNCH(2);
    else QE_EQ_LAUNCH(4);
#undef QE_EQ_LAUNCH
    return hipGetLastError();
}

hipError_t launch_expert_quant(const void* x, int x_dtype, int T, int d_in, const float* smooth,
                               const float* inv_smooth, const float* s_x, int a_bits, const int32_t* perm,
                               const int32_t* expert, int n_r, const uint16_t* mt_re, int rr_pad, int r_r, int ksq,
                               float* vpart, int8_t* codes, uint16_t* v, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    const int nbr = (expert && v) ? rr_pad / 16 : 0;
    if ((nbr != 0 && nbr != 2 && nbr != 4) || d_in % 32 || ksq < 1 || ksq > d_in / 32 || n_r > kMaxRouted || !smooth ||
        !inv_smooth)
        return hipErrorInvalidValue;
    if (ksq > 1 && nbr && !vpart) return hipErrorInvalidValue;
    const dim3 grid((T + EQ_ROWS - 1) / EQ_ROWS, ksq);
    const int qmax = (1 << (a_bits - 1)) - 1;
    hipError_t err = x_dtype == QE_BF16
                         ? launch_eq<QE_BF16>(grid, st, nbr, x, T, d_in, smooth, inv_smooth, s_x, qmax, perm, expert,
                                              n_r, mt_re, r_r, ksq, vpart, codes, v)
                         : launch_eq<QE_F32>(grid, st, nbr, x, T, d_in, smooth, inv_smooth, s_x, qmax, perm, expert,
                                             n_r, mt_re, r_r, ksq, vpart, codes, v);
    if (err != hipSuccess || ksq == 1 || !nbr) return err;
    const size_t n = (size_t)T * rr_pad;
    hipLaunchKernelGGL(vpart_finish_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, vpart, ksq, T, rr_pad,
                       r_r, perm, v);
    return hipGetLastError();
}

// ---------------------------------------------------------------- bucketing
// Single workgroup: counts, exclusive offsets and the permutation of tokens
// sorted by (expert, token index), built chunk by chunk in token order.
__global__ __launch_bounds__(1024) void bucket_kernel(const int32_t* __restrict__ expert, int T, int n_r,
                                                      int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ perm) {
    __shared__ int cnt[kMaxRouted];
    __shared__ int base[kMaxRouted];
    __shared__ int wave_cnt[16][kMaxRouted];
    const int tid = threadIdx.x, wid = tid / kWave, lane = tid % kWave;
    if (tid < kMaxRouted) cnt[tid] = 0;
    __syncthreads();
    for (int t = tid; t < T; t += 1024) atomicAdd(&cnt[min(max(expert[t], 0), n_r - 1)], 1);
    __syncthreads();
    if (tid == 0) {
        int acc = 0;
        for (int e = 0; e < n_r; ++e) {
            base[e] = acc;
            offsets[e] = acc;
            counts[e] = cnt[e];
            acc += cnt[e];
        }
        offsets[n_r] = acc;
    }
    __syncthreads();
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int c0 = 0; c0 < T; c0 += 1024) {
        const int t = c0 + tid;
        const int e = t < T ? min(max(expert[t], 0), n_r - 1) : -1;
        // per-wave counts of each expert
        for (int k = 0; k < n_r; ++k) {
            uint64_t bal = __ballot(e == k);
            if (lane == 0) wave_cnt[wid][k] = __popcll(bal);
        }
        __syncthreads();
        int rank = 0;
        if (e >= 0) {
            for (int w = 0; w < wid; ++w) rank += wave_cnt[w][e];
        }
        // rank within the wave among lanes with the same expert
        for (int k = 0; k < n_r; ++k) {
            uint64_t bal = __ballot(e == k);
            if (e == k) rank += __popcll(bal & lt_mask);
        }
        if (e >= 0) perm[base[e] + rank] = t;
        __syncthreads();
        if (tid < n_r) {
            int tot = 0;
            for (int w = 0; w < 16; ++w) tot += wave_cnt[w][tid];
            base[tid] += tot;
        }
        __syncthreads();
    }
}

hipError_t launch_bucket(const int32_t* expert, int T, int n_r, int32_t* counts, int32_t* offsets, int32_t* perm,
                         hipStream_t st) {
    hipLaunchKernelGGL(bucket_kernel, dim3(1), dim3(1024), 0, st, expert, T, n_r, counts, offsets, perm);
    return hipGetLastError();
}

}  // namespace qe
