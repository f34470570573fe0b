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
#include "qe_splits.h"

namespace qe {

// ---------------------------------------------------------------- helpers
__device__ inline float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

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
// 16-column blocks per wave: 5 (320 columns per workgroup), or 4 for column counts that are a
// multiple of 256 (the routed experts' 8 x 32 input columns), which 5 would pad by a quarter
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

template <int XP_NBW>
__global__ __launch_bounds__(256, 2) void xproj_kernel(const void* __restrict__ x, int x_dtype, int T, int d_in,
                                                       const uint16_t* __restrict__ mt, int col0, int ncols,
                                                       int ncols_pad, int ksplit, float* __restrict__ part) {
    constexpr int XP_COLS = 4 * XP_NBW * 16;
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
    if (ncols_pad % 256 == 0) {
        dim3 grid((T + XP_TOK - 1) / XP_TOK, ksplit, ncols_pad / 256);
        hipLaunchKernelGGL(xproj_kernel<4>, grid, dim3(256), 0, st, x, x_dtype, T, d_in, mt, col0, ncols, ncols_pad,
                           ksplit, part);
    } else {
        dim3 grid((T + XP_TOK - 1) / XP_TOK, ksplit, (ncols_pad + 319) / 320);
        hipLaunchKernelGGL(xproj_kernel<5>, grid, dim3(256), 0, st, x, x_dtype, T, d_in, mt, col0, ncols, ncols_pad,
                           ksplit, part);
    }
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
                                                            uint16_t* __restrict__ u, uint16_t* __restrict__ v,
                                                            int32_t* __restrict__ expert2_out) {
    extern __shared__ float sums[];  // [nq][ncols_pad]: partial sums over split ranges, then the total in row 0
    __shared__ int s_e;
    const int t = blockIdx.x;
    if (t >= T) return;
    const int nq = blockDim.x >> 8;  // 1 or 4 ranges of splits
    const int q = threadIdx.x >> 8, c0 = threadIdx.x & 255;
    const int k0 = ksplit * q / nq, k1 = ksplit * (q + 1) / nq;
    const size_t stride = (size_t)T * ncols_pad;
    // Columns this call reads: only the router's when nothing else is written, only the shared
    // and the given expert's columns when the expert comes in; else every column.
    const bool only_router = router_col >= 0 && !u && !v;
    const int e_in = (router_col < 0 && expert_in) ? min(max(expert_in[t], 0), max(n_r - 1, 0)) : -1;
    auto for_cols = [&](auto&& f) {
        if (only_router) {
            for (int c = c0; c < n_r; c += 256) f(router_col + c);
        } else if (e_in >= 0) {
            if (u && se_col >= 0)
                for (int c = c0; c < rs_pad; c += 256) f(se_col + c);
            if (v && re_col >= 0)
                for (int c = c0; c < rr_pad; c += 256) f(re_col + e_in * rr_pad + c);
        } else {
            for (int c = c0; c < ncols_pad; c += 256) f(c);
        }
    };
    for_cols([&](int c) {
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
    });
    __syncthreads();
    if (q == 0 && nq == 4)
        for_cols([&](int c) {
            sums[c] = ((sums[c] + sums[ncols_pad + c]) + sums[2 * ncols_pad + c]) + sums[3 * ncols_pad + c];
        });
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
            if (expert2_out) {  // top-2 routing: the best of the others, lowest index on ties
                int e2 = -1;
                float b2 = 0.0f;
                for (int j = 0; j < n_r; ++j)
                    if (j != e && (e2 < 0 || sums[router_col + j] < b2)) {
                        b2 = sums[router_col + j];
                        e2 = j;
                    }
                expert2_out[t] = e2;
            }
        } else if (expert_in) {
            e = min(max(expert_in[t], 0), max(n_r - 1, 0));
        }
        s_e = e;
    }
    if (scores && router_col >= 0 && threadIdx.x < n_r) scores[(size_t)t * n_r + threadIdx.x] = sums[router_col + threadIdx.x];
    __syncthreads();
    const int e = s_e;
    if (u && se_col >= 0) {
        for (int c = threadIdx.x; c < rs_pad; c += blockDim.x)
            u[(size_t)t * rs_pad + c] = c < r_s ? (uint16_t)f32_to_bf16_bits(sums[se_col + c]) : (uint16_t)0;
    }
    if (v && re_col >= 0) {
        for (int c = threadIdx.x; c < rr_pad; c += blockDim.x)
            v[(size_t)t * rr_pad + c] = c < r_r ? (uint16_t)f32_to_bf16_bits(sums[re_col + e * rr_pad + c]) : (uint16_t)0;
    }
}

hipError_t launch_xproj_finish(const float* part, int ksplit, int T, int ncols_pad, int col0, int se_col, int r_s,
                               int rs_pad, int re_col, int n_r, int r_r, int rr_pad, int router_col,
                               const int32_t* expert_in, float* scores, int32_t* expert_out, uint16_t* u,
                               uint16_t* v, hipStream_t st, int32_t* expert2_out) {
    if (T <= 0) return hipSuccess;
    if (expert2_out && (router_col < 0 || n_r < 2)) return hipErrorInvalidValue;
    // columns are relative to the projected block that starts at col0
    auto rel = [&](int c) { return c < 0 ? -1 : c - col0; };
    // a call that reads only a few columns (router alone, or one known expert) takes one wave
    // group per token: the dispatch of 16 waves per token would cost more than its loads
    const bool few = (router_col >= 0 && !u && !v) || (router_col < 0 && expert_in);
    const int nq = few ? 1 : 4;
    hipLaunchKernelGGL(xproj_finish_kernel, dim3(T), dim3(256 * nq), nq * (size_t)ncols_pad * sizeof(float), st, part, ksplit, T,
                       ncols_pad, rel(se_col), r_s, rs_pad, rel(re_col), n_r, r_r, rr_pad, rel(router_col), expert_in,
                       scores, expert_out, u, v, expert2_out);
    return hipGetLastError();
}

// ------------------------------------------------------- two-pass prologue (prefill)
// For bf16 activations.  Pass 1 (route_pass): one read of x gives, per token and K
// split, the shared-expert and router projections (the first `ncols` rows of Mt: A_s^T,
// then R^T padded to 16 rows) and the partial max |x / s|.  route_finish turns them into
// the routed expert, u and s_x.  Pass 2 (expert_quant) walks the tokens in expert-sorted
// tiles and, in a second read of x, writes the activation codes and the selected routed
// expert's input v.  Both passes move their operands global -> LDS by DMA through a
// ring of stages with explicit waits, so no load is waited for in the step that uses
// it, and keep per-element arithmetic to the exact float32 operations plus a packed
// range check.

typedef uint16_t v2u16 __attribute__((ext_vector_type(2)));

__device__ inline void bf16x8_unpack(const v4u w, float o[8]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        o[2 * q] = __uint_as_float(w[q] << 16);
        o[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
    }
}

// True when each of the 8 bf16 values is zero or has |x| in [2^-100, 2^100): the domain
// where div_markstein(x, s, 1/s) is the correctly rounded x / s.  Two packed 16-bit
// operations per value: the magnitudes' maximum bounds the exponent from above, the
// minimum of (magnitude - 1) from below while letting zero through (it wraps to 0xFFFF).
__device__ inline bool bf16x8_markstein_ok(const v4u w) {
    v2u16 mx = v2u16{0, 0}, mn = v2u16{0xFFFF, 0xFFFF};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const v2u16 m = __builtin_bit_cast(v2u16, (uint32_t)(w[q] & 0x7FFF7FFFu));
        mx = __builtin_elementwise_max(mx, m);
        mn = __builtin_elementwise_min(mn, m - v2u16{1, 1});
    }
    constexpr uint16_t kHi = (226 << 7) | 0x7F;  // largest magnitude with exponent 2^99
    constexpr uint16_t kLo = (27 << 7) - 1;      // (smallest magnitude 2^-100) - 1
    return mx[0] <= kHi && mx[1] <= kHi && mn[0] >= kLo && mn[1] >= kLo;
}

// x' = x / s for 8 values (x exact in bf16), correctly rounded
__device__ inline void smooth_div8(const v4u w, const v4f s0, const v4f s1, const v4f i0, const v4f i1, float o[8]) {
    float xv[8];
    bf16x8_unpack(w, xv);
    const bool ok = bf16x8_markstein_ok(w);
#pragma unroll
    for (int q = 0; q < 8; ++q) o[q] = div_markstein(xv[q], q < 4 ? s0[q] : s1[q - 4], q < 4 ? i0[q] : i1[q - 4]);
    if (__builtin_expect(__any(!ok), 0)) {
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (!in_markstein_range(xv[q])) o[q] = xv[q] / (q < 4 ? s0[q] : s1[q - 4]);
    }
}

// Codes of 8 smoothed values: clamp(rint(x' / s_x), +-qmax) as int8.  The clamp is a
// med3; adding 1.5 * 2^23 rounds the clamped value to an integer (round half to even,
// the float adder's own rounding) and leaves it in the low mantissa bits, whose low
// byte is the two's complement code.
__device__ inline v2u codes8(const float xs[8], float sx, float inv_sx, bool fast, float fq) {
    float r[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) r[q] = div_markstein(xs[q], sx, inv_sx);
    if (__builtin_expect(__any(!fast), 0)) {  // a wave-uniform branch keeps the division off the common path
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (!fast) r[q] = xs[q] / sx;
    }
    uint32_t cb[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) cb[q] = __float_as_uint(__builtin_amdgcn_fmed3f(r[q], -fq, fq) + 12582912.0f);
    v2u out;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t lo = __builtin_amdgcn_perm(cb[4 * h + 1], cb[4 * h], 0x0c0c0400u);
        const uint32_t hi = __builtin_amdgcn_perm(cb[4 * h + 3], cb[4 * h + 2], 0x0c0c0400u);
        out[h] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    }
    return out;
}

// ---- pass 1
// Workgroup: 64 consecutive tokens (wave w: tokens 16w..16w+15) x a K range, walked in
// groups of 128 channels.  The MFMA sums over K, so the channels of a group may be dealt
// to lanes and steps in any order that A and B share: lane (row l%16, g = l/16) takes
// channels 32g..32g+31 of its row, 8 per step.  x therefore goes straight from memory to
// the A registers (64 contiguous bytes per lane), and the same registers give the
// lane's max |x / s|.  The projection rows of the group and its smoothing factors are
// loaded by all threads in one burst and staged in double-buffered LDS (16-byte chunks
// XOR-swizzled by (row & 15)), one barrier per group.
constexpr int RP_TOK = 64;
constexpr int RP_KG = 128;             // channels per group
constexpr int RP_MAXN = 5;             // up to 80 projected columns

template <int NBK>  // 16-row blocks of projection rows (ncols = 16*NBK <= 80); also the 16-B pieces per thread
__global__ __launch_bounds__(256) void route_pass_kernel(const uint16_t* __restrict__ x, int T, int d_in,
                                                         const uint16_t* __restrict__ mt, int ncols,
                                                         const float* __restrict__ smooth,
                                                         const float* __restrict__ inv_smooth, int ksplit,
                                                         float* __restrict__ part, float* __restrict__ amax_part) {
    constexpr int MP = NBK;  // ncols*16 chunks of 16 B over 256 threads
    constexpr int M_LDS = MP * 256 * 16;
    constexpr int BUF = M_LDS + 1024;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * BUF];
    const int tok0 = blockIdx.x * RP_TOK, ks = blockIdx.y;
    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int ngr = d_in / RP_KG;
    const int g_beg = (int)((long)ks * ngr / ksplit), g_end = (int)((long)(ks + 1) * ngr / ksplit);
    const int row = tok0 + wid * 16 + lr;
    const bool rvalid = row < T;
    const uint16_t* xrow = x + (size_t)min(row, T - 1) * d_in + lg * 32;  // rows past T repeat a valid row

    v4f acc[NBK > 0 ? NBK : 1];
#pragma unroll
    for (int n = 0; n < (NBK > 0 ? NBK : 1); ++n) acc[n] = v4f{0, 0, 0, 0};
    float amax = 0.0f;

    // group g+1's loads are issued before group g is processed (two register sets; loads
    // past the range repeat the last group and are not used)
    struct Regs {
        v4u x[4], m[MP > 0 ? MP : 1];
        v4f s;
    };
    const uint16_t* msrc = ncols > 0 ? mt : x;  // without projection rows: any valid data, never used
    auto load = [&](Regs& R, int g) {
        const size_t k0 = (size_t)g * RP_KG;
#pragma unroll
        for (int q = 0; q < 4; ++q) R.x[q] = *reinterpret_cast<const v4u*>(xrow + k0 + q * 8);
#pragma unroll
        for (int p = 0; p < MP; ++p) {
            const int idx = tid + 256 * p, r = idx >> 4, c = idx & 15;
            R.m[p] = *reinterpret_cast<const v4u*>(msrc + (size_t)min(r, max(ncols - 1, 0)) * d_in + k0 + c * 8);
        }
        R.s = *reinterpret_cast<const v4f*>(((tid & 32) ? inv_smooth : smooth) + k0 + (tid & 31) * 4);
    };
    auto process = [&](const Regs& R, int g) {
        uint8_t* buf = smem + (g & 1) * BUF;
#pragma unroll
        for (int p = 0; p < MP; ++p) {
            const int idx = tid + 256 * p, r = idx >> 4, c = idx & 15;
            if (r < ncols) *reinterpret_cast<v4u*>(buf + r * 256 + ((c ^ (r & 15)) << 4)) = R.m[p];
        }
        if (tid < 64) *reinterpret_cast<v4f*>(buf + M_LDS + tid * 16) = R.s;
        // the stores above are complete in every wave (the other buffer was last read
        // before this barrier); the next group's loads stay in flight
        QE_WAIT_LDS();
        QE_WG_BARRIER();
        if (rvalid) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint8_t* sp = buf + M_LDS + (lg * 32 + q * 8) * 4;
                const v4f s0 = *reinterpret_cast<const v4f*>(sp), s1 = *reinterpret_cast<const v4f*>(sp + 16);
                const v4f i0 = *reinterpret_cast<const v4f*>(sp + 512), i1 = *reinterpret_cast<const v4f*>(sp + 528);
                float xs[8];
                smooth_div8(R.x[q], s0, s1, i0, i1, xs);
#pragma unroll
                for (int e = 0; e < 8; ++e) amax = fmaxf(amax, __builtin_fabsf(xs[e]));
            }
        }
        v8bf bv[4][NBK > 0 ? NBK : 1];  // all B fragments of the group first, then the MFMAs
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int n = 0; n < NBK; ++n) {
                const int rm = n * 16 + lr;
                bv[q][n] = *reinterpret_cast<const v8bf*>(buf + rm * 256 + (((lg * 4 + q) ^ (rm & 15)) << 4));
            }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int n = 0; n < NBK; ++n)
                acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const v8bf*>(&R.x[q]), bv[q][n],
                                                                 acc[n], 0, 0, 0);
    };
    if (g_beg < g_end) {
        Regs A, B;
        load(A, g_beg);
        for (int g = g_beg; g < g_end; g += 2) {
            load(B, min(g + 1, g_end - 1));
            process(A, g);
            load(A, min(g + 2, g_end - 1));
            if (g + 1 < g_end) process(B, g + 1);
        }
    }

    float* out = part + (size_t)ks * T * ncols;
#pragma unroll
    for (int n = 0; n < NBK; ++n) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = tok0 + wid * 16 + lg * 4 + r;
            if (t < T) out[(size_t)t * ncols + n * 16 + lr] = acc[n][r];
        }
    }
    // a row's 128 channels are spread over lanes lr, lr+16, lr+32, lr+48
    float m = amax;
    m = fmaxf(m, __shfl_xor(m, 16, 64));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    if (lg == 0 && rvalid) amax_part[(size_t)ks * T + row] = m;
}

// About two workgroups per compute unit (measured faster than three at 4096 tokens), at least
// two channel groups each, and at most
// 16 splits: the finish kernel loads up to 16 partials of a column at once.
int route_pass_ksplit(int T, int d_in) {
    const int tiles = (T + RP_TOK - 1) / RP_TOK;
    const int ks = std::min({(512 + tiles - 1) / tiles, std::max(1, d_in / (2 * RP_KG)), 16});
    return std::max(ks, 1);
}

hipError_t launch_route_pass(const uint16_t* x, int T, int d_in, const uint16_t* mt, int ncols, const float* smooth,
                             const float* inv_smooth, int ksplit, float* part, float* amax_part, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if (ncols > RP_MAXN * 16 || ncols % 16 || d_in % RP_KG || ksplit < 1 || ksplit > d_in / RP_KG || !smooth ||
        !inv_smooth)
        return hipErrorInvalidValue;
    const dim3 grid((T + RP_TOK - 1) / RP_TOK, ksplit);
#define QE_RP_LAUNCH(NB)                                                                                            \
    hipLaunchKernelGGL(route_pass_kernel<NB>, grid, dim3(256), 0, st, x, T, d_in, mt, ncols, smooth, inv_smooth, \
                       ksplit, part, amax_part)
    switch (ncols / 16) {
        case 0: QE_RP_LAUNCH(0); break;
        case 1: QE_RP_LAUNCH(1); break;
        case 2: QE_RP_LAUNCH(2); break;
        case 3: QE_RP_LAUNCH(3); break;
        case 4: QE_RP_LAUNCH(4); break;
        default: QE_RP_LAUNCH(5); break;
    }
#undef QE_RP_LAUNCH
    return hipGetLastError();
}

// ---- pass 1 for a group of linears that read the same input (q/k/v, gate/up)
// The same tile as route_pass_kernel, for up to RG_MAX linears at once: x is read once per
// 128-channel group and feeds every linear's projection MFMAs (its shared-expert and router
// rows) and every linear's max |x / s_l| (each linear has its own smoothing).  Each linear's
// projection rows and smoothing factors are staged in their own slice of the double-buffered
// LDS; its partial sums go to its own buffers, laid out exactly as route_pass_kernel's.
template <int NL, int NBK>
__global__ __launch_bounds__(256, 2) void route_pass_group_kernel(const uint16_t* __restrict__ x, int T, int d_in,
                                                               RouteGroup G, int ksplit) {
    constexpr int MP = NBK;
    constexpr int M_LDS = MP * 256 * 16;
    constexpr int LBUF = M_LDS + 1024;  // one linear's rows and smoothing factors
    constexpr int BUF = NL * LBUF;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * BUF];
    const int tok0 = blockIdx.x * RP_TOK, ks = blockIdx.y;
    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int ngr = d_in / RP_KG;
    const int g_beg = (int)((long)ks * ngr / ksplit), g_end = (int)((long)(ks + 1) * ngr / ksplit);
    const int row = tok0 + wid * 16 + lr;
    const bool rvalid = row < T;
    const uint16_t* xrow = x + (size_t)min(row, T - 1) * d_in + lg * 32;  // rows past T repeat a valid row

    v4f acc[NL][NBK];
#pragma unroll
    for (int l = 0; l < NL; ++l)
#pragma unroll
        for (int n = 0; n < NBK; ++n) acc[l][n] = v4f{0, 0, 0, 0};
    float amax[NL];
#pragma unroll
    for (int l = 0; l < NL; ++l) amax[l] = 0.0f;

    // x is double-buffered in registers (the next group's rows are requested before a group is
    // processed); each linear's projection rows and smoothing factors are single-buffered: the
    // next group's are requested right after the barrier that retires the current ones, so
    // they are in flight during the current group's arithmetic
    v4u m[NL][MP];
    v4f sv[NL];
    auto load_x = [&](v4u (&xr)[4], int g) {
        const size_t k0 = (size_t)g * RP_KG;
#pragma unroll
        for (int q = 0; q < 4; ++q) xr[q] = *reinterpret_cast<const v4u*>(xrow + k0 + q * 8);
    };
    auto load_m = [&](int g) {
        const size_t k0 = (size_t)g * RP_KG;
#pragma unroll
        for (int l = 0; l < NL; ++l) {
#pragma unroll
            for (int p = 0; p < MP; ++p) {
                const int idx = tid + 256 * p, r = idx >> 4, c = idx & 15;
                m[l][p] = *reinterpret_cast<const v4u*>(G.mt[l] + (size_t)min(r, G.ncols[l] - 1) * d_in + k0 + c * 8);
            }
            sv[l] = *reinterpret_cast<const v4f*>(((tid & 32) ? G.inv_smooth[l] : G.smooth[l]) + k0 + (tid & 31) * 4);
        }
    };
    auto process = [&](const v4u (&xr)[4], int g) {
        uint8_t* buf = smem + (g & 1) * BUF;
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            uint8_t* lb = buf + l * LBUF;
#pragma unroll
            for (int p = 0; p < MP; ++p) {
                const int idx = tid + 256 * p, r = idx >> 4, c = idx & 15;
                if (r < G.ncols[l]) *reinterpret_cast<v4u*>(lb + r * 256 + ((c ^ (r & 15)) << 4)) = m[l][p];
            }
            if (tid < 64) *reinterpret_cast<v4f*>(lb + M_LDS + tid * 16) = sv[l];
        }
        QE_WAIT_LDS();
        QE_WG_BARRIER();
        load_m(min(g + 1, g_end - 1));  // past the range: a harmless repeat of the last group
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            const uint8_t* lb = buf + l * LBUF;
            if (rvalid) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint8_t* sp = lb + M_LDS + (lg * 32 + q * 8) * 4;
                    const v4f s0 = *reinterpret_cast<const v4f*>(sp), s1 = *reinterpret_cast<const v4f*>(sp + 16);
                    const v4f i0 = *reinterpret_cast<const v4f*>(sp + 512), i1 = *reinterpret_cast<const v4f*>(sp + 528);
                    float xs[8];
                    smooth_div8(xr[q], s0, s1, i0, i1, xs);
#pragma unroll
                    for (int e = 0; e < 8; ++e) amax[l] = fmaxf(amax[l], __builtin_fabsf(xs[e]));
                }
            }
            v8bf bv[4][NBK];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int n = 0; n < NBK; ++n) {
                    const int rm = n * 16 + lr;
                    bv[q][n] = *reinterpret_cast<const v8bf*>(lb + rm * 256 + (((lg * 4 + q) ^ (rm & 15)) << 4));
                }
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int n = 0; n < NBK; ++n)
                    acc[l][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const v8bf*>(&xr[q]),
                                                                        bv[q][n], acc[l][n], 0, 0, 0);
        }
    };
    if (g_beg < g_end) {
        v4u xa[4], xb[4];
        load_x(xa, g_beg);
        load_m(g_beg);
        for (int g = g_beg; g < g_end; g += 2) {
            load_x(xb, min(g + 1, g_end - 1));
            process(xa, g);
            load_x(xa, min(g + 2, g_end - 1));
            if (g + 1 < g_end) process(xb, g + 1);
        }
    }

#pragma unroll
    for (int l = 0; l < NL; ++l) {
        const int nc = G.ncols[l];
        float* out = G.part[l] + (size_t)ks * T * nc;
#pragma unroll
        for (int n = 0; n < NBK; ++n) {
            if (n * 16 >= nc) break;  // uniform
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = tok0 + wid * 16 + lg * 4 + r;
                if (t < T) out[(size_t)t * nc + n * 16 + lr] = acc[l][n][r];
            }
        }
        float m = amax[l];
        m = fmaxf(m, __shfl_xor(m, 16, 64));
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        if (lg == 0 && rvalid) G.amax[l][(size_t)ks * T + row] = m;
    }
}

hipError_t launch_route_pass_group(const uint16_t* x, int T, int d_in, const RouteGroup& G, int n_lin, int ksplit,
                                   hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if (n_lin < 2 || n_lin > RG_MAX || d_in % RP_KG || ksplit < 1 || ksplit > d_in / RP_KG) return hipErrorInvalidValue;
    int nbk = 0;
    for (int l = 0; l < n_lin; ++l) {
        if (G.ncols[l] < 16 || G.ncols[l] > RP_MAXN * 16 || G.ncols[l] % 16 || !G.smooth[l] || !G.inv_smooth[l] ||
            !G.mt[l] || !G.part[l] || !G.amax[l])
            return hipErrorInvalidValue;
        nbk = std::max(nbk, G.ncols[l] / 16);
    }
    if (nbk > 3) return hipErrorInvalidValue;  // the grouped tile holds up to 48 projected columns per linear
    const dim3 grid((T + RP_TOK - 1) / RP_TOK, ksplit);
#define QE_RPG_LAUNCH(NLV, NB) \
    hipLaunchKernelGGL((route_pass_group_kernel<NLV, NB>), grid, dim3(256), 0, st, x, T, d_in, G, ksplit)
    if (n_lin == 2) {
        if (nbk == 1) QE_RPG_LAUNCH(2, 1);
        else if (nbk == 2) QE_RPG_LAUNCH(2, 2);
        else QE_RPG_LAUNCH(2, 3);
    } else {
        if (nbk == 1) QE_RPG_LAUNCH(3, 1);
        else if (nbk == 2) QE_RPG_LAUNCH(3, 2);
        else QE_RPG_LAUNCH(3, 3);
    }
#undef QE_RPG_LAUNCH
    return hipGetLastError();
}

// The route finish of RF_TOK consecutive tokens t0 .. t0 + RF_TOK - 1 per workgroup: the
// partial sums of each split are one contiguous block of RF_TOK * ncols floats, read as 16-byte
// vectors, one per thread and split, every split's load in flight together; each thread adds
// its vector's splits in split order starting from zero (the same float32 sums, bit for bit, as
// a sequential sum over the splits), then the sums go through LDS to the per-token steps:
// router argmin (lowest index on ties; for top-2 also the best of the others), u = bf16 of the
// shared projection, s_x = max |x/s| / qmax (a max is exact in any order).
constexpr int RF_TOK = 16;
constexpr int RF_THREADS = 256;

__device__ __forceinline__ void route_finish_block(const float* __restrict__ part, const float* __restrict__ amax_part,
                                                   int ksplit, int T, int ncols, int r_s, int rs_pad, int router_col,
                                                   int n_r, int qmax, int32_t* __restrict__ expert,
                                                   uint16_t* __restrict__ u, float* __restrict__ s_x,
                                                   int32_t* __restrict__ expert2, int t0) {
    __shared__ __attribute__((aligned(16))) float s_sum[RF_TOK * RP_MAXN * 16];
    const int tid = threadIdx.x;
    const int nt = min(RF_TOK, T - t0);
    if (nt <= 0) return;  // uniform
    const int nvec = nt * ncols / 4;  // ncols is a multiple of 16
    const size_t stride = (size_t)T * ncols / 4;  // one split, in 16-byte vectors
    const v4f* blk = reinterpret_cast<const v4f*>(part + (size_t)t0 * ncols);
    constexpr int B = 16;
    for (int i = tid; i < nvec; i += RF_THREADS) {
        v4f sum = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        for (int k0 = 0; k0 < ksplit; k0 += B) {
            v4f a[B];
#pragma unroll
            for (int q = 0; q < B; ++q) a[q] = k0 + q < ksplit ? blk[(size_t)(k0 + q) * stride + i] : v4f{0, 0, 0, 0};
#pragma unroll
            for (int q = 0; q < B; ++q)
                if (k0 + q < ksplit) sum += a[q];
        }
        *reinterpret_cast<v4f*>(s_sum + 4 * i) = sum;
    }
    float m = 0.0f;
    if (tid < nt)
        for (int k = 0; k < ksplit; ++k) m = fmaxf(m, amax_part[(size_t)k * T + t0 + tid]);
    __syncthreads();
    if (tid < nt) {
        const int t = t0 + tid;
        const float* sc = s_sum + tid * ncols;
        if (router_col >= 0) {
            int e = 0;
            float best = sc[router_col];
            for (int j = 1; j < n_r; ++j)
                if (sc[router_col + j] < best) {
                    best = sc[router_col + j];
                    e = j;
                }
            expert[t] = e;
            if (expert2) {  // top-2 routing: the best of the other experts, lowest index on ties
                int e2 = -1;
                float b2 = 0.0f;
                for (int j = 0; j < n_r; ++j)
                    if (j != e && (e2 < 0 || sc[router_col + j] < b2)) {
                        b2 = sc[router_col + j];
                        e2 = j;
                    }
                expert2[t] = e2;
            }
        }
        s_x[t] = m / (float)qmax;
    }
    if (u) {
        for (int i = tid; i < nt * rs_pad; i += RF_THREADS) {
            const int tt = i / rs_pad, c = i - tt * rs_pad;
            u[(size_t)(t0 + tt) * rs_pad + c] = c < r_s ? (uint16_t)f32_to_bf16_bits(s_sum[tt * ncols + c]) : (uint16_t)0;
        }
    }
}

__global__ __launch_bounds__(RF_THREADS) void route_finish_kernel(const float* __restrict__ part,
                                                                  const float* __restrict__ amax_part, int ksplit,
                                                                  int T, int ncols, int r_s, int rs_pad,
                                                                  int router_col, int n_r, int qmax,
                                                                  int32_t* __restrict__ expert,
                                                                  uint16_t* __restrict__ u, float* __restrict__ s_x,
                                                                  int32_t* __restrict__ expert2) {
    route_finish_block(part, amax_part, ksplit, T, ncols, r_s, rs_pad, router_col, n_r, qmax, expert, u, s_x, expert2,
                       blockIdx.x * RF_TOK);
}

// the route finishes of up to RG_MAX linears that read the same x: linear blockIdx.y
__global__ __launch_bounds__(RF_THREADS) void route_finish_group_kernel(FinishGroup G, int ksplit, int T) {
    const FinishLinear& a = G.lin[blockIdx.y];
    route_finish_block(a.part, a.amax, ksplit, T, a.ncols, a.r_s, a.rs_pad, a.router_col, a.n_r, a.qmax, a.expert,
                       a.u, a.s_x, nullptr, blockIdx.x * RF_TOK);
}

hipError_t launch_route_finish_group(const FinishGroup& G, int n_lin, int ksplit, int T, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if (n_lin < 1 || n_lin > RG_MAX) return hipErrorInvalidValue;
    for (int l = 0; l < n_lin; ++l)
        if (G.lin[l].ncols < 0 || G.lin[l].ncols > RP_MAXN * 16 || G.lin[l].ncols % 16) return hipErrorInvalidValue;
    hipLaunchKernelGGL(route_finish_group_kernel, dim3((T + RF_TOK - 1) / RF_TOK, n_lin), dim3(RF_THREADS), 0, st, G,
                       ksplit, T);
    return hipGetLastError();
}

hipError_t launch_route_finish(const float* part, const float* amax_part, int ksplit, int T, int ncols, int r_s,
                               int rs_pad, int router_col, int n_r, int a_bits, int32_t* expert, uint16_t* u,
                               float* s_x, hipStream_t st, int32_t* expert2) {
    if (T <= 0) return hipSuccess;
    if (expert2 && (!expert || router_col < 0 || n_r < 2)) return hipErrorInvalidValue;
    if (ncols < 0 || ncols > RP_MAXN * 16 || ncols % 16 || ksplit < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(route_finish_kernel, dim3((T + RF_TOK - 1) / RF_TOK), dim3(RF_THREADS), 0, st, part, amax_part, ksplit, T, ncols,
                       r_s, rs_pad, router_col, n_r, (1 << (a_bits - 1)) - 1, expert, u, s_x, expert2);
    return hipGetLastError();
}

// ---- few-token prologue
// For up to 128 tokens (256 without a shared expert) the two passes above run a few dozen
// workgroups each, and their four launches (route pass, route finish, expert-sorted pass, v
// finish) cost more than the work.  Here one launch does it all, one workgroup per token (plus
// one more for u when there is a shared expert), with no partials leaving the workgroup:
//   blockIdx.y == 0: x' = x / s and max |x'| (one 8-channel chunk per thread), s_x and the
//     codes; the router scores x.R and their argmin (lowest index on ties); then v = x.A_e
//     for the chosen expert;
//   blockIdx.y == 1: u = x.A_s.
// The token's row is staged in LDS once.  The projections run on bf16 MFMA with the token as
// row 0 of A (the other rows zero): wave w takes the 128-channel groups w, w + 16, ..., lane
// (column l%16, g = l/16) channels 32g .. 32g+31 of each group, 8 per step (any order A and B
// share), so a lane reads 64 contiguous bytes of a projection row per group; the waves' sums
// are added in wave order.  The router's (and u's first) weight fragments are requested with
// the row, before the barrier that publishes it, so two memory rounds are exposed: the row
// with the router weights, then the chosen expert's weights.  Each workgroup streams the
// projection rows it needs once (16 + 32 rows of d_in bf16 values for 8 experts of rank 32),
// which bounds d_in.
constexpr int RW_THREADS = 1024;
constexpr int RW_WAVES = RW_THREADS / 64;
constexpr int RW_MAX_WG = 256;                      // workgroups of one launch (one round)
constexpr int RW_MAX_DIN = RW_THREADS * 8;          // one chunk of 8 channels per thread
constexpr int RW_GPW = RW_MAX_DIN / 128 / RW_WAVES;  // channel groups per wave at the widest

// weight fragments of NG of this wave's groups (its groups i0 .. i0 + NG - 1; a group past the
// range repeats the last one and is not used): NB blocks of 16 rows
// (rows at or past nrows repeat row nrows - 1: the same addresses as a lane that needs them, so
// they add no memory traffic; their columns are not used)
template <int NB, int NG>
__device__ __forceinline__ void row_load_b(const uint16_t* __restrict__ rows, int d_in, int wid, int lane, int i0,
                                           v4u (&b)[NG][NB][4], int nrows = NB * 16) {
    const int lr = lane & 15, lg = lane >> 4, ngr = d_in >> 7;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
        const size_t k0 = (size_t)min(wid + RW_WAVES * (i0 + i), ngr - 1) * 128 + lg * 32;
#pragma unroll
        for (int n = 0; n < NB; ++n)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                b[i][n][s] = *reinterpret_cast<const v4u*>(rows + (size_t)min(n * 16 + lr, nrows - 1) * d_in + k0 + 8 * s);
    }
}

// acc[n] += the token row (LDS) . those fragments, for the groups that exist
template <int NB, int NG>
__device__ __forceinline__ void row_mma(const uint16_t* xl, int d_in, int wid, int lane, int i0,
                                        const v4u (&b)[NG][NB][4], v4f (&acc)[NB]) {
    const int lr = lane & 15, lg = lane >> 4, ngr = d_in >> 7;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
        const int g = wid + RW_WAVES * (i0 + i);
        if (g >= ngr) break;  // uniform in the wave
        const uint16_t* xp = xl + g * 128 + lg * 32;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const v4u w = *reinterpret_cast<const v4u*>(xp + 8 * s);
            const v4u a = lr == 0 ? w : v4u{0, 0, 0, 0};
#pragma unroll
            for (int n = 0; n < NB; ++n)
                acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const v8bf*>(&a),
                                                                 *reinterpret_cast<const v8bf*>(&b[i][n][s]), acc[n], 0,
                                                                 0, 0);
        }
    }
}

// this wave's share of the projection onto NB*16 rows, NG groups' fragments in flight at a time
// (the first batch may already be in b)
template <int NB, int NG>
__device__ __forceinline__ void row_project(const uint16_t* __restrict__ rows, const uint16_t* xl, int d_in, int wid,
                                            int lane, v4u (&b)[NG][NB][4], bool first_loaded, v4f (&acc)[NB]) {
    const int ngr = d_in >> 7;
    const int my = wid < ngr ? (ngr - 1 - wid) / RW_WAVES + 1 : 0;  // this wave's groups
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[n] = v4f{0, 0, 0, 0};
    for (int i0 = 0; i0 < my; i0 += NG) {
        if (i0 > 0 || !first_loaded) row_load_b<NB, NG>(rows, d_in, wid, lane, i0, b);
        row_mma<NB, NG>(xl, d_in, wid, lane, i0, b, acc);
    }
}

// NBS, NBR: 16-column blocks of u (rs_pad / 16) and of v (rr_pad / 16); GPW: channel groups per
// wave the router's fragments are requested for (2 when d_in <= 4096, else RW_GPW)
template <int NBS, int NBR, int GPW>
__global__ __launch_bounds__(RW_THREADS) void row_prologue_kernel(
    const uint16_t* __restrict__ x, int d_in, const float* __restrict__ smooth, const float* __restrict__ inv_smooth,
    int qmax, const uint16_t* __restrict__ mt, int r_s, int col_router, int n_r, int col_re, int r_r,
    int8_t* __restrict__ codes, float* __restrict__ s_x, uint16_t* __restrict__ u, int32_t* __restrict__ expert,
    uint16_t* __restrict__ v) {
    __shared__ __attribute__((aligned(16))) uint16_t xl[RW_MAX_DIN];
    __shared__ float s_part[RW_WAVES][64];
    __shared__ float s_vpart[RW_WAVES][64];
    __shared__ float s_max[RW_WAVES];
    __shared__ float s_sc[16];
    const int t = blockIdx.x;
    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const uint16_t* xrow = x + (size_t)t * d_in;
    const int nch = d_in >> 3;
    const int c = min(tid, nch - 1);  // threads past the row repeat its last chunk (not used)
    const v4u w = *reinterpret_cast<const v4u*>(xrow + (size_t)c * 8);

    if (blockIdx.y == 1) {  // the shared expert's input
        if constexpr (NBS > 0) {
            constexpr int NG = NBS == 2 ? 2 : 1;
            v4u b[NG][NBS][4];
            row_load_b<NBS, NG>(mt, d_in, wid, lane, 0, b);
            if (tid < nch) *reinterpret_cast<v4u*>(xl + tid * 8) = w;
            QE_WAIT_LDS();
            QE_WG_BARRIER();
            v4f acc[NBS];
            row_project<NBS, NG>(mt, xl, d_in, wid, lane, b, true, acc);
            if (lg == 0) {
#pragma unroll
                for (int n = 0; n < NBS; ++n) s_part[wid][n * 16 + lr] = acc[n][0];
            }
            QE_WAIT_LDS();
            QE_WG_BARRIER();
            if (tid < NBS * 16) {
                float a = 0.0f;
#pragma unroll
                for (int q = 0; q < RW_WAVES; ++q) a += s_part[q][tid];
                u[(size_t)t * (NBS * 16) + tid] = tid < r_s ? (uint16_t)f32_to_bf16_bits(a) : (uint16_t)0;
            }
        }
        return;
    }

    // the row's chunk and smoothing factors, and the router's weight fragments, in one round
    const v4f s0 = *reinterpret_cast<const v4f*>(smooth + c * 8), s1 = *reinterpret_cast<const v4f*>(smooth + c * 8 + 4);
    const v4f i0 = *reinterpret_cast<const v4f*>(inv_smooth + c * 8),
              i1 = *reinterpret_cast<const v4f*>(inv_smooth + c * 8 + 4);
    v4u rb[GPW][1][4];
    if constexpr (NBR > 0) row_load_b<1, GPW>(mt + (size_t)col_router * d_in, d_in, wid, lane, 0, rb, n_r);
    if (tid < nch) *reinterpret_cast<v4u*>(xl + tid * 8) = w;
    float xs[8];
    smooth_div8(w, s0, s1, i0, i1, xs);
    float amax = 0.0f;
    if (tid < nch) {
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, __builtin_fabsf(xs[e]));
    }
    amax = wave_max(amax);
    if (lane == 0) s_max[wid] = amax;
    QE_WAIT_LDS();
    QE_WG_BARRIER();  // the row and the maxima are in LDS; the router's fragments stay in flight

    if constexpr (NBR > 0) {  // router scores (the router block is 16 rows)
        v4f racc[1];
        row_project<1, GPW>(mt + (size_t)col_router * d_in, xl, d_in, wid, lane, rb, true, racc);
        if (lg == 0) s_part[wid][lr] = racc[0][0];
    }
    // s_x = max |x'| / qmax (a max is exact in any order), then the codes
    float m = s_max[0];
#pragma unroll
    for (int q = 1; q < RW_WAVES; ++q) m = fmaxf(m, s_max[q]);
    const float sx = m / (float)qmax;
    if (tid == 0) s_x[t] = sx;
    const float inv_sx = sx != 0.0f ? 1.0f / sx : 0.0f;
    const bool fast = (sx >= 0x1p-90f && sx <= 0x1p90f) || sx == 0.0f;
    const v2u cw = codes8(xs, sx, inv_sx, fast, (float)qmax);
    if (tid < nch) *reinterpret_cast<v2u*>(codes + (size_t)t * d_in + (size_t)tid * 8) = cw;

    if constexpr (NBR > 0) {
        // scores summed in wave order by one thread each; then every thread takes the argmin
        // (strict <: the lowest index wins ties).  The barriers order LDS only: the codes'
        // stores need not have landed.
        QE_WAIT_LDS();
        QE_WG_BARRIER();
        if (tid < n_r) {
            float a = 0.0f;
#pragma unroll
            for (int q = 0; q < RW_WAVES; ++q) a += s_part[q][tid];
            s_sc[tid] = a;
        }
        QE_WAIT_LDS();
        QE_WG_BARRIER();
        int e = 0;
        float best = s_sc[0];
        for (int j = 1; j < n_r; ++j) {
            const float sc = s_sc[j];
            if (sc < best) {
                best = sc;
                e = j;
            }
        }
        if (tid == 0) expert[t] = e;
        constexpr int NG = NBR == 2 ? 2 : 1;
        v4u b[NG][NBR][4];
        v4f vacc[NBR];
        row_project<NBR, NG>(mt + (size_t)(col_re + e * NBR * 16) * d_in, xl, d_in, wid, lane, b, false, vacc);
        if (lg == 0) {
#pragma unroll
            for (int n = 0; n < NBR; ++n) s_vpart[wid][n * 16 + lr] = vacc[n][0];
        }
        QE_WAIT_LDS();
        QE_WG_BARRIER();
        if (tid < NBR * 16) {
            float a = 0.0f;
#pragma unroll
            for (int q = 0; q < RW_WAVES; ++q) a += s_vpart[q][tid];
            v[(size_t)t * (NBR * 16) + tid] = tid < r_r ? (uint16_t)f32_to_bf16_bits(a) : (uint16_t)0;
        }
    }
}

// Shapes it takes: every workgroup resident at once (one 1024-thread workgroup per compute unit
// at its register count: a second round of workgroups was measured slower than the two passes)
bool row_prologue_ok(int T, int d_in, int rs_pad, int n_r, int rr_pad) {
    const bool rs_ok = rs_pad == 0 || rs_pad == 32 || rs_pad == 64;
    const bool re_ok = n_r == 0 ? rr_pad == 0 : (n_r <= 16 && (rr_pad == 32 || rr_pad == 64));
    return T > 0 && T * (rs_pad > 0 ? 2 : 1) <= RW_MAX_WG && d_in > 0 && d_in % 128 == 0 && d_in <= RW_MAX_DIN &&
           rs_ok && re_ok;
}

hipError_t launch_row_prologue(const uint16_t* x, int T, int d_in, const float* smooth, const float* inv_smooth,
                               int a_bits, const uint16_t* mt, int r_s, int rs_pad, int col_router, int n_r, int col_re,
                               int r_r, int rr_pad, int8_t* codes, float* s_x, uint16_t* u, int32_t* expert,
                               uint16_t* v, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if (!row_prologue_ok(T, d_in, rs_pad, n_r, rr_pad) || !x || !smooth || !inv_smooth || !mt || !codes || !s_x ||
        (rs_pad > 0 && !u) || (n_r > 0 && (!expert || !v || col_router < 0 || col_re < 0)) || a_bits < 2 ||
        a_bits > 8)
        return hipErrorInvalidValue;
    const dim3 grid(T, rs_pad > 0 ? 2 : 1);
    const int qmax = (1 << (a_bits - 1)) - 1;
    const bool narrow = d_in <= RW_WAVES * 128 * 2;  // at most two channel groups per wave
#define QE_RW_LAUNCH(S, R)                                                                                          \
    if (narrow)                                                                                                     \
        hipLaunchKernelGGL((row_prologue_kernel<S, R, 2>), grid, dim3(RW_THREADS), 0, st, x, d_in, smooth,          \
                           inv_smooth, qmax, mt, r_s, col_router, n_r, col_re, r_r, codes, s_x, u, expert, v);     \
    else                                                                                                            \
        hipLaunchKernelGGL((row_prologue_kernel<S, R, RW_GPW>), grid, dim3(RW_THREADS), 0, st, x, d_in, smooth,     \
                           inv_smooth, qmax, mt, r_s, col_router, n_r, col_re, r_r, codes, s_x, u, expert, v)
#define QE_RW_BY_R(S)                          \
    if (rr_pad == 0) {                         \
        QE_RW_LAUNCH(S, 0);                    \
    } else if (rr_pad == 32) {                 \
        QE_RW_LAUNCH(S, 2);                    \
    } else {                                   \
        QE_RW_LAUNCH(S, 4);                    \
    }
    if (rs_pad == 0) {
        QE_RW_BY_R(0)
    } else if (rs_pad == 32) {
        QE_RW_BY_R(2)
    } else {
        QE_RW_BY_R(4)
    }
#undef QE_RW_BY_R
#undef QE_RW_LAUNCH
    return hipGetLastError();
}

// ---- pass 2
// A workgroup takes 128 token rows of the expert-sorted order, one 16-row block per
// wave, and a K range walked in groups of 128 channels (four 32-wide
// MFMA steps).  As in pass 1, lane (row l%16, g = l/16) takes channels 32g..32g+31 of
// its row: x goes straight to registers (64 contiguous bytes) and the lane writes the
// 32 codes of those channels as 32 contiguous bytes, so each code row segment of 128
// bytes is written whole.  The experts present in the tile are taken ESLOTS at a time;
// each MFMA sees only the rows of its expert (A masked), so one accumulator collects
// every row's own expert exactly.  The group's expert fragments (16 KB, each wave
// loading 2 KB) and smoothing factors are staged in double-buffered LDS for all 8 row
// blocks, one barrier per group.  With K split over workgroups the partial v go to
// `vpart` and vpart_finish adds them in K order.
//   Bucketing is done here too: every workgroup counts the routes (wave ballots over
// contiguous token ranges, so a stable rank is the prefix over waves plus the rank in
// the wave) and picks the tokens of its own positions; the first workgroup of a tile
// writes them to `perm`.  Equal experts keep token order.
constexpr int EQ_W = 8;             // waves per workgroup
constexpr int EQ_ROWS = 16 * EQ_W;  // token rows per workgroup
constexpr int EQ_KG = 128;          // channels per group
constexpr int EQ_TPL = 8;           // routes read per lane and batch while bucketing
constexpr int EQ_FEW_T = 256;       // token counts that take the few-token form

// ESL > 0: the few-token form (a tile then holds most experts): ESL experts per pass, and each
// group's fragments are requested one group ahead (more registers, fewer passes and no
// exposed fragment load per group); ESL == 0: 1 or 2 experts per pass.  sort_rows == false
// keeps the tokens in their order (no bucketing, no permutation written): for few tokens
// whose main product is split over K, whose epilogue does not gain from grouped experts.
template <int NBR, int ESL>
__device__ __forceinline__ void expert_quant_tile(
    const uint16_t* __restrict__ x, int T, int d_in, const float* __restrict__ smooth,
    const float* __restrict__ inv_smooth, const float* __restrict__ s_x, int qmax, const int32_t* __restrict__ expert,
    int n_r, const uint16_t* __restrict__ mt_re, int r_r, int ksq, int32_t* __restrict__ perm_out,
    float* __restrict__ vpart, int8_t* __restrict__ codes, uint16_t* __restrict__ v, bool sort_rows, int tile, int kq) {
    constexpr int RR = NBR * 16;               // padded routed rank
    constexpr int NB1 = NBR ? NBR : 1;
    constexpr int ESLOTS = ESL > 0 ? ESL : NBR == 4 ? 1 : 2;  // experts per pass
    constexpr bool kFew = ESL > 0;
    constexpr int COPIES = NBR ? ESLOTS * NB1 * 4 / EQ_W : 0;  // 1-KB fragment copies per wave and group
    static_assert(NBR == 0 || COPIES * EQ_W == ESLOTS * NB1 * 4, "fragment copies must split evenly over the waves");
    constexpr int B_LDS = NBR ? ESLOTS * NB1 * 4 * 1024 : 0;
    constexpr int BUF = B_LDS + 1024;          // + smoothing factors and reciprocals (128 each)
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * BUF];
    __shared__ uint32_t s_pres[EQ_W];

    __shared__ int s_cnt[EQ_W][kMaxRouted];
    __shared__ int s_tok[EQ_ROWS];
    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int pos0 = tile * EQ_ROWS;
    const bool routed = expert != nullptr && n_r > 0;

    // ---- the tokens of positions pos0 .. pos0 + EQ_ROWS - 1
    if (tid < EQ_ROWS) s_tok[tid] = pos0 + tid < T ? pos0 + tid : -1;
    if (routed && sort_rows) {
        const int tw0 = (int)((long)wid * T / EQ_W), tw1 = (int)((long)(wid + 1) * T / EQ_W);  // wave's tokens
        const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
        int cnt[kMaxRouted];
#pragma unroll
        for (int e = 0; e < kMaxRouted; ++e) cnt[e] = 0;
        // the wave's first batch of routes (clamped into range, -1 past the wave's tokens) stays
        // in registers for the ranking below: with up to 512 tokens per wave it is all of them
        int ev0[EQ_TPL];
        for (int b0 = tw0; b0 < tw1; b0 += 64 * EQ_TPL) {
            int ev[EQ_TPL];
#pragma unroll
            for (int j = 0; j < EQ_TPL; ++j)  // unconditional loads (clamped index), masked after
                ev[j] = expert[min(b0 + 64 * j + lane, T - 1)];
#pragma unroll
            for (int j = 0; j < EQ_TPL; ++j) ev[j] = b0 + 64 * j + lane < tw1 ? min(max(ev[j], 0), n_r - 1) : -1;
            if (b0 == tw0) {
#pragma unroll
                for (int j = 0; j < EQ_TPL; ++j) ev0[j] = ev[j];
            }
#pragma unroll
            for (int j = 0; j < EQ_TPL; ++j)
#pragma unroll
                for (int e = 0; e < kMaxRouted; ++e)
                    if (e < n_r) cnt[e] += __popcll(__ballot(ev[j] == e));
        }
        if (lane == 0)
#pragma unroll
            for (int e = 0; e < kMaxRouted; ++e) s_cnt[wid][e] = cnt[e];
        __syncthreads();
        // expert boundaries, and this wave's base rank in each expert
        int off = 0;
        for (int e = 0; e < n_r; ++e) {
            int tot = 0, base = 0;
#pragma unroll
            for (int w = 0; w < EQ_W; ++w) {
                const int c = s_cnt[w][e];
                base += w < wid ? c : 0;
                tot += c;
            }
            const int lo = max(pos0, off) - off, hi = min(pos0 + EQ_ROWS, off + tot) - off;  // ranks of expert e here
            if (lo < hi && base < hi && base + s_cnt[wid][e] > lo) {
                int rank = base;
                for (int b0 = tw0; b0 < tw1 && rank < hi; b0 += 64 * EQ_TPL) {
                    int ev[EQ_TPL];
                    if (b0 == tw0) {
#pragma unroll
                        for (int j = 0; j < EQ_TPL; ++j) ev[j] = ev0[j];
                    } else {
#pragma unroll
                        for (int j = 0; j < EQ_TPL; ++j) {
                            const int tk = b0 + 64 * j + lane;
                            ev[j] = tk < tw1 ? min(max(expert[min(tk, T - 1)], 0), n_r - 1) : -1;
                        }
                    }
#pragma unroll
                    for (int j = 0; j < EQ_TPL; ++j) {
                        const int tk = b0 + 64 * j + lane;
                        const bool f = ev[j] == e;
                        const uint64_t bal = __ballot(f);
                        const int r = rank + __popcll(bal & lt);
                        if (f && r >= lo && r < hi) s_tok[off + r - pos0] = tk;
                        rank += __popcll(bal);
                    }
                }
            }
            off += tot;
        }
    }
    __syncthreads();
    if (perm_out && kq == 0 && tid < EQ_ROWS && pos0 + tid < T) perm_out[pos0 + tid] = s_tok[tid];

    const int t_row = s_tok[wid * 16 + lr];
    const bool valid = t_row >= 0;
    const int t = valid ? t_row : 0;  // rows past T read row 0 and are never stored
    const int e_row = (NBR && valid && routed) ? min(max(expert[t], 0), n_r - 1) : -1;
    const float sx = valid ? s_x[t] : 0.0f;
    const float inv_sx = sx != 0.0f ? 1.0f / sx : 0.0f;
    const bool fast = (sx >= 0x1p-90f && sx <= 0x1p90f) || sx == 0.0f;
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

    const int ngr = d_in / EQ_KG;
    const int g_beg = (int)((long)kq * ngr / ksq), g_end = (int)((long)(kq + 1) * ngr / ksq);
    const uint16_t* xrow = x + (size_t)t * d_in + lg * 32;
    int8_t* crow = codes + (size_t)t * d_in + lg * 32;

    v4f acc[NB1];
#pragma unroll
    for (int n = 0; n < NB1; ++n) acc[n] = v4f{0, 0, 0, 0};

    uint32_t pm = present;
    bool first = true;
    int gi = 0;  // groups processed (LDS buffer parity)
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
        // fragment copies b = COPIES*wid + q: MFMA step b%4, column block (b/4)%NB1, slot b/(4*NB1)
        const uint16_t* bsrc[COPIES > 0 ? COPIES : 1];
#pragma unroll
        for (int q = 0; q < COPIES; ++q) {
            const int b = COPIES * wid + q, bs = b & 3, bn = (b >> 2) % NB1, bj = b / (4 * NB1);
            int e = max(ex[0], 0);  // empty slots repeat a present expert (never used)
#pragma unroll
            for (int j = 1; j < ESLOTS; ++j)
                if (j == bj && ex[j] >= 0) e = ex[j];
            bsrc[q] = NBR ? mt_re + ((size_t)e * RR + bn * 16 + lr) * d_in + lg * 32 + bs * 8 : nullptr;
        }
        // x of the pass's first group; each group then requests the next one's x (clamped to the
        // last group, so the load is unconditional) before its arithmetic
        v4u xv[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) xv[s] = *reinterpret_cast<const v4u*>(xrow + (size_t)g_beg * EQ_KG + s * 8);
        v4u bv[COPIES > 0 ? COPIES : 1];
        if (NBR && kFew) {  // the first group's fragments; later groups' are requested a group ahead
#pragma unroll
            for (int q = 0; q < COPIES; ++q) bv[q] = *reinterpret_cast<const v4u*>(bsrc[q] + (size_t)g_beg * EQ_KG);
        }
        for (int g = g_beg; g < g_end; ++g, ++gi) {
            uint8_t* buf = smem + (gi & 1) * BUF;
            const size_t k0 = (size_t)g * EQ_KG;
            if (NBR && !kFew) {
#pragma unroll
                for (int q = 0; q < COPIES; ++q) bv[q] = *reinterpret_cast<const v4u*>(bsrc[q] + k0);
            }
            v4f sv = v4f{0, 0, 0, 0};
            if (first && tid < 64)
                sv = *reinterpret_cast<const v4f*>((tid < 32 ? smooth : inv_smooth) + k0 + (tid & 31) * 4);
            if (NBR) {
#pragma unroll
                for (int q = 0; q < COPIES; ++q)
                    *reinterpret_cast<v4u*>(buf + (COPIES * wid + q) * 1024 + lane * 16) = bv[q];
            }
            if (first && tid < 64) *reinterpret_cast<v4f*>(buf + B_LDS + tid * 16) = sv;
            // the stores above are complete in every wave (the other buffer was last read
            // before this barrier); earlier code stores need not have landed
            QE_WAIT_LDS();
            QE_WG_BARRIER();
            v4u xn[4];
            const size_t kn = (size_t)min(g + 1, g_end - 1) * EQ_KG;
#pragma unroll
            for (int s = 0; s < 4; ++s) xn[s] = *reinterpret_cast<const v4u*>(xrow + kn + s * 8);
            if (NBR && kFew) {
#pragma unroll
                for (int q = 0; q < COPIES; ++q) bv[q] = *reinterpret_cast<const v4u*>(bsrc[q] + kn);
            }
            if (first) {
                v2u cw[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const uint8_t* sp = buf + B_LDS + (lg * 32 + s * 8) * 4;
                    const v4f s0 = *reinterpret_cast<const v4f*>(sp), s1 = *reinterpret_cast<const v4f*>(sp + 16);
                    const v4f i0 = *reinterpret_cast<const v4f*>(sp + 512),
                              i1 = *reinterpret_cast<const v4f*>(sp + 528);
                    float xs[8];
                    smooth_div8(xv[s], s0, s1, i0, i1, xs);
                    cw[s] = codes8(xs, sx, inv_sx, fast, fq);
                }
                if (valid) {
                    *reinterpret_cast<v4u*>(crow + k0) = v4u{cw[0][0], cw[0][1], cw[1][0], cw[1][1]};
                    *reinterpret_cast<v4u*>(crow + k0 + 16) = v4u{cw[2][0], cw[2][1], cw[3][0], cw[3][1]};
                }
            }
            if (NBR) {
                const v4u zero4 = v4u{0, 0, 0, 0};
#pragma unroll
                for (int j = 0; j < ESLOTS; ++j) {
                    if (ex[j] < 0) break;  // uniform
                    v8bf bq[4][NB1];  // the slot's fragments of the group first, then its MFMAs
#pragma unroll
                    for (int s = 0; s < 4; ++s)
#pragma unroll
                        for (int n = 0; n < NB1; ++n)
                            bq[s][n] = *reinterpret_cast<const v8bf*>(buf + ((j * NB1 + n) * 4 + s) * 1024 + lane * 16);
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const v4u am = e_row == ex[j] ? xv[s] : zero4;
#pragma unroll
                        for (int n = 0; n < NB1; ++n)
                            acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const v8bf*>(&am),
                                                                             bq[s][n], acc[n], 0, 0, 0);
                    }
                }
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) xv[s] = xn[s];
        }
        first = false;
    } while (pm);
    if (NBR == 0 || !v) return;

    // lane holds column n*16 + lr and rows 4*lg + r of the wave's block
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = lg * 4 + r;
        const int tt = s_tok[wid * 16 + row];
        const int p = pos0 + wid * 16 + row;
#pragma unroll
        for (int n = 0; n < NB1; ++n) {
            const int c = n * 16 + lr;
            if (ksq == 1) {
                if (tt >= 0) v[(size_t)tt * RR + c] = c < r_r ? (uint16_t)f32_to_bf16_bits(acc[n][r]) : (uint16_t)0;
            } else if (p < T) {
                vpart[((size_t)kq * T + p) * RR + c] = acc[n][r];
            }
        }
    }
}

template <int NBR, int ESL>
__global__ __launch_bounds__(64 * EQ_W) void expert_quant_kernel(
    const uint16_t* __restrict__ x, int T, int d_in, const float* __restrict__ smooth,
    const float* __restrict__ inv_smooth, const float* __restrict__ s_x, int qmax, const int32_t* __restrict__ expert,
    int n_r, const uint16_t* __restrict__ mt_re, int r_r, int ksq, int32_t* __restrict__ perm_out,
    float* __restrict__ vpart, int8_t* __restrict__ codes, uint16_t* __restrict__ v, bool sort_rows) {
    expert_quant_tile<NBR, ESL>(x, T, d_in, smooth, inv_smooth, s_x, qmax, expert, n_r, mt_re, r_r, ksq, perm_out, vpart,
                                codes, v, sort_rows, blockIdx.x, blockIdx.y);
}

// the expert-sorted passes of up to RG_MAX linears that read the same x: linear blockIdx.z
template <int NBR, int ESL>
__global__ __launch_bounds__(64 * EQ_W) void expert_quant_group_kernel(const uint16_t* __restrict__ x, int T, int d_in,
                                                                       int ksq, bool sort_rows, EqGroup G) {
    const EqLinear& a = G.lin[blockIdx.z];
    expert_quant_tile<NBR, ESL>(x, T, d_in, a.smooth, a.inv_smooth, a.s_x, a.qmax, a.expert, a.n_r, a.mt_re, a.r_r, ksq,
                                a.perm, a.vpart, a.codes, a.v, sort_rows, blockIdx.x, blockIdx.y);
}

// v[perm[pos]][c] = bf16 of the sum over the splits q of vpart[q][pos][c]: added in split order
// when there are at most VF_SERIAL splits (one thread per entry); with more splits (few tokens
// and wide inputs, one channel group per split) each of a workgroup's four waves adds a quarter
// of the splits in order for 64 entries and the quarters are added in order, so each thread
// waits for one batch of loads instead of a chain of them
constexpr int VF_SERIAL = 64;

__device__ __forceinline__ void vpart_finish_entries(const float* __restrict__ vpart, int ksq, int T, int rr_pad,
                                                     int r_r, const int32_t* __restrict__ perm,
                                                     uint16_t* __restrict__ v, bool quarters) {
    const size_t n = (size_t)T * rr_pad, stride = n;
    if (!quarters) {
        const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
        if (idx >= n) return;
        const int pos = (int)(idx / rr_pad), c = (int)(idx % rr_pad);
        const int tt = perm ? perm[pos] : pos;
        const float a = sum_splits(vpart + idx, stride, ksq);
        v[(size_t)tt * rr_pad + c] = c < r_r ? (uint16_t)f32_to_bf16_bits(a) : (uint16_t)0;
        return;
    }
    __shared__ float s_q[4][64];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const size_t idx = (size_t)blockIdx.x * 64 + lane;
    const bool ok = idx < n;
    const int k0 = (int)((long)w * ksq / 4), k1 = (int)((long)(w + 1) * ksq / 4);
    s_q[w][lane] = ok ? sum_splits<VF_SERIAL>(vpart + (size_t)k0 * stride + idx, stride, k1 - k0) : 0.0f;
    __syncthreads();
    if (w == 0 && ok) {
        const float a = ((s_q[0][lane] + s_q[1][lane]) + s_q[2][lane]) + s_q[3][lane];
        const int pos = (int)(idx / rr_pad), c = (int)(idx % rr_pad);
        const int tt = perm ? perm[pos] : pos;
        v[(size_t)tt * rr_pad + c] = c < r_r ? (uint16_t)f32_to_bf16_bits(a) : (uint16_t)0;
    }
}

__global__ __launch_bounds__(256) void vpart_finish_kernel(const float* __restrict__ vpart, int ksq, int T, int rr_pad,
                                                           int r_r, const int32_t* __restrict__ perm,
                                                           uint16_t* __restrict__ v) {
    vpart_finish_entries(vpart, ksq, T, rr_pad, r_r, perm, v, ksq > VF_SERIAL);
}

// the v finishes of a group: linear blockIdx.y
__global__ __launch_bounds__(256) void vpart_finish_group_kernel(EqGroup G, int ksq, int T, int rr_pad) {
    const EqLinear& a = G.lin[blockIdx.y];
    vpart_finish_entries(a.vpart, ksq, T, rr_pad, a.r_r, a.perm, a.v, ksq > VF_SERIAL);
}

// workgroups of a v finish over n entries
static unsigned vpart_finish_blocks(size_t n, int ksq) {
    return (unsigned)(ksq > VF_SERIAL ? (n + 63) / 64 : (n + 255) / 256);
}

// K splits: about 256 workgroups with at least two channel groups each (measured against 384 and
// 512: the 8B-shaped layer 1.7 % faster than with 512, the 2B-shaped 1 %, the 72B-shaped the same;
// fewer splits also mean fewer v partials to add); few tokens (one or two row tiles) take one
// group per workgroup up to 256 splits (every input here), since each group costs a memory
// latency that so few workgroups cannot hide (the v finish then adds up to 256 partials, 64
// requested at a time)
bool expert_quant_few(int T) { return T <= EQ_FEW_T; }

int expert_quant_ksplit(int T, int d_in) {
    const int tiles = (T + EQ_ROWS - 1) / EQ_ROWS;
    const int ks = T <= EQ_FEW_T ? std::min(d_in / EQ_KG, 256)
                                 : std::min((256 + tiles - 1) / tiles, std::max(1, d_in / (2 * EQ_KG)));
    return std::max(ks, 1);
}

hipError_t launch_expert_quant_group(const uint16_t* x, int T, int d_in, const EqGroup& G0, int n_lin, int rr_pad,
                                     int ksq, bool keep_order, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    const int nbr = rr_pad / 16;
    if (n_lin < 1 || n_lin > RG_MAX || (nbr != 2 && nbr != 4) || d_in % EQ_KG || ksq < 1 || ksq > d_in / EQ_KG)
        return hipErrorInvalidValue;
    const bool few = expert_quant_few(T);
    keep_order = keep_order && few;
    EqGroup G = G0;
    for (int l = 0; l < n_lin; ++l) {
        EqLinear& a = G.lin[l];
        if (!a.expert || !a.v || !a.smooth || !a.inv_smooth || a.n_r < 1 || a.n_r > kMaxRouted) return hipErrorInvalidValue;
        if (ksq > 1 && (!a.vpart || (!a.perm && !keep_order))) return hipErrorInvalidValue;
        if (keep_order) a.perm = nullptr;
    }
    const dim3 grid((T + EQ_ROWS - 1) / EQ_ROWS, ksq, n_lin);
#define QE_EQG_LAUNCH(NB, ESLV) \
    hipLaunchKernelGGL((expert_quant_group_kernel<NB, ESLV>), grid, dim3(64 * EQ_W), 0, st, x, T, d_in, ksq, !keep_order, G)
    if (nbr == 2) {
        if (few) QE_EQG_LAUNCH(2, 8);
        else QE_EQG_LAUNCH(2, 0);
    } else {
        if (few) QE_EQG_LAUNCH(4, 4);
        else QE_EQG_LAUNCH(4, 0);
    }
#undef QE_EQG_LAUNCH
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || ksq == 1) return err;
    const size_t n = (size_t)T * rr_pad;
    hipLaunchKernelGGL(vpart_finish_group_kernel, dim3(vpart_finish_blocks(n, ksq), n_lin), dim3(256), 0, st, G, ksq, T,
                       rr_pad);
    return hipGetLastError();
}

hipError_t launch_expert_quant(const uint16_t* x, int T, int d_in, const float* smooth, const float* inv_smooth,
                               const float* s_x, int a_bits, const int32_t* expert, int n_r, const uint16_t* mt_re,
                               int rr_pad, int r_r, int ksq, int32_t* perm, float* vpart, int8_t* codes, uint16_t* v,
                               bool keep_order, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    const int nbr = (expert && v) ? rr_pad / 16 : 0;
    if ((nbr != 0 && nbr != 2 && nbr != 4) || d_in % EQ_KG || ksq < 1 || ksq > d_in / EQ_KG || n_r > kMaxRouted ||
        !smooth || !inv_smooth)
        return hipErrorInvalidValue;
    const bool few = expert_quant_few(T);
    keep_order = keep_order && few;
    if (ksq > 1 && nbr && (!vpart || (!perm && !keep_order))) return hipErrorInvalidValue;
    const dim3 grid((T + EQ_ROWS - 1) / EQ_ROWS, ksq);
    const int qmax = (1 << (a_bits - 1)) - 1;
#define QE_EQ_LAUNCH(NB, ESLV)                                                                                      \
    hipLaunchKernelGGL((expert_quant_kernel<NB, ESLV>), grid, dim3(64 * EQ_W), 0, st, x, T, d_in, smooth, inv_smooth, \
                       s_x, qmax, expert, n_r, mt_re, r_r, ksq, keep_order ? nullptr : perm, vpart, codes, v, \
                       !keep_order)
    // few tokens: the experts are taken 8 (rank 32) or 4 (rank 64) at a time
    if (nbr == 0) QE_EQ_LAUNCH(0, 0);
    else if (nbr == 2) {
        if (few) QE_EQ_LAUNCH(2, 8);
        else QE_EQ_LAUNCH(2, 0);
    } else {
        if (few) QE_EQ_LAUNCH(4, 4);
        else QE_EQ_LAUNCH(4, 0);
    }
#undef QE_EQ_LAUNCH
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || ksq == 1 || !nbr) return err;
    const size_t n = (size_t)T * rr_pad;
    hipLaunchKernelGGL(vpart_finish_kernel, dim3(vpart_finish_blocks(n, ksq)), dim3(256), 0, st, vpart, ksq, T, rr_pad,
                       r_r, keep_order ? nullptr : perm, v);
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

// Top-2 routing: expert2[t] = the best (smallest-score) expert other than expert1[t], the lower
// index on ties; scores [T][n_r] from the router pass.
__global__ __launch_bounds__(256) void second_expert_kernel(const float* __restrict__ scores,
                                                            const int32_t* __restrict__ expert1, int T, int n_r,
                                                            int32_t* __restrict__ expert2) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= T) return;
    const int e1 = expert1[t];
    int best = -1;
    float bv = 0.0f;
    for (int e = 0; e < n_r; ++e) {
        if (e == e1) continue;
        const float v = scores[(size_t)t * n_r + e];
        if (best < 0 || v < bv) {
            best = e;
            bv = v;
        }
    }
    expert2[t] = best;
}

hipError_t launch_second_expert(const float* scores, const int32_t* expert1, int T, int n_r, int32_t* expert2,
                                hipStream_t st) {
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(second_expert_kernel, dim3((T + 255) / 256), dim3(256), 0, st, scores, expert1, T, n_r, expert2);
    return hipGetLastError();
}

hipError_t launch_bucket(const int32_t* expert, int T, int n_r, int32_t* counts, int32_t* offsets, int32_t* perm,
                         hipStream_t st) {
    hipLaunchKernelGGL(bucket_kernel, dim3(1), dim3(1024), 0, st, expert, T, n_r, counts, offsets, perm);
    return hipGetLastError();
}

}  // namespace qe
