// Weight-only (A16) path of a QE linear for few tokens (decode): the packed
// weights are streamed once from HBM and multiplied with bf16 activations on
// bf16 MFMA; the dequantization and the shared / routed low-rank terms are
// applied in a split-K reduction kernel.
//
//   y[t][i] = s_w[i] * sum_j bf16(x)[t][j] * q_w[i][j] + u[t].B_s[:,i] + v[t].B_{e_t}[:,i]
//
// W3A16 is one of the pages' settings (thelatestinai.com listing, Tables 1-2 text
// and Table 8; MCISLAB DeepRead summary, "Key Results").  Codes are small
// integers, exact in bf16, so the product is exact up to float32 accumulation.
//
// Design: a workgroup owns 128 output channels (8 MFMA N blocks) and a K range;
// its 4 waves split that K range (interleaved 128-wide blocks) and reduce their
// accumulators through LDS, so one float32 partial per (K split, token,
// channel) leaves the workgroup.  Tokens (<= 16 per pass) form the MFMA M side;
// the token tile of x for the workgroup's K range is staged in LDS once.
//
// With quantized activations (W4A6 / W4A8 decode) the same tile streams the 4-bit weights
// against the int8 activation codes on the int8 matrix cores (int32 partials, exact), and
// the finish applies s_x[t] * s_w[i] as the main GEMM's epilogue does.

#include <algorithm>
#include <type_traits>

#include "qe_internal.h"
#include "qe_splits.h"
#include "qe_wfrag.h"

namespace qe {

constexpr int SK_NB = 8;             // 16-channel blocks per workgroup
constexpr int SK_MAX_KBLK = 16;      // max 128-wide K blocks per workgroup
constexpr int SK_LD = SK_MAX_KBLK * 128 * 2 + 16;  // LDS row stride (bytes) of the x tile

// One workgroup's tile of a split-K product:
//   part[ks][t][c] = sum over the K blocks [kb0, kb1) of split ks of bf16(x)[t][k] * W[c][k]
// for tokens t0 .. t0+15 and the NBW 16-channel blocks starting at nb0 (blocks at or past NB
// add nothing and are not written); out_ld = row stride of part, ld = LDS row stride of the
// x tile (>= 256 * (kb1 - kb0) + 16).  WB == 8: x is int8 codes [T][d_in] and part holds the
// exact int32 sums (the float buffer reinterpreted).
template <int WB, int NBW>
__device__ __attribute__((always_inline)) inline void skinny_tile(const void* __restrict__ x, int x_dtype, int T, int t0,
                                                                  int d_in, int NB, int nb0,
                                                                  const uint32_t* __restrict__ w_tiled, int ks,
                                                                  int ksplit, int ld, float* __restrict__ part,
                                                                  int out_ld) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr bool kI8 = WB == 8;
    typedef __attribute__((ext_vector_type(4))) std::conditional_t<kI8, int, float> acc4;
    uint8_t* xs = smem;                          // [ntok][ld] x tile
    acc4* red = reinterpret_cast<acc4*>(smem);   // [4][NBW][64], reuses the LDS after the main loop
    const int KB = d_in >> 7;
    const int kb0 = (int)((long)ks * KB / ksplit), kb1 = (int)((long)(ks + 1) * KB / ksplit);
    const int nkb = kb1 - kb0;
    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int ntok = min(16, T - t0);
    constexpr int FW = Frag<WB>::kWords;
    // the next K block is prefetched into registers except for wide bf16 tiles, whose
    // fragments are 4x larger (two waves per SIMD)
    constexpr bool kPrefetch = WB != 16 || NBW <= 2;

    // weight fragments of this wave's first K block are requested before the x tile is staged.
    // With prefetching, loads are unconditional: channel blocks past NB and K blocks past the
    // wave's range read a valid block instead (discarded), because a branch around a load makes
    // the compiler wait for every load in flight.
    uint32_t f[NBW][FW], fn[NBW][FW];
    int kb = kb0 + wid;
    auto nbc = [&](int j) { return min(nb0 + j, NB - 1); };
    auto kbc = [&](int k) { return min(k, kb1 - 1); };
    if constexpr (kPrefetch) {
#pragma unroll
        for (int j = 0; j < NBW; ++j) load_frag<WB>(w_tiled, nbc(j), NB, kbc(kb), KB, lane, d_in, f[j]);
    } else if (kb < kb1) {
#pragma unroll
        for (int j = 0; j < NBW; ++j) load_frag<WB>(w_tiled, nb0 + j, NB, kb, KB, lane, d_in, f[j]);
    }

    // stage x[t0 .. t0+ntok)[kb0*128 .. kb1*128) as bf16 (or int8 codes), eight independent
    // 16-byte loads per thread in flight per batch
    const int kc8 = nkb * (kI8 ? 8 : 16);  // 16-byte chunks per row
    const int total = ntok * kc8;
    for (int base = 0; base < total; base += 256 * 8) {
        v4u val[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int i = base + q * 256 + tid;
            val[q] = v4u{0, 0, 0, 0};
            if (i < total) {
                const int r = i / kc8, c8 = i % kc8;
                const size_t idx = (size_t)(t0 + r) * d_in + (size_t)kb0 * 128 + c8 * (kI8 ? 16 : 8);
                if constexpr (kI8) {
                    val[q] = *reinterpret_cast<const v4u*>(reinterpret_cast<const int8_t*>(x) + idx);
                } else if (x_dtype == QE_BF16) {
                    val[q] = *reinterpret_cast<const v4u*>(reinterpret_cast<const uint16_t*>(x) + idx);
                } else {
                    const v4f* p = reinterpret_cast<const v4f*>(reinterpret_cast<const float*>(x) + idx);
                    const v4f a = p[0], b = p[1];
                    auto cvt = [](float fv) {
                        uint32_t u = __float_as_uint(fv);
                        return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
                    };
                    val[q][0] = cvt(a[0]) | (cvt(a[1]) << 16);
                    val[q][1] = cvt(a[2]) | (cvt(a[3]) << 16);
                    val[q][2] = cvt(b[0]) | (cvt(b[1]) << 16);
                    val[q][3] = cvt(b[2]) | (cvt(b[3]) << 16);
                }
            }
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int i = base + q * 256 + tid;
            if (i < total) *reinterpret_cast<v4u*>(xs + (i / kc8) * ld + (i % kc8) * 16) = val[q];
        }
    }
    __syncthreads();

    acc4 acc[NBW];
#pragma unroll
    for (int j = 0; j < NBW; ++j) acc[j] = acc4{0, 0, 0, 0};

    // MFMAs of one K block held in w[] (x from the LDS tile; a block past the range gets zero x)
    auto mma = [&](const uint32_t (&w)[NBW][FW], int k) {
        const bool use = lr < ntok && k < kb1;
        if constexpr (kI8) {
            // two 64-wide int8 steps: the lane's 16 codes at K offset 16*lg of each step, and the
            // weight fragment's 8 bytes of that step expanded to 16*code
            const uint8_t* xrow = xs + lr * ld + (kbc(k) - kb0) * 128;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const v4i a = use ? *reinterpret_cast<const v4i*>(xrow + s * 64 + lg * 16) : v4i{0, 0, 0, 0};
#pragma unroll
                for (int j = 0; j < NBW; ++j)
                    acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, unpack_w4x16(w[j][2 * s], w[j][2 * s + 1]),
                                                                   acc[j], 0, 0, 0);
            }
        } else {
            const uint8_t* xrow = xs + lr * ld + (kbc(k) - kb0) * 256;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const v8bf a = use ? *reinterpret_cast<const v8bf*>(xrow + x_step_offset<WB>(s, lg) * 2) : v8bf{};
#pragma unroll
                for (int j = 0; j < NBW; ++j)
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, weight_frag<WB>(w[j], s), acc[j], 0, 0, 0);
            }
        }
    };
    if constexpr (kPrefetch) {
        // two register buffers in turn, one K block (4 apart: the waves interleave) ahead; the
        // trip count is fixed and the body has no branch, so each wait is for the older buffer
        // only and the other stays in flight
        const int npair = (max(kb1 - kb, 0) + 7) / 8;
        for (int p = 0; p < npair; ++p, kb += 8) {
#pragma unroll
            for (int j = 0; j < NBW; ++j) load_frag<WB>(w_tiled, nbc(j), NB, kbc(kb + 4), KB, lane, d_in, fn[j]);
            mma(f, kb);
#pragma unroll
            for (int j = 0; j < NBW; ++j) load_frag<WB>(w_tiled, nbc(j), NB, kbc(kb + 8), KB, lane, d_in, f[j]);
            mma(fn, kb + 4);
        }
    } else {
        for (; kb < kb1; kb += 4) {
            mma(f, kb);
            if (kb + 4 < kb1) {
#pragma unroll
                for (int j = 0; j < NBW; ++j) load_frag<WB>(w_tiled, nb0 + j, NB, kb + 4, KB, lane, d_in, f[j]);
            }
        }
    }
    // reduce the 4 waves' accumulators (fixed order) through LDS
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NBW; ++j) red[(wid * NBW + j) * 64 + lane] = acc[j];
    __syncthreads();
    if (wid == 0) {
        float* out = part + (size_t)ks * T * out_ld;
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            acc4 sum = red[j * 64 + lane];
#pragma unroll
            for (int w = 1; w < 4; ++w) sum += red[(w * NBW + j) * 64 + lane];
            const int nb = nb0 + j;
            if (nb >= NB) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tt = lg * 4 + r;
                if (tt >= ntok) continue;
                if constexpr (kI8)  // 16 * sum exactly: the expanded weights carry a factor 16
                    reinterpret_cast<int32_t*>(out)[(size_t)(t0 + tt) * out_ld + nb * 16 + lr] = sum[r] >> 4;
                else
                    out[(size_t)(t0 + tt) * out_ld + nb * 16 + lr] = sum[r];
            }
        }
    }
}

template <int WB>
__global__ __launch_bounds__(256) void skinny_kernel(const void* __restrict__ x, int x_dtype, int T, int t0, int d_in,
                                                     int n_cols, const uint32_t* __restrict__ w_tiled, int ksplit,
                                                     float* __restrict__ part, int out_ld) {
    skinny_tile<WB, SK_NB>(x, x_dtype, T, t0, d_in, n_cols >> 4, blockIdx.x * SK_NB, w_tiled, blockIdx.y, ksplit,
                           SK_LD, part, out_ld);
}

// Decode GEMV, one launch for both streams of a weight-only linear with T <= 16: the first
// n_pwg workgroups project x onto Mt (the shared-expert, router and routed-expert input
// matrices, bf16 rows) two channel blocks at a time, the rest stream the packed weights
// eight channel blocks at a time; each writes split-K partials for the finish kernel.  The
// register budget is three waves per SIMD: the plan's three workgroups per compute unit.
template <int WB>
__global__ __launch_bounds__(256, 3) void decode_gemv_kernel(const void* __restrict__ x, int x_dtype,
                                                          const int8_t* __restrict__ codes, int T, int d_in,
                                                          int d_out, const uint32_t* __restrict__ w_tiled, int ks_m,
                                                          int ld_m, float* __restrict__ part_m,
                                                          const uint32_t* __restrict__ mt, int ncp, int ks_p, int ld_p,
                                                          float* __restrict__ part_p, int n_pwg) {
    const int bid = blockIdx.x;
    if (bid < n_pwg) {
        const int NBp = ncp >> 4, pgroups = (NBp + 1) >> 1;
        skinny_tile<16, 2>(x, x_dtype, T, 0, d_in, NBp, (bid % pgroups) * 2, mt, bid / pgroups, ks_p, ld_p,
                           part_p, ncp);
    } else {
        const int b = bid - n_pwg, NB = d_out >> 4, groups = (NB + SK_NB - 1) / SK_NB;
        skinny_tile<WB, SK_NB>(WB == 8 ? static_cast<const void*>(codes) : x, x_dtype, T, 0, d_in, NB,
                               (b % groups) * SK_NB, w_tiled, b / groups, ks_m, ld_m, part_m, d_out);
    }
}

constexpr size_t SK_RED_BYTES = 4 * SK_NB * 64 * 4 * sizeof(float);
size_t skinny_lds_bytes(int ntok) { return std::max((size_t)ntok * SK_LD, SK_RED_BYTES); }
size_t skinny_lds_bytes() { return skinny_lds_bytes(16); }

int skinny_ksplit(int d_in, int d_out) {
    const int KB = d_in / 128;
    const int groups = (d_out / 16 + SK_NB - 1) / SK_NB;
    if (groups <= 0 || KB <= 0) return 1;
    int ks = (1024 + groups - 1) / groups;
    ks = max(ks, (KB + SK_MAX_KBLK - 1) / SK_MAX_KBLK);
    ks = min(ks, KB);
    return max(ks, 1);
}

// K splits of the small-T x-projection: few partials per output, so its reduction stays short
int skinny_ksplit_proj(int d_in) { return std::max(1, std::min(d_in / 128, 128)); }

// w_bits 3 / 4: packed tiles; w_bits 16: bf16 rows (the x-projection matrix), n_cols columns
hipError_t launch_skinny(const void* x, int x_dtype, int T, int d_in, int n_cols, int w_bits, const void* w_tiled,
                         int ksplit, float* part, int out_ld, hipStream_t st) {
    const int groups = (n_cols / 16 + SK_NB - 1) / SK_NB;
    const uint32_t* w = reinterpret_cast<const uint32_t*>(w_tiled);
    for (int t0 = 0; t0 < T; t0 += 16) {
        const size_t lds = skinny_lds_bytes(std::min(16, T - t0));
        if (w_bits == 3) {
            hipLaunchKernelGGL(skinny_kernel<3>, dim3(groups, ksplit), dim3(256), lds, st, x, x_dtype, T, t0, d_in,
                               n_cols, w, ksplit, part, out_ld);
        } else if (w_bits == 4) {
            hipLaunchKernelGGL(skinny_kernel<4>, dim3(groups, ksplit), dim3(256), lds, st, x, x_dtype, T, t0, d_in,
                               n_cols, w, ksplit, part, out_ld);
        } else {
            hipLaunchKernelGGL(skinny_kernel<16>, dim3(groups, ksplit), dim3(256), lds, st, x, x_dtype, T, t0, d_in,
                               n_cols, w, ksplit, part, out_ld);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// ------------------------------------------------------------------ fused decode
// Split-K plan of decode_gemv_kernel: workgroups stream about the same number of bytes and
// all of them are resident in one round (three per compute unit: the kernel's register
// footprint), so none starts late and the tail is one memory latency.  The x tile of a
// workgroup fits a third of the LDS.
constexpr int DG_WG_PER_CU = 3;
constexpr int DG_SLOTS = DG_WG_PER_CU * 256;
constexpr int DG_TILE_BUDGET = 52 * 1024;
constexpr int DG_MAX_KBLK = 32;

DecodePlan decode_plan(int d_in, int d_out, int w_bits, int ncp, int T) {
    DecodePlan P{};
    const int KB = d_in / 128, ntok = std::min(16, std::max(T, 1));
    const int groups = (d_out / 16 + SK_NB - 1) / SK_NB;
    const int pgroups = (ncp / 16 + 1) / 2;
    const double mblk = 128.0 * 128.0 * w_bits / 8.0;  // bytes of one main K block (8 channel blocks)
    const double pblk = 32.0 * 128.0 * 2.0;            // bytes of one projection K block (2 channel blocks, bf16)
    const double total = (double)groups * KB * mblk + (double)pgroups * KB * pblk;
    const double per_wg = total / DG_SLOTS;
    const int cap = std::max(1, std::min(DG_MAX_KBLK, (DG_TILE_BUDGET / ntok - 16) / 256));
    const int ks_min = (KB + cap - 1) / cap;  // splits needed for the x tile to fit
    auto clampks = [&](int ks) { return std::max(ks_min, std::min(KB, std::max(1, ks))); };
    P.ks_m = clampks((int)std::lround(KB * mblk / per_wg));
    P.n_mwg = groups * P.ks_m;
    if (pgroups > 0) {
        // the projection takes the slots the main weights leave, at about the same bytes per workgroup
        const int fit = (DG_SLOTS - P.n_mwg) / pgroups;
        P.ks_p = clampks(std::min((int)std::lround(KB * pblk / per_wg), fit));
    }
    P.n_pwg = pgroups * P.ks_p;
    P.ld_m = (KB + P.ks_m - 1) / P.ks_m * 256 + 16;
    P.ld_p = pgroups > 0 ? (KB + P.ks_p - 1) / P.ks_p * 256 + 16 : 0;
    P.lds = std::max({(size_t)ntok * P.ld_m, (size_t)ntok * P.ld_p, SK_RED_BYTES});
    return P;
}

// codes != NULL: quantized activations (W4 only), int32 main partials
hipError_t launch_decode_gemv(const void* x, int x_dtype, const int8_t* codes, int T, int d_in, int d_out, int w_bits,
                              const void* w_tiled, const DecodePlan& P, float* part_m, const uint16_t* mt, int ncp,
                              float* part_p, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if (T > 16 || P.lds > 64 * 1024 || (codes && w_bits != 4)) return hipErrorInvalidValue;
    const uint32_t* w = reinterpret_cast<const uint32_t*>(w_tiled);
    const uint32_t* m = reinterpret_cast<const uint32_t*>(mt);
    const int nwg = P.n_pwg + P.n_mwg;
#define QE_DG_LAUNCH(WBV)                                                                                        \
    hipLaunchKernelGGL(decode_gemv_kernel<WBV>, dim3(nwg), dim3(256), P.lds, st, x, x_dtype, codes, T, d_in, d_out, \
                       w, P.ks_m, P.ld_m, part_m, m, ncp, P.ks_p, P.ld_p, part_p, P.n_pwg)
    if (codes) QE_DG_LAUNCH(8);
    else if (w_bits == 3) QE_DG_LAUNCH(3);
    else QE_DG_LAUNCH(4);
#undef QE_DG_LAUNCH
    return hipGetLastError();
}

// Finish of the fused decode.  Every workgroup turns the projection partials into the routed
// expert of each token (argmin of the router scores, lowest index on ties) and the bf16 adapter
// inputs u (shared expert) and v (the token's routed expert), then writes, for its CH channels
// and all tokens (thread (c, ts) takes channel c of the group and tokens ts, ts + 512/CH, ...),
//   y[t][i] = s_w[i] * sum_ks part_m[ks][t][i] + u[t].Bt_s[i] + v[t].Bt_r[e_t][i]
// or, with quantized activations (s_x != NULL, int32 main partials),
//   y[t][i] = (float)(sum_ks part_m[ks][t][i]) * s_x[t] * s_w[i] + (the same adapter terms).
// Partials are summed in split order.  Two memory rounds are exposed: first everything that
// needs no route (the thread's main partials and shared-expert row, kept in registers, and the
// router and u partials, summed into LDS), then, after one barrier, each thread takes the routes
// of its tokens from the scores in LDS and requests their routed-expert rows together with the
// v partials (measured no faster than the three rounds of loading each phase's operands
// after the previous barrier).  CH is 64 or 32 so that narrower outputs still give every
// compute unit a workgroup.
constexpr int DF_THREADS = 512;

// CH channels per workgroup; KR = 4 or 8: adapter ranks up to 32 or 64 (the register rows' size)
template <int CH, int KR>
__global__ __launch_bounds__(DF_THREADS, KR == 4 ? 4 : 2) void decode_finish_kernel(
    const float* __restrict__ part_m, const float* __restrict__ s_x, int ks_m, int T, int d_out,
    const float* __restrict__ w_scale,
    const float* __restrict__ part_p, int ks_p, int ncp, int col_se, int r_s, int rs_pad, int col_re, int n_r,
    int r_r, int rr_pad, int col_router, const uint16_t* __restrict__ bt_s, const uint16_t* __restrict__ bt_r,
    int32_t* __restrict__ expert_out, float* __restrict__ y, bool y_bf16) {
    constexpr int TS = DF_THREADS / CH;  // token slots
    constexpr int NH = (16 + TS - 1) / TS;  // tokens per thread at T = 16
    constexpr int MP = NH == 1 ? 16 : 4;     // main partials per output requested ahead (the rest after)
    __shared__ float s_sc[16][kMaxRouted];
    __shared__ float s_u[16][kMaxRank];
    __shared__ float s_v[16][kMaxRank];
    const int tid = threadIdx.x;
    const int c = tid % CH, ts = tid / CH;
    const int i = min(blockIdx.x * CH + c, d_out - 1);
    const size_t pstride = (size_t)T * ncp, mstride = (size_t)T * d_out;

    // 1. no route needed: main partials and the shared-expert row (registers), then the router
    //    scores and u (LDS)
    float pm[NH][MP];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const int tt = min(ts + TS * h, T - 1);
#pragma unroll
        for (int q = 0; q < MP; ++q)
            pm[h][q] = (ts + TS * h < T && q < ks_m) ? part_m[(size_t)q * mstride + (size_t)tt * d_out + i] : 0.0f;
    }
    v4u bs[KR];
#pragma unroll
    for (int q = 0; q < KR; ++q)
        bs[q] = 8 * q < rs_pad ? *reinterpret_cast<const v4u*>(bt_s + (size_t)i * rs_pad + 8 * q) : v4u{0, 0, 0, 0};
    const int nsc = T * n_r, nu = T * rs_pad;
    for (int it = tid; it < nsc + nu; it += DF_THREADS) {
        if (it < nsc) {
            const int tt = it / n_r, e = it % n_r;
            s_sc[tt][e] = sum_splits(part_p + (size_t)tt * ncp + col_router + e, pstride, ks_p);
        } else {
            const int tt = (it - nsc) / rs_pad, m = (it - nsc) % rs_pad;
            const float a = m < r_s ? sum_splits(part_p + (size_t)tt * ncp + col_se + m, pstride, ks_p) : 0.0f;
            s_u[tt][m] = __uint_as_float(f32_to_bf16_bits(a) << 16);
        }
    }
    __syncthreads();

    // 2. routes from the scores (strict <: the lowest index wins ties), the routed rows of the
    //    thread's tokens (registers) and v of every token's expert (LDS)
    auto route = [&](int tt) {
        int e = 0;
        float best = s_sc[tt][0];
        for (int j = 1; j < n_r; ++j)
            if (s_sc[tt][j] < best) {
                best = s_sc[tt][j];
                e = j;
            }
        return e;
    };
    int eh[NH];
    v4u br[NH][KR];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const int tt = ts + TS * h;
        eh[h] = (n_r > 0 && tt < T) ? route(tt) : -1;
        const uint16_t* row = bt_r + ((size_t)max(eh[h], 0) * d_out + i) * rr_pad;
#pragma unroll
        for (int q = 0; q < KR; ++q)
            br[h][q] = (eh[h] >= 0 && 8 * q < rr_pad) ? *reinterpret_cast<const v4u*>(row + 8 * q) : v4u{0, 0, 0, 0};
    }
    if (n_r > 0 && expert_out && blockIdx.x == 0 && tid < T) expert_out[tid] = route(tid);
    if (n_r > 0) {
        for (int it = tid; it < T * rr_pad; it += DF_THREADS) {
            const int tt = it / rr_pad, m = it % rr_pad;
            const float a =
                m < r_r ? sum_splits(part_p + (size_t)tt * ncp + col_re + route(tt) * rr_pad + m, pstride, ks_p) : 0.0f;
            s_v[tt][m] = __uint_as_float(f32_to_bf16_bits(a) << 16);
        }
    }
    __syncthreads();

    // 3. the main term (split order), the two dot products, the output
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const int tt = ts + TS * h;
        if (tt >= T) break;  // no barrier follows
        float main;
        if (s_x) {
            int32_t acc = 0;
#pragma unroll
            for (int q = 0; q < MP; ++q) acc += __float_as_int(pm[h][q]);
            if (ks_m > MP)
                acc += sum_splits_i32(reinterpret_cast<const int32_t*>(part_m) + MP * mstride + (size_t)tt * d_out + i,
                                      mstride, ks_m - MP);
            main = (float)acc * s_x[tt] * w_scale[i];
        } else {
            float sum = 0.0f;
#pragma unroll
            for (int q = 0; q < MP; ++q)
                if (q < ks_m) sum += pm[h][q];
            for (int q = MP; q < ks_m; ++q) sum += part_m[(size_t)q * mstride + (size_t)tt * d_out + i];
            main = sum * w_scale[i];
        }
        float du = 0.0f, dv = 0.0f;
#pragma unroll
        for (int q = 0; q < KR; ++q) {
            if (8 * q >= rs_pad) break;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                du = __builtin_fmaf(s_u[tt][8 * q + 2 * k], __uint_as_float(bs[q][k] << 16), du);
                du = __builtin_fmaf(s_u[tt][8 * q + 2 * k + 1], __uint_as_float(bs[q][k] & 0xFFFF0000u), du);
            }
        }
        if (eh[h] >= 0) {
#pragma unroll
            for (int q = 0; q < KR; ++q) {
                if (8 * q >= rr_pad) break;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    dv = __builtin_fmaf(s_v[tt][8 * q + 2 * k], __uint_as_float(br[h][q][k] << 16), dv);
                    dv = __builtin_fmaf(s_v[tt][8 * q + 2 * k + 1], __uint_as_float(br[h][q][k] & 0xFFFF0000u), dv);
                }
            }
        }
        if (blockIdx.x * CH + c < d_out) store_y(y, (size_t)tt * d_out + i, (main + du) + dv, y_bf16);
    }
}

// channels per workgroup: 64, or 32 when 64 would leave compute units without a workgroup
// (the 8192-wide outputs: 256 workgroups instead of 128, measured 1.4 us faster per call;
// 32 for the 29568-wide outputs doubles the grid past one round and is slower)
int decode_finish_channels(int d_out) { return (d_out + 63) / 64 >= 256 ? 64 : 32; }

hipError_t launch_decode_finish(const float* part_m, const float* s_x, int ks_m, int T, int d_out,
                                const float* w_scale, const float* part_p, int ks_p, int ncp, int col_se, int r_s,
                                int rs_pad, int col_re, int n_r, int r_r, int rr_pad, int col_router,
                                const uint16_t* bt_s, const uint16_t* bt_r, int32_t* expert_out, float* y,
                                bool y_bf16, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if (T > 16 || n_r > kMaxRouted || rs_pad > kMaxRank || rr_pad > kMaxRank) return hipErrorInvalidValue;
    const int ch = decode_finish_channels(d_out);
    const bool wide = rs_pad > 32 || rr_pad > 32;
#define QE_DF_LAUNCH(CHV, KRV)                                                                                     \
    hipLaunchKernelGGL((decode_finish_kernel<CHV, KRV>), dim3((d_out + CHV - 1) / CHV), dim3(DF_THREADS), 0, st,   \
                       part_m, s_x, ks_m, T, d_out, w_scale, part_p, ks_p, ncp, col_se, r_s, rs_pad, col_re, n_r,  \
                       r_r, rr_pad, col_router, bt_s, bt_r, expert_out, y, y_bf16)
    if (ch == 64) {
        if (wide) QE_DF_LAUNCH(64, 8);
        else QE_DF_LAUNCH(64, 4);
    } else {
        if (wide) QE_DF_LAUNCH(32, 8);
        else QE_DF_LAUNCH(32, 4);
    }
#undef QE_DF_LAUNCH
    return hipGetLastError();
}

hipError_t skinny_set_attributes() {
    const int lds = (int)skinny_lds_bytes();
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(skinny_kernel<3>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e == hipSuccess)
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(skinny_kernel<4>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e == hipSuccess)
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(skinny_kernel<16>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    return e;
}

// One thread per (token t, channel i):
//   y[t][i] = s_w[i] * sum_ks part[ks][t][i] + u[t].Bt_s[i] + v[t].Bt_r[e_t][i]
// with the adapter rows read as 16-byte vectors (rows are padded to 32 elements).
__device__ inline float dot_bf16_rows(const uint16_t* __restrict__ a, const uint16_t* __restrict__ b, int n) {
    float acc = 0.0f;
    for (int m = 0; m < n; m += 8) {
        const v4u bv = *reinterpret_cast<const v4u*>(b + m);
        const v4u av = *reinterpret_cast<const v4u*>(a + m);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc = __builtin_fmaf(__uint_as_float(av[q] << 16), __uint_as_float(bv[q] << 16), acc);
            acc = __builtin_fmaf(__uint_as_float(av[q] & 0xFFFF0000u), __uint_as_float(bv[q] & 0xFFFF0000u), acc);
        }
    }
    return acc;
}

__global__ __launch_bounds__(256) void skinny_finish_kernel(const float* __restrict__ part, int ksplit, int T,
                                                            int d_out, const float* __restrict__ w_scale,
                                                            const uint16_t* __restrict__ u,
                                                            const uint16_t* __restrict__ bt_s, int rs_pad,
                                                            const uint16_t* __restrict__ v,
                                                            const int32_t* __restrict__ expert,
                                                            const uint16_t* __restrict__ bt_r, int rr_pad,
                                                            float* __restrict__ y, bool y_bf16) {
    const int i = blockIdx.x * 256 + threadIdx.x, t = blockIdx.y;
    if (i >= d_out) return;
    const float* p = part + (size_t)t * d_out + i;
    const size_t stride = (size_t)T * d_out;
    float s = 0.0f;
    int k = 0;
    for (; k + 4 <= ksplit; k += 4) {  // independent loads, summed in order
        const float a0 = p[(size_t)k * stride], a1 = p[(size_t)(k + 1) * stride];
        const float a2 = p[(size_t)(k + 2) * stride], a3 = p[(size_t)(k + 3) * stride];
        s += a0;
        s += a1;
        s += a2;
        s += a3;
    }
    for (; k < ksplit; ++k) s += p[(size_t)k * stride];
    float out = s * w_scale[i];
    if (u) out += dot_bf16_rows(u + (size_t)t * rs_pad, bt_s + (size_t)i * rs_pad, rs_pad);
    if (v && expert) out += dot_bf16_rows(v + (size_t)t * rr_pad, bt_r + ((size_t)expert[t] * d_out + i) * rr_pad, rr_pad);
    store_y(y, (size_t)t * d_out + i, out, y_bf16);
}

hipError_t launch_skinny_finish(const float* part, int ksplit, int T, int d_out, const float* w_scale,
                                const uint16_t* u, const uint16_t* bt_s, int rs_pad, const uint16_t* v,
                                const int32_t* expert, const uint16_t* bt_r, int rr_pad, float* y, bool y_bf16,
                                hipStream_t st) {
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(skinny_finish_kernel, dim3((d_out + 255) / 256, T), dim3(256), 0, st, part, ksplit, T, d_out,
                       w_scale, u, bt_s, rs_pad, v, expert, bt_r, rr_pad, y, y_bf16);
    return hipGetLastError();
}


// Unfused routed experts, grouped by expert bucket: y[perm[p]][i] += v[perm[p]] . Bt_r[e][i] with
// e the bucket of position p.  A workgroup takes 64 bucket positions x 256 channels (wave: 64
// channels); each 16-position block makes one round of bf16 MFMAs per expert present in it (the
// buckets are contiguous, so usually one), with A masked to that expert's rows, and adds its
// result into y in place (every (token, channel) appears once in a grouping).  Column lr of
// channel block nb is channel 64 w + 4 lr + nb, so a lane's four blocks are four consecutive
// channels: each row's update is one 16-byte read-modify-write per lane.
constexpr int RL_P = 64;

__global__ __launch_bounds__(256) void routed_lora_kernel(const uint16_t* __restrict__ v, int rr_pad,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ perm, int n_r,
                                                          const uint16_t* __restrict__ bt_r, int T, int d_out,
                                                          float* __restrict__ y) {
    const int p0 = blockIdx.x * RL_P, tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, lr = lane & 15,
              lg = lane >> 4;
    const int nw = blockIdx.y * 256 + wid * 64;
    auto expert_of = [&](int p) {
        int e = 0;
        while (e + 1 < n_r && offsets[e + 1] <= p) ++e;
        return e;
    };
    // The y rows this lane updates are requested first, at clamped addresses, so their latency
    // overlaps the adapter loads and MFMAs; lane holds positions pb + 4 lg + r and channels
    // ch0 .. ch0 + 3 (d_out is a multiple of 16, so a clamped ch0 stays 16-byte aligned).
    const int ch0 = nw + 4 * lr, ch0c = min(ch0, d_out - 4);
    int tr[4][4];
    v4f yo[4][4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) tr[mb][r] = min(max(perm[min(p0 + 16 * mb + 4 * lg + r, T - 1)], 0), T - 1);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) yo[mb][r] = *reinterpret_cast<const v4f*>(y + (size_t)tr[mb][r] * d_out + ch0c);
    int chs[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) chs[nb] = min(nw + 4 * lr + nb, d_out - 1);  // past d_out: never stored
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        const int pb = p0 + 16 * mb;
        if (pb >= T) break;  // wave-uniform
        v4f acc[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[nb] = v4f{0, 0, 0, 0};
        const int p = min(pb + lr, T - 1);
        const bool prow = pb + lr < T;
        const int e_row = expert_of(p);
        const int t = min(max(perm[p], 0), T - 1);
        const int e_lo = expert_of(pb), e_hi = expert_of(min(pb + 15, T - 1));
        for (int e = e_lo; e <= e_hi; ++e) {  // wave-uniform bounds
            for (int k0 = 0; k0 < rr_pad; k0 += 32) {
                const v8bf av = *reinterpret_cast<const v8bf*>(v + (size_t)t * rr_pad + k0 + lg * 8);
                const v8bf a = (prow && e_row == e) ? av : v8bf{};
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    const v8bf b =
                        *reinterpret_cast<const v8bf*>(bt_r + ((size_t)e * d_out + chs[nb]) * rr_pad + k0 + lg * 8);
                    acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[nb], 0, 0, 0);
                }
            }
        }
        // each (token, channel) appears once in a grouping, so the in-place update is race-free
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (pb + 4 * lg + r >= T || ch0 >= d_out) continue;
            v4f o = yo[mb][r];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) o[nb] += acc[nb][r];
            *reinterpret_cast<v4f*>(y + (size_t)tr[mb][r] * d_out + ch0) = o;
        }
    }
}

hipError_t launch_routed_lora(const uint16_t* v, int rr_pad, const int32_t* offsets, const int32_t* perm, int n_r,
                              const uint16_t* bt_r, int T, int d_out, float* y, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if (rr_pad % 32 || n_r < 1 || d_out % 16) return hipErrorInvalidValue;
    hipLaunchKernelGGL(routed_lora_kernel, dim3((T + RL_P - 1) / RL_P, (d_out + 255) / 256), dim3(256), 0, st, v,
                       rr_pad, offsets, perm, n_r, bt_r, T, d_out, y);
    return hipGetLastError();
}

}  // namespace qe
