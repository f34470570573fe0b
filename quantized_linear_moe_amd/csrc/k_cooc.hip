// Co-occurrence counts of the token-dependent channels over calibration tokens.
//
// MCISLAB DeepRead summary of "Quant Experts", section "Method", and the PaperDaily post
// "西交大提出Quant Experts：token级量化补偿", section "核心设计": O[t][i] says whether token t
// selects the i-th token-dependent channel among its top-k important channels, and the
// co-occurrence matrix counts, for every pair (i, j), the tokens that select both:
// cooc = O^T O.
//
// The contraction runs over tokens with 0/1 operands, so a 32-bit word of a channel's
// token mask carries 32 tokens and one pair-word costs an AND and a popcount-accumulate
// (v_bcnt_u32_b32): about 0.06 VALU operations per multiply-accumulate, which leaves no
// reason to expand the bits to bytes for the int8 matrix cores.  Two kernels:
//   cooc_mask_kernel : one workgroup per 128-token chunk (and 1024-channel range) reads
//                      the chunk's top-k lists once (coalesced), maps channels to
//                      token-dependent slots and ORs token bits into LDS masks, then
//                      writes them word-major: M[word][channel] (workspace).
//   cooc_pair_kernel : one workgroup per 32 x 32 tile of channel pairs on or above the
//                      diagonal and per range of mask words; its four waves take every
//                      fourth word, each lane a 4 x 4 block of pairs in registers; the
//                      waves' sums meet in LDS and one atomic add per pair (and its mirror)
//                      goes to cooc.  Integer adds: the result does not depend on order.

#include <algorithm>

#include "qe_calib.h"

namespace qe {

namespace {

constexpr int CO_THREADS = 256;
constexpr int CO_TOK = 128;            // tokens per chunk
constexpr int CO_WORDS = CO_TOK / 32;  // mask words per chunk
constexpr int CM_CH = 1024;            // channels per mask workgroup (LDS: 4 x 1024 words)
constexpr int CO_BATCH = 16;           // top-k entries per thread held in registers at once
constexpr int CP_TILE = 32;            // channels per side of a pair tile
constexpr int CP_UNROLL = 16;          // mask words per wave whose loads are in flight together

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

inline int channels_padded(int n_dep) { return (n_dep + CP_TILE - 1) / CP_TILE * CP_TILE; }
inline int mask_words(int T) { return (T + CO_TOK - 1) / CO_TOK * CO_WORDS; }

__global__ __launch_bounds__(CO_THREADS) void cooc_mask_kernel(const int32_t* __restrict__ topk, int T, int k,
                                                               const int32_t* __restrict__ slot, int d_in,
                                                               int n_dep, int Cw, uint32_t* __restrict__ M) {
    __shared__ __attribute__((aligned(16))) uint32_t m[CO_WORDS][CM_CH];
    const int tid = threadIdx.x;
    const int t0 = blockIdx.x * CO_TOK;
    const int c0 = blockIdx.y * CM_CH;
    const int nc = min(CM_CH, Cw - c0);  // a multiple of 32

#pragma unroll
    for (int u = 0; u < CO_WORDS * CM_CH / (4 * CO_THREADS); ++u)
        reinterpret_cast<u4*>(&m[0][0])[tid + u * CO_THREADS] = u4{0, 0, 0, 0};
    __syncthreads();

    // element e of the chunk is entry e % k of token e / k; for e = tid + 256 m the token
    // advances by 256 / k per step, with a carry from the remainder (the chunk's 128
    // tokens hold 128 k entries: k / 2 per thread)
    const int n_el = min(CO_TOK, T - t0) * k;
    const int32_t* src = topk + (size_t)t0 * k;
    const int tok_step = CO_THREADS / k, rem_step = CO_THREADS % k;
    int tok = tid / k, rem = tid % k;
    for (int m0 = 0; m0 * CO_THREADS < n_el; m0 += CO_BATCH) {
        int s[CO_BATCH];
#pragma unroll
        for (int u = 0; u < CO_BATCH; ++u) {  // all loads of the batch are issued together
            const int e = tid + (m0 + u) * CO_THREADS;
            s[u] = e < n_el ? src[e] : -1;
        }
#pragma unroll
        for (int u = 0; u < CO_BATCH; ++u) s[u] = (unsigned)s[u] < (unsigned)d_in ? slot[s[u]] : -1;
#pragma unroll
        for (int u = 0; u < CO_BATCH; ++u) {
            const int c = s[u] - c0;
            if ((unsigned)s[u] < (unsigned)n_dep && (unsigned)c < (unsigned)CM_CH)
                atomicOr(&m[tok >> 5][c], 1u << (tok & 31));
            tok += tok_step;
            rem += rem_step;
            if (rem >= k) {
                rem -= k;
                ++tok;
            }
        }
    }
    __syncthreads();

    uint32_t* dst = M + (size_t)blockIdx.x * CO_WORDS * Cw + c0;
#pragma unroll
    for (int u = 0; u < CO_WORDS; ++u)
        for (int c = tid * 4; c < nc; c += CO_THREADS * 4)
            *reinterpret_cast<u4*>(dst + (size_t)u * Cw + c) = *reinterpret_cast<const u4*>(&m[u][c]);
}

__global__ __launch_bounds__(CO_THREADS) void cooc_pair_kernel(const uint32_t* __restrict__ M, int W, int Cw,
                                                               int n_dep, int nt, int wpb,
                                                               uint32_t* __restrict__ cooc) {
    __shared__ uint32_t red[CO_THREADS / 64][CP_TILE * CP_TILE];
    // upper-triangle tile (ti <= tj) of linear index blockIdx.x
    int ti = 0, rest = blockIdx.x;
    while (rest >= nt - ti) {
        rest -= nt - ti;
        ++ti;
    }
    const int tj = ti + rest;
    const int i0 = ti * CP_TILE, j0 = tj * CP_TILE;
    const int tid = threadIdx.x, q = tid >> 6, lane = tid & 63;
    const int lr = lane >> 3, lc = lane & 7;  // rows i0 + 4 lr + a, columns j0 + 4 lc + b
    const int w0 = blockIdx.y * wpb, w1 = min(W, w0 + wpb);

    uint32_t acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = 0;

    // this wave's words: w0 + q, w0 + q + 4, ...; a fixed trip count with clamped, masked
    // loads keeps the loop free of branches around the loads
    const int n_mine = w1 - w0 > q ? (w1 - w0 - q + 3) / 4 : 0;
    const uint32_t* rows = M + i0 + 4 * lr;
    const uint32_t* cols = M + j0 + 4 * lc;
    for (int it = 0; it < n_mine; it += CP_UNROLL) {
        u4 r[CP_UNROLL], c[CP_UNROLL];
#pragma unroll
        for (int u = 0; u < CP_UNROLL; ++u) {
            const int w = min(w0 + q + 4 * (it + u), w1 - 1);
            r[u] = *reinterpret_cast<const u4*>(rows + (size_t)w * Cw);
            c[u] = *reinterpret_cast<const u4*>(cols + (size_t)w * Cw);
        }
#pragma unroll
        for (int u = 0; u < CP_UNROLL; ++u) {
            const uint32_t keep = it + u < n_mine ? ~0u : 0u;
            const uint32_t rv[4] = {r[u].x & keep, r[u].y & keep, r[u].z & keep, r[u].w & keep};
            const uint32_t cv[4] = {c[u].x, c[u].y, c[u].z, c[u].w};
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) acc[a][b] += __builtin_popcount(rv[a] & cv[b]);
        }
    }

#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) red[q][(4 * lr + a) * CP_TILE + 4 * lc + b] = acc[a][b];
    __syncthreads();
#pragma unroll
    for (int r = 0; r < CP_TILE * CP_TILE / CO_THREADS; ++r) {
        const int p = tid + r * CO_THREADS;
        const int i = i0 + p / CP_TILE, j = j0 + p % CP_TILE;
        const uint32_t v = red[0][p] + red[1][p] + red[2][p] + red[3][p];
        if (i < n_dep && j < n_dep && v != 0) {
            atomicAdd(&cooc[(size_t)i * n_dep + j], v);
            if (ti != tj) atomicAdd(&cooc[(size_t)j * n_dep + i], v);
        }
    }
}

}  // namespace

size_t cooccur_workspace_bytes(int T, int n_dep) {
    return (size_t)mask_words(T) * channels_padded(n_dep) * sizeof(uint32_t);
}

hipError_t launch_cooccur(const int32_t* topk, int T, int k, const int32_t* slot, int d_in, int n_dep,
                          uint32_t* cooc, void* ws, hipStream_t st) {
    const int Cw = channels_padded(n_dep);
    const int W = mask_words(T);
    uint32_t* M = static_cast<uint32_t*>(ws);
    hipLaunchKernelGGL(cooc_mask_kernel, dim3(W / CO_WORDS, (Cw + CM_CH - 1) / CM_CH), dim3(CO_THREADS), 0, st,
                       topk, T, k, slot, d_in, n_dep, Cw, M);
    const int nt = Cw / CP_TILE;
    const int n_tri = nt * (nt + 1) / 2;
    // about 256 workgroups where the tokens allow, but at least 64 words per workgroup:
    // every word-range split adds one more round of atomic adds over all pairs
    const int splits = std::max(1, std::min((256 + n_tri - 1) / n_tri, W / 64));
    const int wpb = ((W + splits - 1) / splits + 3) / 4 * 4;
    const int n_split = (W + wpb - 1) / wpb;
    hipLaunchKernelGGL(cooc_pair_kernel, dim3(n_tri, n_split), dim3(CO_THREADS), 0, st, M, W, Cw, n_dep, nt, wpb,
                       cooc);
    return hipGetLastError();
}

}  // namespace qe
