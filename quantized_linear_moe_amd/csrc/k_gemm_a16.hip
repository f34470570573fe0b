// Weight-only (A16) main product for more than 16 tokens: bf16 activations against 3- or
// 4-bit weight codes expanded to bf16 in registers, on bf16 MFMA, with every weight fragment
// used for 64 or 128 tokens.  (The weight-streaming kernels take 16 tokens per pass, which
// would re-read the weights for every 16 tokens.)
//
//   part[ks][t][i] = sum over the K blocks of split ks of bf16(x)[t][j] * q_w[i][j]
//
// then the decode path's finish kernel applies y = s_w * sum + the low-rank terms.  W3A16 is
// one of the pages' settings (thelatestinai.com listing, Tables 1-3 and Table 8).  Codes are
// small integers, exact in bf16, so the product is exact up to float32 accumulation.
//
// Design: a workgroup owns 16*MB tokens x 128 channels (8 channel blocks) and a range of
// 128-wide K blocks; wave w takes channel blocks 2w and 2w+1 for all MB token blocks.  Per K
// block the x tile (16*MB rows x 256 bytes, rows padded by 16 bytes against bank conflicts)
// goes through registers into one of two LDS buffers while the other is read, and each wave
// fetches its weight fragments straight into registers one K block ahead (two register sets
// in turn, so no copy forces a wait).  The K blocks may be split over gridDim.y when the tile
// grid leaves CUs idle.

#include <algorithm>

#include "qe_internal.h"
#include "qe_wfrag.h"

namespace qe {

namespace {

constexpr int GA_NB = 8;               // 16-channel blocks per workgroup
constexpr int GA_LD = 128 * 2 + 16;    // bytes per LDS row of the x tile

__device__ inline v4u load_x8(const void* __restrict__ x, int x_dtype, size_t idx) {
    if (x_dtype == QE_BF16) return *reinterpret_cast<const v4u*>(reinterpret_cast<const uint16_t*>(x) + idx);
    const v4f* p = reinterpret_cast<const v4f*>(reinterpret_cast<const float*>(x) + idx);
    const v4f a = p[0], b = p[1];
    auto cvt = [](float f) {  // round to nearest even (inputs finite)
        const uint32_t u = __float_as_uint(f);
        return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    };
    return v4u{cvt(a[0]) | (cvt(a[1]) << 16), cvt(a[2]) | (cvt(a[3]) << 16), cvt(b[0]) | (cvt(b[1]) << 16),
               cvt(b[2]) | (cvt(b[3]) << 16)};
}

template <int WB, int MB>
__global__ __launch_bounds__(256, 2) void gemm_a16_kernel(const void* __restrict__ x, int x_dtype, int T, int d_in,
                                                          int d_out, const uint32_t* __restrict__ w_tiled, int n_tm,
                                                          float* __restrict__ part) {
    constexpr int BM = 16 * MB;
    constexpr int FW = Frag<WB>::kWords;
    constexpr int XCH = BM * 16 / 256;  // 16-byte chunks of the x tile per thread and K block
    __shared__ __attribute__((aligned(16))) uint8_t xs[2][BM * GA_LD];

    const int tm = blockIdx.x % n_tm, tn = blockIdx.x / n_tm;
    const int m0 = tm * BM;
    const int NB = d_out >> 4, KB = d_in >> 7;
    const int kb0 = (int)((long)blockIdx.y * KB / gridDim.y), kb1 = (int)((long)(blockIdx.y + 1) * KB / gridDim.y);
    const int nk = kb1 - kb0;
    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int nb0 = tn * GA_NB + 2 * wid;  // this wave's two channel blocks

    // x staging: chunk p*256 + tid is row (chunk / 16), 16-byte column (chunk % 16) of the tile
    auto stage = [&](int kb, v4u (&r)[XCH]) {
#pragma unroll
        for (int p = 0; p < XCH; ++p) {
            const int i = p * 256 + tid, row = i >> 4, c = i & 15;
            const int t = min(m0 + row, T - 1);  // rows past T read a valid row; never stored
            r[p] = load_x8(x, x_dtype, (size_t)t * d_in + (size_t)kb * 128 + c * 8);
        }
    };
    auto commit = [&](int buf, const v4u (&r)[XCH]) {
#pragma unroll
        for (int p = 0; p < XCH; ++p) {
            const int i = p * 256 + tid, row = i >> 4, c = i & 15;
            *reinterpret_cast<v4u*>(&xs[buf][row * GA_LD + c * 16]) = r[p];
        }
    };
    // weight fragments of K block kb; blocks past the range (or channel blocks past d_out) are zero
    auto fetch = [&](int kb, uint32_t (&f)[2][FW]) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
            load_frag<WB>(w_tiled, kb < kb1 ? nb0 + j : NB, NB, min(kb, kb1 - 1), KB, lane, d_in, f[j]);
    };

    v4f acc[MB][2];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[m][j] = v4f{0, 0, 0, 0};

    auto mma = [&](int buf, const uint32_t (&f)[2][FW]) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const v8bf b0 = weight_frag<WB>(f[0], s), b1 = weight_frag<WB>(f[1], s);
            const int off = x_step_offset<WB>(s, lg) * 2;
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                const v8bf a = *reinterpret_cast<const v8bf*>(&xs[buf][(m * 16 + lr) * GA_LD + off]);
                acc[m][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b0, acc[m][0], 0, 0, 0);
                acc[m][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b1, acc[m][1], 0, 0, 0);
            }
        }
    };

    uint32_t fa[2][FW], fb[2][FW];
    v4u xr[XCH];
    stage(kb0, xr);
    fetch(kb0, fa);
    commit(0, xr);
    __syncthreads();
    // K blocks in pairs with a fixed trip count: the first of a pair uses register set fa and
    // LDS buffer 0, the second fb and buffer 1; each requests the next block's x and weights
    // before its MFMAs (a block past the range computes with zero weights)
    const int npair = (nk + 1) / 2;
    for (int p = 0; p < npair; ++p) {
        const int kb = kb0 + 2 * p;
        stage(min(kb + 1, kb1 - 1), xr);
        fetch(kb + 1, fb);
        mma(0, fa);
        commit(1, xr);
        __syncthreads();
        stage(min(kb + 2, kb1 - 1), xr);
        fetch(kb + 2, fa);
        mma(1, fb);
        commit(0, xr);
        __syncthreads();
    }

    // lane holds rows 16m + 4lg + r, column lr of each block
    float* out = part + (size_t)blockIdx.y * T * d_out;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int nb = nb0 + j;
        if (nb >= NB) continue;
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = m0 + m * 16 + lg * 4 + r;
                if (t < T) out[(size_t)t * d_out + nb * 16 + lr] = acc[m][j][r];
            }
    }
}

inline int a16_mb(int T) { return T >= 512 ? 8 : 4; }

}  // namespace

// K splits of the A16 product: about 512 workgroups, at least 4 K blocks each, and float
// partials within the packed weights' size.
int gemm_a16_ksplit(int T, int d_in, int d_out, int w_bits) {
    const int BM = 16 * a16_mb(T);
    const long tiles = (long)((T + BM - 1) / BM) * ((d_out / 16 + GA_NB - 1) / GA_NB);
    const long KB = d_in / 128;
    if (T <= 0 || KB <= 0) return 1;
    const long wbytes = (long)d_in * d_out * w_bits / 8;
    long ks = std::min({(512 + tiles - 1) / tiles, std::max(1L, KB / 4), wbytes / std::max(1L, 4L * T * d_out)});
    return (int)std::max(ks, 1L);
}

hipError_t launch_gemm_a16(const void* x, int x_dtype, int T, int d_in, int d_out, int w_bits, const void* w_tiled,
                           int ksplit, float* part, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if ((w_bits != 3 && w_bits != 4) || d_in % 128 || d_out % 16 || ksplit < 1 || ksplit > d_in / 128)
        return hipErrorInvalidValue;
    const int mb = a16_mb(T), BM = 16 * mb;
    const int n_tm = (T + BM - 1) / BM, n_tn = (d_out / 16 + GA_NB - 1) / GA_NB;
    const uint32_t* w = reinterpret_cast<const uint32_t*>(w_tiled);
#define QE_A16_LAUNCH(WBV, MBV)                                                                                   \
    hipLaunchKernelGGL((gemm_a16_kernel<WBV, MBV>), dim3(n_tm * n_tn, ksplit), dim3(256), 0, st, x, x_dtype, T, \
                       d_in, d_out, w, n_tm, part)
    if (w_bits == 3) {
        if (mb == 8) QE_A16_LAUNCH(3, 8);
        else QE_A16_LAUNCH(3, 4);
    } else {
        if (mb == 8) QE_A16_LAUNCH(4, 8);
        else QE_A16_LAUNCH(4, 4);
    }
#undef QE_A16_LAUNCH
    return hipGetLastError();
}

}  // namespace qe
