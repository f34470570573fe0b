// Weight-only (A16) main product for more than 16 tokens: bf16 activations against 3- or
// 4-bit weight codes expanded to bf16 in registers, on bf16 MFMA, with every weight fragment
// used for 64 or 128 tokens.  (The weight-streaming kernels take 16 tokens per pass, which
// would re-read the weights for every 16 tokens.)
//
//   part[ks][t][i] = sum over the K blocks of split ks of bf16(x)[t][j] * q_w[i][j]
//
// then y = s_w * sum + the low-rank terms: in the kernels' epilogue when K is not split, else
// in the decode path's finish kernel.  W3A16 is
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
//
// Many tokens (>= 512): 128 tokens x 256 channels per workgroup (wave tile 128 x 64: each x
// fragment read from LDS feeds four MFMAs, which keeps the LDS traffic at half its bandwidth
// when the matrix cores run at full rate), and both the x tile and the
// weight fragments go global -> LDS by DMA into a three-stage ring of 64-K half blocks (two
// halves in flight, explicit vmcnt waits, no staging registers); x rows are stored with their
// 16-byte chunks XOR-swizzled by row against bank conflicts.  A stage is 24 KB, so two
// workgroups share a CU and each SIMD holds two waves that cover each other's LDS and
// barrier latency.  Its epilogue scales by s_w and adds u.B_s and,
// for every routed expert present among the tile's tokens, (v masked to that expert's rows).B_e
// with bf16 MFMAs, so y is written once and the adapter rows are read once per tile.

#include <algorithm>

#include "qe_dma.h"
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

// Epilogue of a tile whose K range is complete: y = s_w * acc + u.B_s + v.B_{e_t}.  Per 16-row
// block m the low-rank terms go into a small accumulator of their own (bf16 MFMAs; one round
// per routed expert present among the block's rows, v masked to that expert's rows), and the
// block's outputs are written once.  acc is only read here, so no loop carries it.  Lane holds
// rows m0 + 16m + 4lg + r, column 16 (nb0 + j) + lr of each block; the A operands of the
// adapter MFMAs are rows m0 + 16m + lr.
template <int MB, int NBW>
__device__ __attribute__((always_inline)) inline void a16_epilogue(
    v4f (&acc)[MB][NBW], int m0, int nb0, int T, int d_out, int lane, const float* __restrict__ w_scale,
    const uint16_t* __restrict__ u, const uint16_t* __restrict__ bt_s, int rs_pad, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ expert, const uint16_t* __restrict__ bt_r, int rr_pad, int n_r,
    float* __restrict__ y, bool y_bf16) {
    const int NB = d_out >> 4, lr = lane & 15, lg = lane >> 4;
    const bool shared = u != nullptr && bt_s != nullptr && rs_pad > 0;
    const bool routed = v != nullptr && expert != nullptr && bt_r != nullptr && rr_pad > 0 && n_r > 0;
    bool nb_ok[NBW];
    int nbc[NBW];  // fragment sources; blocks past d_out repeat block 0 (never stored)
    float sw[NBW];
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
        nb_ok[j] = nb0 + j < NB;
        nbc[j] = nb_ok[j] ? nb0 + j : 0;
        sw[j] = w_scale[nbc[j] * 16 + lr];
    }
    if constexpr (MB == 1 && NBW == 1) {
        // the finish kernels' 16 x 16 blocks: with rank-32 adapters and at most 8 routed experts,
        // the shared fragments, the v row and every present expert's fragments are requested
        // together (one memory latency instead of one per expert present), then the MFMAs run in
        // the order of the general form below (shared expert, then the experts by index), so the
        // result is bit for bit the same
        if (routed && rr_pad == 32 && n_r <= 8 && (!shared || rs_pad == 32)) {
            const int ar = min(m0 + lr, T - 1);
            const int ex = m0 + lr < T ? min(max(expert[ar], 0), n_r - 1) : -1;
            int el[8];
            int np = 0;
            for (int q = 0; q < n_r; ++q)
                if (__ballot(ex == q)) el[np++] = q;  // wave-uniform
            v8bf ua = v8bf{}, bs = v8bf{};
            if (shared) {
                ua = *reinterpret_cast<const v8bf*>(u + (size_t)ar * rs_pad + lg * 8);
                bs = *reinterpret_cast<const v8bf*>(bt_s + (size_t)(nbc[0] * 16 + lr) * rs_pad + lg * 8);
            }
            const v8bf vrow = *reinterpret_cast<const v8bf*>(v + (size_t)ar * rr_pad + lg * 8);
            v8bf br[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int e = np > 0 ? el[min(i, np - 1)] : 0;  // slots past np repeat a present expert (unused)
                br[i] = *reinterpret_cast<const v8bf*>(bt_r + ((size_t)e * d_out + nbc[0] * 16 + lr) * rr_pad + lg * 8);
            }
            v4f ad = v4f{0, 0, 0, 0};
            if (shared) ad = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ua, bs, ad, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (i >= np) break;  // uniform
                const v8bf va = ex == el[i] ? vrow : v8bf{};
                ad = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, br[i], ad, 0, 0, 0);
            }
            if (nb_ok[0]) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = m0 + lg * 4 + r;
                    if (t < T) store_y(y, (size_t)t * d_out + nb0 * 16 + lr, acc[0][0][r] * sw[0] + ad[r], y_bf16);
                }
            }
            return;
        }
    }
#pragma unroll
    for (int m = 0; m < MB; ++m) {
        const int ar = min(m0 + m * 16 + lr, T - 1);
        v4f ad[NBW];
#pragma unroll
        for (int j = 0; j < NBW; ++j) ad[j] = v4f{0, 0, 0, 0};
        if (shared) {
            for (int k0 = 0; k0 < rs_pad; k0 += 32) {
                const v8bf ua = *reinterpret_cast<const v8bf*>(u + (size_t)ar * rs_pad + k0 + lg * 8);
#pragma unroll
                for (int j = 0; j < NBW; ++j) {
                    const v8bf bs =
                        *reinterpret_cast<const v8bf*>(bt_s + (size_t)(nbc[j] * 16 + lr) * rs_pad + k0 + lg * 8);
                    ad[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ua, bs, ad[j], 0, 0, 0);
                }
            }
        }
        if (routed) {
            const int ex = m0 + m * 16 + lr < T ? min(max(expert[ar], 0), n_r - 1) : -1;
            uint32_t present = 0;
            for (int q = 0; q < n_r; ++q)
                if (__ballot(ex == q)) present |= 1u << q;
            while (present) {  // wave-uniform
                const int e = __builtin_ctz(present);
                present &= present - 1;
                for (int k0 = 0; k0 < rr_pad; k0 += 32) {
                    const v8bf va =
                        ex == e ? *reinterpret_cast<const v8bf*>(v + (size_t)ar * rr_pad + k0 + lg * 8) : v8bf{};
#pragma unroll
                    for (int j = 0; j < NBW; ++j) {
                        const v8bf br = *reinterpret_cast<const v8bf*>(
                            bt_r + ((size_t)e * d_out + nbc[j] * 16 + lr) * rr_pad + k0 + lg * 8);
                        ad[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, br, ad[j], 0, 0, 0);
                    }
                }
            }
        }
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            if (!nb_ok[j]) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = m0 + m * 16 + lg * 4 + r;
                if (t < T) store_y(y, (size_t)t * d_out + (nb0 + j) * 16 + lr, acc[m][j][r] * sw[j] + ad[j][r], y_bf16);
            }
        }
    }
}

template <int WB, int MB>
__global__ __launch_bounds__(256, 2) void gemm_a16_kernel(
    const void* __restrict__ x, int x_dtype, int T, int d_in, int d_out, const uint32_t* __restrict__ w_tiled, int n_tm,
    float* __restrict__ part, const float* __restrict__ w_scale, const uint16_t* __restrict__ u,
    const uint16_t* __restrict__ bt_s, int rs_pad, const uint16_t* __restrict__ v, const int32_t* __restrict__ expert,
    const uint16_t* __restrict__ bt_r, int rr_pad, int n_r, float* __restrict__ y, bool y_bf16) {
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

    if (y != nullptr) {  // K not split: the whole epilogue here
        a16_epilogue<MB, 2>(acc, m0, nb0, T, d_out, lane, w_scale, u, bt_s, rs_pad, v, expert, bt_r, rr_pad, n_r, y, y_bf16);
        return;
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

constexpr int GR_NS = 3;  // ring stages of 64 K: loads run two stages ahead

// x rows in the ring are 128 bytes (eight 16-byte chunks).  At MFMA step s2 of a half block,
// lane (lr, lg) reads logical chunk 4 s2 + lg (3-bit weights) or 2 lg + s2 (4-bit weights); the
// 4-bit layout stores logical chunk 2 a + b at chunk 4 b + a, so both read physical chunk
// 4 s2 + lg, and that chunk is XORed with row & 7.  Measured with the LDS bank-conflict
// counter on this part: no conflicts for either format (XOR with (row & 7) ^ ((row >> 3) & 1)
// doubles the LDS cycles, and so does the 4-bit order without the rotation).
__device__ inline int ring_swz(int row) { return row & 7; }
template <int WB>
__device__ inline int ring_logical_chunk(int pc) { return WB == 4 ? 2 * (pc & 3) + (pc >> 2) : pc; }

template <int WB>
__global__ __launch_bounds__(256, 2) void gemm_a16_ring_kernel(
    const void* __restrict__ x, int T, int d_in, int d_out, const uint32_t* __restrict__ w_tiled, int n_tm,
    float* __restrict__ part, const float* __restrict__ w_scale, const uint16_t* __restrict__ u,
    const uint16_t* __restrict__ bt_s, int rs_pad, const uint16_t* __restrict__ v, const int32_t* __restrict__ expert,
    const uint16_t* __restrict__ bt_r, int rr_pad, int n_r, float* __restrict__ y, bool y_bf16) {
    constexpr int MB = 8, BM = 128, NBW = 4;
    constexpr int X_BYTES = BM * 128;                     // x tile of one 64-K half block
    constexpr int W_WAVE = NBW * 2 * 256;                 // one wave's two fragment dwords per block
    constexpr int STAGE = X_BYTES + 4 * W_WAVE;           // 24 KB: two workgroups fit one CU
    constexpr int X_DMA = X_BYTES / 16 / 256;             // 16-byte x copies per thread and stage
    constexpr int OPS = X_DMA + 2 * NBW;                  // DMA instructions per thread and stage
    __shared__ __attribute__((aligned(1024))) uint8_t smem[GR_NS * STAGE];

    const int tm = blockIdx.x % n_tm, tn = blockIdx.x / n_tm;
    const int m0 = tm * BM;
    const int NB = d_out >> 4, KB = d_in >> 7;
    const int kb0 = (int)((long)blockIdx.y * KB / gridDim.y), kb1 = (int)((long)(blockIdx.y + 1) * KB / gridDim.y);
    const int nh = 2 * (kb1 - kb0);  // 64-K halves
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: LDS bases stay scalar
    const int nb0 = tn * 16 + NBW * wid;
    const uint32_t lds0 = lds_addr(smem);
    const uint16_t* xb = reinterpret_cast<const uint16_t*>(x) + (size_t)kb0 * 128;

    // x copy p of this thread: chunk i = 256 p + tid is LDS slot (row i / 8, slot i % 8) and
    // holds physical chunk slot ^ ring_swz(row) of the row
    const uint16_t* xsrc[X_DMA];
#pragma unroll
    for (int p = 0; p < X_DMA; ++p) {
        const int i = p * 256 + tid, row = i >> 3, slot = i & 7;
        xsrc[p] = xb + (size_t)min(m0 + row, T - 1) * d_in + (ring_logical_chunk<WB>(slot ^ ring_swz(row)) << 3);
    }
    // this lane's fragment dwords of K block kb0 for each of the wave's channel blocks (blocks
    // past d_out repeat a valid block, never stored); a half block uses two of them: W3 the
    // magnitudes of its two steps and the signs, W4 its two steps' codes
    const uint32_t* wsrc[NBW];
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
        const size_t nb = min(nb0 + j, NB - 1);
        wsrc[j] = WB == 3 ? w_tiled + ((nb * KB + kb0) * 64 + lane) * 3 : w_tiled + ((nb * 2 * KB + 2 * kb0) * 64 + lane) * 2;
    }
    auto issue = [&](int stage, int h) {  // half block h of this workgroup's K range into `stage`
        const uint32_t base = lds0 + stage * STAGE;
#pragma unroll
        for (int p = 0; p < X_DMA; ++p) dma16(xsrc[p] + h * 64, base + (p * 256 + wid * 64) * 16);
        const uint32_t wbase = base + X_BYTES + wid * W_WAVE;
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            if constexpr (WB == 3) {
                const uint32_t* q = wsrc[j] + (h >> 1) * 192;
                dma4(q + (h & 1), wbase + (j * 2) * 256);
                dma4(q + 2, wbase + (j * 2 + 1) * 256);
            } else {
                const uint32_t* q = wsrc[j] + h * 128;
                dma4(q, wbase + (j * 2) * 256);
                dma4(q + 1, wbase + (j * 2 + 1) * 256);
            }
        }
    };

    v4f acc[MB][NBW];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int j = 0; j < NBW; ++j) acc[m][j] = v4f{0, 0, 0, 0};

#pragma unroll
    for (int st = 0; st < GR_NS - 1; ++st) issue(st, min(st, nh - 1));
    QE_WAIT_VMCNT_LDS((GR_NS - 2) * OPS);
    QE_WG_BARRIER();

    auto half = [&](int i, auto hh_c) {  // half i (of parity hh) of the K range
        constexpr int hh = decltype(hh_c)::value;
        // refill the slot consumed in the previous half (past the end: a harmless repeat)
        issue((i + GR_NS - 1) % GR_NS, min(i + GR_NS - 1, nh - 1));
        const uint8_t* st = smem + (i % GR_NS) * STAGE;
        const uint32_t* wl = reinterpret_cast<const uint32_t*>(st + X_BYTES + wid * W_WAVE);
        uint32_t f[NBW][Frag<WB>::kWords];
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            const uint32_t g0 = wl[(j * 2) * 64 + lane], g1 = wl[(j * 2 + 1) * 64 + lane];
#pragma unroll
            for (int q = 0; q < Frag<WB>::kWords; ++q) f[j][q] = 0;
            if constexpr (WB == 3) {
                f[j][hh] = g0;
                f[j][2] = g1;
            } else {
                f[j][2 * hh] = g0;
                f[j][2 * hh + 1] = g1;
            }
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int s = 2 * hh + s2;
            v8bf b[NBW];
#pragma unroll
            for (int j = 0; j < NBW; ++j) b[j] = weight_frag<WB>(f[j], s);
            const int c = 4 * s2 + lg;  // physical chunk of the step's 8 activations
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                const int row = m * 16 + lr;
                const v8bf a = *reinterpret_cast<const v8bf*>(st + row * 128 + ((c ^ ring_swz(row)) << 4));
#pragma unroll
                for (int j = 0; j < NBW; ++j)
                    acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[j], acc[m][j], 0, 0, 0);
            }
        }
        // the slot read here is refilled in the next half: every LDS read must have completed,
        // and the next half must have landed (the later one may still be in flight)
        __builtin_amdgcn_sched_barrier(0);
        QE_WAIT_VMCNT_LDS((GR_NS - 2) * OPS);
        QE_WG_BARRIER();
    };
    for (int i = 0; i < nh; i += 2) {
        half(i, std::integral_constant<int, 0>{});
        half(i + 1, std::integral_constant<int, 1>{});
    }
    QE_WAIT_VMCNT(0);

    // lane holds rows 16m + 4lg + r, column 16 nb + lr of each block; the A operands of the
    // adapter MFMAs are rows 16m + lr
    if (y != nullptr) {  // K not split: the whole epilogue here
        a16_epilogue<MB, NBW>(acc, m0, nb0, T, d_out, lane, w_scale, u, bt_s, rs_pad, v, expert, bt_r, rr_pad, n_r, y, y_bf16);
        return;
    }

    float* out = part + (size_t)blockIdx.y * T * d_out;
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
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

// Finish of a K-split A16 product: a workgroup sums the float partials of a 16-token x 64-channel
// tile (a 16 x 16 block per wave, small enough that narrow outputs still give hundreds of
// workgroups) straight into the MFMA accumulator layout (fixed split order) and applies the
// epilogue of the unsplit kernels, so each adapter row is read once per 16 tokens (a thread per
// output re-read them for every token).
__global__ __launch_bounds__(256) void gemm_a16_finish_kernel(
    const float* __restrict__ part, int ksplit, int T, int d_out, int n_tm, const float* __restrict__ w_scale,
    const uint16_t* __restrict__ u, const uint16_t* __restrict__ bt_s, int rs_pad, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ expert, const uint16_t* __restrict__ bt_r, int rr_pad, int n_r,
    float* __restrict__ y, bool y_bf16) {
    constexpr int MB = 1, NBW = 1;
    const int tm = blockIdx.x % n_tm, tn = blockIdx.x / n_tm;
    const int m0 = tm * 16;
    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int nb0 = tn * 4 + NBW * wid;
    const int NB = d_out >> 4;
    v4f acc[MB][NBW];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int j = 0; j < NBW; ++j) acc[m][j] = v4f{0, 0, 0, 0};
    // lane holds rows m0 + 16m + 4lg + r and column 16 (nb0 + j) + lr; rows and blocks past the
    // ends read a valid partial (never stored)
    size_t off[MB][NBW][4];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                off[m][j][r] = (size_t)min(m0 + 16 * m + 4 * lg + r, T - 1) * d_out + min(nb0 + j, NB - 1) * 16 + lr;
    for (int ks = 0; ks < ksplit; ++ks) {
        const float* pk = part + (size_t)ks * T * d_out;
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int j = 0; j < NBW; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[m][j][r] += pk[off[m][j][r]];
    }
    a16_epilogue<MB, NBW>(acc, m0, nb0, T, d_out, lane, w_scale, u, bt_s, rs_pad, v, expert, bt_r, rr_pad, n_r, y, y_bf16);
}

// Finish of a K-split int8 main product (A6 / A8 with few tokens): the int32 partials of a 16 x 64
// tile summed in split order (exact), times s_x[t], then the same epilogue (times s_w, low-rank
// terms on MFMA, adapter rows read once per 16 tokens).  The main term is ((float)acc * s_x) * s_w,
// as in the unsplit GEMM.
__global__ __launch_bounds__(256) void gemm_i8_finish_kernel(
    const int32_t* __restrict__ part, int ksplit, int T, int d_out, int n_tm, const float* __restrict__ s_x,
    const float* __restrict__ w_scale, const uint16_t* __restrict__ u, const uint16_t* __restrict__ bt_s, int rs_pad,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ expert, const uint16_t* __restrict__ bt_r,
    int rr_pad, int n_r, float* __restrict__ y, bool y_bf16) {
    const int tm = blockIdx.x % n_tm, tn = blockIdx.x / n_tm;
    const int m0 = tm * 16;
    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int nb0 = tn * 4 + wid;
    const int NB = d_out >> 4;
    size_t off[4];
    int32_t si[4] = {0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < 4; ++r) off[r] = (size_t)min(m0 + 4 * lg + r, T - 1) * d_out + min(nb0, NB - 1) * 16 + lr;
    for (int ks = 0; ks < ksplit; ++ks) {
        const int32_t* pk = part + (size_t)ks * T * d_out;
#pragma unroll
        for (int r = 0; r < 4; ++r) si[r] += pk[off[r]];
    }
    v4f acc[1][1];
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[0][0][r] = (float)si[r] * s_x[min(m0 + 4 * lg + r, T - 1)];
    a16_epilogue<1, 1>(acc, m0, nb0, T, d_out, lane, w_scale, u, bt_s, rs_pad, v, expert, bt_r, rr_pad, n_r, y, y_bf16);
}

inline int a16_mb(int T) { return T >= 512 ? 8 : 4; }
// channel blocks per workgroup: the ring kernel (many tokens, bf16 x) takes 16
inline int a16_nbg(int T, int x_dtype) { return T >= 512 && x_dtype == QE_BF16 ? 16 : GA_NB; }

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

// The whole A16 main product with its epilogue: y = s_w * (x . q_w^T) + u.B_s + v.B_{e_t}.
// part: float [ksplit][T][d_out] scratch (unused when the many-token kernel finishes in place).
hipError_t launch_gemm_a16(const void* x, int x_dtype, int T, int d_in, int d_out, int w_bits, const void* w_tiled,
                           int ksplit, float* part, const float* w_scale, const uint16_t* u, const uint16_t* bt_s,
                           int rs_pad, const uint16_t* v, const int32_t* expert, const uint16_t* bt_r, int rr_pad,
                           int n_r, float* y, bool y_bf16, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if ((w_bits != 3 && w_bits != 4) || d_in % 128 || d_out % 16 || ksplit < 1 || ksplit > d_in / 128)
        return hipErrorInvalidValue;
    const int mb = a16_mb(T), BM = 16 * mb, nbg = a16_nbg(T, x_dtype);
    const int n_tm = (T + BM - 1) / BM, n_tn = (d_out / 16 + nbg - 1) / nbg;
    const uint32_t* w = reinterpret_cast<const uint32_t*>(w_tiled);
    const bool ring = mb == 8 && x_dtype == QE_BF16;
    const bool fused = ksplit == 1;
#define QE_A16_LAUNCH(WBV, MBV)                                                                                      \
    hipLaunchKernelGGL((gemm_a16_kernel<WBV, MBV>), dim3(n_tm * n_tn, ksplit), dim3(256), 0, st, x, x_dtype, T,    \
                       d_in, d_out, w, n_tm, part, w_scale, u, bt_s, rs_pad, v, expert, bt_r, rr_pad, n_r,        \
                       fused ? y : nullptr, y_bf16)
#define QE_RING_LAUNCH(WBV)                                                                                         \
    hipLaunchKernelGGL(gemm_a16_ring_kernel<WBV>, dim3(n_tm * n_tn, ksplit), dim3(256), 0, st, x, T, d_in, d_out, w, \
                       n_tm, part, w_scale, u, bt_s, rs_pad, v, expert, bt_r, rr_pad, n_r, fused ? y : nullptr, y_bf16)
    if (ring) {  // many tokens: the DMA ring (bf16 rows copied as they are)
        if (w_bits == 3) QE_RING_LAUNCH(3);
        else QE_RING_LAUNCH(4);
    } else if (w_bits == 3) {
        if (mb == 8) QE_A16_LAUNCH(3, 8);
        else QE_A16_LAUNCH(3, 4);
    } else {
        if (mb == 8) QE_A16_LAUNCH(4, 8);
        else QE_A16_LAUNCH(4, 4);
    }
#undef QE_A16_LAUNCH
#undef QE_RING_LAUNCH
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || fused) return e;
    const int f_tm = (T + 15) / 16;
    hipLaunchKernelGGL(gemm_a16_finish_kernel, dim3(f_tm * ((d_out / 16 + 3) / 4)), dim3(256), 0, st, part,
                       ksplit, T, d_out, f_tm, w_scale, u, bt_s, rs_pad, v, expert, bt_r, rr_pad, n_r, y, y_bf16);
    return hipGetLastError();
}

hipError_t launch_gemm_split_finish(const int32_t* part, int ksplit, int T, int d_out, const float* s_x,
                                    const float* w_scale, const uint16_t* u, const uint16_t* bt_s, int rs_pad,
                                    const uint16_t* v, const int32_t* expert, int n_r, const uint16_t* bt_r,
                                    int rr_pad, float* y, bool y_bf16, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if (d_out % 16) return hipErrorInvalidValue;
    const int n_tm = (T + 15) / 16;
    hipLaunchKernelGGL(gemm_i8_finish_kernel, dim3(n_tm * ((d_out / 16 + 3) / 4)), dim3(256), 0, st, part, ksplit, T,
                       d_out, n_tm, s_x, w_scale, u, bt_s, rs_pad, v, expert, bt_r, rr_pad, n_r, y, y_bf16);
    return hipGetLastError();
}

}  // namespace qe
