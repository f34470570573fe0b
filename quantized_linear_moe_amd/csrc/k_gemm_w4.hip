// Quantized main product of a QE linear on int8 MFMA (gfx950), with the
// dequantization and both low-rank corrections fused into the epilogue.
//
//   acc[t][i] = sum_j codes[t][j] * q_w[i][j]              (exact int32)
//   y[t][i]   = acc * s_x[t] * s_w[i] + u[t] . B_s[:, i] + v[t] . B_{e_t}[:, i]
//
// The s*d^2 term of the thelatestinai.com listing's Table 7 (complexity of a QE
// linear) plus the shared and routed low-rank terms of the MCISLAB DeepRead
// summary, "Method".
//
// Design (CDNA4, wave64):
//   * v_mfma_i32_16x16x64_i8.  4-bit weight codes are expanded to int8 in
//     registers as 16*code (the nibble is moved into the high half of its byte:
//     one AND or one shift+AND per 4 codes, no sign extension), so the int32
//     accumulator holds 16*acc exactly (|16*acc| < 2^31 for d_in <= 150000 at A8)
//     and an arithmetic shift recovers acc.
//   * Weights are pre-tiled at load time: 512 contiguous bytes per 16 channels x
//     one 64-wide K step, each lane's 8 bytes being exactly its MFMA fragment.
//   * Both operands go global -> LDS by DMA (global_load_lds_dwordx4) into a
//     4-stage ring, three K steps ahead of the MFMAs, with no staging registers;
//     the activation-code rows use an XOR swizzle of their 16-byte chunks
//     against bank conflicts.
//   * Workgroup tile 128 tokens x 256 channels; wave tile 128 x 64
//     (8 x 4 MFMA blocks, 128 accumulator registers); 64-token tiles when the
//     grid would otherwise leave CUs idle (narrow projections).
//   * Tokens may be visited in an expert-sorted order (`perm`): code rows are
//     gathered and output rows scattered, so a tile meets one or two routed
//     experts instead of all of them.
//   * Epilogue: int32 -> float, scale by s_x and s_w, then bf16 MFMA
//     16x16x32 steps accumulate u.B_s and, for every routed expert present in
//     the tile, (v masked to that expert's tokens).B_e on top of it.
//   * Few tokens (a grid far below the CU count): the K steps are split over
//     gridDim.y workgroups that store their exact int32 partial sums; a finish
//     kernel adds them in split order (still exact) and applies the epilogue.

#include <algorithm>

#include "qe_dma.h"
#include "qe_internal.h"

namespace qe {

constexpr int G_BN = 256;
constexpr int G_BK = 64;   // K per pipeline stage (one int8 MFMA K step)
constexpr int G_NS = 4;    // stages in the LDS ring of 128-token tiles: loads run three stages ahead
constexpr int G_NBW = 4;   // N blocks per wave

// A tile rows are 64 bytes (four 16-byte chunks); chunk c of row r is stored at
// c ^ ((r >> 1) & 3), which spreads the 16-byte reads of 8 consecutive rows over all banks.
__device__ inline int a_swz(int row) { return (row >> 1) & 3; }

// MB: 16-row M blocks per workgroup (tile MB*16 tokens x 256 channels).  Tile rows are
// positions in `perm` order when perm != NULL (tokens grouped by routed expert, so a
// tile meets few experts in the epilogue), else token order.
// kFast: adapter ranks <= 32 and no accumulator dump; the epilogue then reads every
// operand from LDS (see below).
template <int MB, bool kFast>
__global__ __launch_bounds__(256, 2) void gemm_w4_kernel(
    const int8_t* __restrict__ codes, const float* __restrict__ s_x, const uint8_t* __restrict__ w_tiled,
    const float* __restrict__ w_scale, int T, int d_in, int d_out, const uint16_t* __restrict__ u,
    const uint16_t* __restrict__ bt_s, int rs_pad, const uint16_t* __restrict__ v, const int32_t* __restrict__ expert,
    const uint16_t* __restrict__ bt_r, int rr_pad, int n_r, const int32_t* __restrict__ perm, float* __restrict__ y,
    int32_t* __restrict__ acc_debug, int n_tm, int32_t* __restrict__ part) {
    constexpr int BM = MB * 16;
    constexpr int A_STAGE = BM * G_BK;            // bytes of codes per stage
    constexpr int B_STAGE = 4 * G_NBW * 512;      // 4 waves x 4 N blocks x 512 B of packed weights
    constexpr int STAGE = A_STAGE + B_STAGE;
    constexpr int A_DMA = A_STAGE / 1024 / 4;     // A copies per wave per stage
    constexpr int OPS = A_DMA + 2;                // DMA instructions per thread per stage
    // ring depth: 64-token tiles run few workgroups per CU with short K steps, so their loads
    // run further ahead to cover the memory latency
    constexpr int NS = MB == 4 ? 8 : G_NS;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * STAGE];

    const int tm = blockIdx.x % n_tm, tn = blockIdx.x / n_tm;
    const int m0 = tm * BM;
    const int NB = d_out >> 4, KB = d_in / G_BK;
    // K steps of this workgroup: all of them, or split gridDim.y of `part`'s partial sums
    const int kb_beg = (int)((long)blockIdx.y * KB / gridDim.y), nk = (int)((long)(blockIdx.y + 1) * KB / gridDim.y) - kb_beg;
    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
    const int nb0 = tn * (G_BN / 16) + wid * G_NBW;
    const int lr = lane & 15, lg = lane >> 4;
    auto token = [&](int pos) {
        pos = min(pos, T - 1);
        return perm ? perm[pos] : pos;
    };
    const uint32_t lds0 = lds_addr(smem);

    // The tile's rows, read once: token, activation scale and routed expert (clamped into
    // range) go to LDS for the DMA sources and the epilogue; every wave derives the set of
    // experts present.  Two bursts of loads: the tokens, then what they index.
    __shared__ int s_tok[BM];
    __shared__ __attribute__((aligned(16))) float s_sx[BM];
    __shared__ int s_ex[BM];
    const bool routed = v != nullptr && expert != nullptr && bt_r != nullptr && rr_pad > 0 && n_r > 0;
    uint32_t present = 0;
    {
        constexpr int RPL = (BM + 63) / 64;  // rows per lane
        int tk[RPL], ex[RPL];
        float sx[RPL];
#pragma unroll
        for (int i = 0; i < RPL; ++i) tk[i] = perm ? perm[min(m0 + 64 * i + lane, T - 1)] : min(m0 + 64 * i + lane, T - 1);
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            sx[i] = s_x[tk[i]];
            ex[i] = routed ? expert[tk[i]] : 0;
        }
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            const int r = 64 * i + lane;
            const int e = (routed && m0 + r < T) ? min(max(ex[i], 0), n_r - 1) : -1;
            if (routed)
                for (int q = 0; q < n_r; ++q)
                    if (__ballot(e == q)) present |= 1u << q;
            if (wid == 0) {
                s_tok[r] = tk[i];
                s_sx[r] = sx[i];
                s_ex[r] = e;
            }
        }
    }
    __syncthreads();


    // DMA sources.  A: copy q = wid + 4p covers tile rows 16q..16q+15; lane i fetches the
    // logical chunk stored at its LDS slot (row 16q + i/4, slot i%4).
    const int8_t* a_src[A_DMA];
#pragma unroll
    for (int p = 0; p < A_DMA; ++p) {
        const int q = wid + 4 * p, r = 16 * q + (lane >> 2), c = (lane & 3) ^ a_swz(r);
        a_src[p] = codes + (size_t)s_tok[r] * d_in + c * 16;
    }
    // B: copy p of this wave moves the 512-byte K-step tiles of N blocks 2p and 2p+1
    // (lanes 0-31 and 32-63); blocks past d_out fetch block 0 and are never stored.
    const uint8_t* b_src[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int nb = nb0 + 2 * p + (lane >> 5);
        b_src[p] = w_tiled + (size_t)(nb < NB ? nb : 0) * KB * 512 + (lane & 31) * 16;
    }
    auto issue = [&](int stage, int i) {  // copy the workgroup's K step i into ring slot `stage`
        const uint32_t base = lds0 + stage * STAGE;
        const int kb = kb_beg + i;
#pragma unroll
        for (int p = 0; p < A_DMA; ++p) dma16(a_src[p] + (size_t)kb * G_BK, base + (wid + 4 * p) * 1024);
#pragma unroll
        for (int p = 0; p < 2; ++p) dma16(b_src[p] + (size_t)kb * 512, base + A_STAGE + wid * 2048 + p * 1024);
    };

    bool nb_ok[G_NBW];
#pragma unroll
    for (int j = 0; j < G_NBW; ++j) nb_ok[j] = (nb0 + j) < NB;

    v4i acc[MB][G_NBW];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int j = 0; j < G_NBW; ++j) acc[m][j] = v4i{0, 0, 0, 0};

    // prologue: three stages in flight, then wait for the first
#pragma unroll
    for (int st = 0; st < NS - 1; ++st) issue(st, min(st, nk - 1));
    QE_WAIT_VMCNT_LDS((NS - 2) * OPS);
    QE_WG_BARRIER();

    for (int kb = 0; kb < nk; ++kb) {
        // refill the slot consumed in the previous step (past the end: a harmless repeat)
        issue((kb + NS - 1) % NS, min(kb + NS - 1, nk - 1));
        const uint8_t* st = smem + (kb % NS) * STAGE;
        v2u bp[G_NBW];
#pragma unroll
        for (int j = 0; j < G_NBW; ++j)
            bp[j] = *reinterpret_cast<const v2u*>(st + A_STAGE + wid * 2048 + j * 512 + lane * 8);
        v4i a[MB];
#pragma unroll
        for (int m = 0; m < MB; ++m) {
            const int row = m * 16 + lr;
            a[m] = *reinterpret_cast<const v4i*>(st + row * G_BK + ((lg ^ a_swz(row)) << 4));
        }
        v4i bop[G_NBW];
#pragma unroll
        for (int j = 0; j < G_NBW; ++j) bop[j] = unpack_w4x16(bp[j][0], bp[j][1]);
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int j = 0; j < G_NBW; ++j)
                acc[m][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[m], bop[j], acc[m][j], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, MB + G_NBW, 0);  // LDS reads first
        __builtin_amdgcn_sched_group_barrier(0x002, 3 * G_NBW, 0);    // weight unpack
        __builtin_amdgcn_sched_group_barrier(0x008, MB * G_NBW, 0);   // then the MFMAs
        // nothing of this step may move below the barrier: the slot read here is the
        // DMA target of the next step, so every LDS read must have completed (lgkmcnt 0);
        // and step kb+1 must have landed (the NS-2 later steps may still be in flight)
        __builtin_amdgcn_sched_barrier(0);
        QE_WAIT_VMCNT_LDS((NS - 2) * OPS);
        QE_WG_BARRIER();
    }
    QE_WAIT_VMCNT(0);

    if (part) {  // split K: this workgroup's exact partial sums, in token order
        int32_t* pt = part + (size_t)blockIdx.y * T * d_out;
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m * 16 + lg * 4 + r;
                if (m0 + row >= T) continue;
                int32_t* prow = pt + (size_t)s_tok[row] * d_out;
#pragma unroll
                for (int j = 0; j < G_NBW; ++j)
                    if (nb_ok[j]) prow[(nb0 + j) * 16 + lr] = acc[m][j][r] >> 4;
            }
        return;
    }

    // ------------------------------------------------------------ epilogue
    // lane holds column (nb*16 + lr) and rows (m*16 + lg*4 + r) of each block; the A
    // operands of the adapter MFMAs are rows (m*16 + lr).
    //
    // Common case (kFast): the ring is free now, so the u and v rows of the tile, this
    // wave's B_s fragments and the B_e fragments of up to NSLOT experts present arrive by
    // DMA in one burst; each 16-row block is then dequantized, corrected and stored with
    // every operand read from LDS.  A tile with more experts than the ring holds adds the
    // rest in further rounds, reading back the y rows it stored.
    const bool have_se = u != nullptr && bt_s != nullptr && rs_pad > 0;
    if constexpr (kFast) {
        constexpr int U_OFF = 0, V_OFF = MB * 1024, BS_OFF = 2 * MB * 1024, BR_OFF = BS_OFF + 16384;
        constexpr int NSLOT = (NS * STAGE - BR_OFF) / 16384;  // experts per round
        static_assert(NSLOT >= 1, "LDS ring too small for the epilogue operands");
        QE_WAIT_VMCNT_LDS(0);
        QE_WG_BARRIER();  // every wave is done with the ring
        int nbj[G_NBW];   // fragment sources; blocks past d_out repeat a valid block (never stored)
#pragma unroll
        for (int j = 0; j < G_NBW; ++j) nbj[j] = nb_ok[j] ? nb0 + j : 0;
        if (have_se) {
#pragma unroll
            for (int p = 0; p < MB / 4; ++p) {
                const int m = wid + 4 * p;
                dma16(u + (size_t)s_tok[m * 16 + lr] * rs_pad + lg * 8, lds0 + U_OFF + m * 1024);
            }
#pragma unroll
            for (int j = 0; j < G_NBW; ++j)
                dma16(bt_s + (size_t)(nbj[j] * 16 + lr) * rs_pad + lg * 8, lds0 + BS_OFF + (wid * G_NBW + j) * 1024);
        }
        if (present) {
#pragma unroll
            for (int p = 0; p < MB / 4; ++p) {
                const int m = wid + 4 * p;
                dma16(v + (size_t)s_tok[m * 16 + lr] * rr_pad + lg * 8, lds0 + V_OFF + m * 1024);
            }
        }
        int es[NSLOT];
        uint32_t pend = present;
        auto stage_experts = [&]() {
#pragma unroll
            for (int sl = 0; sl < NSLOT; ++sl) {
                es[sl] = -1;
                if (pend) {
                    es[sl] = __builtin_ctz(pend);
                    pend &= pend - 1;
#pragma unroll
                    for (int j = 0; j < G_NBW; ++j)
                        dma16(bt_r + ((size_t)es[sl] * d_out + nbj[j] * 16 + lr) * rr_pad + lg * 8,
                              lds0 + BR_OFF + sl * 16384 + (wid * G_NBW + j) * 1024);
                }
            }
        };
        stage_experts();
        float sw[G_NBW];
#pragma unroll
        for (int j = 0; j < G_NBW; ++j) sw[j] = nb_ok[j] ? w_scale[(nb0 + j) * 16 + lr] : 0.0f;
        QE_WAIT_VMCNT_LDS(0);
        QE_WG_BARRIER();
        auto routed = [&](int m, v4f (&yv)[G_NBW]) {  // y += (v masked to expert e's rows) . B_e
            const int exm = s_ex[m * 16 + lr];
#pragma unroll
            for (int sl = 0; sl < NSLOT; ++sl) {
                if (es[sl] < 0) break;  // uniform
                const bool mine = exm == es[sl];
                if (__ballot(mine) == 0) continue;  // no row of this block uses the expert
                const v8bf va = mine ? *reinterpret_cast<const v8bf*>(smem + V_OFF + m * 1024 + lane * 16) : v8bf{};
                const uint8_t* lbr = smem + BR_OFF + sl * 16384 + wid * G_NBW * 1024 + lane * 16;
#pragma unroll
                for (int j = 0; j < G_NBW; ++j)
                    yv[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, *reinterpret_cast<const v8bf*>(lbr + j * 1024),
                                                                    yv[j], 0, 0, 0);
            }
        };
        const uint8_t* lbs = smem + BS_OFF + wid * G_NBW * 1024 + lane * 16;
#pragma unroll
        for (int m = 0; m < MB; ++m) {
            const v4f sx = *reinterpret_cast<const v4f*>(&s_sx[m * 16 + lg * 4]);
            v4f yv[G_NBW];
#pragma unroll
            for (int j = 0; j < G_NBW; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) yv[j][r] = (float)(acc[m][j][r] >> 4) * sx[r] * sw[j];
            if (have_se) {  // y += u . B_s
                const v8bf ua = *reinterpret_cast<const v8bf*>(smem + U_OFF + m * 1024 + lane * 16);
#pragma unroll
                for (int j = 0; j < G_NBW; ++j)
                    yv[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ua, *reinterpret_cast<const v8bf*>(lbs + j * 1024),
                                                                    yv[j], 0, 0, 0);
            }
            routed(m, yv);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m * 16 + lg * 4 + r;
                if (m0 + row >= T) continue;
                float* yrow = y + (size_t)s_tok[row] * d_out;
#pragma unroll
                for (int j = 0; j < G_NBW; ++j)
                    if (nb_ok[j]) yrow[(nb0 + j) * 16 + lr] = yv[j][r];
            }
            __builtin_amdgcn_sched_barrier(0);  // one block at a time: keeps register pressure flat
        }
        while (pend) {  // more experts than one round holds (uniform; rare)
            QE_WAIT_VMCNT_LDS(0);
            QE_WG_BARRIER();
            stage_experts();
            QE_WAIT_VMCNT_LDS(0);
            QE_WG_BARRIER();
            for (int m = 0; m < MB; ++m) {
                v4f yv[G_NBW];
#pragma unroll
                for (int r = 0; r < 4; ++r) {  // this lane's own stores of the first round
                    const int row = m * 16 + lg * 4 + r;
                    const float* yrow = y + (size_t)s_tok[row] * d_out;
#pragma unroll
                    for (int j = 0; j < G_NBW; ++j)
                        yv[j][r] = (nb_ok[j] && m0 + row < T) ? yrow[(nb0 + j) * 16 + lr] : 0.0f;
                }
                routed(m, yv);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = m * 16 + lg * 4 + r;
                    if (m0 + row >= T) continue;
                    float* yrow = y + (size_t)s_tok[row] * d_out;
#pragma unroll
                    for (int j = 0; j < G_NBW; ++j)
                        if (nb_ok[j]) yrow[(nb0 + j) * 16 + lr] = yv[j][r];
                }
            }
        }
        return;
    }

    // General case (larger ranks, or the accumulator dump): operands straight from memory.
    if constexpr (!kFast) {
    // lane holds column (nb*16 + lr) and rows (m*16 + lg*4 + r) of each block; the
    // A operands of the adapter MFMAs are rows (m*16 + lr).  Processed one M block at
    // a time to keep register pressure at the main loop's level.
    v8bf bs[G_NBW];
    if (have_se) {  // issued before the dequantization math
#pragma unroll
        for (int j = 0; j < G_NBW; ++j)
            bs[j] = nb_ok[j] ? *reinterpret_cast<const v8bf*>(bt_s + (size_t)((nb0 + j) * 16 + lr) * rs_pad + lg * 8)
                             : v8bf{};
    }
    float sw[G_NBW];
#pragma unroll
    for (int j = 0; j < G_NBW; ++j) sw[j] = nb_ok[j] ? w_scale[(nb0 + j) * 16 + lr] : 0.0f;

    v4f yv[MB][G_NBW];
#pragma unroll
    for (int m = 0; m < MB; ++m) {
        float sx[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) sx[r] = s_x[token(m0 + m * 16 + lg * 4 + r)];
        if (acc_debug) {
#pragma unroll
            for (int j = 0; j < G_NBW; ++j) {
                if (!nb_ok[j]) continue;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (m0 + m * 16 + lg * 4 + r < T)
                        acc_debug[(size_t)token(m0 + m * 16 + lg * 4 + r) * d_out + (nb0 + j) * 16 + lr] = acc[m][j][r] >> 4;
            }
        }
#pragma unroll
        for (int j = 0; j < G_NBW; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) yv[m][j][r] = (float)(acc[m][j][r] >> 4) * sx[r] * sw[j];
        // shared expert: y += u . B_s (one bf16 MFMA K step per 32 of rank)
        if (have_se) {
            const int arow = token(m0 + m * 16 + lr);
            for (int k0 = 0; k0 < rs_pad; k0 += 32) {
                if (k0 > 0) {
#pragma unroll
                    for (int j = 0; j < G_NBW; ++j)
                        bs[j] = nb_ok[j] ? *reinterpret_cast<const v8bf*>(bt_s + (size_t)((nb0 + j) * 16 + lr) * rs_pad + k0 + lg * 8)
                                         : v8bf{};
                }
                const v8bf ua = *reinterpret_cast<const v8bf*>(u + (size_t)arow * rs_pad + k0 + lg * 8);
#pragma unroll
                for (int j = 0; j < G_NBW; ++j) yv[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ua, bs[j], yv[m][j], 0, 0, 0);
            }
            if (rs_pad > 32 && m + 1 < MB) {  // restore the first K step for the next block
#pragma unroll
                for (int j = 0; j < G_NBW; ++j)
                    bs[j] = nb_ok[j] ? *reinterpret_cast<const v8bf*>(bt_s + (size_t)((nb0 + j) * 16 + lr) * rs_pad + lg * 8)
                                     : v8bf{};
            }
        }
    }

    // routed experts: for every expert present among the tile's tokens,
    // y += (v masked to that expert's rows) . B_e
    if (v && expert) {
        int ex[MB];
#pragma unroll
        for (int m = 0; m < MB; ++m) ex[m] = (m0 + m * 16 + lr < T) ? expert[token(m0 + m * 16 + lr)] : -1;
        uint32_t present = 0;
#pragma unroll
        for (int m = 0; m < MB; ++m) {
            for (int e = 0; e < n_r; ++e)
                if (__ballot(ex[m] == e)) present |= 1u << e;
        }
        while (present) {
            const int e = __builtin_ctz(present);
            present &= present - 1;
            for (int k0 = 0; k0 < rr_pad; k0 += 32) {
                v8bf br[G_NBW];
#pragma unroll
                for (int j = 0; j < G_NBW; ++j)
                    br[j] = nb_ok[j] ? *reinterpret_cast<const v8bf*>(
                                           bt_r + ((size_t)e * d_out + (nb0 + j) * 16 + lr) * rr_pad + k0 + lg * 8)
                                     : v8bf{};
#pragma unroll
                for (int m = 0; m < MB; ++m) {
                    if (__ballot(ex[m] == e) == 0) continue;  // no row of this block uses expert e
                    const v8bf va = ex[m] == e ? *reinterpret_cast<const v8bf*>(v + (size_t)token(m0 + m * 16 + lr) * rr_pad + k0 + lg * 8)
                                               : v8bf{};
#pragma unroll
                    for (int j = 0; j < G_NBW; ++j)
                        yv[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, br[j], yv[m][j], 0, 0, 0);
                }
            }
        }
    }

#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int pos = m0 + m * 16 + lg * 4 + r;
            if (pos >= T) continue;
            const size_t rowoff = (size_t)token(pos) * d_out;
#pragma unroll
            for (int j = 0; j < G_NBW; ++j)
                if (nb_ok[j]) y[rowoff + (nb0 + j) * 16 + lr] = yv[m][j][r];
        }
    }
}

// K splits of the main product (fast epilogue only): 1 unless the 64-token-tile grid
// leaves CUs idle.  The 64-token tiles hold one workgroup per CU (their LDS ring), so the
// split grid is kept to one round of 256 workgroups; each split keeps at least 8 K steps,
// and the int32 partials (written and read once) stay within twice the packed weights.
int gemm_ksplit(int T, int d_in, int d_out) {
    const long tiles = (long)((T + 63) / 64) * ((d_out + G_BN - 1) / G_BN);
    if (T <= 0 || tiles >= 128) return 1;
    const long ks = std::min({256 / tiles, (long)(d_in / G_BK / 8), (long)d_in / (4L * T)});
    return (int)std::max(ks, 1L);
}

hipError_t launch_gemm_w4(const int8_t* codes, const float* s_x, const uint8_t* w_tiled, const float* w_scale, int T,
                          int d_in, int d_out, const uint16_t* u, const uint16_t* bt_s, int rs_pad, const uint16_t* v,
                          const int32_t* expert, const uint16_t* bt_r, int rr_pad, int n_r, const int32_t* perm,
                          float* y, int32_t* acc_debug, int ksplit, int32_t* part, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    const int n_tn = (d_out + G_BN - 1) / G_BN;
    // 128-token tiles unless that leaves the chip less than two workgroups per CU
    const bool small = (long)((T + 127) / 128) * n_tn < 512;
    const uint8_t* w = w_tiled;
    const bool split = ksplit > 1 && part != nullptr && acc_debug == nullptr && rs_pad <= 32 && rr_pad <= 32;
    if (split && !small) return hipErrorInvalidValue;
    const bool fast = !acc_debug && rs_pad <= 32 && rr_pad <= 32;
    const int ks = split ? ksplit : 1;
    int32_t* pp = split ? part : nullptr;
#define QE_GEMM_LAUNCH(MBV, FAST, NTM)                                                                     \
    hipLaunchKernelGGL((gemm_w4_kernel<MBV, FAST>), dim3((NTM) * n_tn, ks), dim3(256), 0, st, codes, s_x, w, \
                       w_scale, T, d_in, d_out, u, bt_s, rs_pad, v, expert, bt_r, rr_pad, n_r, perm, y, acc_debug, NTM, pp)
    if (small) {
        const int n_tm = (T + 63) / 64;
        if (fast) QE_GEMM_LAUNCH(4, true, n_tm);
        else QE_GEMM_LAUNCH(4, false, n_tm);
    } else {
        const int n_tm = (T + 127) / 128;
        if (fast) QE_GEMM_LAUNCH(8, true, n_tm);
        else QE_GEMM_LAUNCH(8, false, n_tm);
    }
#undef QE_GEMM_LAUNCH
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !split) return e;
    const bool routed = v != nullptr && expert != nullptr && bt_r != nullptr && rr_pad > 0 && n_r > 0;
    return launch_gemm_split_finish(part, ks, T, d_out, s_x, w_scale, rs_pad > 0 ? u : nullptr, bt_s, rs_pad,
                                    routed ? v : nullptr, routed ? expert : nullptr, n_r, bt_r, rr_pad, y, st);
}

}  // namespace qe
