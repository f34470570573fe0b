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
//     the tile, (v masked to that expert's tokens).B_e on top of it; the tile
//     stays in registers through the expert rounds and leaves as whole 128-byte
//     lines (a wave-private LDS transpose) with non-temporal stores.  Top-2
//     routing adds each token's second expert in the same rounds.
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
// One workgroup's tile: block `bid` of `nblk` (the tile grid of this linear) and K split `ky` of
// `nky`; gemm_w4_kernel runs one linear's grid, gemm_w4_group_kernel the grids of several
// linears in one launch.
// kTop2: top-2 routing; every token also takes the correction of a second expert
// (expert2, with its adapter input v2), added in the same epilogue rounds.
template <int MB, bool kFast, bool kTop2 = false>
__device__ __attribute__((always_inline)) inline void gemm_w4_tile(
    const int8_t* __restrict__ codes, const float* __restrict__ s_x, const uint8_t* __restrict__ w_tiled,
    const float* __restrict__ w_scale, int T, int d_in, int d_out, const uint16_t* __restrict__ u,
    const uint16_t* __restrict__ bt_s, int rs_pad, const uint16_t* __restrict__ v, const int32_t* __restrict__ expert,
    const uint16_t* __restrict__ bt_r, int rr_pad, int n_r, const int32_t* __restrict__ perm, float* __restrict__ y,
    int32_t* __restrict__ acc_debug, int n_tm, int32_t* __restrict__ part, bool y_bf16, int bid, int nblk, int ky,
    int nky, const uint16_t* __restrict__ v2 = nullptr, const int32_t* __restrict__ expert2 = nullptr) {
    static_assert(!kTop2 || (kFast && MB == 8), "top-2 routing takes the fast epilogue of 128-token tiles");
    constexpr int BM = MB * 16;
    constexpr int A_STAGE = BM * G_BK;            // bytes of codes per stage
    constexpr int B_STAGE = 4 * G_NBW * 512;      // 4 waves x 4 N blocks x 512 B of packed weights
    constexpr int STAGE = A_STAGE + B_STAGE;
    constexpr int A_DMA = A_STAGE / 1024 / 4;     // A copies per wave per stage
    constexpr int OPS = A_DMA + 2;                // DMA instructions per thread per stage
    // ring depth: 64-token tiles run few workgroups per CU with short K steps, so their loads
    // run further ahead to cover the memory latency
    constexpr int NS = MB == 4 ? 8 : G_NS;
    // top-2: the second expert's v rows after the ring
    constexpr int V2_OFF = NS * STAGE;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * STAGE + (kTop2 ? MB * 1024 : 0)];

    // Tile order.  Workgroups are handed to the 8 XCDs in turn (block b to XCD b % 8), each
    // XCD with its own L2: the block index is renumbered so that every XCD walks a contiguous
    // range of logical tiles, and logical tiles run down groups of 8 token tiles across the
    // channel tiles.  An XCD then touches 8 token tiles and a band of channel tiles, so every
    // activation tile is fetched by about 2 XCDs and every weight tile by about 4 (the plain
    // order made all 8 fetch every weight tile); the result does not depend on the order.
    int tm, tn;
    {
        const int G = nblk, n_tn = G / n_tm;
        int L = bid;
        if ((G & 7) == 0) L = (L & 7) * (G >> 3) + (L >> 3);
        constexpr int GM = 8;
        const int per_group = GM * n_tn;
        const int g = L / per_group, first = g * GM, gs = min(n_tm - first, GM), r = L - g * per_group;
        tm = first + r % gs;
        tn = r / gs;
    }
    const int m0 = tm * BM;
    const int NB = d_out >> 4, KB = d_in / G_BK;
    // K steps of this workgroup: all of them, or split nky of `part`'s partial sums
    const int kb_beg = (int)((long)ky * KB / nky), nk = (int)((long)(ky + 1) * KB / nky) - kb_beg;
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
    __shared__ int s_ex2[kTop2 ? BM : 1];
    const bool routed = v != nullptr && expert != nullptr && bt_r != nullptr && rr_pad > 0 && n_r > 0;
    uint32_t present = 0;  // experts of the tile's rows (first and, top-2, second)
    {
        constexpr int RPL = (BM + 63) / 64;  // rows per lane
        int tk[RPL], ex[RPL], ex2[RPL];
        float sx[RPL];
#pragma unroll
        for (int i = 0; i < RPL; ++i) tk[i] = perm ? perm[min(m0 + 64 * i + lane, T - 1)] : min(m0 + 64 * i + lane, T - 1);
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            sx[i] = s_x[tk[i]];
            ex[i] = routed ? expert[tk[i]] : 0;
            if constexpr (kTop2) ex2[i] = routed ? expert2[tk[i]] : 0;
        }
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            const int r = 64 * i + lane;
            const int e = (routed && m0 + r < T) ? min(max(ex[i], 0), n_r - 1) : -1;
            const int e2 = (kTop2 && routed && m0 + r < T) ? min(max(ex2[i], 0), n_r - 1) : -1;
            if (routed)
                for (int q = 0; q < n_r; ++q)
                    if (__ballot(e == q || e2 == q)) present |= 1u << q;
            if (wid == 0) {
                s_tok[r] = tk[i];
                s_sx[r] = sx[i];
                s_ex[r] = e;
                if constexpr (kTop2) s_ex2[r] = e2;
            }
        }
    }
    __syncthreads();
    if constexpr (kTop2) {  // the second expert's v rows, into LDS past the ring (landed by the ring's first wait)
        if (present) {
#pragma unroll
            for (int p = 0; p < MB / 4; ++p) {
                const int m = wid + 4 * p;
                dma16(v2 + (size_t)s_tok[m * 16 + lr] * rr_pad + lg * 8, lds0 + V2_OFF + m * 1024);
            }
        }
    }


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

    // Operands of the fast epilogue (see below): the u and v rows of the tile, this wave's
    // B_s fragments and the B_e fragments of up to NSLOT routed experts present, in the ring.
    // 128-token tiles with at least NS K steps load them during their last NS-1 K steps,
    // whose ring slots take no further K step: slot nk%NS the u and v rows, slot (nk+1)%NS
    // the B_s fragments, slot (nk+2)%NS the first expert's B_e fragments (a second expert
    // goes to the last K step's slot after the loop).  Other tiles load them all after the
    // loop at fixed places.  Each tail step issues exactly OPS copies, as a K step does, so
    // the ring's vmcnt waits keep their meaning (an operand the tile does not use is
    // replaced by a copy of a valid code row that is never read).
    const bool have_se = u != nullptr && bt_s != nullptr && rs_pad > 0;
    constexpr int NSLOT = (NS * STAGE - 2 * MB * 1024 - 16384) / 16384;  // experts per round
    static_assert(NSLOT >= 1, "LDS ring too small for the epilogue operands");
    const bool pre = kFast && MB == 8 && part == nullptr && nk >= NS;
    static_assert(MB != 8 || (2 * (MB / 4) == OPS && G_NBW == OPS), "tail steps must issue OPS copies");
    int nbj[G_NBW];  // fragment sources; blocks past d_out repeat a valid block (never stored)
#pragma unroll
    for (int j = 0; j < G_NBW; ++j) nbj[j] = nb_ok[j] ? nb0 + j : 0;
    int u_off = 0, bs_off = 2 * MB * 1024, br_off[NSLOT];
#pragma unroll
    for (int sl = 0; sl < NSLOT; ++sl) br_off[sl] = bs_off + 16384 * (sl + 1);
    if (pre) {
        u_off = (nk % NS) * STAGE;
        bs_off = ((nk + 1) % NS) * STAGE;
        br_off[0] = ((nk + 2) % NS) * STAGE;
        br_off[NSLOT - 1] = ((nk + 3) % NS) * STAGE;
    }
    const int v_off = u_off + MB * 1024;
    int es[NSLOT];  // experts of the current round (-1: none), taken in index order from `pend`
    uint32_t pend = present;
    auto pick_experts = [&]() {
#pragma unroll
        for (int sl = 0; sl < NSLOT; ++sl) {
            es[sl] = -1;
            if (pend) {
                es[sl] = __builtin_ctz(pend);
                pend &= pend - 1;
            }
        }
    };
    pick_experts();
    float sw[G_NBW];
#pragma unroll
    for (int j = 0; j < G_NBW; ++j) sw[j] = nb_ok[j] ? w_scale[(nb0 + j) * 16 + lr] : 0.0f;
    auto prefetch_epilogue = [&](int part_j) {  // tail step part_j = 0, 1, 2 (pre only)
        const int8_t* dummy = a_src[0];
        if (part_j == 0) {
#pragma unroll
            for (int p = 0; p < MB / 4; ++p) {
                const int m = wid + 4 * p;
                const void* src = have_se ? (const void*)(u + (size_t)s_tok[m * 16 + lr] * rs_pad + lg * 8) : dummy;
                dma16(src, lds0 + u_off + m * 1024);
            }
#pragma unroll
            for (int p = 0; p < MB / 4; ++p) {
                const int m = wid + 4 * p;
                const void* src = es[0] >= 0 ? (const void*)(v + (size_t)s_tok[m * 16 + lr] * rr_pad + lg * 8) : dummy;
                dma16(src, lds0 + v_off + m * 1024);
            }
        } else if (part_j == 1) {
#pragma unroll
            for (int j = 0; j < G_NBW; ++j) {
                const void* src = have_se ? (const void*)(bt_s + (size_t)(nbj[j] * 16 + lr) * rs_pad + lg * 8) : dummy;
                dma16(src, lds0 + bs_off + (wid * G_NBW + j) * 1024);
            }
        } else {
#pragma unroll
            for (int j = 0; j < G_NBW; ++j) {
                const void* src = es[0] >= 0 ? (const void*)(bt_r + ((size_t)es[0] * d_out + nbj[j] * 16 + lr) * rr_pad + lg * 8)
                                             : dummy;
                dma16(src, lds0 + br_off[0] + (wid * G_NBW + j) * 1024);
            }
        }
    };

    // prologue: three stages in flight, then wait for the first
#pragma unroll
    for (int st = 0; st < NS - 1; ++st) issue(st, min(st, nk - 1));
    QE_WAIT_VMCNT_LDS((NS - 2) * OPS);
    QE_WG_BARRIER();

    auto k_step = [&](int kb) {  // the MFMAs of K step kb (ring slot kb % NS)
        const uint8_t* st = smem + (kb % NS) * STAGE;
        v2u bp[G_NBW];
#pragma unroll
        for (int j = 0; j < G_NBW; ++j)
            bp[j] = *reinterpret_cast<const v2u*>(st + A_STAGE + wid * 2048 + j * 512 + lane * 8);
        // the weight fragments are requested first: their unpacking then overlaps the
        // activation reads, and the first MFMAs wait for one activation row only (left to
        // itself the compiler may issue them last, and every MFMA then waits for all reads)
        __builtin_amdgcn_sched_barrier(0);
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
        __builtin_amdgcn_sched_group_barrier(0x100, MB, 0);           // activation reads first
        __builtin_amdgcn_sched_group_barrier(0x002, 3 * G_NBW, 0);    // weight unpack
        __builtin_amdgcn_sched_group_barrier(0x008, MB * G_NBW, 0);   // then the MFMAs
        // nothing of this step may move below the barrier: the slot read here is the
        // DMA target of the next step, so every LDS read must have completed (lgkmcnt 0);
        // and step kb+1 must have landed (the NS-2 later steps may still be in flight)
        __builtin_amdgcn_sched_barrier(0);
        QE_WAIT_VMCNT_LDS((NS - 2) * OPS);
        QE_WG_BARRIER();
    };
    // each step first refills the slot consumed in the previous one; past the end that is a
    // harmless repeat, or (pre) the epilogue's operands, in a loop of its own so that their
    // addresses are not held in registers through the main loop
    const int nk_main = pre ? nk - (NS - 1) : nk;
    int kb = 0;
    for (; kb < nk_main; ++kb) {
        issue((kb + NS - 1) % NS, min(kb + NS - 1, nk - 1));
        k_step(kb);
    }
    for (; kb < nk; ++kb) {
        prefetch_epilogue(kb + NS - 1 - nk);
        k_step(kb);
    }
    QE_WAIT_VMCNT(0);

    if (part) {  // split K: this workgroup's exact partial sums, in token order
        int32_t* pt = part + (size_t)ky * T * d_out;
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
    // Common case (kFast): every operand is read from LDS (loaded into the ring as set out
    // above); the tile is dequantized and corrected in registers, round by round of experts,
    // then stored.
    if constexpr (kFast) {
        QE_WAIT_VMCNT_LDS(0);
        QE_WG_BARRIER();  // every wave is done with the ring; the tail's copies have landed
        auto stage_experts = [&](int first) {
#pragma unroll
            for (int sl = 0; sl < NSLOT; ++sl) {
                if (sl < first || es[sl] < 0) continue;  // uniform
#pragma unroll
                for (int j = 0; j < G_NBW; ++j)
                    dma16(bt_r + ((size_t)es[sl] * d_out + nbj[j] * 16 + lr) * rr_pad + lg * 8,
                          lds0 + br_off[sl] + (wid * G_NBW + j) * 1024);
            }
        };
        if (!pre) {
            if (have_se) {
#pragma unroll
                for (int p = 0; p < MB / 4; ++p) {
                    const int m = wid + 4 * p;
                    dma16(u + (size_t)s_tok[m * 16 + lr] * rs_pad + lg * 8, lds0 + u_off + m * 1024);
                }
#pragma unroll
                for (int j = 0; j < G_NBW; ++j)
                    dma16(bt_s + (size_t)(nbj[j] * 16 + lr) * rs_pad + lg * 8, lds0 + bs_off + (wid * G_NBW + j) * 1024);
            }
            if (present) {
#pragma unroll
                for (int p = 0; p < MB / 4; ++p) {
                    const int m = wid + 4 * p;
                    dma16(v + (size_t)s_tok[m * 16 + lr] * rr_pad + lg * 8, lds0 + v_off + m * 1024);
                }
            }
            stage_experts(0);
        } else {
            stage_experts(1);  // the first expert's fragments came with the tail
        }
        if (!pre || (NSLOT > 1 && es[1] >= 0)) {  // uniform
            QE_WAIT_VMCNT_LDS(0);
            QE_WG_BARRIER();
        }
        auto routed = [&](int m, v4f (&yv)[G_NBW]) {  // y += (v masked to expert e's rows) . B_e
            const int exm = s_ex[m * 16 + lr];
            const int exm2 = kTop2 ? s_ex2[m * 16 + lr] : -1;
#pragma unroll
            for (int sl = 0; sl < NSLOT; ++sl) {
                if (es[sl] < 0) break;  // uniform
                const bool mine = exm == es[sl];
                const bool mine2 = kTop2 && exm2 == es[sl];  // top-2: rows whose second expert it is
                if (__ballot(mine || mine2) == 0) continue;  // no row of this block uses the expert
                const v8bf va = mine    ? *reinterpret_cast<const v8bf*>(smem + v_off + m * 1024 + lane * 16)
                                : mine2 ? *reinterpret_cast<const v8bf*>(smem + V2_OFF + m * 1024 + lane * 16)
                                        : v8bf{};
                const uint8_t* lbr = smem + br_off[sl] + wid * G_NBW * 1024 + lane * 16;
#pragma unroll
                for (int j = 0; j < G_NBW; ++j)
                    yv[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, *reinterpret_cast<const v8bf*>(lbr + j * 1024),
                                                                    yv[j], 0, 0, 0);
            }
        };
        const uint8_t* lbs = smem + bs_off + wid * G_NBW * 1024 + lane * 16;
        // The whole tile stays in registers through the expert rounds (the accumulators
        // become y in place): a tile with more experts than one round holds (always, for
        // top-2, whose tiles meet most experts as second ones) adds the rest in further rounds
        // without reading back stored rows.
        v4f yt[MB][G_NBW];
#pragma unroll
        for (int m = 0; m < MB; ++m) {
            const v4f sx = *reinterpret_cast<const v4f*>(&s_sx[m * 16 + lg * 4]);
#pragma unroll
            for (int j = 0; j < G_NBW; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) yt[m][j][r] = (float)(acc[m][j][r] >> 4) * sx[r] * sw[j];
            if (have_se) {  // y += u . B_s
                const v8bf ua = *reinterpret_cast<const v8bf*>(smem + u_off + m * 1024 + lane * 16);
#pragma unroll
                for (int j = 0; j < G_NBW; ++j)
                    yt[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        ua, *reinterpret_cast<const v8bf*>(lbs + j * 1024), yt[m][j], 0, 0, 0);
            }
            routed(m, yt[m]);
        }
        while (pend) {  // uniform
            QE_WAIT_VMCNT_LDS(0);
            QE_WG_BARRIER();
            pick_experts();
            stage_experts(0);
            QE_WAIT_VMCNT_LDS(0);
            QE_WG_BARRIER();
#pragma unroll
            for (int m = 0; m < MB; ++m) routed(m, yt[m]);
        }
        // Stores.  A lane holds 16 single columns of four rows; through a wave-private LDS
        // buffer (16 rows x 64 columns, rows padded to 68 floats so a lane group's 16 writes hit
        // distinct banks) each store instruction instead writes four rows x 256 contiguous bytes,
        // whole 128-byte lines, marked non-temporal: y is not read again here, and full-line
        // streaming stores keep the K loops' operands in the caches (partial lines written
        // non-temporally cost more than they save).
        QE_WAIT_LDS();
        QE_WG_BARRIER();  // every wave is done with the operands in the ring
        constexpr int YLD = 68;
        static_assert(4 * 16 * YLD * 4 <= NS * STAGE, "store buffers must fit in the ring");
        float* ybuf = reinterpret_cast<float*>(smem) + wid * 16 * YLD;
        const int sr = lane >> 4, sc = (lane & 15) * 4;  // read-back: row sr + 4i, columns sc..sc+3
        const bool col_ok = nb_ok[(lane & 15) >> 2];
#pragma unroll
        for (int m = 0; m < MB; ++m) {
#pragma unroll
            for (int j = 0; j < G_NBW; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) ybuf[(lg * 4 + r) * YLD + j * 16 + lr] = yt[m][j][r];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = m * 16 + sr + 4 * i;
                const v4f val = *reinterpret_cast<const v4f*>(&ybuf[(sr + 4 * i) * YLD + sc]);
                if (col_ok && m0 + row < T)
                    __builtin_nontemporal_store(val, reinterpret_cast<v4f*>(y + (size_t)s_tok[row] * d_out + nb0 * 16 + sc));
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
                if (nb_ok[j]) store_y(y, rowoff + (nb0 + j) * 16 + lr, yv[m][j][r], y_bf16);
        }
    }
}

template <int MB, bool kFast>
__global__ __launch_bounds__(256, 2) void gemm_w4_kernel(
    const int8_t* __restrict__ codes, const float* __restrict__ s_x, const uint8_t* __restrict__ w_tiled,
    const float* __restrict__ w_scale, int T, int d_in, int d_out, const uint16_t* __restrict__ u,
    const uint16_t* __restrict__ bt_s, int rs_pad, const uint16_t* __restrict__ v, const int32_t* __restrict__ expert,
    const uint16_t* __restrict__ bt_r, int rr_pad, int n_r, const int32_t* __restrict__ perm, float* __restrict__ y,
    int32_t* __restrict__ acc_debug, int n_tm, int32_t* __restrict__ part, bool y_bf16) {
    gemm_w4_tile<MB, kFast>(codes, s_x, w_tiled, w_scale, T, d_in, d_out, u, bt_s, rs_pad, v, expert, bt_r, rr_pad, n_r,
                            perm, y, acc_debug, n_tm, part, y_bf16, blockIdx.x, gridDim.x, blockIdx.y, gridDim.y);
}

// Several linears' 128-token-tile grids in one launch (linears that read the same input: the
// narrow k / v projections then run with q's tiles instead of a grid of their own that leaves
// compute units idle).  Block b belongs to linear l with begin[l] <= b < begin[l + 1]; every
// linear's grid starts at a multiple of 8, so its tiles keep their XCD assignment.
// top-2 routing: 128-token tiles, fast epilogue, both experts' corrections in it
__global__ __launch_bounds__(256, 2) void gemm_w4_top2_kernel(
    const int8_t* __restrict__ codes, const float* __restrict__ s_x, const uint8_t* __restrict__ w_tiled,
    const float* __restrict__ w_scale, int T, int d_in, int d_out, const uint16_t* __restrict__ u,
    const uint16_t* __restrict__ bt_s, int rs_pad, const uint16_t* __restrict__ v, const int32_t* __restrict__ expert,
    const uint16_t* __restrict__ bt_r, int rr_pad, int n_r, const int32_t* __restrict__ perm, float* __restrict__ y,
    int n_tm, const uint16_t* __restrict__ v2, const int32_t* __restrict__ expert2) {
    gemm_w4_tile<8, true, true>(codes, s_x, w_tiled, w_scale, T, d_in, d_out, u, bt_s, rs_pad, v, expert, bt_r, rr_pad,
                                n_r, perm, y, nullptr, n_tm, nullptr, false, blockIdx.x, gridDim.x, 0, 1, v2, expert2);
}

template <int MB>
__global__ __launch_bounds__(256, 2) void gemm_w4_group_kernel(GemmGroup G) {
    int l = 0;
#pragma unroll
    for (int i = 1; i < GG_MAX; ++i)
        if (i < G.n && (int)blockIdx.x >= G.begin[i]) l = i;
    const GemmLinear& a = G.lin[l];
    const int nblk = (l + 1 < G.n ? G.begin[l + 1] : (int)gridDim.x) - G.begin[l];
    gemm_w4_tile<MB, true>(a.codes, a.s_x, a.w_tiled, a.w_scale, G.T, a.d_in, a.d_out, a.u, a.bt_s, a.rs_pad, a.v,
                           a.expert, a.bt_r, a.rr_pad, a.n_r, a.perm, a.y, nullptr, (G.T + MB * 16 - 1) / (MB * 16),
                           nullptr, false, (int)blockIdx.x - G.begin[l], nblk, 0, 1);
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
                          float* y, int32_t* acc_debug, int ksplit, int32_t* part, bool y_bf16, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    const int n_tn = (d_out + G_BN - 1) / G_BN;
    // 128-token tiles unless that leaves the chip less than two workgroups per CU
    const bool small = (long)((T + 127) / 128) * n_tn < 512;
    const uint8_t* w = w_tiled;
    const bool split = ksplit > 1 && part != nullptr && acc_debug == nullptr && rs_pad <= 32 && rr_pad <= 32;
    if (split && !small) return hipErrorInvalidValue;
    // bf16 outputs take the general epilogue, which stores every output once from registers (the
    // fast one adds the routed terms of tiles with many experts onto the stored y)
    const bool fast = !acc_debug && !y_bf16 && rs_pad <= 32 && rr_pad <= 32;
    const int ks = split ? ksplit : 1;
    int32_t* pp = split ? part : nullptr;
#define QE_GEMM_LAUNCH(MBV, FAST, NTM)                                                                     \
    hipLaunchKernelGGL((gemm_w4_kernel<MBV, FAST>), dim3((NTM) * n_tn, ks), dim3(256), 0, st, codes, s_x, w, \
                       w_scale, T, d_in, d_out, u, bt_s, rs_pad, v, expert, bt_r, rr_pad, n_r, perm, y, acc_debug, NTM, pp, y_bf16)
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
                                    routed ? v : nullptr, routed ? expert : nullptr, n_r, bt_r, rr_pad, y, y_bf16, st);
}

// Top-2 routing in the main product's epilogue: for the launches that take 128-token tiles with
// the fast epilogue and no K split (float32 y, ranks <= 32); gemm_w4_top2_ok says which.
bool gemm_w4_top2_ok(int T, int d_out, int rs_pad, int rr_pad, int ksplit, bool y_bf16) {
    const int n_tn = (d_out + G_BN - 1) / G_BN;
    const bool small = (long)((T + 127) / 128) * n_tn < 512;
    return T > 0 && !small && ksplit <= 1 && !y_bf16 && rs_pad <= 32 && rr_pad > 0 && rr_pad <= 32;
}

hipError_t launch_gemm_w4_top2(const int8_t* codes, const float* s_x, const uint8_t* w_tiled, const float* w_scale,
                               int T, int d_in, int d_out, const uint16_t* u, const uint16_t* bt_s, int rs_pad,
                               const uint16_t* v, const int32_t* expert, const uint16_t* v2, const int32_t* expert2,
                               const uint16_t* bt_r, int rr_pad, int n_r, const int32_t* perm, float* y,
                               hipStream_t st) {
    if (T <= 0) return hipSuccess;
    if (!gemm_w4_top2_ok(T, d_out, rs_pad, rr_pad, 1, false) || !v || !expert || !v2 || !expert2 || !bt_r || n_r < 2 ||
        d_in % G_BK)
        return hipErrorInvalidValue;
    const int n_tn = (d_out + G_BN - 1) / G_BN, n_tm = (T + 127) / 128;
    hipLaunchKernelGGL(gemm_w4_top2_kernel, dim3(n_tm * n_tn), dim3(256), 0, st, codes, s_x, w_tiled, w_scale, T, d_in,
                       d_out, rs_pad > 0 ? u : nullptr, bt_s, rs_pad, v, expert, bt_r, rr_pad, n_r, perm, y, n_tm, v2,
                       expert2);
    return hipGetLastError();
}

// The grouped launch is for linears on the fast path without a K split: float32 y, ranks <= 32,
// no accumulator dump, every linear's tile grid a multiple of 8.  Returns hipErrorInvalidValue
// (nothing launched) otherwise, and the caller then launches the linears one by one.
hipError_t launch_gemm_w4_group(const GemmGroup& G0, hipStream_t st) {
    GemmGroup G = G0;
    if (G.n < 1 || G.n > GG_MAX || G.T <= 0) return hipErrorInvalidValue;
    // 128-token tiles unless the group's grid would leave the chip less than two workgroups per
    // CU, as for one linear (launch_gemm_w4); then 64-token tiles
    long tiles128 = 0;
    for (int l = 0; l < G.n; ++l) tiles128 += (long)((G.T + 127) / 128) * ((G.lin[l].d_out + G_BN - 1) / G_BN);
    const int bm = tiles128 < 512 ? 64 : 128;
    const int n_tm = (G.T + bm - 1) / bm;
    int begin = 0;
    for (int l = 0; l < G.n; ++l) {
        const GemmLinear& a = G.lin[l];
        if (a.rs_pad > 32 || a.rr_pad > 32 || a.d_out % 16 || a.d_in % G_BK) return hipErrorInvalidValue;
        const int tiles = n_tm * ((a.d_out + G_BN - 1) / G_BN);
        if (tiles % 8) return hipErrorInvalidValue;
        G.begin[l] = begin;
        begin += tiles;
    }
    if (bm == 128) hipLaunchKernelGGL(gemm_w4_group_kernel<8>, dim3(begin), dim3(256), 0, st, G);
    else hipLaunchKernelGGL(gemm_w4_group_kernel<4>, dim3(begin), dim3(256), 0, st, G);
    return hipGetLastError();
}

}  // namespace qe
