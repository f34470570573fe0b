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
//   * Weights are pre-tiled at load time so that every lane fetches its own
//     16-byte fragment with one coalesced dwordx4 load (1 KB per wave per
//     16 channels x 128 K); they go global -> VGPR without LDS.
//   * Activation codes (shared by the 4 waves) are staged in LDS, double
//     buffered, with an XOR swizzle of the 16-byte chunks against bank conflicts.
//   * Workgroup tile 128 tokens x 256 channels; wave tile 128 x 64
//     (8 x 4 MFMA blocks, 128 accumulator registers).
//   * Epilogue: int32 -> float, scale by s_x and s_w, then bf16 MFMA
//     16x16x32 steps accumulate u.B_s and, for every routed expert present in
//     the tile, (v masked to that expert's tokens).B_e on top of it.

#include "qe_internal.h"

namespace qe {

constexpr int G_BM = 128;
constexpr int G_BN = 256;
constexpr int G_BK = 128;
constexpr int G_MB = G_BM / 16;  // M blocks per wave
constexpr int G_NBW = 4;         // N blocks per wave

__device__ inline v4i unpack_w4x16(uint32_t p0, uint32_t p1) {
    // tiled byte b of p holds code b (low nibble) and code b+4 (high nibble)
    v4i r;
    r[0] = (int)((p0 << 4) & 0xF0F0F0F0u);
    r[1] = (int)(p0 & 0xF0F0F0F0u);
    r[2] = (int)((p1 << 4) & 0xF0F0F0F0u);
    r[3] = (int)(p1 & 0xF0F0F0F0u);
    return r;
}

__device__ inline int lds_a_offset(int row, int chunk) { return row * G_BK + ((chunk ^ (row & 7)) << 4); }

__global__ __launch_bounds__(256, 2) void gemm_w4_kernel(
    const int8_t* __restrict__ codes, const float* __restrict__ s_x, const v4u* __restrict__ w_tiled,
    const float* __restrict__ w_scale, int T, int d_in, int d_out, const uint16_t* __restrict__ u,
    const uint16_t* __restrict__ bt_s, int rs_pad, const uint16_t* __restrict__ v, const int32_t* __restrict__ expert,
    const uint16_t* __restrict__ bt_r, int rr_pad, int n_r, float* __restrict__ y, int32_t* __restrict__ acc_debug,
    int n_tm) {
    __shared__ __attribute__((aligned(16))) uint8_t As[2][G_BM * G_BK];

    const int tm = blockIdx.x % n_tm, tn = blockIdx.x / n_tm;
    const int m0 = tm * G_BM;
    const int NB = d_out >> 4, KB = d_in / G_BK;
    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
    const int nb0 = tn * (G_BN / 16) + wid * G_NBW;
    const int lr = lane & 15, lg = lane >> 4;

    // activation-code tile loads: 4 x 16 B per thread, 8 threads per 128-byte row
    const int a_c = tid & 7;
    const int8_t* a_ptr[4];
    int a_lds[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int r = (tid >> 3) + 32 * p;
        const int gr = min(m0 + r, T - 1);
        a_ptr[p] = codes + (size_t)gr * d_in + a_c * 16;
        a_lds[p] = lds_a_offset(r, a_c);
    }
    // weight fragment pointers (one per N block of this wave)
    const v4u* b_ptr[G_NBW];
    bool nb_ok[G_NBW];
#pragma unroll
    for (int j = 0; j < G_NBW; ++j) {
        nb_ok[j] = (nb0 + j) < NB;
        b_ptr[j] = w_tiled + ((size_t)(nb_ok[j] ? nb0 + j : 0) * KB) * 64 + lane;
    }

    v4i acc[G_MB][G_NBW];
#pragma unroll
    for (int m = 0; m < G_MB; ++m)
#pragma unroll
        for (int j = 0; j < G_NBW; ++j) acc[m][j] = v4i{0, 0, 0, 0};

    v4u a_reg[4], b_reg[G_NBW];
#pragma unroll
    for (int p = 0; p < 4; ++p) a_reg[p] = *reinterpret_cast<const v4u*>(a_ptr[p]);
#pragma unroll
    for (int j = 0; j < G_NBW; ++j) b_reg[j] = nb_ok[j] ? b_ptr[j][0] : v4u{0, 0, 0, 0};
#pragma unroll
    for (int p = 0; p < 4; ++p) *reinterpret_cast<v4u*>(&As[0][a_lds[p]]) = a_reg[p];
    __syncthreads();

    for (int kb = 0; kb < KB; ++kb) {
        const int cur = kb & 1;
        v4u b_cur[G_NBW];
#pragma unroll
        for (int j = 0; j < G_NBW; ++j) b_cur[j] = b_reg[j];
        const bool more = (kb + 1) < KB;
        if (more) {
#pragma unroll
            for (int p = 0; p < 4; ++p)
                a_reg[p] = *reinterpret_cast<const v4u*>(a_ptr[p] + (size_t)(kb + 1) * G_BK);
#pragma unroll
            for (int j = 0; j < G_NBW; ++j)
                b_reg[j] = nb_ok[j] ? b_ptr[j][(size_t)(kb + 1) * 64] : v4u{0, 0, 0, 0};
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            v4i bop[G_NBW];
#pragma unroll
            for (int j = 0; j < G_NBW; ++j) bop[j] = unpack_w4x16(b_cur[j][2 * s], b_cur[j][2 * s + 1]);
            v4i a[G_MB];  // all A fragments of this K step in flight at once
#pragma unroll
            for (int m = 0; m < G_MB; ++m)
                a[m] = *reinterpret_cast<const v4i*>(&As[cur][lds_a_offset(m * 16 + lr, s * 4 + lg)]);
#pragma unroll
            for (int m = 0; m < G_MB; ++m)
#pragma unroll
                for (int j = 0; j < G_NBW; ++j)
                    acc[m][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[m], bop[j], acc[m][j], 0, 0, 0);
            // keep the eight LDS reads ahead of the 32 MFMAs that consume them
            __builtin_amdgcn_sched_group_barrier(0x100, G_MB, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, G_MB * G_NBW, 0);
        }
        if (more) {
#pragma unroll
            for (int p = 0; p < 4; ++p) *reinterpret_cast<v4u*>(&As[cur ^ 1][a_lds[p]]) = a_reg[p];
        }
        __syncthreads();
    }

    // ------------------------------------------------------------ epilogue
    // lane holds column (nb*16 + lr) and rows (m*16 + lg*4 + r) of each block
    float sx[G_MB][4];
#pragma unroll
    for (int m = 0; m < G_MB; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) sx[m][r] = s_x[min(m0 + m * 16 + lg * 4 + r, T - 1)];
    float sw[G_NBW];
#pragma unroll
    for (int j = 0; j < G_NBW; ++j) sw[j] = nb_ok[j] ? w_scale[(nb0 + j) * 16 + lr] : 0.0f;

    if (acc_debug) {
#pragma unroll
        for (int m = 0; m < G_MB; ++m)
#pragma unroll
            for (int j = 0; j < G_NBW; ++j) {
                if (!nb_ok[j]) continue;
                const int col = (nb0 + j) * 16 + lr;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = m0 + m * 16 + lg * 4 + r;
                    if (row < T) acc_debug[(size_t)row * d_out + col] = acc[m][j][r] >> 4;
                }
            }
    }

    v4f yv[G_MB][G_NBW];
#pragma unroll
    for (int m = 0; m < G_MB; ++m)
#pragma unroll
        for (int j = 0; j < G_NBW; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) yv[m][j][r] = (float)(acc[m][j][r] >> 4) * sx[m][r] * sw[j];

    // shared expert: y += u . B_s
    if (u) {
        for (int k0 = 0; k0 < rs_pad; k0 += 32) {
            v8bf bs[G_NBW];
#pragma unroll
            for (int j = 0; j < G_NBW; ++j)
                bs[j] = nb_ok[j] ? *reinterpret_cast<const v8bf*>(bt_s + (size_t)((nb0 + j) * 16 + lr) * rs_pad + k0 + lg * 8)
                                 : v8bf{};
#pragma unroll
            for (int m = 0; m < G_MB; ++m) {
                const int row = min(m0 + m * 16 + lr, T - 1);
                const v8bf a = *reinterpret_cast<const v8bf*>(u + (size_t)row * rs_pad + k0 + lg * 8);
#pragma unroll
                for (int j = 0; j < G_NBW; ++j) yv[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bs[j], yv[m][j], 0, 0, 0);
            }
        }
    }

    // routed experts: for every expert present among the tile's tokens,
    // y += (v masked to that expert's rows) . B_e
    if (v && expert) {
        int ex[G_MB];
#pragma unroll
        for (int m = 0; m < G_MB; ++m) {
            const int row = m0 + m * 16 + lr;
            ex[m] = row < T ? expert[row] : -1;
        }
        const int e0 = (m0 + lane < T) ? expert[m0 + lane] : -1;
        const int e1 = (m0 + 64 + lane < T) ? expert[m0 + 64 + lane] : -1;
        for (int e = 0; e < n_r; ++e) {
            if (__ballot(e0 == e || e1 == e) == 0) continue;
            for (int k0 = 0; k0 < rr_pad; k0 += 32) {
                v8bf br[G_NBW];
#pragma unroll
                for (int j = 0; j < G_NBW; ++j)
                    br[j] = nb_ok[j] ? *reinterpret_cast<const v8bf*>(
                                           bt_r + ((size_t)e * d_out + (nb0 + j) * 16 + lr) * rr_pad + k0 + lg * 8)
                                     : v8bf{};
#pragma unroll
                for (int m = 0; m < G_MB; ++m) {
                    const int row = min(m0 + m * 16 + lr, T - 1);
                    v8bf a = *reinterpret_cast<const v8bf*>(v + (size_t)row * rr_pad + k0 + lg * 8);
                    if (ex[m] != e) a = v8bf{};
#pragma unroll
                    for (int j = 0; j < G_NBW; ++j)
                        yv[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, br[j], yv[m][j], 0, 0, 0);
                }
            }
        }
    }

#pragma unroll
    for (int m = 0; m < G_MB; ++m)
#pragma unroll
        for (int j = 0; j < G_NBW; ++j) {
            if (!nb_ok[j]) continue;
            const int col = (nb0 + j) * 16 + lr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + m * 16 + lg * 4 + r;
                if (row < T) y[(size_t)row * d_out + col] = yv[m][j][r];
            }
        }
}

hipError_t launch_gemm_w4(const int8_t* codes, const float* s_x, const uint8_t* w_tiled, const float* w_scale, int T,
                          int d_in, int d_out, const uint16_t* u, const uint16_t* bt_s, int rs_pad, const uint16_t* v,
                          const int32_t* expert, const uint16_t* bt_r, int rr_pad, int n_r, float* y,
                          int32_t* acc_debug, hipStream_t st) {
    if (T <= 0) return hipSuccess;
    const int n_tm = (T + G_BM - 1) / G_BM;
    const int n_tn = (d_out + G_BN - 1) / G_BN;
    hipLaunchKernelGGL(gemm_w4_kernel, dim3(n_tm * n_tn), dim3(256), 0, st, codes, s_x,
                       reinterpret_cast<const v4u*>(w_tiled), w_scale, T, d_in, d_out, u, bt_s, rs_pad, v, expert,
                       bt_r, rr_pad, n_r, y, acc_debug, n_tm);
    return hipGetLastError();
}

}  // namespace qe
