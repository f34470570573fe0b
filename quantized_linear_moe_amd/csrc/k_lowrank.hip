// Expert construction: the low-rank factors of the shared and routed experts.
//
// MCISLAB DeepRead summary of "Quant Experts", section "Method" (Shared Expert, Routed
// Experts): the layer's quantization error E = W_f - W_q is reconstructed by a low-rank shared
// expert, and the error left after it by one low-rank routed expert per cluster of
// token-dependent channels.  PaperDaily post "西交大提出Quant Experts：token级量化补偿",
// section "核心设计": the decomposition is a whitening SVD, which balances the scales of the
// directions before the SVD.  Here the whitening is diagonal (input channel j weighted by the
// RMS c_j of its calibration activations), and the truncated SVD of M = diag(w) E^T is the
// randomized subspace iteration of Halko, Martinsson and Tropp, "Finding structure with
// randomness" (SIAM Review 2011), Algorithms 4.4 and 5.1, with the Gaussian test matrix an
// input:
//   Y = M omega, Q = qr(Y); power_iters times: Q~ = qr(M^T Q), Q = qr(M Q~);
//   Z = M^T Q (= B^T with B = Q^T M);  B B^T = Z^T Z = U~ S^2 U~^T;  U = Q U~, V = Z U~ S^-1;
//   A = diag(1/w) U_r S_r^(1/2) (rows with w = 0 are zero), B = S_r^(1/2) V_r^T.
//
// Everything that touches a d-long dimension runs on the GPU: the thin products M X and M^T X
// with X of k <= 128 columns over E (d_out x d_in float32, up to ~1 GB for the largest
// linears; float32 FMAs, LDS tiles, contraction split over workgroups with atomic adds), the
// k x k Gram matrices X^T X (float64 sums) and the products X S with k x k matrices S.  The
// host only solves k x k symmetric eigenproblems in double.  Orthonormalization is by the Gram
// matrix (the scheme of CholeskyQR2, Fukaya et al. 2014, with the eigenvalue decomposition in
// place of the Cholesky factor): X = Y V diag(lambda)^(-1/2), directions whose eigenvalue is
// below 1e-11 of the largest dropped as null (they give zero columns), then, when the kept
// eigenvalues span more than 1e4, the same on X, which restores orthogonality to working
// precision.

#include <algorithm>
#include <cmath>
#include <vector>

#include "qe_calib.h"
#include "qe_internal.h"
#include "qe_lowrank.h"

namespace qe {

namespace {

// ---------------------------------------------------------------- quantization error
// One workgroup per output channel: the row maximum of |W_f * s|, s_w = max / qmax, then
// the codes exactly as the weight quantizer takes them (float32, ties to even, clamp) and
// E = W_f - s_w * code / s.
__global__ __launch_bounds__(256) void quant_error_kernel(const float* __restrict__ W, const float* __restrict__ s,
                                                          int d_in, float qmax, float* __restrict__ E) {
    __shared__ float red[256];
    const float* row = W + (size_t)blockIdx.x * d_in;
    float* out = E + (size_t)blockIdx.x * d_in;
    const int tid = threadIdx.x;
    float amax = 0.0f;
    for (int j = tid; j < d_in; j += 256) amax = fmaxf(amax, fabsf(s ? row[j] * s[j] : row[j]));
    red[tid] = amax;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if (tid < h) red[tid] = fmaxf(red[tid], red[tid + h]);
        __syncthreads();
    }
    amax = red[0];
    const float sw = amax / qmax;
    for (int j = tid; j < d_in; j += 256) {
        const float v = s ? row[j] * s[j] : row[j];
        const float c = amax > 0.0f ? fminf(fmaxf(rintf(v / sw), -qmax), qmax) : 0.0f;
        float wq = sw * c;
        if (s) wq = wq / s[j];
        out[j] = row[j] - wq;
    }
}

// --------------------------------------------------------------------- channel RMS
constexpr int RMS_TOK = 256;  // tokens per partial sum

__global__ __launch_bounds__(256) void channel_sumsq_kernel(const void* __restrict__ x, int x_dtype, int T, int d_in,
                                                            double* __restrict__ part) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= d_in) return;
    const int t0 = blockIdx.y * RMS_TOK, t1 = min(T, t0 + RMS_TOK);
    double acc = 0.0;
    if (x_dtype == QE_BF16) {
        const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
        for (int t = t0; t < t1; ++t) {
            const float v = __uint_as_float((uint32_t)xb[(size_t)t * d_in + j] << 16);
            acc += (double)v * (double)v;
        }
    } else {
        const float* xf = reinterpret_cast<const float*>(x);
        for (int t = t0; t < t1; ++t) {
            const float v = xf[(size_t)t * d_in + j];
            acc += (double)v * (double)v;
        }
    }
    part[(size_t)blockIdx.y * d_in + j] = acc;
}

__global__ __launch_bounds__(256) void channel_rms_finish_kernel(const double* __restrict__ part, int nb, int T,
                                                                 int d_in, float* __restrict__ c) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= d_in) return;
    double sum = 0.0;
    for (int y = 0; y < nb; ++y) sum += part[(size_t)y * d_in + j];
    c[j] = (float)sqrt(sum / T);
}

// ------------------------------------------------------------------ thin products
constexpr int TH_A = 64;  // output rows per workgroup
constexpr int TH_B = 32;  // contraction chunk

// TRANS == false: C[a][l] += sum_b E[a][b] w[b] S[b][l]   (a < d_out, b < d_in): Z = M^T S
// TRANS == true : C[a][l] += w[a] sum_b E[b][a] S[b][l]   (a < d_in, b < d_out): Y = M S
// S [n_b][k], C [n_a][k] row-major float32, k <= KP; C is zeroed by the caller.  Each thread
// owns 4 rows x KP/16 columns; the contraction range of blockIdx.y is [y bpb, (y+1) bpb).
template <int KP, bool TRANS>
__global__ __launch_bounds__(256) void thin_kernel(const float* __restrict__ E, int d_out, int d_in,
                                                   const float* __restrict__ S, int k, const float* __restrict__ w,
                                                   int bpb, float* __restrict__ C) {
    __shared__ float Et[TH_B][TH_A + 4];  // [b][a]
    __shared__ float St[TH_B][KP];
    constexpr int LU = KP / 16;
    const int n_a = TRANS ? d_in : d_out, n_b = TRANS ? d_out : d_in;
    const int a0 = blockIdx.x * TH_A;
    const int b_beg = blockIdx.y * bpb, b_end = min(n_b, b_beg + bpb);
    const int tid = threadIdx.x, ag = tid >> 4, lg = tid & 15;
    float acc[4][LU];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int u = 0; u < LU; ++u) acc[r][u] = 0.0f;

    for (int b0 = b_beg; b0 < b_end; b0 += TH_B) {
        if constexpr (!TRANS) {  // rows a of E, 8 contiguous b per thread
            const int ar = tid >> 2, bs = (tid & 3) * 8, a = a0 + ar;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int b = b0 + bs + q;
                Et[bs + q][ar] = (a < n_a && b < b_end) ? E[(size_t)a * d_in + b] : 0.0f;
            }
        } else {  // rows b of E, 8 contiguous a per thread
            const int br = tid >> 3, as = (tid & 7) * 8, b = b0 + br;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int a = a0 + as + q;
                Et[br][as + q] = (b < b_end && a < n_a) ? E[(size_t)b * d_in + a] : 0.0f;
            }
        }
        for (int e = tid; e < TH_B * KP; e += 256) {
            const int br = e / KP, l = e % KP, b = b0 + br;
            float v = (b < b_end && l < k) ? S[(size_t)b * k + l] : 0.0f;
            if (!TRANS && w != nullptr && b < b_end) v *= w[b];
            St[br][l] = v;
        }
        __syncthreads();
#pragma unroll 4
        for (int bi = 0; bi < TH_B; ++bi) {
            float ea[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) ea[r] = Et[bi][ag * 4 + r];
#pragma unroll
            for (int u = 0; u < LU; ++u) {
                const float sv = St[bi][lg + 16 * u];
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r][u] += ea[r] * sv;
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int a = a0 + ag * 4 + r;
        if (a >= n_a) continue;
        const float wa = (TRANS && w != nullptr) ? w[a] : 1.0f;
#pragma unroll
        for (int u = 0; u < LU; ++u) {
            const int l = lg + 16 * u;
            if (l < k) atomicAdd(&C[(size_t)a * k + l], acc[r][u] * wa);
        }
    }
}

// ------------------------------------------------------- passes over E (matrix cores)
// The two products that read the whole of E, on v_mfma_f32_16x16x4_f32 (float32 in, float32
// sums): lane (i = lane % 16, g = lane / 16) supplies A[i][g] and B[g][i], and holds
// D[4g + r][i].  Each workgroup (4 waves) reads a contiguous slice of E once; the k-column
// operand is staged in LDS (rows padded against bank conflicts) and shared by the waves.  The
// contraction is split over gridDim.y into long ranges, so few partial sums meet in the
// atomic adds.  NL: 16-column blocks of the k columns (k <= 16 NL).
typedef float v4f_t __attribute__((ext_vector_type(4)));
typedef float v2f_t __attribute__((ext_vector_type(2)));
constexpr int PX_ROWS = 64;  // E rows per stage of the M X pass
constexpr int PT_COLS = 64;  // E columns per stage of the M^T X pass

// Y[a][l] += w[a] sum_b E[b][a] X[b][l]: a over d_in (a wave owns 32 consecutive a, two
// 16-blocks, as float2 per lane: a = a0 + 2 i + j for block j), b over the E rows of the split.
// The next stage's E values and X rows are loaded into registers while the current stage's
// MFMAs run; X goes through two LDS buffers (one barrier per stage).
template <int NL, bool VEC>
__global__ __launch_bounds__(256) void pass_mx_kernel(const float* __restrict__ E, int d_out, int d_in,
                                                      const float* __restrict__ X, int k, const float* __restrict__ w,
                                                      int bpb, float* __restrict__ Y) {
    constexpr int LD = NL * 16 + 4;
    constexpr int NS = PX_ROWS / 4;                        // MFMA K steps per stage
    constexpr int XR = (PX_ROWS * NL * 16 + 255) / 256;    // X values per thread and stage
    __shared__ float Xs[2][PX_ROWS][LD];
    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, li = lane & 15, lg = lane >> 4;
    const int a0 = (blockIdx.x * 4 + wid) * 32;
    const int b_beg = blockIdx.y * bpb, b_end = min(d_out, b_beg + bpb);
    const int a = a0 + 2 * li;
    v4f_t acc[2][NL];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int lb = 0; lb < NL; ++lb) acc[j][lb] = v4f_t{0, 0, 0, 0};
    // Every load is unconditional at a clamped address and nothing uses its value before the
    // next stage, so the loads of a stage are all in flight together.  Clamped E rows (b past the
    // range) meet X rows that are zeroed in LDS, and clamped E columns (a past d_in) feed output
    // rows that are never stored, so E needs no masking; X is masked when it is written to LDS.
    const int a_lo = min(a, d_in - 1), a_hi = min(a + 1, d_in - 1);
    const int a_v = min(a, d_in - 2);  // VEC (d_in even): an aligned pair inside the row
    auto load = [&](int b0, v2f_t (&ev)[NS], float (&xr)[XR]) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const float* row = E + (size_t)min(b0 + 4 * s + lg, b_end - 1) * d_in;
            if constexpr (VEC) {
                ev[s] = *reinterpret_cast<const v2f_t*>(row + a_v);
            } else {
                ev[s][0] = row[a_lo];
                ev[s][1] = row[a_hi];
            }
        }
#pragma unroll
        for (int u = 0; u < XR; ++u) {
            const int e = tid + 256 * u, br = e / (NL * 16), l = e % (NL * 16);
            xr[u] = X[(size_t)min(b0 + br, b_end - 1) * k + min(l, k - 1)];
        }
    };
    v2f_t ev[NS], en[NS];
    float xr[XR], xn[XR];
    load(b_beg, en, xn);
    int buf = 0;
    for (int b0 = b_beg; b0 < b_end; b0 += PX_ROWS) {
#pragma unroll
        for (int s = 0; s < NS; ++s) ev[s] = en[s];
#pragma unroll
        for (int u = 0; u < XR; ++u) xr[u] = xn[u];
#pragma unroll
        for (int u = 0; u < XR; ++u) {
            const int e = tid + 256 * u, br = e / (NL * 16), l = e % (NL * 16);
            if (e < PX_ROWS * NL * 16) Xs[buf][br][l] = (b0 + br < b_end && l < k) ? xr[u] : 0.0f;
        }
        __syncthreads();  // also orders this buffer's previous reads (two stages ago) before the writes above
        if (b0 + PX_ROWS < b_end) load(b0 + PX_ROWS, en, xn);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
#pragma unroll
            for (int lb = 0; lb < NL; ++lb) {
                const float bv = Xs[buf][4 * s + lg][16 * lb + li];
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[j][lb] = __builtin_amdgcn_mfma_f32_16x16x4f32(ev[s][j], bv, acc[j][lb], 0, 0, 0);
            }
        }
        buf ^= 1;
    }
    // block j, row 4 lg + r <-> a = a0 + 2 (4 lg + r) + j; column 16 lb + li
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ao = a0 + 2 * (4 * lg + r) + j;
            if (ao >= d_in) continue;
            const float wa = w ? w[ao] : 1.0f;
#pragma unroll
            for (int lb = 0; lb < NL; ++lb) {
                const int l = 16 * lb + li;
                if (l < k) atomicAdd(&Y[(size_t)ao * k + l], acc[j][lb][r] * wa);
            }
        }
}

// Z[a][l] += sum_b E[a][b] w[b] Q[b][l]: a over d_out (a wave owns 32 rows, two 16-blocks),
// b over the E columns of the split, 16 per MFMA group: lane (i, g) loads E[row][b0 + 4 g ..
// + 3] as float4 and MFMA q of the group takes component q (K slot g <-> b = b0 + 4 g + q).
// Pipelined like pass_mx_kernel.
template <int NL, bool VEC>
__global__ __launch_bounds__(256) void pass_mtx_kernel(const float* __restrict__ E, int d_out, int d_in,
                                                       const float* __restrict__ Q, int k, const float* __restrict__ w,
                                                       int bpb, float* __restrict__ Z) {
    constexpr int LD = NL * 16 + 4;
    constexpr int NC = PT_COLS / 16;                        // MFMA groups per stage
    constexpr int QR = (PT_COLS * NL * 16 + 255) / 256;     // Q values per thread and stage
    __shared__ float Qs[2][PT_COLS][LD];
    const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, li = lane & 15, lg = lane >> 4;
    const int a0 = (blockIdx.x * 4 + wid) * 32;
    const int b_beg = blockIdx.y * bpb, b_end = min(d_in, b_beg + bpb);
    v4f_t acc[2][NL];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int lb = 0; lb < NL; ++lb) acc[j][lb] = v4f_t{0, 0, 0, 0};
    const float* rows[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) rows[j] = E + (size_t)min(a0 + 16 * j + li, d_out - 1) * d_in;
    // unconditional loads at clamped addresses whose values are used only at the next stage
    // (see pass_mx_kernel): clamped columns meet Q rows zeroed in LDS, clamped rows feed output
    // rows never stored; Q is masked and scaled by w when it is written to LDS.  The vector form
    // needs d_in % 4 == 0, so a clamped column stays aligned.
    auto load = [&](int b0, v4f_t (&ev)[NC][2], float (&qr)[QR], float (&wr)[QR]) {
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int b = b0 + 16 * c + 4 * lg;
                if constexpr (VEC) {
                    ev[c][j] = *reinterpret_cast<const v4f_t*>(rows[j] + min(b, d_in - 4));
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) ev[c][j][q] = rows[j][min(b + q, d_in - 1)];
                }
            }
#pragma unroll
        for (int u = 0; u < QR; ++u) {
            const int e = tid + 256 * u, br = e / (NL * 16), l = e % (NL * 16);
            const int bc = min(b0 + br, b_end - 1);
            qr[u] = Q[(size_t)bc * k + min(l, k - 1)];
            wr[u] = w != nullptr ? w[bc] : 1.0f;
        }
    };
    v4f_t ev[NC][2], en[NC][2];
    float qr[QR], qn[QR], wr[QR], wn[QR];
    load(b_beg, en, qn, wn);
    int buf = 0;
    for (int b0 = b_beg; b0 < b_end; b0 += PT_COLS) {
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int j = 0; j < 2; ++j) ev[c][j] = en[c][j];
#pragma unroll
        for (int u = 0; u < QR; ++u) {
            qr[u] = qn[u];
            wr[u] = wn[u];
        }
#pragma unroll
        for (int u = 0; u < QR; ++u) {
            const int e = tid + 256 * u, br = e / (NL * 16), l = e % (NL * 16);
            if (e < PT_COLS * NL * 16) Qs[buf][br][l] = (b0 + br < b_end && l < k) ? qr[u] * wr[u] : 0.0f;
        }
        __syncthreads();  // also orders this buffer's previous reads (two stages ago) before the writes above
        if (b0 + PT_COLS < b_end) load(b0 + PT_COLS, en, qn, wn);
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int lb = 0; lb < NL; ++lb) {
                    const float bv = Qs[buf][16 * c + 4 * lg + q][16 * lb + li];
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[j][lb] = __builtin_amdgcn_mfma_f32_16x16x4f32(ev[c][j][q], bv, acc[j][lb], 0, 0, 0);
                }
        buf ^= 1;
    }
    // block j, row 4 lg + r <-> a = a0 + 16 j + 4 lg + r; column 16 lb + li
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ao = a0 + 16 * j + 4 * lg + r;
            if (ao >= d_out) continue;
#pragma unroll
            for (int lb = 0; lb < NL; ++lb) {
                const int l = 16 * lb + li;
                if (l < k) atomicAdd(&Z[(size_t)ao * k + l], acc[j][lb][r]);
            }
        }
}

__global__ __launch_bounds__(256) void zero_kernel(float* __restrict__ p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0.0f;
}

// ------------------------------------------------------------- rank-r subtraction
// E[i][j] -= sum_l A[j][l] B[l][i]: 64 x 64 tiles of E, A and B slices in LDS, 4 x 4 per thread.
__global__ __launch_bounds__(256) void sub_lowrank_kernel(float* __restrict__ E, int d_out, int d_in,
                                                          const float* __restrict__ A, const float* __restrict__ B,
                                                          int r) {
    __shared__ float At[64][65];  // [j][l]
    __shared__ float Bt[64][65];  // [l][i]
    const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64, tid = threadIdx.x;
    for (int e = tid; e < 64 * 64; e += 256) {
        const int jj = e >> 6, l = e & 63;
        At[jj][l] = (j0 + jj < d_in && l < r) ? A[(size_t)(j0 + jj) * r + l] : 0.0f;
        const int l2 = e >> 6, ii = e & 63;
        Bt[l2][ii] = (l2 < r && i0 + ii < d_out) ? B[(size_t)l2 * d_out + i0 + ii] : 0.0f;
    }
    __syncthreads();
    const int ty = tid >> 4, tx = tid & 15;
    float acc[4][4] = {};
    for (int l = 0; l < r; ++l) {
        float bi[4], aj[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            bi[q] = Bt[l][ty * 4 + q];
            aj[q] = At[tx * 4 + q][l];
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[a][b] += aj[b] * bi[a];
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int i = i0 + ty * 4 + a;
        if (i >= d_out) continue;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int j = j0 + tx * 4 + b;
            if (j < d_in) E[(size_t)i * d_in + j] -= acc[a][b];
        }
    }
}

// C = thin product (see thin_kernel), zeroing C first
hipError_t thin(bool trans, const float* E, int d_out, int d_in, const float* S, int k, const float* w, float* C,
                hipStream_t st) {
    const int n_a = trans ? d_in : d_out, n_b = trans ? d_out : d_in;
    const size_t nc = (size_t)n_a * k;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)std::min<size_t>((nc + 255) / 256, 4096)), dim3(256), 0, st, C, nc);
    const int tiles = (n_a + TH_A - 1) / TH_A;
    const int chunks = (n_b + TH_B - 1) / TH_B;
    // about 2048 workgroups, at least 8 contraction chunks each
    const int splits = std::max(1, std::min((2048 + tiles - 1) / tiles, chunks / 8));
    const int bpb = (chunks + splits - 1) / splits * TH_B;
    const int ny = (n_b + bpb - 1) / bpb;
    const dim3 grid(tiles, ny);
#define QE_THIN(KPV)                                                                                                \
    do {                                                                                                            \
        if (trans) hipLaunchKernelGGL((thin_kernel<KPV, true>), grid, dim3(256), 0, st, E, d_out, d_in, S, k, w, bpb, C); \
        else hipLaunchKernelGGL((thin_kernel<KPV, false>), grid, dim3(256), 0, st, E, d_out, d_in, S, k, w, bpb, C); \
    } while (0)
    if (k <= 32) QE_THIN(32);
    else if (k <= 64) QE_THIN(64);
    else QE_THIN(128);
#undef QE_THIN
    return hipGetLastError();
}

// One pass over E on the matrix cores: trans ? (C = diag(w) E^T S, [d_in][k]) : (C = E diag(w) S,
// [d_out][k]); C zeroed first.  About 512 workgroups, each with a long contraction range.
hipError_t pass_over_e(bool trans, const float* E, int d_out, int d_in, const float* S, int k, const float* w, float* C,
                       hipStream_t st) {
    const int n_a = trans ? d_in : d_out, n_b = trans ? d_out : d_in;
    const size_t nc = (size_t)n_a * k;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)std::min<size_t>((nc + 255) / 256, 4096)), dim3(256), 0, st, C, nc);
    const int step = trans ? PX_ROWS : PT_COLS;
    const int tiles = (n_a + 127) / 128;
    const int steps = (n_b + step - 1) / step;
    const int splits = std::max(1, std::min((512 + tiles - 1) / tiles, steps / 4));
    const int bpb = (steps + splits - 1) / splits * step;
    const dim3 grid(tiles, (n_b + bpb - 1) / bpb);
    const int nl = (k + 15) / 16;
#define QE_PASS(NLV)                                                                                          \
    do {                                                                                                      \
        if (trans) {                                                                                          \
            if (d_in % 2 == 0)                                                                                \
                hipLaunchKernelGGL((pass_mx_kernel<NLV, true>), grid, dim3(256), 0, st, E, d_out, d_in, S, k, w, bpb, C); \
            else                                                                                              \
                hipLaunchKernelGGL((pass_mx_kernel<NLV, false>), grid, dim3(256), 0, st, E, d_out, d_in, S, k, w, bpb, C); \
        } else if (d_in % 4 == 0) {                                                                           \
            hipLaunchKernelGGL((pass_mtx_kernel<NLV, true>), grid, dim3(256), 0, st, E, d_out, d_in, S, k, w, bpb, C); \
        } else {                                                                                              \
            hipLaunchKernelGGL((pass_mtx_kernel<NLV, false>), grid, dim3(256), 0, st, E, d_out, d_in, S, k, w, bpb, C); \
        }                                                                                                     \
    } while (0)
    switch (nl) {
        case 1: QE_PASS(1); break;
        case 2: QE_PASS(2); break;
        case 3: QE_PASS(3); break;
        case 4: QE_PASS(4); break;
        case 5: QE_PASS(5); break;
        case 6: QE_PASS(6); break;
        case 7: QE_PASS(7); break;
        default: QE_PASS(8); break;
    }
#undef QE_PASS
    return hipGetLastError();
}

// ------------------------------------------------------------------ router fit
constexpr int RT_TOK = 128;  // calibration tokens per chunk of the target computation

// XT[j][t] = x[t0 + t][j] as float32, t < kc (32 x 32 tiles through LDS)
__global__ __launch_bounds__(256) void transpose_chunk_kernel(const void* __restrict__ x, int x_dtype, int t0, int kc,
                                                              int d_in, float* __restrict__ XT) {
    __shared__ float tile[32][33];
    const int j0 = blockIdx.x * 32, tt0 = blockIdx.y * 32, tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    for (int r = ty; r < 32; r += 8) {
        const int t = tt0 + r, j = j0 + tx;
        float v = 0.0f;
        if (t < kc && j < d_in) {
            const size_t idx = (size_t)(t0 + t) * d_in + j;
            v = x_dtype == QE_BF16 ? __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(x)[idx] << 16)
                                   : reinterpret_cast<const float*>(x)[idx];
        }
        tile[r][tx] = v;
    }
    __syncthreads();
    for (int r = ty; r < 32; r += 8) {
        const int j = j0 + r, t = tt0 + tx;
        if (j < d_in && t < kc) XT[(size_t)j * kc + t] = tile[tx][r];
    }
}

__global__ __launch_bounds__(256) void to_f32_kernel(const void* __restrict__ x, int x_dtype, size_t n,
                                                     float* __restrict__ out) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
        out[i] = x_dtype == QE_BF16 ? __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(x)[i] << 16)
                                    : reinterpret_cast<const float*>(x)[i];
}

// target[t0 + t][g] = mean_i |Z[i][t] - sum_l B_g[l][i] U_g[t][l]|   (one workgroup per (t, g))
__global__ __launch_bounds__(256) void router_target_kernel(const float* __restrict__ Z, int kc, int d_out,
                                                            const float* __restrict__ B_r, int r_r,
                                                            const float* __restrict__ U, int t0, int n_r,
                                                            float* __restrict__ target) {
    __shared__ float u[64];
    __shared__ double red[256];
    const int t = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
    if (tid < r_r) u[tid] = U[((size_t)g * kc + t) * r_r + tid];
    __syncthreads();
    const float* Bg = B_r + (size_t)g * r_r * d_out;
    double acc = 0.0;
    for (int i = tid; i < d_out; i += 256) {
        float v = Z[(size_t)i * kc + t];
        for (int l = 0; l < r_r; ++l) v -= Bg[(size_t)l * d_out + i] * u[l];
        acc += fabs((double)v);
    }
    red[tid] = acc;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if (tid < h) red[tid] += red[tid + h];
        __syncthreads();
    }
    if (tid == 0) target[(size_t)(t0 + t) * n_r + g] = (float)(red[0] / d_out);
}

// out[g] = sum_j a[j][g] b[j][g] (float64), one workgroup per column g of [d][n] matrices
__global__ __launch_bounds__(256) void coldot_kernel(const float* __restrict__ a, const float* __restrict__ b, int d,
                                                     int n, double* __restrict__ out) {
    __shared__ double red[256];
    const int g = blockIdx.x, tid = threadIdx.x;
    double acc = 0.0;
    for (int j = tid; j < d; j += 256) acc += (double)a[(size_t)j * n + g] * (double)b[(size_t)j * n + g];
    red[tid] = acc;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if (tid < h) red[tid] += red[tid + h];
        __syncthreads();
    }
    if (tid == 0) out[g] = red[0];
}

// sum of squares of n floats (float64), accumulated into *out (zeroed by the caller)
__global__ __launch_bounds__(256) void sumsq_kernel(const float* __restrict__ a, size_t n, double* __restrict__ out) {
    __shared__ double red[256];
    double acc = 0.0;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
        acc += (double)a[i] * (double)a[i];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if (threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0) atomicAdd(out, red[0]);
}

// conjugate-gradient updates on [d][n] matrices with per-column scalars (float64 on the device):
//   mode 0: q += lam p;  mode 1: R += alpha p, r -= alpha q;  mode 2: p = r + beta p
__global__ __launch_bounds__(256) void cg_update_kernel(int mode, int d, int n, double lam,
                                                        const double* __restrict__ coef, float* __restrict__ R,
                                                        float* __restrict__ r, float* __restrict__ p,
                                                        float* __restrict__ q) {
    const size_t total = (size_t)d * n;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (size_t)gridDim.x * 256) {
        const int g = (int)(i % n);
        if (mode == 0) {
            q[i] = (float)((double)q[i] + lam * p[i]);
        } else if (mode == 1) {
            R[i] = (float)((double)R[i] + coef[g] * p[i]);
            r[i] = (float)((double)r[i] - coef[g] * q[i]);
        } else {
            p[i] = (float)((double)r[i] + coef[g] * p[i]);
        }
    }
}

// ------------------------------------------------------------------ Gram matrices
// G[a][l] += sum_r Y[r][a] Y[r][l] over the rows of blockIdx.x (Y float32 [m][k], G double
// [k][k], zeroed by the caller); float64 products and sums.
template <int KP>
__global__ __launch_bounds__(256) void gram_kernel(const float* __restrict__ Y, int m, int k, int rpb,
                                                   double* __restrict__ G) {
    __shared__ float Ys[32][KP];
    constexpr int NP = KP * KP / 256;
    const int tid = threadIdx.x;
    const int r_beg = blockIdx.x * rpb, r_end = min(m, r_beg + rpb);
    double acc[NP];
#pragma unroll
    for (int u = 0; u < NP; ++u) acc[u] = 0.0;
    for (int r0 = r_beg; r0 < r_end; r0 += 32) {
        for (int e = tid; e < 32 * KP; e += 256) {
            const int br = e / KP, l = e % KP, r = r0 + br;
            Ys[br][l] = (r < r_end && l < k) ? Y[(size_t)r * k + l] : 0.0f;
        }
        __syncthreads();
        for (int br = 0; br < 32; ++br) {
#pragma unroll
            for (int u = 0; u < NP; ++u) {
                const int p = tid + 256 * u;
                acc[u] += (double)Ys[br][p / KP] * (double)Ys[br][p % KP];
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < NP; ++u) {
        const int p = tid + 256 * u, a = p / KP, l = p % KP;
        if (a < k && l < k) atomicAdd(&G[(size_t)a * k + l], acc[u]);
    }
}

hipError_t gram(const float* Y, int m, int k, double* G, hipStream_t st) {
    hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(256), 0, st, reinterpret_cast<float*>(G), (size_t)2 * k * k);
    const int blocks = std::max(1, std::min(256, (m + 31) / 32));
    const int rpb = ((m + blocks - 1) / blocks + 31) / 32 * 32;
    const int nb = (m + rpb - 1) / rpb;
    if (k <= 32) hipLaunchKernelGGL(gram_kernel<32>, dim3(nb), dim3(256), 0, st, Y, m, k, rpb, G);
    else if (k <= 64) hipLaunchKernelGGL(gram_kernel<64>, dim3(nb), dim3(256), 0, st, Y, m, k, rpb, G);
    else hipLaunchKernelGGL(gram_kernel<128>, dim3(nb), dim3(256), 0, st, Y, m, k, rpb, G);
    return hipGetLastError();
}

// Host: eigen-decomposition of the symmetric k x k matrix G (double, from the device) into
// ascending eigenvalues lam and eigenvector columns V (row-major [k][k]).  Returns false when
// the iteration does not converge.
bool host_eigen(const std::vector<double>& Gh, int k, std::vector<double>& lam, std::vector<double>& V) {
    std::vector<double> A(Gh);
    for (int a = 0; a < k; ++a)  // symmetrize the float64 sums (their order differs per entry)
        for (int b = a + 1; b < k; ++b) A[(size_t)a * k + b] = A[(size_t)b * k + a] = 0.5 * (A[(size_t)a * k + b] + A[(size_t)b * k + a]);
    lam.resize(k);
    V.resize((size_t)k * k);
    return symmetric_eigen(A.data(), k, lam.data(), V.data()) == 0;
}

// The k x k side of a randomized fit: Gram matrices of device [m][k] matrices (double sums on
// the GPU, eigen-decomposition on the host), products with host k x k matrices, and the
// orthonormalization by the Gram matrix.  Device scratch: G (k x k double), S (k x k float)
// and T ([m_max][k] float) for the first pass of a two-pass orthonormalization.
struct SmallOps {
    int k;
    hipStream_t st;
    double* Gd;
    float* Sd;
    float* Td;
    std::vector<double> Gh, lam, V;
    std::vector<float> Sh;
    SmallOps(int k_, hipStream_t st_, double* G, float* S, float* T)
        : k(k_), st(st_), Gd(G), Sd(S), Td(T), Gh((size_t)k_ * k_), Sh((size_t)k_ * k_) {}
    // eigen-decomposition (ascending) of X^T X for a device [m][k] matrix X
    hipError_t gram_eigen(const float* X, int m) {
        hipError_t r;
        if ((r = gram(X, m, k, Gd, st)) != hipSuccess) return r;
        if ((r = hipMemcpyAsync(Gh.data(), Gd, (size_t)k * k * 8, hipMemcpyDeviceToHost, st)) != hipSuccess) return r;
        if ((r = hipStreamSynchronize(st)) != hipSuccess) return r;
        return host_eigen(Gh, k, lam, V) ? hipSuccess : hipErrorNotSupported;
    }
    // dst = src Sh ([m][k] times the host [k][cols] matrix Sh; dst may not alias src)
    hipError_t apply(const float* src, int m, int cols, float* dst) {
        hipError_t r;
        if ((r = hipMemcpyAsync(Sd, Sh.data(), (size_t)k * cols * 4, hipMemcpyHostToDevice, st)) != hipSuccess) return r;
        if ((r = thin(false, src, m, k, Sd, cols, nullptr, dst, st)) != hipSuccess) return r;
        return hipStreamSynchronize(st);  // Sh is refilled by the next step
    }
    // orthonormal basis of the columns of src [m][k], written to dst (may alias src).  The
    // second pass is needed only when the kept eigenvalues span more than 1e4 (a condition
    // number above 100, where float32 rounding of the first product leaves columns measurably
    // non-orthogonal); otherwise the first product goes straight to dst.
    hipError_t orth(const float* src, int m, float* dst) {
        hipError_t r;
        const float* in = src;
        for (int pass = 0; pass < 2; ++pass) {
            if ((r = gram_eigen(in, m)) != hipSuccess) return r;
            const double top = std::max(lam[k - 1], 0.0);
            double low = top;
            for (int i = 0; i < k; ++i)
                if (lam[i] > 1e-11 * top) low = std::min(low, lam[i]);
            for (int a = 0; a < k; ++a)
                for (int i = 0; i < k; ++i)
                    Sh[(size_t)a * k + i] = lam[i] > 1e-11 * top ? (float)(V[(size_t)a * k + i] / std::sqrt(lam[i])) : 0.0f;
            const bool last = pass == 1 || low >= 1e-4 * top;
            float* out = last ? dst : Td;
            if ((r = apply(in, m, k, out)) != hipSuccess) return r;
            if (last) break;
            in = out;
        }
        return hipSuccess;
    }
};

}  // namespace

hipError_t launch_quant_error(const float* W_f, const float* s, int d_out, int d_in, int w_bits, float* E,
                              hipStream_t st) {
    hipLaunchKernelGGL(quant_error_kernel, dim3(d_out), dim3(256), 0, st, W_f, s, d_in, w_bits == 4 ? 7.0f : 3.0f, E);
    return hipGetLastError();
}

size_t channel_rms_workspace_bytes(int T, int d_in) {
    return (size_t)((T + RMS_TOK - 1) / RMS_TOK) * d_in * sizeof(double);
}

hipError_t launch_channel_rms(const void* x, int x_dtype, int T, int d_in, float* c, void* ws, hipStream_t st) {
    const int nb = (T + RMS_TOK - 1) / RMS_TOK;
    double* part = static_cast<double*>(ws);
    hipLaunchKernelGGL(channel_sumsq_kernel, dim3((d_in + 255) / 256, nb), dim3(256), 0, st, x, x_dtype, T, d_in,
                       part);
    hipLaunchKernelGGL(channel_rms_finish_kernel, dim3((d_in + 255) / 256), dim3(256), 0, st, part, nb, T, d_in, c);
    return hipGetLastError();
}

hipError_t launch_sub_lowrank(float* E, int d_out, int d_in, const float* A, const float* B, int r, hipStream_t st) {
    hipLaunchKernelGGL(sub_lowrank_kernel, dim3((d_in + 63) / 64, (d_out + 63) / 64), dim3(256), 0, st, E, d_out,
                       d_in, A, B, r);
    return hipGetLastError();
}

// device workspace (float32 unless noted): Y, Q [d_in][k]; Z, Q~ [d_out][k]; T [max(d_in,
// d_out)][k]; G [k][k] double; S [k][k]
size_t lowrank_workspace_bytes(int d_out, int d_in, int k) {
    return align256((size_t)2 * d_in * k * 4) + align256((size_t)2 * d_out * k * 4) +
           align256((size_t)std::max(d_in, d_out) * k * 4) + align256((size_t)k * k * 8) + align256((size_t)k * k * 4);
}

hipError_t lowrank_fit(const float* E, int d_out, int d_in, const float* w, const float* omega, int k, int rank,
                       int power_iters, float* A, float* B, double* sigma, void* ws, hipStream_t st) {
    char* p = static_cast<char*>(ws);
    float* Yd = reinterpret_cast<float*>(p);
    float* Qd = Yd + (size_t)d_in * k;
    p += align256((size_t)2 * d_in * k * 4);
    float* Zd = reinterpret_cast<float*>(p);
    float* Qtd = Zd + (size_t)d_out * k;
    p += align256((size_t)2 * d_out * k * 4);
    float* Td = reinterpret_cast<float*>(p);
    p += align256((size_t)std::max(d_in, d_out) * k * 4);
    double* Gd = reinterpret_cast<double*>(p);
    p += align256((size_t)k * k * 8);
    float* Sd = reinterpret_cast<float*>(p);
    SmallOps so(k, st, Gd, Sd, Td);
    std::vector<double>& lam = so.lam;
    std::vector<double>& V = so.V;
    std::vector<float>& Sh = so.Sh;
    hipError_t e;
#define QE_TRY(expr)                              \
    do {                                          \
        if ((e = (expr)) != hipSuccess) return e; \
    } while (0)
    auto gram_eigen = [&](const float* X, int m) { return so.gram_eigen(X, m); };
    auto apply = [&](const float* src, int m, int cols, float* dst) { return so.apply(src, m, cols, dst); };
    auto orth = [&](const float* src, int m, float* dst) { return so.orth(src, m, dst); };
    QE_TRY(pass_over_e(true, E, d_out, d_in, omega, k, w, Yd, st));  // Y = M omega
    QE_TRY(orth(Yd, d_in, Qd));
    for (int it = 0; it < power_iters; ++it) {
        QE_TRY(pass_over_e(false, E, d_out, d_in, Qd, k, w, Zd, st));  // M^T Q
        QE_TRY(orth(Zd, d_out, Qtd));
        QE_TRY(pass_over_e(true, E, d_out, d_in, Qtd, k, w, Yd, st));  // M Q~
        QE_TRY(orth(Yd, d_in, Qd));
    }
    QE_TRY(pass_over_e(false, E, d_out, d_in, Qd, k, w, Zd, st));  // Z = M^T Q = B^T
    // B B^T = Z^T Z = U~ S^2 U~^T (ascending); U = Q U~, V = Z U~ S^-1
    QE_TRY(gram_eigen(Zd, d_out));
    std::vector<double> root(rank), inv(rank);
    for (int l = 0; l < rank; ++l) {
        const double sg = std::sqrt(std::max(lam[k - 1 - l], 0.0));
        sigma[l] = sg;
        root[l] = std::sqrt(sg);
        inv[l] = sg > 0.0 ? root[l] / sg : 0.0;
    }
    // U_r S_r^(1/2) = Q (U~ S^(1/2)) -> Yd [d_in][rank]; V_r S_r^(1/2) = Z (U~ S^(-1/2)) -> Qtd [d_out][rank]
    for (int a = 0; a < k; ++a)
        for (int l = 0; l < rank; ++l) Sh[(size_t)a * rank + l] = (float)(V[(size_t)a * k + (k - 1 - l)] * root[l]);
    QE_TRY(apply(Qd, d_in, rank, Yd));
    for (int a = 0; a < k; ++a)
        for (int l = 0; l < rank; ++l) Sh[(size_t)a * rank + l] = (float)(V[(size_t)a * k + (k - 1 - l)] * inv[l]);
    QE_TRY(apply(Zd, d_out, rank, Qtd));
    std::vector<float> us((size_t)d_in * rank), vs((size_t)d_out * rank), wv;
    QE_TRY(hipMemcpyAsync(us.data(), Yd, us.size() * 4, hipMemcpyDeviceToHost, st));
    QE_TRY(hipMemcpyAsync(vs.data(), Qtd, vs.size() * 4, hipMemcpyDeviceToHost, st));
    if (w) {
        wv.resize(d_in);
        QE_TRY(hipMemcpyAsync(wv.data(), w, (size_t)d_in * 4, hipMemcpyDeviceToHost, st));
    }
    QE_TRY(hipStreamSynchronize(st));
#undef QE_TRY
    for (int j = 0; j < d_in; ++j) {
        const float wj = w ? wv[j] : 1.0f;
        for (int l = 0; l < rank; ++l) A[(size_t)j * rank + l] = wj > 0.0f ? us[(size_t)j * rank + l] / wj : 0.0f;
    }
    for (int l = 0; l < rank; ++l)
        for (int i = 0; i < d_out; ++i) B[(size_t)l * d_out + i] = vs[(size_t)i * rank + l];
    return hipSuccess;
}

size_t build_experts_workspace_bytes(int d_out, int d_in, int k, int r_max) {
    return align256((size_t)d_out * d_in * sizeof(float)) + align256(lowrank_workspace_bytes(d_out, d_in, k)) +
           align256((size_t)d_in * sizeof(float)) + align256((size_t)d_in * r_max * sizeof(float)) +
           align256((size_t)r_max * d_out * sizeof(float));
}

// The SE on the whole quantization error (weights c), then each RE on the residual with the
// weights of its cluster's channels only.  Host outputs; synchronizes `st`.
hipError_t build_experts(const float* W_f, const float* s, int d_out, int d_in, int w_bits, const float* c,
                         const int32_t* dep, const int32_t* labels, int n_dep, int n_r, int r_s, int r_r,
                         const float* omegas, int k, int power_iters, float* A_s, float* B_s, float* A_r, float* B_r,
                         double* sigma_s, double* sigma_r, void* ws, hipStream_t st) {
    const int r_max = std::max(r_s, r_r);
    char* p = static_cast<char*>(ws);
    float* E = reinterpret_cast<float*>(p);
    p += align256((size_t)d_out * d_in * sizeof(float));
    void* lws = p;
    p += align256(lowrank_workspace_bytes(d_out, d_in, k));
    float* wd = reinterpret_cast<float*>(p);
    p += align256((size_t)d_in * sizeof(float));
    float* Ad = reinterpret_cast<float*>(p);
    p += align256((size_t)d_in * r_max * sizeof(float));
    float* Bd = reinterpret_cast<float*>(p);
    hipError_t e;
#define QE_TRY(expr)                              \
    do {                                          \
        if ((e = (expr)) != hipSuccess) return e; \
    } while (0)
    QE_TRY(launch_quant_error(W_f, s, d_out, d_in, w_bits, E, st));
    if (r_s > 0) {
        QE_TRY(lowrank_fit(E, d_out, d_in, c, omegas, k, r_s, power_iters, A_s, B_s, sigma_s, lws, st));
        QE_TRY(hipMemcpyAsync(Ad, A_s, (size_t)d_in * r_s * sizeof(float), hipMemcpyHostToDevice, st));
        QE_TRY(hipMemcpyAsync(Bd, B_s, (size_t)r_s * d_out * sizeof(float), hipMemcpyHostToDevice, st));
        QE_TRY(launch_sub_lowrank(E, d_out, d_in, Ad, Bd, r_s, st));  // E_1 = E - (A_s B_s)^T
    }
    if (n_r > 0) {
        std::vector<float> ch(d_in), wg(d_in);
        QE_TRY(hipMemcpyAsync(ch.data(), c, (size_t)d_in * sizeof(float), hipMemcpyDeviceToHost, st));
        QE_TRY(hipStreamSynchronize(st));
        for (int g = 0; g < n_r; ++g) {
            std::fill(wg.begin(), wg.end(), 0.0f);
            for (int t = 0; t < n_dep; ++t)
                if (labels[t] == g) wg[dep[t]] = ch[dep[t]];
            QE_TRY(hipMemcpyAsync(wd, wg.data(), (size_t)d_in * sizeof(float), hipMemcpyHostToDevice, st));
            QE_TRY(hipStreamSynchronize(st));  // wg is refilled for the next cluster
            QE_TRY(lowrank_fit(E, d_out, d_in, wd, omegas + (size_t)(1 + g) * d_out * k, k, r_r, power_iters,
                               A_r + (size_t)g * d_in * r_r, B_r + (size_t)g * r_r * d_out, sigma_r + (size_t)g * r_r,
                               lws, st));
        }
    }
    QE_TRY(hipStreamSynchronize(st));
#undef QE_TRY
    return hipSuccess;
}


// ---------------------------------------------------------------- covariance whitening
// The SE minimizes sum_t |(E - A_hat) x_t|^2 over the calibration tokens (PaperDaily post,
// "核心设计": the residual of the error minus the compensations, times the input token), and
// the whitening is by the covariance of the error outputs C = Z Z^T, Z = E diag(m) X^T
// (d_out x T; m a 0/1 channel mask, all ones for the SE, the cluster's channels for an RE).
// Eckart-Young on Z: A_hat = U_r U_r^T E diag(m) with U_r the top-r left singular vectors of
// Z.  They come from the randomized subspace iteration (Halko, Martinsson and Tropp,
// Algorithms 4.4 and 5.1) on the operator Z, applied through passes over E and over a float32
// copy of X, never forming Z or C:
//   Y = E diag(m) X^T omega, Q = orth(Y); power_iters times: H = orth(X diag(m) E^T Q),
//   Q = orth(E diag(m) X^T H); then P = diag(m) E^T Q, H = X P = Z^T Q, H^T H = U~ S^2 U~^T,
//   U_r = Q U~_r, A = P U~_r = diag(m) E^T U_r, B = U_r^T.
// Directions whose eigenvalue is below 1e-11 of the largest are dropped (zero columns).

// device workspace (float32 unless noted): P [d_in][k]; Y, Q [d_out][k]; H, H2 [T][k];
// T [max(d_in, d_out, T)][k]; G [k][k] double; S [k][k]
size_t lowrank_cov_workspace_bytes(int d_out, int d_in, int T, int k) {
    return align256((size_t)d_in * k * 4) + 2 * align256((size_t)d_out * k * 4) + 2 * align256((size_t)T * k * 4) +
           align256((size_t)std::max(std::max(d_in, d_out), T) * k * 4) + align256((size_t)k * k * 8) +
           align256((size_t)k * k * 4);
}

hipError_t lowrank_fit_cov(const float* E, int d_out, int d_in, const float* X, int T, const float* mask,
                           const float* omega, int k, int rank, int power_iters, float* A, float* B, double* sigma,
                           void* ws, hipStream_t st) {
    char* p = static_cast<char*>(ws);
    auto take = [&p](size_t bytes) {
        float* q = reinterpret_cast<float*>(p);
        p += align256(bytes);
        return q;
    };
    float* Pd = take((size_t)d_in * k * 4);
    float* Yd = take((size_t)d_out * k * 4);
    float* Qd = take((size_t)d_out * k * 4);
    float* Hd = take((size_t)T * k * 4);
    float* H2d = take((size_t)T * k * 4);
    float* Td = take((size_t)std::max(std::max(d_in, d_out), T) * k * 4);
    double* Gd = reinterpret_cast<double*>(take((size_t)k * k * 8));
    float* Sd = take((size_t)k * k * 4);
    SmallOps so(k, st, Gd, Sd, Td);
    hipError_t e;
#define QE_TRY(expr)                              \
    do {                                          \
        if ((e = (expr)) != hipSuccess) return e; \
    } while (0)
    QE_TRY(pass_over_e(true, X, T, d_in, omega, k, mask, Pd, st));  // P = diag(m) X^T omega
    QE_TRY(pass_over_e(false, E, d_out, d_in, Pd, k, nullptr, Yd, st));  // Y = E P
    QE_TRY(so.orth(Yd, d_out, Qd));
    for (int it = 0; it < power_iters; ++it) {
        QE_TRY(pass_over_e(true, E, d_out, d_in, Qd, k, mask, Pd, st));   // P = diag(m) E^T Q
        QE_TRY(pass_over_e(false, X, T, d_in, Pd, k, nullptr, Hd, st));   // H = X P = Z^T Q
        QE_TRY(so.orth(Hd, T, H2d));
        QE_TRY(pass_over_e(true, X, T, d_in, H2d, k, mask, Pd, st));      // P = diag(m) X^T H
        QE_TRY(pass_over_e(false, E, d_out, d_in, Pd, k, nullptr, Yd, st));  // Y = E P = Z H
        QE_TRY(so.orth(Yd, d_out, Qd));
    }
    QE_TRY(pass_over_e(true, E, d_out, d_in, Qd, k, mask, Pd, st));  // P = diag(m) E^T Q
    QE_TRY(pass_over_e(false, X, T, d_in, Pd, k, nullptr, Hd, st));  // H = Z^T Q
    QE_TRY(so.gram_eigen(Hd, T));  // Q^T Z Z^T Q = U~ S^2 U~^T (ascending)
    const double top = std::max(so.lam[k - 1], 0.0);
    for (int a = 0; a < k; ++a)
        for (int l = 0; l < rank; ++l) {
            const int c = k - 1 - l;
            so.Sh[(size_t)a * rank + l] = so.lam[c] > 1e-11 * top ? (float)so.V[(size_t)a * k + c] : 0.0f;
        }
    for (int l = 0; l < rank; ++l) {
        const double lv = so.lam[k - 1 - l];
        sigma[l] = lv > 1e-11 * top ? std::sqrt(lv) : 0.0;
    }
    QE_TRY(so.apply(Pd, d_in, rank, Td));  // A = P U~_r  [d_in][rank]
    QE_TRY(so.apply(Qd, d_out, rank, Yd));  // U_r = Q U~_r [d_out][rank]
    std::vector<float> ud((size_t)d_out * rank);
    QE_TRY(hipMemcpyAsync(A, Td, (size_t)d_in * rank * 4, hipMemcpyDeviceToHost, st));
    QE_TRY(hipMemcpyAsync(ud.data(), Yd, ud.size() * 4, hipMemcpyDeviceToHost, st));
    QE_TRY(hipStreamSynchronize(st));
#undef QE_TRY
    for (int l = 0; l < rank; ++l)
        for (int i = 0; i < d_out; ++i) B[(size_t)l * d_out + i] = ud[(size_t)i * rank + l];
    return hipSuccess;
}

size_t build_experts_cov_workspace_bytes(int d_out, int d_in, int T, int k, int r_max) {
    return align256((size_t)d_out * d_in * 4) + align256((size_t)T * d_in * 4) +
           align256(lowrank_cov_workspace_bytes(d_out, d_in, T, k)) + align256((size_t)d_in * 4) +
           align256((size_t)d_in * r_max * 4) + align256((size_t)r_max * d_out * 4);
}

// SE on the whole error, then each RE on the residual's cluster columns, both by covariance
// whitening over the calibration tokens x.  Host outputs; synchronizes `st`.
hipError_t build_experts_cov(const float* W_f, const float* s, int d_out, int d_in, int w_bits, const void* x,
                             int x_dtype, int T, const int32_t* dep, const int32_t* labels, int n_dep, int n_r,
                             int r_s, int r_r, const float* omegas, int k, int power_iters, float* A_s, float* B_s,
                             float* A_r, float* B_r, double* sigma_s, double* sigma_r, void* ws, hipStream_t st) {
    const int r_max = std::max(r_s, r_r);
    char* p = static_cast<char*>(ws);
    float* E = reinterpret_cast<float*>(p);
    p += align256((size_t)d_out * d_in * 4);
    float* Xf = reinterpret_cast<float*>(p);
    p += align256((size_t)T * d_in * 4);
    void* lws = p;
    p += align256(lowrank_cov_workspace_bytes(d_out, d_in, T, k));
    float* md = reinterpret_cast<float*>(p);
    p += align256((size_t)d_in * 4);
    float* Ad = reinterpret_cast<float*>(p);
    p += align256((size_t)d_in * r_max * 4);
    float* Bd = reinterpret_cast<float*>(p);
    hipError_t e;
#define QE_TRY(expr)                              \
    do {                                          \
        if ((e = (expr)) != hipSuccess) return e; \
    } while (0)
    const size_t nx = (size_t)T * d_in;
    hipLaunchKernelGGL(to_f32_kernel, dim3((unsigned)std::min<size_t>((nx + 255) / 256, 4096)), dim3(256), 0, st, x,
                       x_dtype, nx, Xf);
    QE_TRY(hipGetLastError());
    QE_TRY(launch_quant_error(W_f, s, d_out, d_in, w_bits, E, st));
    if (r_s > 0) {
        QE_TRY(lowrank_fit_cov(E, d_out, d_in, Xf, T, nullptr, omegas, k, r_s, power_iters, A_s, B_s, sigma_s, lws,
                               st));
        QE_TRY(hipMemcpyAsync(Ad, A_s, (size_t)d_in * r_s * 4, hipMemcpyHostToDevice, st));
        QE_TRY(hipMemcpyAsync(Bd, B_s, (size_t)r_s * d_out * 4, hipMemcpyHostToDevice, st));
        QE_TRY(launch_sub_lowrank(E, d_out, d_in, Ad, Bd, r_s, st));  // E_1 = E - (A_s B_s)^T
    }
    std::vector<float> mh(d_in);
    for (int g = 0; g < n_r; ++g) {
        std::fill(mh.begin(), mh.end(), 0.0f);
        for (int t = 0; t < n_dep; ++t)
            if (labels[t] == g) mh[dep[t]] = 1.0f;
        QE_TRY(hipMemcpyAsync(md, mh.data(), (size_t)d_in * 4, hipMemcpyHostToDevice, st));
        QE_TRY(hipStreamSynchronize(st));  // mh is refilled for the next cluster
        QE_TRY(lowrank_fit_cov(E, d_out, d_in, Xf, T, md, omegas + (size_t)(1 + g) * T * k, k, r_r, power_iters,
                               A_r + (size_t)g * d_in * r_r, B_r + (size_t)g * r_r * d_out, sigma_r + (size_t)g * r_r,
                               lws, st));
    }
    QE_TRY(hipStreamSynchronize(st));
#undef QE_TRY
    return hipSuccess;
}

// ---------------------------------------------------------------- router targets and fit
size_t router_targets_workspace_bytes(int d_out, int d_in, int n_r, int r_r) {
    return align256((size_t)d_in * RT_TOK * 4) + align256((size_t)d_out * RT_TOK * 4) +
           align256((size_t)n_r * RT_TOK * r_r * 4);
}

// target[t][g] = mean_i |x_t (E_1^T - A_g B_g)|_i for T calibration tokens, 128 at a time: one
// pass over E_1 per chunk gives x E_1^T, then the tiny products x A_g and the reduction.
hipError_t router_targets(const float* E1, int d_out, int d_in, const void* x, int x_dtype, int T, const float* A_r,
                          const float* B_r, int n_r, int r_r, float* target, void* ws, hipStream_t st) {
    char* p = static_cast<char*>(ws);
    float* XT = reinterpret_cast<float*>(p);
    p += align256((size_t)d_in * RT_TOK * 4);
    float* Zc = reinterpret_cast<float*>(p);
    p += align256((size_t)d_out * RT_TOK * 4);
    float* U = reinterpret_cast<float*>(p);
    hipError_t e;
    for (int t0 = 0; t0 < T; t0 += RT_TOK) {
        const int kc = std::min(RT_TOK, T - t0);
        hipLaunchKernelGGL(transpose_chunk_kernel, dim3((d_in + 31) / 32, (kc + 31) / 32), dim3(256), 0, st, x,
                           x_dtype, t0, kc, d_in, XT);
        if ((e = pass_over_e(false, E1, d_out, d_in, XT, kc, nullptr, Zc, st)) != hipSuccess) return e;  // Z = E_1 X^T
        for (int g = 0; g < n_r; ++g)  // U_g = X A_g  ([kc][r_r]; XT as a [d_in][kc] matrix)
            if ((e = pass_over_e(true, XT, d_in, kc, A_r + (size_t)g * d_in * r_r, r_r, nullptr,
                                 U + (size_t)g * kc * r_r, st)) != hipSuccess)
                return e;
        hipLaunchKernelGGL(router_target_kernel, dim3(kc, n_r), dim3(256), 0, st, Zc, kc, d_out, B_r, r_r, U, t0, n_r,
                           target);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

size_t router_fit_workspace_bytes(int T, int d_in, int n_r) {
    return align256((size_t)T * d_in * 4) + 5 * align256((size_t)d_in * n_r * 4) + align256((size_t)T * n_r * 4) +
           align256(((size_t)n_r + 1) * 8);
}

// Ridge least squares (X^T X + lam I) R = X^T target, lam = ridge * |X|_F^2 / d_in, by conjugate
// gradients on the normal equations, one independent system per column; the products with X
// are the passes over a float32 copy of X.  Stops when every column's residual is below
// tol times its right-hand side, or after max_iters.  R: host [d_in][n_r].
hipError_t router_fit(const void* x, int x_dtype, int T, int d_in, const float* target, int n_r, double ridge,
                      int max_iters, double tol, float* R, int* iters_done, void* ws, hipStream_t st) {
    char* p = static_cast<char*>(ws);
    float* Xf = reinterpret_cast<float*>(p);
    p += align256((size_t)T * d_in * 4);
    float* vec[5];
    for (int v = 0; v < 5; ++v) {
        vec[v] = reinterpret_cast<float*>(p);
        p += align256((size_t)d_in * n_r * 4);
    }
    float *Rd = vec[0], *rd = vec[1], *pd = vec[2], *qd = vec[3], *bd = vec[4];
    float* Xp = reinterpret_cast<float*>(p);
    p += align256((size_t)T * n_r * 4);
    double* dd = reinterpret_cast<double*>(p);  // [n_r] dots, then one sum of squares
    const size_t nv = (size_t)d_in * n_r;
    const unsigned gv = (unsigned)std::min<size_t>((nv + 255) / 256, 1024);
    std::vector<double> rr(n_r), rr_new(n_r), bb(n_r), pq(n_r), coef(n_r);
    hipError_t e;
#define QE_TRY(expr)                              \
    do {                                          \
        if ((e = (expr)) != hipSuccess) return e; \
    } while (0)
    auto dots = [&](const float* a, const float* b, std::vector<double>& out) -> hipError_t {
        hipLaunchKernelGGL(coldot_kernel, dim3(n_r), dim3(256), 0, st, a, b, d_in, n_r, dd);
        hipError_t r;
        if ((r = hipMemcpyAsync(out.data(), dd, (size_t)n_r * 8, hipMemcpyDeviceToHost, st)) != hipSuccess) return r;
        return hipStreamSynchronize(st);
    };
    auto upload_coef = [&]() -> hipError_t {
        hipError_t r;
        if ((r = hipMemcpyAsync(dd, coef.data(), (size_t)n_r * 8, hipMemcpyHostToDevice, st)) != hipSuccess) return r;
        return hipStreamSynchronize(st);  // coef is refilled by the next step
    };
    const size_t nx = (size_t)T * d_in;
    hipLaunchKernelGGL(to_f32_kernel, dim3((unsigned)std::min<size_t>((nx + 255) / 256, 4096)), dim3(256), 0, st, x,
                       x_dtype, nx, Xf);
    hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(256), 0, st, reinterpret_cast<float*>(dd + n_r), (size_t)2);
    hipLaunchKernelGGL(sumsq_kernel, dim3(1024), dim3(256), 0, st, Xf, nx, dd + n_r);
    double fro = 0.0;
    QE_TRY(hipMemcpyAsync(&fro, dd + n_r, 8, hipMemcpyDeviceToHost, st));
    QE_TRY(hipStreamSynchronize(st));
    const double lam = ridge * fro / d_in;
    QE_TRY(pass_over_e(true, Xf, T, d_in, target, n_r, nullptr, bd, st));  // b = X^T target
    hipLaunchKernelGGL(zero_kernel, dim3(gv), dim3(256), 0, st, Rd, nv);
    QE_TRY(hipMemcpyAsync(rd, bd, nv * 4, hipMemcpyDeviceToDevice, st));
    QE_TRY(hipMemcpyAsync(pd, bd, nv * 4, hipMemcpyDeviceToDevice, st));
    QE_TRY(dots(bd, bd, bb));
    rr = bb;
    int it = 0;
    for (; it < max_iters; ++it) {
        bool done = true;
        for (int g = 0; g < n_r; ++g) done = done && rr[g] <= tol * tol * bb[g];
        if (done) break;
        QE_TRY(pass_over_e(false, Xf, T, d_in, pd, n_r, nullptr, Xp, st));  // X p
        QE_TRY(pass_over_e(true, Xf, T, d_in, Xp, n_r, nullptr, qd, st));   // X^T X p
        hipLaunchKernelGGL(cg_update_kernel, dim3(gv), dim3(256), 0, st, 0, d_in, n_r, lam, dd, Rd, rd, pd, qd);
        QE_TRY(dots(pd, qd, pq));
        for (int g = 0; g < n_r; ++g) coef[g] = pq[g] > 0.0 ? rr[g] / pq[g] : 0.0;  // alpha
        QE_TRY(upload_coef());
        hipLaunchKernelGGL(cg_update_kernel, dim3(gv), dim3(256), 0, st, 1, d_in, n_r, lam, dd, Rd, rd, pd, qd);
        QE_TRY(dots(rd, rd, rr_new));
        for (int g = 0; g < n_r; ++g) coef[g] = rr[g] > 0.0 ? rr_new[g] / rr[g] : 0.0;  // beta
        QE_TRY(upload_coef());
        hipLaunchKernelGGL(cg_update_kernel, dim3(gv), dim3(256), 0, st, 2, d_in, n_r, lam, dd, Rd, rd, pd, qd);
        rr = rr_new;
    }
    if (iters_done) *iters_done = it;
    QE_TRY(hipMemcpyAsync(R, Rd, nv * 4, hipMemcpyDeviceToHost, st));
    QE_TRY(hipStreamSynchronize(st));
#undef QE_TRY
    return hipGetLastError();
}

}  // namespace qe
