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
// matrix, twice (the two-pass scheme of CholeskyQR2, Fukaya et al. 2014, with the eigenvalue
// decomposition in place of the Cholesky factor): X = Y V diag(lambda)^(-1/2), directions whose
// eigenvalue is below 1e-11 of the largest dropped as null (they give zero columns), then the
// same on X, which restores orthogonality to working precision.

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
    std::vector<double> Gh((size_t)k * k), lam, V;
    std::vector<float> Sh((size_t)k * k);
    hipError_t e;
#define QE_TRY(expr)                              \
    do {                                          \
        if ((e = (expr)) != hipSuccess) return e; \
    } while (0)
    // Gram matrix of a device [m][kk] matrix -> host eigen-decomposition
    auto gram_eigen = [&](const float* X, int m) -> hipError_t {
        hipError_t r;
        if ((r = gram(X, m, k, Gd, st)) != hipSuccess) return r;
        if ((r = hipMemcpyAsync(Gh.data(), Gd, (size_t)k * k * 8, hipMemcpyDeviceToHost, st)) != hipSuccess) return r;
        if ((r = hipStreamSynchronize(st)) != hipSuccess) return r;
        return host_eigen(Gh, k, lam, V) ? hipSuccess : hipErrorNotSupported;
    };
    // dst = src S with the k x k matrix S on the device (dst may not alias src)
    auto apply = [&](const float* src, int m, int cols, float* dst) -> hipError_t {
        hipError_t r;
        if ((r = hipMemcpyAsync(Sd, Sh.data(), (size_t)k * cols * 4, hipMemcpyHostToDevice, st)) != hipSuccess) return r;
        if ((r = thin(false, src, m, k, Sd, cols, nullptr, dst, st)) != hipSuccess) return r;
        return hipStreamSynchronize(st);  // Sh is refilled by the next step
    };
    // orthonormal basis of the columns of src [m][k], written to dst (may alias src)
    auto orth = [&](const float* src, int m, float* dst) -> hipError_t {
        hipError_t r;
        const float* in = src;
        for (int pass = 0; pass < 2; ++pass) {
            if ((r = gram_eigen(in, m)) != hipSuccess) return r;
            const double top = std::max(lam[k - 1], 0.0);
            for (int a = 0; a < k; ++a)
                for (int i = 0; i < k; ++i)
                    Sh[(size_t)a * k + i] = lam[i] > 1e-11 * top ? (float)(V[(size_t)a * k + i] / std::sqrt(lam[i])) : 0.0f;
            float* out = pass == 0 ? Td : dst;
            if ((r = apply(in, m, k, out)) != hipSuccess) return r;
            in = out;
        }
        return hipSuccess;
    };
    QE_TRY(thin(true, E, d_out, d_in, omega, k, w, Yd, st));  // Y = M omega
    QE_TRY(orth(Yd, d_in, Qd));
    for (int it = 0; it < power_iters; ++it) {
        QE_TRY(thin(false, E, d_out, d_in, Qd, k, w, Zd, st));  // M^T Q
        QE_TRY(orth(Zd, d_out, Qtd));
        QE_TRY(thin(true, E, d_out, d_in, Qtd, k, w, Yd, st));  // M Q~
        QE_TRY(orth(Yd, d_in, Qd));
    }
    QE_TRY(thin(false, E, d_out, d_in, Qd, k, w, Zd, st));  // Z = M^T Q = B^T
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

}  // namespace qe
